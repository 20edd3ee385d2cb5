"""Seeded randomized GPU parity sweep: small workloads drawn at random, each
run in lockstep with the oracle and compared bit for bit (slot maps,
counters, LRU state, eviction logs, slot bytes).

The draws cover every items-per-thread shape of the resolve kernel (the
cache size C picks it: 1, 2, 3, 4, 6, 8, 12 and 16 items per thread, with
and without the early host reads of the fused copy), every structure of the
five workloads (one request, a resident window, growth by appends -- fused
into the resolve call in even cases, a separate launch in odd ones -- shared
selections, 18 KiB page rows), both miss-fetch paths, the copy-free and
duplicate-checking flags, and several query tokens per request."""
import numpy as np
import pytest

from workload import WORKLOADS

N_CASES = 120
# C for each items-per-thread shape: max(k, C) <= 1024 x items
C_FOR_IPT = {1: 700, 2: 1500, 3: 2500, 4: 3900, 6: 5000, 8: 7000, 12: 10000, 16: 15000}


def draw_case(i):
    """Case i of the sweep: (base workload id, overrides, queries, flags
    names, fetch mode).  Pure function of i."""
    rng = np.random.default_rng(7000 + i)
    ipt = list(C_FOR_IPT)[i % len(C_FOR_IPT)]
    base = [1, 2, 3, 4, 5][int(rng.integers(0, 5))]
    pages = base == 5
    C = C_FOR_IPT[ipt] if not pages else int(rng.integers(40, 1500))
    queries = int(rng.choice([1, 1, 2, 3])) if C <= 5000 else 1
    k_max = min(C, 4096 if queries == 1 else 2048)
    k = int(rng.integers(1, k_max + 1))
    if rng.random() < 0.2:
        k = k_max                                    # rows as wide as allowed
    k -= k % queries
    k = max(k, queries)
    R = int(rng.choice([0, 1, 7, 64])) if base != 1 else 0
    B = int(rng.integers(1, 4))
    layers = int(rng.integers(1, 3)) if base in (3, 4, 5) else 1
    per_query = k // queries
    # enough positions that the cache turns over, few enough for a quick oracle;
    # new positions avoid the whole previous row, and the Zipf-over-distance
    # workloads need more room still to draw them
    lo = 2 * per_query + R + 8 if base not in (2, 4) else 4 * per_query + R + 64
    L0 = int(rng.integers(lo, max(lo + 1, (3 if pages else 4) * C)))
    if pages:
        L0 = min(L0, 6000)
    steps = int(rng.integers(3, 7))
    carry = int(rng.integers(0, 96))
    flags = str(rng.choice(["none", "none", "no_io", "debug"])) if queries == 1 else \
        str(rng.choice(["none", "no_io"]))
    mode = str(rng.choice(["auto", "fused", "split"]))
    kw = dict(B=B, layers=layers, L0=L0, C=C, R=R, k=k, steps=steps, carry_pct=carry)
    return base, kw, queries, flags, mode


def test_sweep_draws_cover_every_shape():
    """Every items-per-thread shape, every base workload and every option is
    drawn at least once (a CPU-side property of the draws)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert {b for b, *_ in cases} == {1, 2, 3, 4, 5}
    assert {q for _, _, q, _, _ in cases} >= {1, 2}
    assert {f for *_, f, _ in cases} == {"none", "no_io", "debug"}
    assert {m for *_, m in cases} == {"auto", "fused", "split"}
    token_c = {kw["C"] for b, kw, *_ in cases if b != 5}
    assert set(C_FOR_IPT.values()) <= token_c


def test_sweep_traces_generate():
    """Every drawn case's selection trace can be generated on the host (the
    context leaves the generator enough free positions)."""
    from tests.harness import make_trace
    for i in range(N_CASES):
        base, kw, queries, _, _ = draw_case(i)
        cfg = WORKLOADS[base].scaled(**kw)
        tr = make_trace(cfg, queries=queries)
        assert tr.shape == (cfg.steps, cfg.layers, cfg.B, cfg.k), i


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_parity(i, monkeypatch):
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    base, kw, queries, flags, mode = draw_case(i)
    if mode != "auto":
        monkeypatch.setenv("HISPARSE_FETCH_MODE", mode)
    fl = {"none": 0, "no_io": hb.HISPARSE_NO_IO, "debug": hb.HISPARSE_DEBUG_VALIDATE}[flags]
    cfg = WORKLOADS[base].scaled(**kw)
    print(f"[sweep {i}] base={base} {kw} queries={queries} flags={flags} mode={mode}", flush=True)
    run = LockstepRun(cfg, flags=fl, queries=queries)
    try:
        for s in range(cfg.steps):
            if s > 0 and cfg.growth and i % 2 == 0:
                run.append_and_step(s)         # append fused into the resolve call
            else:
                if s > 0 and cfg.growth:
                    run.append_rows(s)         # separate append launch
                run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s), full_state=(s == cfg.steps - 1),
                             contents=(s == cfg.steps - 1))
        assert run.gpu.status() == 0
    finally:
        run.close()
