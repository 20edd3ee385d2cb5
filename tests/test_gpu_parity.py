"""GPU parity: libhisparse (HIP, through the C ABI) against the CPU oracle,
element by element, bit-exact, on reduced workloads that span several tiles
and ragged tails, and on the edge cases of the method."""
import numpy as np
import pytest

from tests import pins
from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def _run_lockstep(cfg, flags=0, oracle_streams=None):
    from tests.gpu_harness import LockstepRun
    import torch
    run = LockstepRun(cfg, oracle_streams=oracle_streams, flags=flags)
    try:
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.append_rows(s)
            run.gpu_step(s)
            torch.cuda.synchronize()
            res = run.oracle_step(s)
            run.compare_step(s, res)
        assert run.gpu.status() == 0
    finally:
        run.close()


CASES = {
    # name: (base config, overrides)
    "one_request_ragged": (1, dict(L0=4096, C=700, k=300, steps=10)),
    "mix_window_two_rounds": (2, dict(B=3, L0=8192, C=1500, k=700, steps=12)),
    "independent_layers_growth": (3, dict(B=2, layers=3, L0=6000, C=2500, R=37, k=1000, steps=8)),
    "shared_layers_full_stream_shape": (4, dict(B=2, layers=2, L0=20000, steps=6)),
    "pages": (5, dict(B=2, layers=2, L0=3000, steps=10)),
    "cache_equals_k": (1, dict(L0=5000, C=256, k=256, steps=8, carry_pct=0)),
    "k_one": (2, dict(B=2, L0=500, C=4, R=3, k=1, steps=20, carry_pct=0)),
    "largest_supported_shape": (1, dict(L0=60000, C=12000, k=3000, steps=4)),
    "window_covers_context": (3, dict(B=2, layers=1, L0=40, C=64, R=64, k=32, steps=12)),
    # ten requests: a forced split fetch takes the flat fan-out kernel (below eight
    # streams per call the grid is sliced per stream instead)
    "many_requests": (2, dict(B=10, L0=8192, C=1500, k=700, steps=6)),
    # the context grows past the window (58 .. 69 rows, R = 64): the first steps are all
    # resident, then the oldest positions leave the window and are fetched when selected
    "window_boundary_crossing": (3, dict(B=2, layers=1, L0=58, C=64, R=64, k=24, steps=12)),
    # the largest cache and selection the library accepts (C = 16384, k = 4096)
    "maximum_cache_and_k": (1, dict(L0=70000, C=16384, k=4096, steps=4)),
    # more streams per call than the GPU has CUs: the resolve grid runs in several rounds
    "more_requests_than_cus": (2, dict(B=300, L0=2000, C=96, R=8, k=48, steps=4)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_parity_reduced(name):
    base, kw = CASES[name]
    _parity_case(name, base, kw)


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("name", ["one_request_ragged", "independent_layers_growth", "pages",
                                  "largest_supported_shape", "many_requests",
                                  "maximum_cache_and_k", "more_requests_than_cus"])
def test_parity_fetch_modes(name, mode, monkeypatch):
    """Both miss-fetch paths (copies by the resolve workgroups themselves, or
    by a separate fan-out kernel: sliced per stream below eight streams per
    call, flat above) on the same cases."""
    monkeypatch.setenv("HISPARSE_FETCH_MODE", mode)
    base, kw = CASES[name]
    _parity_case(name, base, kw)


def _parity_case(name, base, kw):
    cfg = WORKLOADS[base].scaled(**kw)
    print(f"[parity] {name}: B={cfg.B} L={cfg.layers} L0={cfg.L0} C={cfg.C} R={cfg.R} "
          f"k={cfg.k} steps={cfg.steps}", flush=True)
    _run_lockstep(cfg)


APPEND_CASES = {
    # growing contexts: (base, overrides); R = 0 takes the two-launch path
    "window_37": (3, dict(B=2, layers=3, L0=6000, C=2500, R=37, k=1000, steps=8)),
    "window_1": (3, dict(B=3, layers=2, L0=3000, C=900, R=1, k=400, steps=10)),
    "window_covers_context": (3, dict(B=2, layers=1, L0=40, C=64, R=64, k=32, steps=12)),
    "no_window": (3, dict(B=2, layers=2, L0=3000, C=900, R=0, k=400, steps=10)),
    "pages_window": (5, dict(B=2, layers=2, L0=3000, R=3, growth=1, steps=8)),
}


@pytest.mark.parametrize("name,queries", [("window_37", 2), ("window_1", 3), ("no_window", 2),
                                          ("pages_window", 2)])
def test_append_resolve_multi_parity(name, queries):
    """hisparse_append_resolve_multi equals the oracle's append followed by
    its multi-query step."""
    import torch
    from tests.gpu_harness import LockstepRun
    base, kw = APPEND_CASES[name]
    cfg = WORKLOADS[base].scaled(**kw)
    cfg = cfg.scaled(k=(cfg.k // queries) * queries)
    print(f"[append_resolve_multi] {name} Q={queries}: k={cfg.k}", flush=True)
    run = LockstepRun(cfg, queries=queries)
    try:
        for s in range(cfg.steps):
            if s > 0:
                run.append_and_step(s)
            else:
                run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


@pytest.mark.parametrize("flags", ["none", "no_io"])
@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("name", sorted(APPEND_CASES))
def test_append_resolve_parity(name, mode, flags, monkeypatch):
    """hisparse_append_resolve (one launch with a window, two without) equals
    the oracle's append followed by its step, state and slot bytes."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    monkeypatch.setenv("HISPARSE_FETCH_MODE", mode)
    base, kw = APPEND_CASES[name]
    cfg = WORKLOADS[base].scaled(**kw)
    fl = hb.HISPARSE_NO_IO if flags == "no_io" else 0
    print(f"[append_resolve] {name} {mode} {flags}: B={cfg.B} L={cfg.layers} L0={cfg.L0} "
          f"C={cfg.C} R={cfg.R} k={cfg.k} steps={cfg.steps}", flush=True)
    run = LockstepRun(cfg, flags=fl)
    try:
        for s in range(cfg.steps):
            if s > 0:
                run.append_and_step(s)
            else:
                run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


@pytest.mark.parametrize("name", ["mix_window_two_rounds", "pages"])
def test_parity_reduced_no_io(name):
    base, kw = CASES[name]
    cfg = WORKLOADS[base].scaled(**kw)
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    _run_lockstep(cfg, flags=hb.HISPARSE_NO_IO)


@pytest.mark.parametrize("golden", ["lru_hand_example.txt", "resident_window_example.txt"])
def test_hand_examples_on_gpu(golden):
    """The hand-derived examples reproduced by the GPU path itself."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import GpuInstance
    from workload.configs import Workload
    spec, events = pins.parse_golden(golden)
    steps = [ev for kind, ev in events if kind == "step"]
    k = len(steps[0]["sel"])
    cfg = Workload(name="hand", B=1, layers=1, L0=spec["L"], growth=0, row_elems=8,
                   C=spec["C"], R=spec["R"], k=k, steps=len(steps), carry_pct=0,
                   replacement="uniform")
    g = GpuInstance(cfg)
    try:
        host = g.host(0, 0)
        for p in range(spec["L"]):
            host[p] = (p * 7 + np.arange(cfg.row_bytes)) % 251
        ctx0 = torch.tensor([steps[0]["ctx"][0]], dtype=torch.int32, device="cuda")
        hb.hisparse_load_window(g.h, g.stream, 0, ctx0.data_ptr())
        out = torch.empty((1, k), dtype=torch.int32, device="cuda")
        for kind, ev in events:
            if kind == "append":
                row = ((ev * 13 + np.arange(cfg.row_bytes)) % 241).astype(np.uint8)
                rows = torch.from_numpy(row[None]).cuda()
                pos = torch.tensor([ev], dtype=torch.int32, device="cuda")
                hb.hisparse_append(g.h, g.stream, 0, rows.data_ptr(), pos.data_ptr())
                continue
            sel = torch.tensor([ev["sel"]], dtype=torch.int32, device="cuda")
            ctx = torch.tensor(ev["ctx"], dtype=torch.int32, device="cuda")
            hb.hisparse_resolve(g.h, g.stream, sel.data_ptr(), ctx.data_ptr(), 0, out.data_ptr())
            torch.cuda.synchronize()
            st = g.state(0, 0)
            assert out.cpu().numpy()[0].tolist() == ev["out"]
            m = len(ev["log"])
            assert [tuple(x) for x in st["evict"][:m].tolist()] == ev["log"]
            assert st["slot2pos"].tolist() == ev["slot2pos"]
            assert st["last_use"].tolist() == ev["last_use"]
            dev = g.slots(0, 0)
            for i, p in enumerate(ev["sel"]):
                if p >= 0:
                    assert (dev[ev["out"][i]] == host[p]).all()
        assert g.status() == 0
    finally:
        g.close()


def test_long_run_many_cache_turnovers():
    """400 steps on small caches (the LRU order, stamps and the position map
    turn over dozens of times), compared with the oracle every step; full
    state and slot bytes every 50 steps."""
    import torch
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=2, L0=20000, C=1200, R=16, k=600, steps=400, carry_pct=60)
    print(f"[long run] {cfg.steps} steps, C={cfg.C}, k={cfg.k}", flush=True)
    run = LockstepRun(cfg)
    try:
        for s in range(cfg.steps):
            run.gpu_step(s)
            torch.cuda.synchronize()
            full = s % 50 == 49
            run.compare_step(s, run.oracle_step(s), full_state=full, contents=full)
            if full:
                print(f"[long run] step {s + 1} matches", flush=True)
        assert run.gpu.status() == 0
        hdr = run.gpu.hdr(0, 0)
        assert int(hdr[0]) == cfg.steps
    finally:
        run.close()


# One (k, C) per instantiation of the resolve kernel: (selection items, order
# items) per thread, from the smallest cache that yields the pair (the largest
# k there), so both sides run their full item counts.
KERNEL_SHAPES = {
    (1, 1): (1, 1), (1, 2): (576, 1025), (1, 3): (704, 2049), (1, 4): (832, 3073),
    (1, 6): (704, 4097), (1, 8): (832, 6145), (1, 12): (704, 8193), (1, 16): (832, 12289),
    (2, 2): (1025, 1025), (2, 3): (1408, 2049), (2, 4): (1664, 3073), (2, 6): (1408, 4097),
    (2, 8): (1664, 6145), (2, 12): (1408, 8193), (2, 16): (1664, 12289), (3, 3): (2049, 2049),
    (4, 4): (3073, 3073), (4, 6): (2816, 4097), (4, 8): (3328, 6145), (4, 12): (2816, 8193),
    (4, 16): (3328, 12289), (6, 6): (4096, 4097), (8, 8): (4096, 6145), (12, 12): (4096, 8193),
    (16, 16): (4096, 12289),
}


@pytest.mark.parametrize("pair", sorted(KERNEL_SHAPES), ids=lambda p: f"sel{p[0]}_ord{p[1]}")
def test_every_resolve_kernel_instantiation(pair):
    """Every (selection, LRU-order) items-per-thread instantiation of the
    resolve kernel, against the oracle for three steps (one request, half
    the selections carried over, so later steps hit, miss and evict)."""
    k, C = KERNEL_SHAPES[pair]
    cfg = WORKLOADS[1].scaled(L0=2 * C + 1000, C=C, k=k, steps=3, carry_pct=50)
    print(f"[shape] items {pair}: k={k} C={C}", flush=True)
    _run_lockstep(cfg)
