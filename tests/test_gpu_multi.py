"""GPU parity of the multi-query step (several query tokens per request
resolved in one pass, hisparse_resolve_multi) against the oracle's
resolve_multi, element by element and bit-exact: slot maps, counters, LRU
state, eviction logs and slot bytes; plus the hand-derived example, graph
replay, rejection of bad rows and the call's own argument checks."""
import numpy as np
import pytest

from tests import pins
from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def _run(cfg, queries, flags=0, oracle_streams=None):
    import torch
    from tests.gpu_harness import LockstepRun
    print(f"[multi] Q={queries} B={cfg.B} L={cfg.layers} L0={cfg.L0} C={cfg.C} R={cfg.R} "
          f"k={cfg.k} steps={cfg.steps} flags={flags}", flush=True)
    run = LockstepRun(cfg, oracle_streams=oracle_streams, flags=flags, queries=queries)
    try:
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.append_rows(s)
            run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


CASES = {
    # name: (base config, queries, overrides); k = queries x per-query count
    "two_tokens_window": (2, 2, dict(B=3, L0=8192, C=1500, k=1200, steps=8)),
    "three_tokens_ragged": (1, 3, dict(L0=5000, C=1000, k=699, steps=8)),
    "four_tokens_growth_layers": (3, 4, dict(B=2, layers=2, L0=6000, C=2500, R=37, k=1000,
                                             steps=6)),
    "two_tokens_shared_layers": (4, 2, dict(B=2, layers=2, L0=20000, k=2048, steps=5)),
    "two_tokens_pages": (5, 2, dict(B=2, layers=2, L0=3000, k=128, steps=8)),
    "tiny_cache_many_tokens": (2, 8, dict(B=2, L0=600, C=64, R=3, k=64, steps=12)),
    # 12 entries per thread, 12000 slots and a 8192-cell deduplication table
    "largest_shape_two_tokens": (1, 2, dict(L0=60000, C=12000, k=3000, steps=4)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_multi_parity(name):
    base, q, kw = CASES[name]
    _run(WORKLOADS[base].scaled(**kw), q)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_multi_parity_fetch_modes(mode, monkeypatch):
    monkeypatch.setenv("HISPARSE_FETCH_MODE", mode)
    base, q, kw = CASES["four_tokens_growth_layers"]
    _run(WORKLOADS[base].scaled(**kw), q)


def test_multi_parity_debug_validate():
    """Repeated positions are the point of a multi-query row: with the debug
    flag set they must not be reported as duplicates, and parity holds."""
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    base, q, kw = CASES["two_tokens_window"]
    _run(WORKLOADS[base].scaled(**kw), q, flags=hb.HISPARSE_DEBUG_VALIDATE)


def test_multi_parity_no_io():
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    base, q, kw = CASES["two_tokens_window"]
    _run(WORKLOADS[base].scaled(**kw), q, flags=hb.HISPARSE_NO_IO)


def test_multi_full_size_two_tokens():
    """Two query tokens of 2048 selections each on the 16-request, 6144-slot
    shape of the independent-layers workload (two layers, sampled streams):
    the 4096-entry rows use the largest deduplication table."""
    cfg = WORKLOADS[3].scaled(layers=2, k=4096, steps=4)
    _run(cfg, 2, oracle_streams=[(0, 0), (7, 1), (15, 0)])


def test_multi_hand_example_on_gpu():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import GpuInstance
    from workload.configs import Workload
    spec, events = pins.parse_golden("multi_query_example.txt")
    Q, kq = len(events[0][1]["sel"]), len(events[0][1]["sel"][0])
    cfg = Workload(name="hand_multi", B=1, layers=1, L0=spec["L"], growth=0, row_elems=8,
                   C=spec["C"], R=spec["R"], k=Q * kq, steps=len(events), carry_pct=0,
                   replacement="uniform")
    g = GpuInstance(cfg)
    try:
        host = g.host(0, 0)
        for p in range(spec["L"]):
            host[p] = (p * 5 + 3 * np.arange(cfg.row_bytes)) % 239
        ctx0 = torch.tensor([events[0][1]["ctx"][0]], dtype=torch.int32, device="cuda")
        hb.hisparse_load_window(g.h, g.stream, 0, ctx0.data_ptr())
        out = torch.empty((1, Q, kq), dtype=torch.int32, device="cuda")
        for _, ev in events:
            sel = torch.tensor([ev["sel"]], dtype=torch.int32, device="cuda")
            ctx = torch.tensor(ev["ctx"], dtype=torch.int32, device="cuda")
            hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), Q, kq, ctx.data_ptr(), 0,
                                      out.data_ptr())
            torch.cuda.synchronize()
            where = f"call at t={ev['mstep'][0]}"
            assert out.cpu().numpy()[0].tolist() == ev["out"], where
            st = g.state(0, 0)
            hdr = st["hdr"]
            assert hdr[hb.HDR_T] == ev["mstep"][0], where
            assert hdr[hb.HDR_STATUS] == ev["status"][0], where
            if ev["status"][0] == 0:
                got = [int(hdr[i]) for i in (hb.HDR_PAD, hb.HDR_RES, hb.HDR_HIT, hb.HDR_MISS,
                                             hb.HDR_EVICT)]
                assert got == ev["counts"], where
                m = len(ev["log"])
                assert [tuple(x) for x in st["evict"][:m].tolist()] == ev["log"], where
            assert st["slot2pos"].tolist() == ev["slot2pos"], where
            assert st["last_use"].tolist() == ev["last_use"], where
            dev = g.slots(0, 0)
            if ev["status"][0] == 0:
                for q, row in enumerate(ev["sel"]):
                    for i, p in enumerate(row):
                        if p >= 0:
                            assert (dev[ev["out"][q][i]] == host[p]).all(), where
        assert g.status(clear=True) == hb.HISPARSE_STATUS_SEL_RANGE
    finally:
        g.close()


def test_multi_graph_replay_equals_eager():
    """A captured multi-query step replayed with new selections each step
    equals an eager instance and the oracle, bit for bit."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=3, L0=8192, C=1500, k=1200, steps=6)
    Q = 3
    run = LockstepRun(cfg, queries=Q)
    try:
        sel_buf = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda")
        ctx_buf = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                hb.hisparse_resolve_multi(run.gpu.h, torch.cuda.current_stream().cuda_stream,
                                          sel_buf.data_ptr(), Q, cfg.k // Q, ctx_buf.data_ptr(),
                                          0, run.out_dev[0].data_ptr())
        torch.cuda.synchronize()
        for s in range(cfg.steps):
            sel_buf.copy_(run.sel_dev[s, 0])
            ctx_buf.copy_(run.ctx_dev[s])
            run.out_dev.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_multi_rejects_bad_rows_per_request():
    """A row with an entry out of range is rejected (-1 everywhere, stream
    untouched, clock kept); the other requests are resolved as the oracle
    resolves them."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=3, L0=6000, C=800, k=400, steps=2)
    Q = 2
    run = LockstepRun(cfg, queries=Q)
    try:
        run.gpu_step(0)
        torch.cuda.synchronize()
        run.compare_step(0, run.oracle_step(0))
        snap = run.gpu.state(1, 0)
        trace = run.trace.copy()
        trace[1, 0, 1, 250] = cfg.ctx_at(1)          # request 1, query 1: out of range
        run.trace = trace
        run.sel_dev = torch.from_numpy(trace).cuda()
        run.gpu_step(1)
        torch.cuda.synchronize()
        res = run.oracle_step(1)
        assert res[(1, 0)].status == hb.HISPARSE_STATUS_SEL_RANGE
        assert (run.out_dev[0, 1] == -1).all()
        st1 = run.gpu.state(1, 0)
        for key in ("slot2pos", "last_use", "order", "pos2slot"):
            np.testing.assert_array_equal(st1[key], snap[key])
        assert st1["hdr"][hb.HDR_T] == snap["hdr"][hb.HDR_T]
        assert st1["hdr"][hb.HDR_STATUS] == hb.HISPARSE_STATUS_SEL_RANGE
        del res[(1, 0)]
        run.compare_step(1, res)
        assert run.gpu.status(clear=True) == hb.HISPARSE_STATUS_SEL_RANGE
    finally:
        run.close()


def test_multi_argument_checks():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import GpuInstance
    cfg = WORKLOADS[4].scaled(B=2, layers=2, L0=5000, C=512, R=8, k=256, steps=1)
    g = GpuInstance(cfg)
    try:
        sel = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device="cuda")
        out = torch.empty_like(sel)
        for q, kq in ((0, 16), (2, 0), (3, 100), (257, 1)):
            with pytest.raises(hb.HisparseError) as e:
                hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), q, kq, ctx.data_ptr(),
                                          0, out.data_ptr())
            assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
        with pytest.raises(hb.HisparseError):
            hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), 2, 128, ctx.data_ptr(),
                                      2, out.data_ptr())
        # a pending prefetch of the layer must be joined by hisparse_resolve first
        side = torch.cuda.Stream()
        hb.hisparse_prefetch(g.h, g.stream, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1)
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), 2, 128, ctx.data_ptr(), 1,
                                      out.data_ptr())
        assert e.value.code == hb.HISPARSE_ERR_STATE
        hb.hisparse_resolve(g.h, g.stream, sel.data_ptr(), ctx.data_ptr(), 1, out.data_ptr())
        # all padding: nothing happens except the clock
        hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), 4, 64, ctx.data_ptr(), 0,
                                  out.data_ptr())
        torch.cuda.synchronize()
        assert (out == -1).all()
        hdr = g.hdr(0, 0)
        assert hdr[hb.HDR_T] == 1 and hdr[hb.HDR_PAD] == cfg.k and hdr[hb.HDR_MISS] == 0
        assert g.status() == 0
    finally:
        g.close()
