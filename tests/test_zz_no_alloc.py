"""The attention entry point that allocates nothing
(hisparse_sparse_mla_decode_noalloc), through the C ABI, against the same
attention with a caller workspace (hisparse_sparse_mla_decode).

Both run the same kernels on the same inputs and the split/merge order is
fixed, so the results must be identical bit for bit (stricter than the
attention's tolerance against the float64 oracle, which the regular
attention tests cover).  Two calls in a row, the second with a smaller input
(fewer requests, selections and heads, on another handle), as the scratch
array keeps the previous call's contents; then the same call captured into a
HIP graph and replayed with eager work in between; and a shape whose
workspace exceeds the array is rejected before anything is launched.
"""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def _instance(cfg):
    import torch
    from tests.gpu_harness import LockstepRun
    run = LockstepRun(cfg, oracle_streams=[])
    for s in range(cfg.steps):
        run.gpu_step(s)
    torch.cuda.synchronize()
    assert run.gpu.status() == 0
    return run


def _both(run, layer, H):
    """(out, lse) of the no-alloc call and of the workspace call."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from workload.rows import make_queries
    cfg = run.cfg
    q = torch.from_numpy(make_queries(cfg.B, H, 3000 + cfg.data_seed, layer)).to("cuda")
    scale = 1.0 / np.sqrt(576.0)
    res = []
    for noalloc in (True, False):
        out = torch.full((cfg.B, H, 512), np.nan, dtype=torch.float32, device="cuda")
        lse = torch.full((cfg.B, H), np.nan, dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        if noalloc:
            hb.hisparse_sparse_mla_decode_noalloc(run.gpu.h, st, layer, q.data_ptr(),
                                                  run.out_dev[layer].data_ptr(), H, scale,
                                                  out.data_ptr(), lse.data_ptr())
        else:
            ws = torch.empty(hb.hisparse_mla_workspace_bytes(run.gpu.h, H), dtype=torch.uint8,
                             device="cuda")
            hb.hisparse_sparse_mla_decode(run.gpu.h, st, layer, q.data_ptr(),
                                          run.out_dev[layer].data_ptr(), H, scale,
                                          ws.data_ptr(), out.data_ptr(), lse.data_ptr())
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res, q, scale


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    big = _instance(WORKLOADS[4].scaled(B=16, layers=2, L0=40000, steps=2))
    small = _instance(WORKLOADS[2].scaled(B=3, L0=8192, C=1500, k=700, steps=2))
    try:
        for run, layer, H in ((big, 1, 64), (small, 0, 16)):   # the second is smaller
            need = hb.hisparse_mla_workspace_bytes(run.gpu.h, H)
            assert need <= hb.HISPARSE_NOALLOC_SCRATCH_BYTES
            (o_n, l_n), (o_w, l_w) = _both(run, layer, H)[0]
            assert np.isfinite(o_n).all() and np.isfinite(l_n).all()
            np.testing.assert_array_equal(o_n, o_w, err_msg=f"out, {run.cfg.B} requests x {H} heads")
            np.testing.assert_array_equal(l_n, l_w, err_msg=f"lse, {run.cfg.B} requests x {H} heads")
            print(f"[noalloc] {run.cfg.B} requests x {H} heads ({need} B of scratch): "
                  f"identical to the workspace call", flush=True)
        torch.cuda.synchronize()
    finally:
        small.close()
        big.close()


def test_noalloc_replays_in_a_graph():
    """Captured (no allocation happens in the call), replayed three times
    with eager work and synchronizations between the replays; every replay
    equals the eager workspace call."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    run = _instance(WORKLOADS[4].scaled(B=8, layers=1, L0=30000, steps=1))
    try:
        H = 32
        res, q, scale = _both(run, 0, H)
        o_w, l_w = res[1]
        out = torch.zeros((run.cfg.B, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.zeros((run.cfg.B, H), dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                hb.hisparse_sparse_mla_decode_noalloc(
                    run.gpu.h, torch.cuda.current_stream().cuda_stream, 0, q.data_ptr(),
                    run.out_dev[0].data_ptr(), H, scale, out.data_ptr(), lse.data_ptr())
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(np.nan)
            lse.fill_(np.nan)
            _both(run, 0, 16)            # eager work on the same scratch in between
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(out.cpu().numpy(), o_w, err_msg=f"replay {rep}")
            np.testing.assert_array_equal(lse.cpu().numpy(), l_w, err_msg=f"replay {rep}")
    finally:
        run.close()


def test_noalloc_rejects_a_workspace_beyond_its_array():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    run = _instance(WORKLOADS[4].scaled(B=16, layers=1, L0=20000, steps=1))
    try:
        H = 4096    # 256 head blocks x 16 requests: partials far beyond the array
        assert hb.hisparse_mla_workspace_bytes(run.gpu.h, H) > hb.HISPARSE_NOALLOC_SCRATCH_BYTES
        q = torch.zeros(16, dtype=torch.uint8, device="cuda")
        out = torch.zeros(16, dtype=torch.float32, device="cuda")
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_sparse_mla_decode_noalloc(run.gpu.h, torch.cuda.current_stream().cuda_stream,
                                                  0, q.data_ptr(), run.out_dev[0].data_ptr(), H,
                                                  0.04, out.data_ptr(), out.data_ptr())
        assert e.value.code == hb.HISPARSE_ERR_UNSUPPORTED
        assert "workspace" in hb.hisparse_last_error()
        torch.cuda.synchronize()
        assert run.gpu.status() == 0
    finally:
        run.close()
