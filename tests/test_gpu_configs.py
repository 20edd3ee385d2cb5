"""GPU parity at the five workloads' full sizes: eager per-layer resolve
calls (the benchmark's kernel-timing pass), and every step of a workload
captured as one HIP graph and replayed (the benchmark's timed region).

The GPU runs every stream of the workload; the oracle recomputes a sample of
streams (all of them where that is cheap) -- streams are independent, so a
sampled stream's expected values are exact.  Slot maps, counters and
eviction logs are compared every step; the full position->slot table and the
slot contents at the first, middle and last step.  Shared-selection
workloads also check that every layer of a request stays identical.
"""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu

SAMPLED = {
    1: None,                                   # every stream
    2: None,
    3: [(0, 0), (7, 3), (15, 7), (3, 6)],
    4: [(0, 0), (9, 4), (15, 7)],
    5: None,
}


def _run_full(cfg_id, flags=0):
    import torch
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[cfg_id]
    print(f"[full] {cfg.name} flags={flags}: building inputs", flush=True)
    run = LockstepRun(cfg, oracle_streams=SAMPLED[cfg_id], flags=flags)
    checkpoints = {0, cfg.steps // 2, cfg.steps - 1}
    try:
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.append_rows(s)
            run.gpu_step(s)
            torch.cuda.synchronize()
            if cfg.shared_selection:
                out = run.out_dev
                for l in range(1, cfg.layers):
                    assert torch.equal(out[0], out[l]), f"layer {l} diverged at step {s}"
            res = run.oracle_step(s)
            full = s in checkpoints
            run.compare_step(s, res, full_state=full, contents=full)
            if full:
                print(f"[full] {cfg.name}: step {s} matches (full state)", flush=True)
        assert run.gpu.status() == 0
    finally:
        run.close()


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_full_size_parity(cfg_id):
    _run_full(cfg_id)


def test_full_size_pages_no_io():
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    _run_full(5, flags=hb.HISPARSE_NO_IO)


@pytest.mark.parametrize("cfg_id,fused_append", [(2, False), (3, False), (3, True)])
def test_full_size_graph_of_all_steps(cfg_id, fused_append):
    """All steps (and, for the growing workload, the appends: separate calls,
    or fused into the resolve calls) captured as one HIP graph on a side
    stream and replayed once from a cold cache, as the benchmark times them.  The slot map buffer is rewritten by every step, so
    the last step's map is compared; the LRU state, eviction log, counters,
    running totals and slot bytes of the sampled streams after the last step
    must equal the oracle's after all steps."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    from tests.harness import appended_row
    cfg = WORKLOADS[cfg_id]
    print(f"[graph] {cfg.name}: building inputs", flush=True)
    run = LockstepRun(cfg, oracle_streams=SAMPLED[cfg_id] or [(0, 0), (cfg.B - 1, 0)])
    try:
        rows = None
        if cfg.growth:
            rows = torch.from_numpy(np.stack([
                np.stack([np.stack([appended_row(cfg, b, l, cfg.ctx_at(s) - 1)
                                    for b in range(cfg.B)]) for l in range(cfg.layers)])
                if s > 0 else np.zeros((cfg.layers, cfg.B, cfg.row_bytes), np.uint8)
                for s in range(cfg.steps)])).to("cuda")
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                st = torch.cuda.current_stream().cuda_stream
                for s in range(cfg.steps):
                    for l in range(cfg.layers):
                        if cfg.growth and s > 0 and fused_append:
                            hb.hisparse_append_resolve(
                                run.gpu.h, st, l, rows[s, l].data_ptr(), run.pos_dev[s].data_ptr(),
                                run.sel_dev[s, l].data_ptr(), run.ctx_dev[s].data_ptr(),
                                run.out_dev[l].data_ptr())
                            continue
                        if cfg.growth and s > 0:
                            hb.hisparse_append(run.gpu.h, st, l, rows[s, l].data_ptr(),
                                               run.pos_dev[s].data_ptr())
                        hb.hisparse_resolve(run.gpu.h, st, run.sel_dev[s, l].data_ptr(),
                                            run.ctx_dev[s].data_ptr(), l,
                                            run.out_dev[l].data_ptr())
        torch.cuda.synchronize()
        print(f"[graph] {cfg.name}: captured {cfg.steps} steps, replaying", flush=True)
        g.replay()
        torch.cuda.synchronize()
        res = None
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.oracle.append(s)
            res = run.oracle_step(s)
        last = cfg.steps - 1
        run.compare_step(last, res, full_state=True, contents=True)
        for (b, l), st_o in run.oracle.st.items():
            hdr = run.gpu.hdr(b, l)
            assert int(hdr[hb.HDR_T]) == int(st_o.t[0]) == cfg.steps
        assert run.gpu.status() == 0
    finally:
        run.close()
