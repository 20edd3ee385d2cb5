"""GPU parity at the five workloads' full sizes: eager per-layer resolve
calls, the layer-wise prefetch schedule of the shared-selection workload, and
every step of a workload captured as one HIP graph and replayed (the
benchmark's timed region).

The oracle runs every stream of every workload.  Slot maps, clocks,
counters, eviction logs, miss lists, slot2pos, last_use and the LRU order of
every stream are compared every step; the full position->slot table and the
slot contents at the first, middle and last step, on a sample of streams
where a workload has many (each of those copies is a whole stream's table or
cache).  Shared-selection workloads also check that every layer of a request
stays identical.
"""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu

# streams whose position->slot table and slot bytes are compared at the
# checkpoints (None: every stream)
DEEP = {
    1: None,
    2: None,
    3: [(0, 0), (7, 3), (15, 7), (3, 6)],
    4: [(0, 0), (9, 4), (15, 7), (4, 2)],
    5: None,
}


def _layers_identical(run, s):
    out = run.out_dev
    for l in range(1, run.cfg.layers):
        assert bool((out[0] == out[l]).all()), f"layer {l} diverged at step {s}"


def _run_full(cfg_id, flags=0, prefetch=False):
    import torch
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[cfg_id]
    print(f"[full] {cfg.name} flags={flags} prefetch={prefetch}: building inputs", flush=True)
    run = LockstepRun(cfg, flags=flags)
    checkpoints = {0, cfg.steps // 2, cfg.steps - 1}
    main = torch.cuda.Stream() if prefetch else None
    side = torch.cuda.Stream() if prefetch else None
    try:
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.append_rows(s)
            if prefetch:
                torch.cuda.synchronize()
                run.prefetch_step(s, main.cuda_stream, side.cuda_stream)
            else:
                run.gpu_step(s)
            torch.cuda.synchronize()
            if cfg.shared_selection:
                _layers_identical(run, s)
            res = run.oracle_step(s)
            full = s in checkpoints
            run.compare_step(s, res, full_state=full, contents=full, full_streams=DEEP[cfg_id])
            if full:
                print(f"[full] {cfg.name}: step {s} matches on all {len(res)} streams "
                      f"(deep checks on {len(DEEP[cfg_id] or res)})", flush=True)
        assert run.gpu.status() == 0
    finally:
        run.close()


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_full_size_parity(cfg_id):
    _run_full(cfg_id)


def test_full_size_pages_no_io():
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    _run_full(5, flags=hb.HISPARSE_NO_IO)


def test_full_size_prefetch_schedule():
    """The shared-selection workload as it is defined: layer 0 resolved on
    the main stream, then every layer l+1 prefetched on a second stream
    (forked after layer l) and joined by its resolve; every stream's slot
    map, cache state, logs and counters against the oracle every step."""
    _run_full(4, prefetch=True)


@pytest.mark.parametrize("cfg_id,schedule", [(2, "plain"), (3, "append"), (3, "fused_append"),
                                             (4, "plain"), (4, "prefetch")])
def test_full_size_graph_of_all_steps(cfg_id, schedule):
    """All steps captured as one HIP graph and replayed once from a cold
    cache, as the benchmark times them: plain resolves; for the growing
    workload the appends as separate calls or fused into the resolve calls;
    for the shared-selection workload also its layer-wise prefetch schedule
    (a second stream forked and joined inside the graph).  Each step writes
    its own slot-map buffer, so every step's slot map of every stream is
    compared with the oracle; after the last step, the cache state, eviction
    log, counters and running totals of every stream, and the position->slot
    table and slot bytes of the sampled streams."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    from tests.harness import appended_row
    cfg = WORKLOADS[cfg_id]
    print(f"[graph] {cfg.name} ({schedule}): building inputs", flush=True)
    run = LockstepRun(cfg)
    try:
        rows = None
        if cfg.growth:
            rows = torch.from_numpy(np.stack([
                np.stack([np.stack([appended_row(cfg, b, l, cfg.ctx_at(s) - 1)
                                    for b in range(cfg.B)]) for l in range(cfg.layers)])
                if s > 0 else np.zeros((cfg.layers, cfg.B, cfg.row_bytes), np.uint8)
                for s in range(cfg.steps)])).to("cuda")
        outs = torch.full((cfg.steps, cfg.layers, cfg.B, cfg.k), -7, dtype=torch.int32,
                          device="cuda")
        main = torch.cuda.Stream()
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            with torch.cuda.graph(g, stream=main):
                st = torch.cuda.current_stream().cuda_stream
                for s in range(cfg.steps):
                    if schedule == "prefetch":
                        run.prefetch_step(s, st, side.cuda_stream, out=outs[s])
                        continue
                    for l in range(cfg.layers):
                        sel = run.sel_dev[s, l].data_ptr()
                        ctx = run.ctx_dev[s].data_ptr()
                        out = outs[s, l].data_ptr()
                        if cfg.growth and s > 0 and schedule == "fused_append":
                            hb.hisparse_append_resolve(run.gpu.h, st, l, rows[s, l].data_ptr(),
                                                       run.pos_dev[s].data_ptr(), sel, ctx, out)
                            continue
                        if cfg.growth and s > 0:
                            hb.hisparse_append(run.gpu.h, st, l, rows[s, l].data_ptr(),
                                               run.pos_dev[s].data_ptr())
                        hb.hisparse_resolve(run.gpu.h, st, sel, ctx, l, out)
        torch.cuda.synchronize()
        print(f"[graph] {cfg.name}: captured {cfg.steps} steps, replaying", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = outs.cpu().numpy()
        res = None
        for s in range(cfg.steps):
            if s > 0 and cfg.growth:
                run.oracle.append(s)
            res = run.oracle_step(s)
            for (b, l), r in res.items():
                np.testing.assert_array_equal(got[s, l, b], r.out,
                                              err_msg=f"out_slot step {s} stream (b={b}, l={l})")
        last = cfg.steps - 1
        run.out_dev.copy_(outs[last])
        torch.cuda.synchronize()
        run.compare_step(last, res, full_state=True, contents=True, full_streams=DEEP[cfg_id])
        snap = run.gpu.meta_snapshot()
        for (b, l), st_o in run.oracle.st.items():
            hdr = run.gpu.hdr(b, l, snap)
            assert int(hdr[hb.HDR_T]) == int(st_o.t[0]) == cfg.steps
        assert run.gpu.status() == 0
        print(f"[graph] {cfg.name} ({schedule}): every step's slot map matches on all "
              f"{len(res)} streams", flush=True)
    finally:
        run.close()
