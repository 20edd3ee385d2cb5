"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (eager per-layer resolve calls, miss fetch on).

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
