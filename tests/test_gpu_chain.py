"""The whole per-layer path on the GPU, end to end, against the oracle chain:
indexer scores -> hisparse_topk -> hisparse_append_resolve (the newest row
appended in the same launch, misses fetched from pinned host memory) ->
hisparse_sparse_mla_decode over the slot map, for every layer of several
decode steps of a growing context with independent per-layer selections.

Each piece is compared where it is exact: the selections bit for bit with
the oracle's top-k of the same scores, the cache state and slot bytes bit for
bit with the oracle's resolution of those selections, and the attention
output within the float64 oracle's stated tolerance over the *host* rows at
the selected positions ("HiSparse: Scaling Sparse-Attention Decoding with
Hierarchical KV Cache Management", Abstract: resolution only changes where
rows live, so attention outputs are unchanged)."""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def test_scores_topk_resolve_attention_chain():
    import torch
    from oracle.topk import topk_rows
    from tests.gpu_harness import LockstepRun
    from tests.test_gpu_mla import Attn
    from tests.test_gpu_topk import Topk, _scores
    cfg = WORKLOADS[3].scaled(B=3, layers=2, L0=10000, C=1500, R=37, k=600, steps=5)
    print(f"[chain] {cfg.B} requests x {cfg.layers} layers, ctx {cfg.L0}.., k={cfg.k}, "
          f"C={cfg.C}, R={cfg.R}, {cfg.steps} steps", flush=True)
    run = LockstepRun(cfg, fill_all=True)
    t = Topk(cfg.B, cfg.l_cap)
    attn = Attn(run, 16)
    trace = np.full_like(run.trace, -1)
    worst = 0.0
    try:
        for s in range(cfg.steps):
            ctx = cfg.ctx_at(s)
            for l in range(cfg.layers):
                sc = _scores(cfg.B, cfg.l_cap, 4600 + 10 * l, step=s, ties=True)
                t.scores[:, :cfg.l_cap].copy_(torch.from_numpy(sc))
                t.ctx.copy_(run.ctx_dev[s])
                t.launch(cfg.k, run.sel_dev[s, l])
                trace[s, l] = topk_rows(sc, [ctx] * cfg.B, cfg.k)
            if s > 0:
                run.append_and_step(s)     # every layer: append + resolve, one launch
            else:
                run.gpu_step(s)
            torch.cuda.synchronize()
            run.trace[s] = trace[s]        # the attention check reads the step's selections
            for l in range(cfg.layers):
                np.testing.assert_array_equal(run.sel_dev[s, l].cpu().numpy(), trace[s, l],
                                              err_msg=f"top-k step {s} layer {l}")
            run.compare_step(s, run.oracle.step(s, trace), full_state=(s == cfg.steps - 1),
                             contents=True)
            for l in range(cfg.layers):
                attn.launch(l, run.out_dev[l])
                torch.cuda.synchronize()
                worst = max(worst, attn.check(s, l))
        assert run.gpu.status() == 0
    finally:
        run.close()
    print(f"[chain] max |attention out - oracle| = {worst:.3e}")
