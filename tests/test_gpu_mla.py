"""GPU sparse-MLA decode attention over the slot map, against the float64
oracle attention over the *host* rows at the selected positions.

This is the exactness claim of the method on the GPU path: resolution only
changes where rows live, so attention through the slot map must equal
attention over the full history ("HiSparse: Scaling Sparse-Attention Decoding
with Hierarchical KV Cache Management", Abstract).

Tolerance (derived from the arithmetic, stated once): q and the rows are
exact bf16; each product is exact in fp32 and the 576-term score sums in fp32
(error ~ sqrt(576) * 2^-24 * |q||k| ~ 1e-6 after the 1/sqrt(576) scale); the
softmax weights enter the value product as bf16 hi + lo (~2^-16 relative);
the output is a weighted mean of N(0,1) values, so its absolute error stays
below ~2^-16 * E|v| ~ 1.2e-5.  We allow 5e-5 absolute on out and 2e-5 on lse.
"""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu

OUT_ATOL = 5e-5
LSE_ATOL = 2e-5


def _reference(cfg, host, sel, q_bytes, scale):
    """float64 oracle over the host rows at the selected positions."""
    from oracle.attention import bf16_to_f64, mla_decode_attention_lse
    T = cfg.row_bytes // 1152
    pos = sel[sel >= 0]
    rows = host[pos].reshape(-1, 1152) if T > 1 else host[pos]
    q = bf16_to_f64(q_bytes)
    return mla_decode_attention_lse(q, bf16_to_f64(rows), scale)


class Attn:
    def __init__(self, run, H):
        import torch
        from hierarchical_kv_cache_hisparse_amd import binding as hb
        self.run, self.H, self.hb, self.torch = run, H, hb, torch
        cfg = run.cfg
        ws = hb.hisparse_mla_workspace_bytes(run.gpu.h, H)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")   # needs no initialisation
        self.out = torch.empty((cfg.B, H, 512), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((cfg.B, H), dtype=torch.float32, device="cuda")
        from workload.rows import make_queries
        self.q_bytes = {l: make_queries(cfg.B, H, 3000 + cfg.data_seed, l) for l in range(cfg.layers)}
        self.q = {l: torch.from_numpy(self.q_bytes[l]).to("cuda") for l in self.q_bytes}
        self.scale = 1.0 / np.sqrt(576.0)

    def launch(self, layer, out_slot):
        self.hb.hisparse_sparse_mla_decode(
            self.run.gpu.h, self.torch.cuda.current_stream().cuda_stream, layer,
            self.q[layer].data_ptr(), out_slot.data_ptr(), self.H, self.scale,
            self.ws.data_ptr(), self.out.data_ptr(), self.lse.data_ptr())

    def check(self, s, layer, requests=None):
        cfg = self.run.cfg
        out = self.out.cpu().numpy()
        lse = self.lse.cpu().numpy()
        worst = 0.0
        for b in (range(cfg.B) if requests is None else requests):
            sel = self.run.trace[s, layer, b]
            ref, ref_lse = _reference(cfg, self.run.gpu.host(b, layer), sel,
                                      self.q_bytes[layer][b], self.scale)
            err = np.abs(out[b] - ref).max()
            worst = max(worst, err)
            assert err <= OUT_ATOL, f"step {s} layer {layer} request {b}: out error {err}"
            np.testing.assert_allclose(lse[b], ref_lse, atol=LSE_ATOL, rtol=0,
                                       err_msg=f"lse step {s} layer {layer} request {b}")
        return worst


def _run(cfg, H, steps=None, requests=None):
    import torch
    from tests.gpu_harness import LockstepRun
    run = LockstepRun(cfg, oracle_streams=[])
    attn = Attn(run, H)
    worst = 0.0
    try:
        for s in range(cfg.steps if steps is None else steps):
            if s > 0 and cfg.growth:
                run.append_rows(s)
            run.gpu_step(s)
            for l in range(cfg.layers):
                attn.launch(l, run.out_dev[l])
                torch.cuda.synchronize()
                worst = max(worst, attn.check(s, l, requests))
        assert run.gpu.status() == 0
    finally:
        run.close()
    print(f"[mla] max |out - oracle| = {worst:.3e}")


@pytest.mark.parametrize("H", [16, 48])
def test_attention_over_token_slots(H):
    cfg = WORKLOADS[2].scaled(B=3, L0=8192, C=1500, k=700, steps=3)
    _run(cfg, H)


@pytest.mark.parametrize("fused_append", [True, False])
def test_attention_over_a_growing_context(fused_append):
    """Independent per-layer selections over a context that grows by one row
    per step: the newest row reaches its ring slot through the append (fused
    into the resolve launch, or a separate append launch) and is attended
    from there, the oldest leaves the window; every step's attention equals
    the oracle over the host rows."""
    import torch
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[3].scaled(B=3, layers=2, L0=6000, C=1200, R=37, k=500, steps=5)
    run = LockstepRun(cfg, oracle_streams=[])
    attn = Attn(run, 16)
    worst = 0.0
    try:
        for s in range(cfg.steps):
            if s > 0 and fused_append:
                run.append_and_step(s)
            else:
                if s > 0:
                    run.append_rows(s)
                run.gpu_step(s)
            for l in range(cfg.layers):
                attn.launch(l, run.out_dev[l])
                torch.cuda.synchronize()
                worst = max(worst, attn.check(s, l))
        assert run.gpu.status() == 0
    finally:
        run.close()
    print(f"[mla] growing context, max |out - oracle| = {worst:.3e}")


def test_attention_over_page_slots():
    cfg = WORKLOADS[5].scaled(B=2, layers=2, L0=3000, C=64, k=40, steps=3)
    _run(cfg, 16)


def test_attention_full_shared_selection_step():
    """The 16-request, 2048-selection shape of the shared-selection workload
    (one layer), 128 heads, sampled requests."""
    cfg = WORKLOADS[4].scaled(layers=1, steps=2)
    _run(cfg, 128, requests=[0, 7, 15])


def test_attention_skips_padding_and_empty_rows():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=3, L0=4000, C=512, k=200, steps=1)
    run = LockstepRun(cfg, oracle_streams=[])
    attn = Attn(run, 16)
    try:
        trace = run.trace.copy()
        trace[0, 0, 1, ::3] = -1          # request 1: a third padding
        trace[0, 0, 2, :] = -1            # request 2: nothing selected
        run.trace = trace
        sel = torch.from_numpy(trace[0, 0]).cuda()
        hb.hisparse_resolve(run.gpu.h, run.gpu.stream, sel.data_ptr(), run.ctx_dev[0].data_ptr(),
                            0, run.out_dev[0].data_ptr())
        attn.launch(0, run.out_dev[0])
        torch.cuda.synchronize()
        attn.check(0, 0, requests=[0, 1])
        assert (attn.out[2] == 0).all() and torch.isinf(attn.lse[2]).all()
        assert (attn.lse[2] < 0).all()
    finally:
        run.close()


def test_attention_graph_replays_are_bit_reproducible():
    """Captured once (split attention + merge), replayed several times with
    eager work in between: every replay equals the eager launch bit for bit."""
    import torch
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=4, L0=6000, C=1024, k=512, steps=1)
    run = LockstepRun(cfg, oracle_streams=[])
    attn = Attn(run, 32)
    try:
        run.gpu_step(0)
        torch.cuda.synchronize()
        attn.launch(0, run.out_dev[0])
        torch.cuda.synchronize()
        eager = attn.out.clone()
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                attn.launch(0, run.out_dev[0])
        torch.cuda.synchronize()
        for _ in range(4):
            attn.out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(attn.out, eager)
        attn.check(0, 0)
    finally:
        run.close()


MULTI_CASES = {
    # name: (base workload, query tokens, overrides); k = tokens x per-token count
    "tokens_two": (2, 2, dict(B=3, L0=8192, C=1500, k=1200, steps=3)),
    "tokens_three_shared_layers": (4, 3, dict(B=2, layers=2, L0=20000, k=1536, steps=2)),
    "pages_four": (5, 4, dict(B=2, layers=1, L0=3000, C=300, k=160, steps=3)),
}


@pytest.mark.parametrize("name", sorted(MULTI_CASES))
def test_attention_multi_query(name):
    """Several query tokens per request over the multi-query slot map: token
    j of request b attends to the slots of its own selections, and equals the
    float64 oracle over the host rows at those positions."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    from workload.rows import make_queries
    base, Q, kw = MULTI_CASES[name]
    cfg = WORKLOADS[base].scaled(**kw)
    H, per = 16, cfg.k // Q
    print(f"[mla multi] {name}: B={cfg.B} Q={Q} per_query={per} H={H}", flush=True)
    run = LockstepRun(cfg, oracle_streams=[], queries=Q)
    try:
        ws = torch.empty(hb.hisparse_mla_workspace_bytes_multi(run.gpu.h, Q, per, H),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((cfg.B * Q, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((cfg.B * Q, H), dtype=torch.float32, device="cuda")
        scale = 1.0 / np.sqrt(576.0)
        for s in range(cfg.steps):
            run.gpu_step(s)
            for l in range(cfg.layers):
                q_bytes = make_queries(cfg.B * Q, H, 3100 + cfg.data_seed, l)
                q = torch.from_numpy(q_bytes).to("cuda")
                hb.hisparse_sparse_mla_decode_multi(
                    run.gpu.h, torch.cuda.current_stream().cuda_stream, l, Q, per, q.data_ptr(),
                    run.out_dev[l].data_ptr(), H, scale, ws.data_ptr(), out.data_ptr(),
                    lse.data_ptr())
                torch.cuda.synchronize()
                o, g = out.cpu().numpy(), lse.cpu().numpy()
                for b in range(cfg.B):
                    sel_q = run.trace[s, l, b].reshape(Q, per)
                    for j in range(Q):
                        r = b * Q + j
                        ref, ref_lse = _reference(cfg, run.gpu.host(b, l), sel_q[j], q_bytes[r],
                                                  scale)
                        err = np.abs(o[r] - ref).max()
                        assert err <= OUT_ATOL, f"step {s} layer {l} request {b} token {j}: {err}"
                        np.testing.assert_allclose(g[r], ref_lse, atol=LSE_ATOL, rtol=0)
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_attention_multi_with_one_token_is_the_single_call():
    """queries = 1, per_query = top_k: the multi entry is the single-token
    attention, bit for bit."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=3, L0=6000, C=1024, k=512, steps=1)
    run = LockstepRun(cfg, oracle_streams=[])
    attn = Attn(run, 32)
    try:
        run.gpu_step(0)
        torch.cuda.synchronize()
        attn.launch(0, run.out_dev[0])
        torch.cuda.synchronize()
        want, want_lse = attn.out.clone(), attn.lse.clone()
        assert hb.hisparse_mla_workspace_bytes_multi(run.gpu.h, 1, cfg.k, 32) == \
            hb.hisparse_mla_workspace_bytes(run.gpu.h, 32)
        attn.out.zero_()
        hb.hisparse_sparse_mla_decode_multi(
            run.gpu.h, torch.cuda.current_stream().cuda_stream, 0, 1, cfg.k, attn.q[0].data_ptr(),
            run.out_dev[0].data_ptr(), 32, attn.scale, attn.ws.data_ptr(), attn.out.data_ptr(),
            attn.lse.data_ptr())
        torch.cuda.synchronize()
        assert torch.equal(attn.out, want) and torch.equal(attn.lse, want_lse)
        for bad in ((0, 16), (2, 0), (3, cfg.k)):
            with pytest.raises(hb.HisparseError) as e:
                hb.hisparse_mla_workspace_bytes_multi(run.gpu.h, bad[0], bad[1], 32)
            assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
    finally:
        run.close()


@pytest.mark.parametrize("i", range(24))
def test_attention_random_shapes(i):
    """Seeded random shapes over real slot maps: token rows or 16-token pages,
    1-4 requests, 16-128 heads, any selection width up to the cache, with and
    without a resident window."""
    rng = np.random.default_rng(9500 + i)
    pages = rng.random() < 0.3
    B = int(rng.integers(1, 5))
    H = int(rng.choice([16, 32, 48, 64, 128]))
    if pages:
        C = int(rng.integers(8, 300))
        k = int(rng.integers(1, min(C, 128) + 1))
        L0 = int(rng.integers(4 * k + 40, 4 * k + 2000))
        R = int(rng.choice([0, 1, 4]))
        cfg = WORKLOADS[5].scaled(B=B, layers=1, L0=L0, C=C, R=R, k=k, steps=2)
    else:
        C = int(rng.integers(16, 5000))
        k = int(rng.integers(1, min(C, 4096) + 1))
        R = int(rng.choice([0, 1, 37, 128]))
        L0 = int(rng.integers(4 * k + R + 64, 4 * k + R + 20000))
        cfg = WORKLOADS[2].scaled(B=B, layers=1, L0=L0, C=C, R=R, k=k, steps=2)
    print(f"[mla random {i}] pages={pages} B={B} H={H} C={C} k={k} R={R} L0={L0}", flush=True)
    _run(cfg, H)
