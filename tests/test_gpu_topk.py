"""GPU top-k selection (hisparse_topk, through the C ABI) against the oracle's
topk_select, bit-exact per row: seeded drifting N(0,1) scores with and
without bfloat16 ties and special values, ragged lengths, per-row context
lengths, all-equal rows (every position a boundary candidate), the full
per-layer shapes of the token and page workloads, rows on both sides of the
finish kernel's 2^18-position LDS bitmap limit, workspace reuse, graph
replay, and the selection fed straight into the resolver."""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu


class Topk:
    def __init__(self, rows, max_len, row_stride=None):
        import torch
        from hierarchical_kv_cache_hisparse_amd import binding as hb
        self.torch, self.hb = torch, hb
        self.rows, self.max_len = rows, max_len
        self.stride = row_stride or ((max_len + 3) // 4) * 4
        n = hb.hisparse_topk_workspace_bytes(rows, max_len)
        self.ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        self.scores = torch.zeros((rows, self.stride), dtype=torch.float32, device="cuda")
        self.ctx = torch.zeros(rows, dtype=torch.int32, device="cuda")

    def run(self, scores_np, ctx_np, k):
        torch = self.torch
        self.scores[:, :scores_np.shape[1]].copy_(torch.from_numpy(scores_np))
        self.ctx.copy_(torch.from_numpy(np.asarray(ctx_np, np.int32)))
        out = torch.full((self.rows, k), -7, dtype=torch.int32, device="cuda")
        self.launch(k, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def launch(self, k, out):
        self.hb.hisparse_topk(self.torch.cuda.current_stream().cuda_stream,
                              self.scores.data_ptr(), self.stride, self.rows, self.max_len,
                              self.ctx.data_ptr(), k, self.ws.data_ptr(), out.data_ptr())


def _scores(rows, n, seed, step=0, **kw):
    from workload.scores import score_rows
    return score_rows(rows, n, seed, 0, step, **kw)


def _check(got, scores, ctx, k, where):
    from oracle.topk import topk_select
    for b in range(len(ctx)):
        want = topk_select(scores[b], int(min(max(ctx[b], 0), scores.shape[1])), k)
        np.testing.assert_array_equal(got[b], want, err_msg=f"{where} row {b}")


CASES = {
    # name: (rows, max_len, k, ctx per row or None for all max_len, score options)
    "small_ragged": (3, 10001, 300, [10001, 9000, 4097], {}),
    "ties_and_specials": (4, 20003, 700, [20003, 20000, 12345, 4096], {"ties": True, "specials": True}),
    "short_rows": (5, 5000, 512, [0, 1, 511, 512, 513], {"ties": True}),
    "k_one": (2, 70000, 1, None, {"ties": True}),
    "k_max": (2, 30000, 4096, [30000, 4100], {"ties": True, "specials": True}),
    "one_chunk": (3, 4096, 64, None, {}),
    # the longest rows whose bitmap the finish kernel keeps in LDS (2^18)
    "overlay_max_len": (2, 262144, 1000, [262144, 262143], {"specials": True}),
    # longer rows: the finish kernel marks and reads the global bitmap
    "long_rows": (3, 300001, 2048, [300001, 270000, 5000], {"ties": True}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_topk_parity(name):
    rows, n, k, ctx, kw = CASES[name]
    ctx = [n] * rows if ctx is None else ctx
    print(f"[topk] {name}: rows={rows} n={n} k={k} ctx={ctx}", flush=True)
    t = Topk(rows, n)
    s = _scores(rows, n, 4000 + len(name), **kw)
    _check(t.run(s, ctx, k), s, ctx, k, name)


def test_topk_all_equal_and_plateaus():
    """Rows where the boundary bin holds every position (all scores equal),
    or a plateau of equal scores straddles the boundary."""
    n, k = 50000, 1000
    t = Topk(3, n)
    s = np.zeros((3, n), np.float32)
    s[0] = 1.0                                     # all equal: lowest k positions
    s[1] = -0.0
    s[1, ::2] = 0.0                                # -0 and +0 mixed: all equal
    s[2] = 2.0
    s[2, 1000:3000] = 3.0                          # 2000 highest, k=1000 of them
    s[2, 40000:40500] = 5.0
    got = t.run(s, [n, n, n], k)
    _check(got, s, [n, n, n], k, "plateaus")
    assert got[0].tolist() == list(range(k))


def test_topk_row_stride_and_ctx_clamp():
    n, stride, k = 9000, 9216, 256
    t = Topk(2, n, row_stride=stride)
    s = _scores(2, n, 4100, ties=True)
    got = t.run(s, [-5, n + 100], k)       # clamped to 0 and n
    assert (got[0] == -1).all()
    _check(got[1:], s[1:], [n], k, "clamp")


def test_topk_workspace_reuse_and_graph_replay():
    """Consecutive calls on one workspace (the second with shorter rows and a
    smaller k), then one captured graph replayed on new scores each time:
    every result equals the oracle's."""
    import torch
    n = 40000
    t = Topk(4, n)
    s1 = _scores(4, n, 4200, ties=True)
    _check(t.run(s1, [n] * 4, 2048), s1, [n] * 4, 2048, "first call")
    s2 = _scores(4, n, 4201, specials=True)
    ctx2 = [30000, 100, 5000, n]
    _check(t.run(s2, ctx2, 300), s2, ctx2, 300, "second call")
    out = torch.empty((4, 512), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            t.launch(512, out)
    torch.cuda.synchronize()
    for rep in range(4):
        s = _scores(4, n, 4300, step=rep, ties=True)
        ctx = [n, n - 7 * rep, 20000, 600 + rep]
        t.scores[:, :n].copy_(torch.from_numpy(s))
        t.ctx.copy_(torch.tensor(ctx, dtype=torch.int32))
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(out.cpu().numpy(), s, ctx, 512, f"replay {rep}")


@pytest.mark.parametrize("cfg_id", [3, 4, 5])
def test_topk_full_layer_shapes(cfg_id):
    """One layer call at the workload's shape: 16 x 131072 tokens (k 2048),
    16 x 262144 tokens (k 2048), 4 x 65536 pages (k 128)."""
    cfg = WORKLOADS[cfg_id]
    print(f"[topk] full shape {cfg.name}: rows={cfg.B} n={cfg.L0} k={cfg.k}", flush=True)
    t = Topk(cfg.B, cfg.L0)
    s = _scores(cfg.B, cfg.L0, 4400 + cfg_id, ties=True)
    _check(t.run(s, [cfg.L0] * cfg.B, cfg.k), s, [cfg.L0] * cfg.B, cfg.k, cfg.name)


def test_topk_feeds_the_resolver():
    """Scores -> hisparse_topk -> hisparse_resolve over several drifting
    steps equals oracle top-k -> oracle resolve, state and slot bytes."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from oracle.topk import topk_rows
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=3, L0=12000, C=1500, k=600, steps=6)
    run = LockstepRun(cfg, fill_all=True)
    t = Topk(cfg.B, cfg.L0)
    try:
        trace = np.full_like(run.trace, -1)
        for s in range(cfg.steps):
            sc = _scores(cfg.B, cfg.L0, 4500, step=s)
            t.scores[:, :cfg.L0].copy_(torch.from_numpy(sc))
            t.ctx.copy_(run.ctx_dev[s])
            t.launch(cfg.k, run.sel_dev[s, 0])
            hb.hisparse_resolve(run.gpu.h, run.gpu.stream, run.sel_dev[s, 0].data_ptr(),
                                run.ctx_dev[s].data_ptr(), 0, run.out_dev[0].data_ptr())
            torch.cuda.synchronize()
            trace[s, 0] = topk_rows(sc, [cfg.ctx_at(s)] * cfg.B, cfg.k)
            np.testing.assert_array_equal(run.sel_dev[s, 0].cpu().numpy(), trace[s, 0])
            run.compare_step(s, run.oracle.step(s, trace))
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_topk_argument_checks():
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    t = Topk(2, 5000)
    out = torch.empty((2, 64), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    bad = [
        dict(k=0), dict(k=4097), dict(row_stride=4999), dict(row_stride=5002),
        dict(num_rows=0), dict(max_len=0), dict(scores_off=4),
    ]
    for b in bad:
        kw = dict(k=64, row_stride=t.stride, num_rows=2, max_len=5000, scores_off=0)
        kw.update(b)
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_topk(s, t.scores.data_ptr() + kw["scores_off"], kw["row_stride"],
                             kw["num_rows"], kw["max_len"], t.ctx.data_ptr(), kw["k"],
                             t.ws.data_ptr(), out.data_ptr())
        assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG, b


def _random_topk_case(i):
    """Seeded random shape: rows, row length (short, mid, or past the finish
    kernel's 2^18-position LDS bitmap), k, ragged per-row contexts, bf16 ties,
    special values and plateaus of equal scores.  Pure function of i."""
    from workload.scores import score_rows
    rng = np.random.default_rng(9000 + i)
    rows = int(rng.integers(1, 9))
    n = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 70000)),
                        int(rng.integers(250000, 300000))]))
    k = int(rng.integers(1, 4097))
    ctx = [int(rng.choice([n, int(rng.integers(0, n + 1)), min(n, k), max(0, k - 1)]))
           for _ in range(rows)]
    kw = [{}, {"ties": True}, {"specials": True}, {"ties": True, "specials": True}][
        int(rng.integers(0, 4))]
    sc = score_rows(rows, n, 9100 + i, 0, 0, **kw)
    if rng.random() < 0.15:
        a = int(rng.integers(0, n))
        b = int(rng.integers(a, n + 1))
        sc[:, a:b] = np.float32(rng.choice([0.0, -0.0, 1.5, np.inf, -np.inf]))
    return rows, n, k, ctx, sc


@pytest.mark.parametrize("i", range(40))
def test_topk_random_shapes(i):
    rows, n, k, ctx, sc = _random_topk_case(i)
    print(f"[topk random {i}] rows={rows} n={n} k={k} ctx={ctx}", flush=True)
    t = Topk(rows, n)
    _check(t.run(sc, ctx, k), sc, ctx, k, f"random case {i}")
