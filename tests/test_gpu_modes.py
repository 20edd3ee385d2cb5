"""GPU mode tests of the resolve path, all through the C ABI:

  graph replay equals eager launches (the step is graph-capturable);
  prefetch on a second stream equals no prefetch (exact layer-wise prefetch);
  copies suppressed (no-IO) leave the metadata unchanged and read no rows;
  hits read no host bytes (host rows of cached positions are poisoned);
  invalid rows leave their stream untouched and are reported;
  snapshot / restore of the caller-owned state replays identically;
  resetting one request's stream leaves the others alone.
"""
import numpy as np
import pytest

from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _hb():
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    return hb


def _pair(cfg, flags_a=0, flags_b=0):
    """Two instances over the same pinned host histories."""
    from tests.gpu_harness import GpuInstance
    from tests.harness import fill_host, make_trace
    a = GpuInstance(cfg, flags=flags_a)
    b = GpuInstance(cfg, flags=flags_b, hosts=a.hosts)
    trace = make_trace(cfg)
    fill_host(cfg, a.host, trace, [(bb, l) for bb in range(cfg.B) for l in range(cfg.layers)])
    return a, b, trace


def _assert_same_state(a, b, cfg, contents=True):
    for l in range(cfg.layers):
        for bb in range(cfg.B):
            sa, sb = a.state(bb, l), b.state(bb, l)
            for key in ("hdr", "slot2pos", "last_use", "order", "pos2slot"):
                np.testing.assert_array_equal(sa[key], sb[key], err_msg=f"{key} (b={bb}, l={l})")
            m = int(sa["hdr"][5])
            np.testing.assert_array_equal(sa["evict"][:m], sb["evict"][:m])
            if contents:
                filled = np.nonzero(sa["slot2pos"] >= 0)[0]
                np.testing.assert_array_equal(a.slots(bb, l)[filled], b.slots(bb, l)[filled])


def _load_windows(inst, ctx_dev):
    _hb().hisparse_load_window(inst.h, inst.stream, -1, ctx_dev.data_ptr())


def test_graph_replay_equals_eager():
    """One captured graph (reading the selections from a fixed buffer) is
    replayed every step, with eager copies and synchronizations in between;
    every replay must equal an eager instance bit for bit."""
    torch, hb = _torch(), _hb()
    cfg = WORKLOADS[3].scaled(B=3, layers=2, L0=9000, C=2048, k=1024, steps=8)
    a, b, trace = _pair(cfg)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.ctx_at(0), dtype=torch.int32, device=dev)
        _load_windows(a, ctx)
        _load_windows(b, ctx)
        sel_buf = torch.empty((cfg.layers, cfg.B, cfg.k), dtype=torch.int32, device=dev)
        ctx_buf = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
        out_g = torch.empty_like(sel_buf)
        out_e = torch.empty_like(sel_buf)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                s = torch.cuda.current_stream().cuda_stream
                for l in range(cfg.layers):
                    hb.hisparse_resolve(a.h, s, sel_buf[l].data_ptr(), ctx_buf.data_ptr(), l,
                                        out_g[l].data_ptr())
        torch.cuda.synchronize()
        trace_dev = torch.from_numpy(trace).to(dev)
        from tests.harness import appended_row
        for step in range(cfg.steps):
            if step > 0:   # growth: append through the library on both instances
                p = cfg.ctx_at(step) - 1
                pos = torch.full((cfg.B,), p, dtype=torch.int32, device=dev)
                for l in range(cfg.layers):
                    rows = torch.from_numpy(np.stack([appended_row(cfg, bb, l, p)
                                                      for bb in range(cfg.B)])).to(dev)
                    hb.hisparse_append(a.h, a.stream, l, rows.data_ptr(), pos.data_ptr())
                    hb.hisparse_append(b.h, b.stream, l, rows.data_ptr(), pos.data_ptr())
            sel_buf.copy_(trace_dev[step])
            ctx_buf.fill_(cfg.ctx_at(step))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(cfg.layers):
                hb.hisparse_resolve(b.h, b.stream, trace_dev[step, l].data_ptr(),
                                    ctx_buf.data_ptr(), l, out_e[l].data_ptr())
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), f"step {step}"
            _assert_same_state(a, b, cfg)
        assert a.status() == 0 and b.status() == 0
    finally:
        b.close()
        a.close()


@pytest.mark.parametrize("captured", [False, True])
def test_prefetch_equals_no_prefetch(captured):
    """Shared selections across layers: layer l+1 resolved early on a second
    stream (forked after layer l) must give the same slot maps and state as
    resolving every layer in order on one stream."""
    torch, hb = _torch(), _hb()
    cfg = WORKLOADS[4].scaled(B=2, layers=4, L0=30000, steps=6)
    a, b, trace = _pair(cfg)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        _load_windows(a, ctx)
        _load_windows(b, ctx)
        trace_dev = torch.from_numpy(trace).to(dev)
        sel_buf = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev)
        out_p = torch.empty((cfg.layers, cfg.B, cfg.k), dtype=torch.int32, device=dev)
        out_s = torch.empty_like(out_p)
        main = torch.cuda.Stream()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()

        def prefetched_step():
            ms, ss = main.cuda_stream, side.cuda_stream
            hb.hisparse_resolve(a.h, ms, sel_buf.data_ptr(), ctx.data_ptr(), 0, out_p[0].data_ptr())
            for l in range(cfg.layers - 1):
                hb.hisparse_prefetch(a.h, ms, ss, sel_buf.data_ptr(), ctx.data_ptr(), l + 1)
                # (layer l's attention would run on `main` here)
                hb.hisparse_resolve(a.h, ms, sel_buf.data_ptr(), ctx.data_ptr(), l + 1,
                                    out_p[l + 1].data_ptr())

        graph = None
        if captured:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(main):
                with torch.cuda.graph(graph, stream=main):
                    prefetched_step()
            torch.cuda.synchronize()
        for step in range(cfg.steps):
            sel_buf.copy_(trace_dev[step, 0])
            torch.cuda.synchronize()
            if captured:
                graph.replay()
            else:
                with torch.cuda.stream(main):
                    prefetched_step()
            torch.cuda.synchronize()
            for l in range(cfg.layers):
                hb.hisparse_resolve(b.h, b.stream, sel_buf.data_ptr(), ctx.data_ptr(), l,
                                    out_s[l].data_ptr())
            torch.cuda.synchronize()
            assert torch.equal(out_p, out_s), f"step {step}"
            _assert_same_state(a, b, cfg)
            # shared selections: every layer ends in the same state
            for l in range(1, cfg.layers):
                assert torch.equal(out_s[0], out_s[l])
        assert a.status() == 0 and b.status() == 0
    finally:
        b.close()
        a.close()


def test_prefetch_with_a_growing_context():
    """Shared selections over a context that grows by one row per step: each
    layer's new row goes in through hisparse_append_resolve while the layer
    after it has been prefetched on a second stream (the append then runs as
    its own launch before the join).  Slot maps, state, slot bytes and the
    resident ring equal appending and resolving every layer in order."""
    torch, hb = _torch(), _hb()
    from tests.harness import appended_row
    cfg = WORKLOADS[4].scaled(B=2, layers=3, L0=20000, growth=1, steps=6)
    a, b, trace = _pair(cfg)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        _load_windows(a, ctx)
        _load_windows(b, ctx)
        trace_dev = torch.from_numpy(trace).to(dev)
        sel_buf = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev)
        pos_buf = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
        rows_dev = torch.empty((cfg.layers, cfg.B, cfg.row_bytes), dtype=torch.uint8, device=dev)
        out_p = torch.empty((cfg.layers, cfg.B, cfg.k), dtype=torch.int32, device=dev)
        out_s = torch.empty_like(out_p)
        main = torch.cuda.Stream()
        side = torch.cuda.Stream()

        def layer_call(inst, st, l, grow, out):
            if grow:
                hb.hisparse_append_resolve(inst.h, st, l, rows_dev[l].data_ptr(),
                                           pos_buf.data_ptr(), sel_buf.data_ptr(),
                                           ctx.data_ptr(), out[l].data_ptr())
            else:
                hb.hisparse_resolve(inst.h, st, sel_buf.data_ptr(), ctx.data_ptr(), l,
                                    out[l].data_ptr())

        for step in range(cfg.steps):
            c = cfg.ctx_at(step)
            grow = step > 0
            ctx.fill_(c)
            pos_buf.fill_(c - 1)
            sel_buf.copy_(trace_dev[step, 0])
            rows_dev.copy_(torch.from_numpy(np.stack([
                np.stack([appended_row(cfg, bb, l, c - 1) for bb in range(cfg.B)])
                for l in range(cfg.layers)])))
            torch.cuda.synchronize()
            with torch.cuda.stream(main):
                ms, ss = main.cuda_stream, side.cuda_stream
                layer_call(a, ms, 0, grow, out_p)
                for l in range(cfg.layers - 1):
                    hb.hisparse_prefetch(a.h, ms, ss, sel_buf.data_ptr(), ctx.data_ptr(), l + 1)
                    layer_call(a, ms, l + 1, grow, out_p)
            torch.cuda.synchronize()
            for l in range(cfg.layers):
                layer_call(b, b.stream, l, grow, out_s)
            torch.cuda.synchronize()
            assert torch.equal(out_p, out_s), f"step {step}"
            _assert_same_state(a, b, cfg)
            for l in range(cfg.layers):
                for bb in range(cfg.B):
                    np.testing.assert_array_equal(a.slots(bb, l)[cfg.C:], b.slots(bb, l)[cfg.C:],
                                                  err_msg=f"ring step {step} b={bb} l={l}")
        assert a.status() == 0 and b.status() == 0
    finally:
        b.close()
        a.close()


@pytest.mark.parametrize("captured,k,direct", [(False, 1500, True), (True, 1500, True),
                                                (False, 1001, False), (True, 1500, False)])
def test_prefetch_schedule_against_the_oracle(captured, k, direct):
    """Shared selections, layer-wise prefetch: layer 0 resolved on the main
    stream, then every layer l+1 prefetched on a second stream and joined by
    its resolve.  Every step (eager, or one captured step replayed with
    eager copies in between) is compared with the oracle resolving every
    layer in order: slot maps, clocks, counters, eviction logs, LRU state,
    position->slot tables and slot bytes of every stream.  direct: the
    prefetch writes the slot-map buffer the join passes (the join is an event
    wait), else the library's own buffer (the join copies it; an odd k leaves
    the rows unaligned for its 16-byte copies, the scalar path)."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[4].scaled(B=3, layers=4, L0=30000, C=3000, k=k, steps=10)
    run = LockstepRun(cfg)
    try:
        main, side = torch.cuda.Stream(), torch.cuda.Stream()
        sel_buf = torch.empty_like(run.sel_dev[0])
        ctx_buf = torch.empty_like(run.ctx_dev[0])
        graph = None
        if captured:
            graph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.stream(main):
                with torch.cuda.graph(graph, stream=main):
                    run.prefetch_step(0, main.cuda_stream, side.cuda_stream, sel=sel_buf,
                                      ctx=ctx_buf, direct=direct)
            torch.cuda.synchronize()
        for s in range(cfg.steps):
            if captured:
                sel_buf.copy_(run.sel_dev[s])
                ctx_buf.copy_(run.ctx_dev[s])
                torch.cuda.synchronize()
                graph.replay()
            else:
                torch.cuda.synchronize()
                run.prefetch_step(s, main.cuda_stream, side.cuda_stream, direct=direct)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


@pytest.mark.parametrize("captured", [False, True])
def test_two_prefetches_in_flight_against_the_oracle(captured):
    """Two layers resolved at once: each layer l+1 is prefetched on one of
    two side streams before layer l is joined, so the launches of layers l and
    l+1 overlap on the GPU (with 8 requests the misses are copied by the
    resolve launches themselves).  Each layer keeps its own state, so every
    step must still equal the oracle resolving the layers in order."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[4].scaled(B=8, layers=5, L0=30000, C=3000, k=1500, steps=8)
    run = LockstepRun(cfg)
    try:
        main, sides = torch.cuda.Stream(), (torch.cuda.Stream(), torch.cuda.Stream())
        side_ptrs = tuple(x.cuda_stream for x in sides)
        sel_buf = torch.empty_like(run.sel_dev[0])
        ctx_buf = torch.empty_like(run.ctx_dev[0])
        graph = None
        if captured:
            graph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.stream(main):
                with torch.cuda.graph(graph, stream=main):
                    run.prefetch_ahead_step(0, main.cuda_stream, side_ptrs, sel=sel_buf, ctx=ctx_buf)
            torch.cuda.synchronize()
        for s in range(cfg.steps):
            if captured:
                sel_buf.copy_(run.sel_dev[s])
                ctx_buf.copy_(run.ctx_dev[s])
                torch.cuda.synchronize()
                graph.replay()
            else:
                torch.cuda.synchronize()
                run.prefetch_ahead_step(s, main.cuda_stream, side_ptrs)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_prefetch_over_a_growing_context_against_the_oracle():
    """Shared selections over a context that grows by one row per step: each
    layer's new row goes in through hisparse_append_resolve while the layer
    after it is prefetched on a second stream (the pending layers append in
    a launch of their own before the join).  Compared every step with the
    oracle appending and resolving every layer in order, resident ring and
    slot bytes included."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    from tests.harness import appended_row
    cfg = WORKLOADS[4].scaled(B=2, layers=3, L0=20000, growth=1, C=2500, k=1200, steps=7)
    run = LockstepRun(cfg)
    try:
        main, side = torch.cuda.Stream(), torch.cuda.Stream()
        h = run.gpu.h
        for s in range(cfg.steps):
            p = cfg.ctx_at(s) - 1
            rows = torch.from_numpy(np.stack([
                np.stack([appended_row(cfg, bb, l, p) for bb in range(cfg.B)])
                for l in range(cfg.layers)])).to("cuda")
            sel, ctx, pos, out = run.sel_dev[s], run.ctx_dev[s], run.pos_dev[s], run.out_dev
            torch.cuda.synchronize()
            ms, ss = main.cuda_stream, side.cuda_stream

            def call(l):
                if s > 0:
                    hb.hisparse_append_resolve(h, ms, l, rows[l].data_ptr(), pos.data_ptr(),
                                               sel[l].data_ptr(), ctx.data_ptr(),
                                               out[l].data_ptr())
                else:
                    hb.hisparse_resolve(h, ms, sel[l].data_ptr(), ctx.data_ptr(), l,
                                        out[l].data_ptr())

            call(0)
            for l in range(cfg.layers - 1):
                hb.hisparse_prefetch(h, ms, ss, sel[l + 1].data_ptr(), ctx.data_ptr(), l + 1)
                call(l + 1)
            torch.cuda.synchronize()
            if s > 0:
                run.oracle.append(s)
            run.compare_step(s, run.oracle_step(s))
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_append_resolve_after_a_prefetch_without_a_window_is_rejected():
    """Without a resident window the appended position may be selected, and
    a pending prefetch may already have read its host row: the call is
    rejected before anything is launched, and the prefetch can still be
    joined."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import GpuInstance
    cfg = WORKLOADS[1].scaled(layers=2, L0=5000, growth=1, C=512, k=256, steps=2)
    g = GpuInstance(cfg)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        pos = torch.full((cfg.B,), cfg.L0 - 1, dtype=torch.int32, device=dev)
        sel = torch.from_numpy(np.random.default_rng(5).choice(cfg.L0, (cfg.B, cfg.k),
                                                                replace=False).astype(np.int32)).to(dev)
        rows = torch.zeros((cfg.B, cfg.row_bytes), dtype=torch.uint8, device=dev)
        out = torch.empty_like(sel)
        side = torch.cuda.Stream()
        s = g.stream
        hb.hisparse_prefetch(g.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1)
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_append_resolve(g.h, s, 1, rows.data_ptr(), pos.data_ptr(),
                                       sel.data_ptr(), ctx.data_ptr(), out.data_ptr())
        assert e.value.code == hb.HISPARSE_ERR_STATE
        hb.hisparse_resolve(g.h, s, sel.data_ptr(), ctx.data_ptr(), 1, out.data_ptr())
        torch.cuda.synchronize()
        assert g.status() == 0
        assert bool((out >= 0).all())
    finally:
        g.close()


def test_prefetch_misuse_is_reported():
    torch, hb = _torch(), _hb()
    cfg = WORKLOADS[4].scaled(B=2, layers=2, L0=5000, steps=2)
    from tests.gpu_harness import GpuInstance
    g = GpuInstance(cfg)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        sel = torch.from_numpy(np.stack([np.random.default_rng(b).choice(cfg.L0 - 100, cfg.k,
                                        replace=False) for b in range(cfg.B)]).astype(np.int32)).to(dev)
        other = sel.flip(1).contiguous()
        out = torch.empty_like(sel)
        s = g.stream
        side = torch.cuda.Stream()
        hb.hisparse_prefetch(g.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1)
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_prefetch(g.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1)
        assert e.value.code == hb.HISPARSE_ERR_STATE
        hb.hisparse_resolve(g.h, s, other.data_ptr(), ctx.data_ptr(), 1, out.data_ptr())
        torch.cuda.synchronize()
        assert g.status(clear=True) & hb.HISPARSE_STATUS_PREFETCH_MISMATCH
        assert g.status() == 0
    finally:
        g.close()


def test_prefetch_into_the_callers_buffer_joins():
    """A prefetch told the joining call's slot-map buffer writes it directly;
    a join that passes another buffer gets a copy, and one that passes other
    selections is checked (with equal contents no status bit, with different
    contents PREFETCH_MISMATCH); the maps equal a plain resolve's."""
    torch, hb = _torch(), _hb()
    cfg = WORKLOADS[4].scaled(B=2, layers=4, L0=5000, steps=2)
    from tests.gpu_harness import GpuInstance
    a = GpuInstance(cfg)
    b = GpuInstance(cfg, hosts=a.hosts)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        _load_windows(a, ctx)
        _load_windows(b, ctx)
        sel = torch.from_numpy(np.stack([np.random.default_rng(7 + bb).choice(
            cfg.L0 - 100, cfg.k, replace=False) for bb in range(cfg.B)]).astype(np.int32)).to(dev)
        sel_same = sel.clone()              # another buffer, same contents
        other = sel.flip(1).contiguous()    # another buffer, other contents
        out = torch.full((cfg.layers, cfg.B, cfg.k), -7, dtype=torch.int32, device=dev)
        ref = torch.full_like(out, -9)
        side = torch.cuda.Stream()
        s = a.stream
        # layer 1: same buffers -> event wait only
        hb.hisparse_prefetch(a.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1,
                             out[1].data_ptr())
        hb.hisparse_resolve(a.h, s, sel.data_ptr(), ctx.data_ptr(), 1, out[1].data_ptr())
        # layer 2: written to a spare buffer, joined into out[2] -> copied
        spare = torch.full_like(out[2], -5)
        hb.hisparse_prefetch(a.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 2,
                             spare.data_ptr())
        hb.hisparse_resolve(a.h, s, sel.data_ptr(), ctx.data_ptr(), 2, out[2].data_ptr())
        # layer 3: same out, another selection buffer with the same contents
        hb.hisparse_prefetch(a.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 3,
                             out[3].data_ptr())
        hb.hisparse_resolve(a.h, s, sel_same.data_ptr(), ctx.data_ptr(), 3, out[3].data_ptr())
        hb.hisparse_resolve(a.h, s, sel.data_ptr(), ctx.data_ptr(), 0, out[0].data_ptr())
        torch.cuda.synchronize()
        assert a.status() == 0
        for l in range(cfg.layers):
            hb.hisparse_resolve(b.h, b.stream, sel.data_ptr(), ctx.data_ptr(), l, ref[l].data_ptr())
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(spare, ref[2])
        _assert_same_state(a, b, cfg)
        # a join with other contents in another buffer is reported
        hb.hisparse_prefetch(a.h, s, side.cuda_stream, sel.data_ptr(), ctx.data_ptr(), 1,
                             out[1].data_ptr())
        hb.hisparse_resolve(a.h, s, other.data_ptr(), ctx.data_ptr(), 1, out[1].data_ptr())
        torch.cuda.synchronize()
        assert a.status(clear=True) & hb.HISPARSE_STATUS_PREFETCH_MISMATCH
        assert a.status() == 0
    finally:
        b.close()
        a.close()


def test_no_io_equals_io_metadata_and_reads_nothing():
    torch, hb = _torch(), _hb()
    cfg = WORKLOADS[2].scaled(B=4, L0=20000, steps=10)
    a, b, trace = _pair(cfg, 0, hb.HISPARSE_NO_IO)
    try:
        dev = "cuda:0"
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
        _load_windows(a, ctx)
        b.cache.fill_(0xA5)           # no-IO instance: LRU slots must never change
        _load_windows(b, ctx)
        trace_dev = torch.from_numpy(trace).to(dev)
        out_a = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev)
        out_b = torch.empty_like(out_a)
        for step in range(cfg.steps):
            hb.hisparse_resolve(a.h, a.stream, trace_dev[step, 0].data_ptr(), ctx.data_ptr(), 0,
                                out_a.data_ptr())
            hb.hisparse_resolve(b.h, b.stream, trace_dev[step, 0].data_ptr(), ctx.data_ptr(), 0,
                                out_b.data_ptr())
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b)
            for bb in range(cfg.B):
                sa, sb = a.state(bb, 0), b.state(bb, 0)
                for key in ("slot2pos", "last_use", "order", "pos2slot"):
                    np.testing.assert_array_equal(sa[key], sb[key])
                np.testing.assert_array_equal(sa["hdr"][:7], sb["hdr"][:7])
                assert sb["hdr"][7] == 0 and sa["hdr"][7] == sa["hdr"][5] * cfg.row_bytes
                assert (b.slots(bb, 0)[: cfg.C] == 0xA5).all()
    finally:
        b.close()
        a.close()


@pytest.mark.parametrize("noncoherent", [False, True])
def test_hits_read_no_host_bytes(noncoherent):
    """After every step the host rows of every cached position are poisoned;
    hit slots must keep the bytes fetched earlier, and every slot must still
    match the oracle reading the same (poisoned) host memory."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=2, L0=12000, C=1024, k=512, steps=10)
    flags = hb.HISPARSE_HOST_NONCOHERENT if noncoherent else hb.HISPARSE_HOST_COHERENT
    run = LockstepRun(cfg, host_flags=flags)
    try:
        before = {}
        for s in range(cfg.steps):
            run.gpu_step(s)
            torch.cuda.synchronize()
            res = run.oracle_step(s)
            run.compare_step(s, res, host_rows=False)   # host rows are poisoned on purpose
            for (b, l), r in res.items():
                st = run.oracle.st[(b, l)]
                dev = run.gpu.slots(b, l)
                fetched = set(r.log_slot.tolist())
                hit_slots = [x for x in r.out.tolist() if 0 <= x < cfg.C and x not in fetched]
                for x in hit_slots:                       # bytes from before the poisoning
                    assert (dev[x] == before[(b, l)][x]).all(), f"hit slot {x} re-read host memory"
                held = st.slot2pos[st.slot2pos >= 0]
                run.gpu.host(b, l)[held] ^= 0x5A          # poison every cached position
                before[(b, l)] = dev.copy()
        assert run.gpu.status() == 0
    finally:
        run.close()


def test_invalid_rows_are_rejected_per_request():
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import GpuInstance
    cfg = WORKLOADS[2].scaled(B=3, L0=6000, C=512, k=256, steps=1)
    for flags in (0, hb.HISPARSE_DEBUG_VALIDATE):
        g = GpuInstance(cfg, flags=flags)
        try:
            dev = "cuda:0"
            rng = np.random.default_rng(11)
            sel = np.stack([rng.choice(cfg.L0, cfg.k, replace=False) for _ in range(cfg.B)]).astype(np.int32)
            ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device=dev)
            out = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev)
            # a clean first step everywhere
            hb.hisparse_resolve(g.h, g.stream, torch.from_numpy(sel).to(dev).data_ptr(),
                                ctx.data_ptr(), 0, out.data_ptr())
            torch.cuda.synchronize()
            snap = [g.state(b, 0) for b in range(cfg.B)]
            bad = sel.copy()
            bad[1, 17] = cfg.L0                  # out of range in request 1
            expect = hb.HISPARSE_STATUS_SEL_RANGE
            if flags & hb.HISPARSE_DEBUG_VALIDATE:
                bad[2, 5] = bad[2, 9]            # repeated position in request 2
                expect |= hb.HISPARSE_STATUS_SEL_DUP
            hb.hisparse_resolve(g.h, g.stream, torch.from_numpy(bad).to(dev).data_ptr(),
                                ctx.data_ptr(), 0, out.data_ptr())
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            assert (o[1] == -1).all()
            st1 = g.state(1, 0)
            for key in ("slot2pos", "last_use", "order", "pos2slot"):
                np.testing.assert_array_equal(st1[key], snap[1][key])
            assert st1["hdr"][0] == snap[1]["hdr"][0]          # clock not advanced
            assert st1["hdr"][1] == hb.HISPARSE_STATUS_SEL_RANGE
            assert g.state(0, 0)["hdr"][0] == snap[0]["hdr"][0] + 1   # request 0 ran
            if flags & hb.HISPARSE_DEBUG_VALIDATE:
                assert (o[2] == -1).all() and g.state(2, 0)["hdr"][1] == hb.HISPARSE_STATUS_SEL_DUP
            assert g.status(clear=True) == expect
            # a bad context length
            ctx_bad = torch.tensor([cfg.L0, cfg.l_cap + 1, -3], dtype=torch.int32, device=dev)
            hb.hisparse_resolve(g.h, g.stream, torch.from_numpy(sel).to(dev).data_ptr(),
                                ctx_bad.data_ptr(), 0, out.data_ptr())
            torch.cuda.synchronize()
            assert g.status(clear=True) & hb.HISPARSE_STATUS_CTX_RANGE
            o = out.cpu().numpy()
            assert (o[1] == -1).all() and (o[2] == -1).all() and (o[0] >= 0).all()
        finally:
            g.close()


def test_snapshot_restore_replays_identically():
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[2].scaled(B=2, L0=15000, steps=12)
    run = LockstepRun(cfg)
    try:
        for s in range(5):
            run.gpu_step(s)
        torch.cuda.synchronize()
        meta0, cache0 = run.gpu.meta.clone(), run.gpu.cache.clone()
        outs = []
        for s in range(5, cfg.steps):
            run.gpu_step(s)
            torch.cuda.synchronize()
            outs.append(run.out_dev.clone())
        meta1, cache1 = run.gpu.meta.clone(), run.gpu.cache.clone()
        run.gpu.meta.copy_(meta0)
        run.gpu.cache.copy_(cache0)
        torch.cuda.synchronize()
        for i, s in enumerate(range(5, cfg.steps)):
            run.gpu_step(s)
            torch.cuda.synchronize()
            assert torch.equal(run.out_dev, outs[i]), f"step {s}"
        assert torch.equal(run.gpu.meta, meta1) and torch.equal(run.gpu.cache, cache1)
    finally:
        run.close()


def test_reset_one_request_leaves_the_others():
    torch, hb = _torch(), _hb()
    from oracle.oracle import OracleStream
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[3].scaled(B=3, layers=2, L0=8000, C=1024, k=512, steps=8, growth=0)
    run = LockstepRun(cfg)
    try:
        for s in range(4):
            run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
        hb.hisparse_reset(run.gpu.h, run.gpu.stream, 1, 2)     # layer 1, request 2
        torch.cuda.synchronize()
        st = run.gpu.state(2, 1)
        assert (st["slot2pos"] == -1).all() and (st["pos2slot"] == -1).all()
        assert (st["last_use"] == 0).all() and (st["order"] == np.arange(cfg.C)).all()
        assert st["hdr"][0] == 0
        fresh = OracleStream(cfg.C, cfg.R, cfg.l_cap, cfg.row_bytes, host=run.gpu.host(2, 1))
        fresh.slots[:] = run.oracle.st[(2, 1)].slots   # the ring slots are not reset
        run.oracle.st[(2, 1)] = fresh
        for s in range(4, cfg.steps):
            run.gpu_step(s)
            torch.cuda.synchronize()
            run.compare_step(s, run.oracle_step(s))
    finally:
        run.close()


def test_timing_counts_every_launch():
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import LockstepRun
    cfg = WORKLOADS[3].scaled(B=2, layers=3, L0=5000, C=1024, k=512, steps=4, growth=0)
    run = LockstepRun(cfg, oracle_streams=[])
    try:
        hb.hisparse_set_timing(run.gpu.h, True)
        for s in range(cfg.steps):
            run.gpu_step(s)
        t = hb.hisparse_get_timing(run.gpu.h)
        assert t["resolve_launches"] == cfg.steps * cfg.layers
        assert t["fetch_launches"] == cfg.steps * cfg.layers
        assert t["resolve_ms"] > 0 and t["fetch_ms"] > 0
    finally:
        run.close()


def test_append_resolve_argument_checks():
    """hisparse_append_resolve rejects a bad layer, NULL buffers and
    misaligned rows before any launch, and leaves the streams untouched."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import GpuInstance
    cfg = WORKLOADS[3].scaled(B=2, layers=2, L0=3000, C=900, R=8, k=400, steps=2)
    g = GpuInstance(cfg)
    try:
        rows = torch.zeros(cfg.B * cfg.row_bytes + 16, dtype=torch.uint8, device="cuda")
        pos = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device="cuda")
        sel = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
        ctx = torch.full((cfg.B,), cfg.L0 + 1, dtype=torch.int32, device="cuda")
        out = torch.empty_like(sel)
        good = dict(layer=0, rows=rows.data_ptr(), pos=pos.data_ptr(), sel=sel.data_ptr(),
                    ctx=ctx.data_ptr(), out=out.data_ptr())
        for bad in (dict(layer=2), dict(layer=-1), dict(rows=0), dict(pos=0), dict(sel=0),
                    dict(ctx=0), dict(out=0), dict(rows=rows.data_ptr() + 4)):
            kw = dict(good, **bad)
            with pytest.raises(hb.HisparseError) as e:
                hb.hisparse_append_resolve(g.h, g.stream, kw["layer"], kw["rows"], kw["pos"],
                                           kw["sel"], kw["ctx"], kw["out"])
            assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG, bad
        torch.cuda.synchronize()
        for l in range(cfg.layers):
            for b in range(cfg.B):
                assert int(g.hdr(b, l)[hb.HDR_T]) == 0
        # a well-formed all-padding call: the clock ticks, the row lands
        rows[:cfg.B * cfg.row_bytes] = 7
        hb.hisparse_append_resolve(g.h, g.stream, 1, rows.data_ptr(), pos.data_ptr(),
                                   sel.data_ptr(), ctx.data_ptr(), out.data_ptr())
        torch.cuda.synchronize()
        assert (out == -1).all()
        for b in range(cfg.B):
            assert int(g.hdr(b, 1)[hb.HDR_T]) == 1
            assert (g.host(b, 1)[cfg.L0] == 7).all()
            assert (g.slots(b, 1)[cfg.C + cfg.L0 % cfg.R] == 7).all()
        assert g.status() == 0
    finally:
        g.close()


def test_overlapping_output_is_rejected():
    """out_slot sharing bytes with sel or ctx_len is refused on the host (the
    kernel reads them while it writes out_slot)."""
    torch, hb = _torch(), _hb()
    from tests.gpu_harness import GpuInstance
    cfg = WORKLOADS[2].scaled(B=2, L0=5000, C=800, R=8, k=256, steps=1)
    g = GpuInstance(cfg)
    try:
        buf = torch.full((3 * cfg.B * cfg.k,), -1, dtype=torch.int32, device="cuda")
        ctx = torch.full((cfg.B,), cfg.L0, dtype=torch.int32, device="cuda")
        sel = buf[:cfg.B * cfg.k]
        for out_ptr in (sel.data_ptr(), sel.data_ptr() + 4 * (cfg.B * cfg.k - 1), ctx.data_ptr()):
            with pytest.raises(hb.HisparseError) as e:
                hb.hisparse_resolve(g.h, g.stream, sel.data_ptr(), ctx.data_ptr(), 0, out_ptr)
            assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
            with pytest.raises(hb.HisparseError):
                hb.hisparse_resolve_multi(g.h, g.stream, sel.data_ptr(), 2, cfg.k // 2,
                                          ctx.data_ptr(), 0, out_ptr)
        # adjacent, not overlapping: accepted
        out = buf[cfg.B * cfg.k: 2 * cfg.B * cfg.k]
        hb.hisparse_resolve(g.h, g.stream, sel.data_ptr(), ctx.data_ptr(), 0, out.data_ptr())
        torch.cuda.synchronize()
        assert (out == -1).all() and int(g.hdr(0, 0)[hb.HDR_T]) == 1
        assert g.status() == 0
    finally:
        g.close()


@pytest.mark.parametrize("workgroups", [1, 7, 64])
def test_link_probe_copies_host_bytes_exactly(workgroups):
    """The link probe (the zero-copy read kernel the benchmark's link peak and
    counter scaling use) moves pinned host bytes to device memory unchanged,
    at any grid size, including a size that does not divide evenly."""
    torch, hb = _torch(), _hb()
    from hierarchical_kv_cache_hisparse_amd.instance import host_view
    nbytes = (3 << 20) + 16 * 37
    ptr = hb.hisparse_host_alloc(nbytes, hb.HISPARSE_HOST_COHERENT)
    try:
        view = host_view(ptr, nbytes)
        view[:] = np.random.default_rng(workgroups).integers(0, 256, nbytes, dtype=np.uint8)
        dev = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
        hb.hisparse_probe_host_read(torch.cuda.current_stream().cuda_stream, ptr, dev.data_ptr(),
                                    nbytes, workgroups)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dev.cpu().numpy(), view)
    finally:
        hb.hisparse_host_free(ptr)


def test_device_numa_node_is_a_host_node_or_none():
    """The GPU's NUMA node is -1 (the device reports none) or a node of this
    host."""
    import glob
    hb = _hb()
    _torch()
    node = hb.hisparse_device_numa_node()
    nodes = {int(p.rsplit("node", 1)[1]) for p in glob.glob("/sys/devices/system/node/node[0-9]*")}
    assert node == -1 or node in nodes, (node, nodes)

