"""Invariants of the method, checked on the oracle over reduced copies of the
five workloads (no GPU):

  I1 every served slot holds the bytes of the selected host row;
  I2 resident positions map to ring slot C + p mod R;
  I3 hits fetch nothing: bytes = n_miss * row_bytes;
  I5 attention through the slot map equals attention over the full history
     (the pages: only placement changes, outputs are unchanged);
  I8 copies suppressed (no-IO) leave every metadata output unchanged;
  I9 pos2slot and slot2pos are mutual inverses; the four classes add to k.
"""
import numpy as np
import pytest

from oracle.attention import bf16_to_f64, mla_decode_attention, masked_dense_attention
from tests.harness import OracleRun, fill_host, make_trace, small_variant
from workload import WORKLOADS


def _small(cfg_id):
    cfg = WORKLOADS[cfg_id]
    if cfg.row_elems > 576:   # page rows
        return small_variant(cfg, B=2, layers=2, L0=2048, C=64, k=32, steps=12)
    return small_variant(cfg, B=2, layers=2, L0=8192, C=768, k=384, steps=10)


def _hosts(cfg):
    return {(b, l): np.zeros((cfg.l_cap, cfg.row_bytes), np.uint8)
            for b in range(cfg.B) for l in range(cfg.layers)}


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_invariants_on_reduced_workloads(cfg_id):
    cfg = _small(cfg_id)
    streams = [(b, l) for b in range(cfg.B) for l in range(cfg.layers)]
    trace = make_trace(cfg)
    hosts = _hosts(cfg)
    fill_host(cfg, lambda b, l: hosts[(b, l)], trace, streams)
    run = OracleRun(cfg, streams, host_of=lambda b, l: hosts[(b, l)])
    meta_only = OracleRun(cfg, streams, with_data=False)
    for s in range(cfg.steps):
        if s > 0 and cfg.growth:
            run.append(s)
        ctx = cfg.ctx_at(s)
        res = run.step(s, trace)
        res_noio = meta_only.step(s, trace, no_io=True)
        for (b, l), r in res.items():
            st = run.st[(b, l)]
            sel = trace[s, l, b]
            assert r.status == 0
            c = r.counters
            # I9 (counts) and I3 (bytes)
            assert c["n_pad"] + c["n_res"] + c["n_hit"] + c["n_miss"] == cfg.k
            assert c["bytes"] == c["n_miss"] * cfg.row_bytes
            # I2
            res_mask = sel >= ctx - cfg.R if cfg.R else np.zeros_like(sel, bool)
            assert (r.out[res_mask] == cfg.C + sel[res_mask] % cfg.R).all()
            assert (r.out[~res_mask] < cfg.C).all() and (r.out >= 0).all()
            # I1
            host = hosts[(b, l)]
            assert (st.slots[r.out] == host[sel]).all()
            # I9 (inverse maps)
            held = np.nonzero(st.slot2pos >= 0)[0]
            assert (st.pos2slot[st.slot2pos[held]] == held).all()
            assert np.count_nonzero(st.pos2slot >= 0) == held.size
            # I8
            rn = res_noio[(b, l)]
            assert rn.counters["bytes"] == 0
            assert (rn.out == r.out).all()
            assert (rn.log_slot == r.log_slot).all() and (rn.log_old == r.log_old).all()
            sn = meta_only.st[(b, l)]
            assert (sn.pos2slot == st.pos2slot).all() and (sn.last_use == st.last_use).all()


def test_attention_through_slot_map_is_unchanged():
    """I5: gathered attention over the slots equals attention over the host
    rows at the selected positions bit for bit (same bytes, same order), and a
    masked dense attention over the whole history in position order agrees to
    rounding (float64, relative 1e-12)."""
    cfg = small_variant(WORKLOADS[2], B=1, layers=1, L0=4096, C=512, k=256, steps=6)
    streams = [(0, 0)]
    trace = make_trace(cfg)
    host = np.zeros((cfg.l_cap, cfg.row_bytes), np.uint8)
    # the dense reference reads every row, so fill the whole history
    from workload.rows import fill_range
    fill_range(host, cfg.row_elems, 0, cfg.l_cap, cfg.data_seed, 0, 0)
    run = OracleRun(cfg, streams, host_of=lambda b, l: host)
    st = run.st[(0, 0)]
    rng = np.random.default_rng(3002)
    q = rng.standard_normal((16, 576))
    scale = 1.0 / np.sqrt(576.0)
    all_rows = bf16_to_f64(host)
    for s in range(cfg.steps):
        r = run.step(s, trace)[(0, 0)]
        sel = trace[s, 0, 0]
        via_slots = mla_decode_attention(q, bf16_to_f64(st.slots[r.out]), scale)
        via_host = mla_decode_attention(q, bf16_to_f64(host[sel]), scale)
        assert np.array_equal(via_slots, via_host)
        mask = np.zeros(cfg.l_cap, bool)
        mask[sel] = True
        dense = masked_dense_attention(q, all_rows[: cfg.ctx_at(s)], mask[: cfg.ctx_at(s)], scale)
        np.testing.assert_allclose(via_slots, dense, rtol=1e-12, atol=1e-14)


def test_attention_check_detects_a_wrong_row():
    """The I5 check is sensitive: swapping one served row changes the output."""
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((64, 576))
    q = rng.standard_normal((4, 576))
    a = mla_decode_attention(q, rows, 0.05)
    bad = rows.copy()
    bad[10] = rng.standard_normal(576)
    assert not np.allclose(a, mla_decode_attention(q, bad, 0.05), rtol=1e-9)


def test_attention_lse_closed_forms():
    """lse of one row is its score; of n identical rows, score + log n; the
    output of identical rows is the row's latent part; no rows -> 0, -inf."""
    from oracle.attention import mla_decode_attention_lse
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 576))
    row = rng.standard_normal(576)
    out, lse = mla_decode_attention_lse(q, row[None, :], 0.1)
    np.testing.assert_allclose(lse, 0.1 * q @ row, rtol=1e-13)
    np.testing.assert_allclose(out, np.repeat(row[None, :512], 3, axis=0), rtol=1e-13)
    out, lse = mla_decode_attention_lse(q, np.repeat(row[None, :], 7, axis=0), 0.1)
    np.testing.assert_allclose(lse, 0.1 * q @ row + np.log(7), rtol=1e-13)
    out, lse = mla_decode_attention_lse(q, np.zeros((0, 576)), 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()
    # agrees with the plain version
    rows = rng.standard_normal((50, 576))
    o1 = mla_decode_attention(q, rows, 0.05)
    o2, _ = mla_decode_attention_lse(q, rows, 0.05)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
