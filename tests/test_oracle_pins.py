"""The CPU oracle against values fixed independently of it: hand-derived
examples, closed forms and degenerate cases (no GPU)."""
import numpy as np
import pytest

from oracle.oracle import OracleStream
from tests import pins
from workload import WORKLOADS
from workload.traces import stream_trace


def test_lru_hand_example():
    fetched, evicted = pins.check_golden("lru_hand_example.txt")
    assert (fetched, evicted) == (7, 4)


def test_resident_window_example():
    pins.check_golden("resident_window_example.txt")


def test_validation_leaves_state_untouched():
    pins.check_validation()


def test_no_eviction_closed_form_config1():
    """When C covers every distinct non-resident position ever selected, the
    n-th distinct position (in step, then selection order) takes slot n-1 and
    nothing is evicted.  The 1-request workload (C=4096, k=2048, 8 steps, 90%
    carry-over) is such a case."""
    cfg = WORKLOADS[1]
    trace = stream_trace(cfg, 0, 0)
    st = OracleStream(cfg.C, cfg.R, cfg.l_cap, cfg.row_bytes)
    first_seen = {}
    for s in range(cfg.steps):
        for p in trace[s].tolist():
            if p not in first_seen:
                first_seen[p] = len(first_seen)
        r = st.resolve(trace[s], cfg.ctx_at(s))
        assert r.status == 0
        assert r.counters["n_evict"] == 0
        assert (r.log_old == -1).all()
        expect = np.array([first_seen[p] for p in trace[s].tolist()], np.int32)
        assert (r.out == expect).all()
    assert len(first_seen) < cfg.C
    assert st.slot2pos[: len(first_seen)].tolist() == list(first_seen.keys())
    assert (st.slot2pos[len(first_seen):] == -1).all()


def test_full_carry_over_hits_everything():
    """Repeating the same selection: after the first step every row hits and
    no byte is fetched."""
    rng = np.random.default_rng(0)
    C, k, L, rb = 64, 48, 1000, 32
    host = rng.integers(0, 256, (L, rb), dtype=np.uint8)
    st = OracleStream(C, 0, L, rb, host=host)
    sel = rng.choice(L, k, replace=False)
    r0 = st.resolve(sel, L)
    assert r0.counters["n_miss"] == k and r0.counters["bytes"] == k * rb
    for _ in range(5):
        r = st.resolve(rng.permutation(sel), L)
        assert r.counters["n_hit"] == k and r.counters["n_miss"] == 0
        assert r.counters["bytes"] == 0


def test_cache_equal_to_k_with_fresh_rows():
    """C = k and all-new positions every step: every slot is evicted each step
    and the j-th miss takes slot j."""
    C = k = 16
    L = 16 * 10
    st = OracleStream(C, 0, L, 16)
    for s in range(10):
        sel = np.arange(s * k, (s + 1) * k)[::-1].copy()
        r = st.resolve(sel, L)
        assert r.out.tolist() == list(range(k))
        assert r.log_slot.tolist() == list(range(k))
        assert r.counters["n_evict"] == (0 if s == 0 else k)
        if s:
            assert r.log_old.tolist() == list(range((s - 1) * k, s * k))[::-1]


def test_window_covering_context_is_all_resident():
    """R >= ctx: every valid position is resident at C + p mod R; the LRU
    state never changes except for the clock."""
    C, R, k = 8, 32, 8
    st = OracleStream(C, R, 64, 16)
    rng = np.random.default_rng(1)
    for s, ctx in enumerate((8, 20, 32)):
        sel = rng.choice(ctx, k, replace=False)
        r = st.resolve(sel, ctx)
        assert r.out.tolist() == [C + p % R for p in sel]
        assert r.counters["n_res"] == k
        assert (st.slot2pos == -1).all() and (st.last_use == 0).all()
        assert int(st.t[0]) == s + 1


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_config_step0_fills_free_slots_in_order(cfg_id):
    """Closed form for the first step of every workload: all non-resident
    selections miss and take free slots 0, 1, 2, ... in selection order."""
    cfg = WORKLOADS[cfg_id]
    trace = stream_trace(cfg, 0, 0, steps=1)
    st = OracleStream(cfg.C, cfg.R, cfg.l_cap, cfg.row_bytes)
    r = st.resolve(trace[0], cfg.ctx_at(0))
    ctx = cfg.ctx_at(0)
    nxt = 0
    for i, p in enumerate(trace[0].tolist()):
        if cfg.R > 0 and p >= ctx - cfg.R:
            assert r.out[i] == cfg.C + p % cfg.R
        else:
            assert r.out[i] == nxt
            nxt += 1
    assert r.counters["n_miss"] == nxt and r.counters["n_evict"] == 0
