"""The oracle's multi-query step (several query tokens of a request resolved
in one step) against values fixed independently of it: a hand-derived
example, an entry-wise brute-force formulation, the cases that reduce to the
single-query step, and planted mistakes (no GPU)."""
import inspect

import numpy as np
import pytest

from oracle import oracle as oracle_mod
from oracle.oracle import OracleStream, StepResult, resolve_multi
from tests import pins


def test_multi_query_hand_example():
    pins.check_golden_multi()


def test_multi_query_bruteforce():
    pins.check_bruteforce_multi(n_traces=400)


def test_one_query_is_the_single_query_step():
    """Q = 1: the union is the selection row itself."""
    rng = np.random.default_rng(21)
    a = OracleStream(40, 3, 300, 16)
    b = OracleStream(40, 3, 300, 16)
    for s in range(30):
        ctx = 200 + s
        sel = rng.choice(ctx, 24, replace=False).astype(np.int32)
        sel[rng.random(24) < 0.1] = -1
        ra = resolve_multi(a, sel[None, :], ctx)
        rb = b.resolve(sel, ctx)
        assert ra.status == rb.status == 0
        assert np.array_equal(ra.out[0], rb.out)
        assert np.array_equal(ra.log_slot, rb.log_slot) and np.array_equal(ra.log_old, rb.log_old)
        assert ra.counters == rb.counters
        assert np.array_equal(a.pos2slot, b.pos2slot) and np.array_equal(a.last_use, b.last_use)


def test_repeated_query_is_the_single_query_step():
    """Q identical rows: every query is served exactly as the single step
    serves the row; the extra Q-1 copies count as padding."""
    rng = np.random.default_rng(22)
    a = OracleStream(64, 0, 500, 16)
    b = OracleStream(64, 0, 500, 16)
    for s in range(20):
        sel = rng.choice(500, 16, replace=False).astype(np.int32)
        ra = resolve_multi(a, np.stack([sel] * 3), 500)
        rb = b.resolve(sel, 500)
        assert (ra.out == rb.out[None, :]).all()
        assert np.array_equal(ra.log_slot, rb.log_slot)
        assert ra.counters["n_pad"] == rb.counters["n_pad"] + 2 * 16
        for key in ("n_res", "n_hit", "n_miss", "n_evict", "bytes"):
            assert ra.counters[key] == rb.counters[key]
        assert np.array_equal(a.slot2pos, b.slot2pos)


def test_cached_set_does_not_depend_on_entry_order():
    """The victim set is the first M unreferenced slots whatever order the
    distinct misses come in; only their pairing with the victims follows the
    order.  So, from the same state, permuting the entries changes which slot
    a position gets but not the set of cached positions nor the set of
    refilled slots (later steps then diverge: their hits land on other
    slots)."""
    rng = np.random.default_rng(23)
    a = OracleStream(30, 2, 100, 16)
    b = OracleStream(30, 2, 100, 16)
    for s in range(25):
        sel = np.stack([rng.choice(100, 5, replace=False) for _ in range(3)]).astype(np.int32)
        perm = rng.permutation(sel.reshape(-1)).reshape(sel.shape)
        b.restore(a.snapshot())
        ra = resolve_multi(a, sel, 100)
        rb = resolve_multi(b, perm, 100)
        assert set(ra.log_slot.tolist()) == set(rb.log_slot.tolist())
        assert set(np.nonzero(a.pos2slot >= 0)[0]) == set(np.nonzero(b.pos2slot >= 0)[0])
        assert ra.counters == rb.counters


def test_missing_row_is_fetched_once_and_served_to_every_entry():
    rng = np.random.default_rng(24)
    host = rng.integers(0, 256, (300, 32), dtype=np.uint8)
    st = OracleStream(48, 4, 300, 32, host=host)
    st.seed_window(300)
    for s in range(15):
        base = rng.choice(300, 12, replace=False)
        sel = np.stack([base, rng.permutation(base), rng.choice(300, 12, replace=False)])
        sel = sel.astype(np.int32)
        r = resolve_multi(st, sel, 300)
        assert r.status == 0
        distinct = np.unique(sel)
        assert r.counters["n_pad"] == sel.size - distinct.size
        assert r.counters["bytes"] == r.counters["n_miss"] * 32
        assert len(set(r.log_slot.tolist())) == r.counters["n_miss"]
        for q in range(3):
            for i in range(12):
                assert (st.slots[r.out[q, i]] == host[sel[q, i]]).all()
        # equal positions, equal slots
        for p in distinct:
            assert len(set(r.out[sel == p].tolist())) == 1


MULTI_MUTANTS = {
    "union_in_last_occurrence_order": ("for p in flat:\n", "for p in reversed(flat):\n"),
    "union_not_padded": ("r = stream.resolve(union, ctx", "r = stream.resolve(union[:len(first)], ctx"),
    "no_dedup_across_entries": ("if p != -1 and p not in first:", "if p != -1:"),
    "index_major_entries": ("flat = sel.reshape(-1).tolist()", "flat = sel.T.reshape(-1).tolist()"),
}


@pytest.mark.parametrize("name", sorted(MULTI_MUTANTS))
def test_planted_multi_mistake_is_caught(name):
    old, new = MULTI_MUTANTS[name]
    src = inspect.getsource(oracle_mod.resolve_multi)
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    ns = {"np": np, "StepResult": StepResult, "OracleStream": OracleStream}
    exec(src.replace(old, new), ns)
    bad = ns["resolve_multi"]
    with pytest.raises(Exception):
        pins.check_golden_multi(resolve_multi=bad)
        pins.check_bruteforce_multi(n_traces=150, resolve_multi=bad)
