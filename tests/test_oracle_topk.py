"""The top-k oracle (oracle/topk.py) against values fixed independently of
it: hand-derived examples, exhaustive search on tiny rows, the defining
property of the selected set on larger rows, closed forms and planted
mistakes (no GPU)."""
import inspect
import os

import numpy as np
import pytest

from oracle import topk as otopk
from oracle.topk import topk_select
from tests.bruteforce import brute_topk
from workload.scores import score_row

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "topk_hand_example.txt")


def _golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = [p.split() for p in line.split("|")]
        cases.append((parts[0][0], int(parts[1][1]), int(parts[2][1]),
                      np.array([float(x) for x in parts[3][1:]], np.float32),
                      [int(x) for x in parts[4][1:]]))
    return cases


def check_golden(fn=topk_select):
    for name, k, ctx, scores, out in _golden():
        assert fn(scores, ctx, k).tolist() == out, f"hand example {name}"


def check_brute(fn=topk_select, n: int = 400, seed: int = 5):
    rng = np.random.default_rng(seed)
    for t in range(n):
        ctx = int(rng.integers(0, 9))
        k = int(rng.integers(1, 7))
        vals = rng.choice([-np.inf, -2.0, -0.0, 0.0, 1.0, 1.5, 3.0, np.inf], ctx + 2)
        scores = vals.astype(np.float32)
        assert fn(scores, ctx, k).tolist() == brute_topk(scores, ctx, k), \
            f"trace {t}: {scores.tolist()} ctx {ctx} k {k}"


def check_defining_property(fn=topk_select, seed: int = 6):
    """The chosen set S (|S| = min(k, ctx)) is the top-k iff every chosen
    score >= every unchosen one, and at the boundary value every chosen
    position is lower than every unchosen position with that value."""
    for t, (n, k, kw) in enumerate([(5000, 300, {}), (5000, 300, {"ties": True}),
                                    (4097, 4096, {"ties": True, "specials": True}),
                                    (20000, 2048, {"ties": True, "specials": True}),
                                    (3000, 1, {"ties": True})]):
        s = score_row(n, seed, t, 0, 0, **kw)
        ctx = n - 3
        out = fn(s, ctx, k)
        chosen = out[out >= 0]
        assert chosen.size == min(k, ctx) and np.all(np.diff(chosen) > 0)
        mask = np.zeros(ctx, bool)
        mask[chosen] = True
        sc = s[:ctx].astype(np.float64)
        if mask.all():
            continue
        lo, hi = sc[mask].min(), sc[~mask].max()
        assert lo >= hi, f"case {t}: a chosen score is below an unchosen one"
        if lo == hi:
            tie_in = np.nonzero(mask & (sc == lo))[0]
            tie_out = np.nonzero(~mask & (sc == lo))[0]
            assert tie_in.max() < tie_out.min(), f"case {t}: tie not broken by position"


def test_topk_hand_examples():
    check_golden()


def test_topk_matches_exhaustive_search():
    check_brute()


def test_topk_defining_property():
    check_defining_property()


def test_topk_closed_forms():
    n = 1000
    dec = np.linspace(5, -5, n).astype(np.float32)
    assert topk_select(dec, n, 100).tolist() == list(range(100))
    assert topk_select(dec[::-1].copy(), n, 100).tolist() == list(range(900, 1000))
    assert topk_select(np.ones(n, np.float32), n, 77).tolist() == list(range(77))
    assert topk_select(dec, 40, 100).tolist() == list(range(40)) + [-1] * 60
    assert topk_select(dec, 0, 5).tolist() == [-1] * 5
    # distinct scores: the set equals numpy's argpartition set
    s = score_row(10000, 9, 0, 0, 0)
    want = np.sort(np.argpartition(-s.astype(np.float64), 500)[:500])
    assert topk_select(s, 10000, 500).tolist() == want.tolist()


def test_topk_rejects_nan():
    with pytest.raises(ValueError):
        topk_select(np.array([1.0, np.nan], np.float32), 2, 1)


TOPK_MUTANTS = {
    "ties_to_higher_position": ("order = np.lexsort((pos, -s))", "order = np.lexsort((-pos, -s))"),
    "smallest_scores": ("order = np.lexsort((pos, -s))", "order = np.lexsort((pos, s))"),
    "score_order_output": ("chosen = np.sort(order[:k])", "chosen = order[:k]"),
    "ctx_ignored": ("s = np.asarray(scores, dtype=np.float64)[:ctx]",
                    "s = np.asarray(scores, dtype=np.float64)[:ctx + 1][:ctx]\n"
                    "    s = np.asarray(scores, dtype=np.float64)[:len(scores)]"),
    "signed_zero_ordered": ("order = np.lexsort((pos, -s))",
                            "order = np.lexsort((pos, -s - 1e-300 * np.signbit(s)))"),
    "off_by_one_k": ("chosen = np.sort(order[:k])", "chosen = np.sort(order[:max(k - 1, 1)])"),
}


@pytest.mark.parametrize("name", sorted(TOPK_MUTANTS))
def test_planted_topk_mistake_is_caught(name):
    old, new = TOPK_MUTANTS[name]
    src = inspect.getsource(otopk.topk_select)
    assert src.count(old) == 1, name
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    bad = ns["topk_select"]
    caught = False
    for check in (check_golden, check_brute, check_defining_property):
        try:
            check(bad)
        except (AssertionError, ValueError):
            caught = True
            break
    assert caught, f"mistake {name} not caught"
