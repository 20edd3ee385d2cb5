"""Checks that pin the CPU oracle to something other than itself.

Each function takes an oracle library handle (the normal build, or a copy
with a planted mistake) and raises AssertionError on disagreement.  Used by
the oracle tests and by the planted-mistake test, which checks that every
plausible mistake in the oracle is caught by at least one of these.
"""
from __future__ import annotations

import os

import numpy as np

from oracle.oracle import OracleStream, resolve_multi as _oracle_resolve_multi
from tests.bruteforce import BruteStream

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_golden(name: str):
    cfg, events = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("mstep"):
                ev = {}
                for part in line.split("|"):
                    key, *vals = part.split()
                    if key == "log":
                        ev[key] = [tuple(int(x) for x in v.split(":")) for v in vals]
                    elif key in ("sel", "out"):
                        ev[key] = [[int(x) for x in q.split()] for q in " ".join(vals).split(";")]
                    else:
                        ev[key] = [int(v) for v in vals]
                events.append(("mstep", ev))
            elif line.startswith("step"):
                ev = {}
                for part in line.split("|"):
                    key, *vals = part.split()
                    if key == "log":
                        ev[key] = [tuple(int(x) for x in v.split(":")) for v in vals]
                    else:
                        ev[key] = [int(v) for v in vals]
                events.append(("step", ev))
            elif line.startswith("append"):
                events.append(("append", int(line.split()[1])))
            else:
                key, val = line.split()
                cfg[key] = int(val)
    return cfg, events


def check_golden(name: str, lib=None):
    cfg, events = parse_golden(name)
    C, R, L = cfg["C"], cfg["R"], cfg["L"]
    row_bytes = 16
    host = np.zeros((L, row_bytes), np.uint8)
    for p in range(L):
        host[p] = (p * 7 + np.arange(row_bytes)) % 251
    st = OracleStream(C, R, L, row_bytes, host=host, lib=lib)
    first_ctx = next(ev["ctx"][0] for kind, ev in events if kind == "step")
    st.seed_window(first_ctx)
    fetched = evicted = 0
    for kind, ev in events:
        if kind == "append":
            row = ((ev * 13 + np.arange(row_bytes)) % 241).astype(np.uint8)
            st.append(row, ev)
            continue
        r = st.resolve(ev["sel"], ev["ctx"][0])
        assert r.status == 0, f"{name} step {ev['step']}: status {r.status}"
        assert r.out.tolist() == ev["out"], f"{name} step {ev['step']}: out {r.out.tolist()} != {ev['out']}"
        got_log = list(zip(r.log_slot.tolist(), r.log_old.tolist()))
        assert got_log == ev["log"], f"{name} step {ev['step']}: log {got_log} != {ev['log']}"
        assert st.slot2pos.tolist() == ev["slot2pos"], f"{name} step {ev['step']}: slot2pos"
        assert st.last_use.tolist() == ev["last_use"], f"{name} step {ev['step']}: last_use"
        assert int(st.t[0]) == ev["step"][0]
        assert r.counters["bytes"] == len(ev["log"]) * row_bytes
        fetched += r.counters["n_miss"]
        evicted += r.counters["n_evict"]
        # every served slot holds the row of the selected position
        for i, p in enumerate(ev["sel"]):
            if p >= 0:
                assert (st.slots[r.out[i]] == host[p]).all(), f"{name}: slot bytes of position {p}"
    return fetched, evicted


def _compare_with_brute(st: OracleStream, br: BruteStream, sel, ctx, where: str):
    r = st.resolve(sel, ctx)
    b = br.resolve(list(sel), ctx)
    if b is None:
        assert r.status != 0, f"{where}: oracle accepted an invalid row"
        return
    assert r.status == 0, f"{where}: oracle rejected a valid row"
    out, log = b
    assert r.out.tolist() == out, f"{where}: out {r.out.tolist()} != {out}"
    assert list(zip(r.log_slot.tolist(), r.log_old.tolist())) == log, f"{where}: eviction log"
    assert st.slot2pos.tolist() == br.slot2pos(), f"{where}: slot2pos"
    # pos2slot is the inverse of slot2pos
    inv = {p: s for s, p in enumerate(st.slot2pos.tolist()) if p >= 0}
    cached = {p: int(s) for p, s in enumerate(st.pos2slot.tolist()) if s >= 0}
    assert inv == cached, f"{where}: pos2slot is not the inverse of slot2pos"


def check_bruteforce_random(lib=None, n_traces: int = 300, seed: int = 7):
    """Random tiny traces: L <= 12, k <= 5, C in [k, k+4], R in {0..3},
    up to 25 steps, context growth, padding and occasional invalid rows."""
    rng = np.random.default_rng(seed)
    for n in range(n_traces):
        k = int(rng.integers(1, 6))
        C = k + int(rng.integers(0, 5))
        R = int(rng.integers(0, 4))
        L = int(rng.integers(max(k, 3), 13))
        grow = bool(rng.integers(0, 2))
        steps = int(rng.integers(3, 26))
        l_cap = L + (steps if grow else 0)
        st = OracleStream(C, R, l_cap, 16, lib=lib)
        br = BruteStream(C, R)
        ctx = L
        for s in range(steps):
            n_pad = int(rng.integers(0, k + 1)) if rng.random() < 0.2 else 0
            sel = list(rng.choice(ctx, k - n_pad, replace=False)) + [-1] * n_pad
            sel = [int(x) for x in rng.permutation(sel)]
            if rng.random() < 0.03:
                sel[int(rng.integers(0, k))] = ctx + int(rng.integers(0, 3))  # out of range
            _compare_with_brute(st, br, sel, ctx, f"trace {n} step {s}")
            if grow:
                ctx += 1


def check_bruteforce_exhaustive(lib=None):
    """Every 3-step sequence of ordered distinct pairs over 5 positions, for
    C in {2,3,4} and R in {0,1,2}; every 3-step sequence of single selections
    (padding included) over 7 positions for C in {1,2,3}, R in {0,1,2}."""
    import itertools
    L = 5
    pairs = [p for p in itertools.permutations(range(L), 2)]
    for C in (2, 3, 4):
        for R in (0, 1, 2):
            for seq in itertools.product(pairs, repeat=3):
                st = OracleStream(C, R, L, 16, lib=lib)
                br = BruteStream(C, R)
                for s, sel in enumerate(seq):
                    _compare_with_brute(st, br, list(sel), L, f"C{C} R{R} {seq} step {s}")
    L = 7
    singles = [(p,) for p in range(-1, L)]
    for C in (1, 2, 3):
        for R in (0, 1, 2):
            for seq in itertools.product(singles, repeat=3):
                st = OracleStream(C, R, L, 16, lib=lib)
                br = BruteStream(C, R)
                for s, sel in enumerate(seq):
                    _compare_with_brute(st, br, list(sel), L, f"C{C} R{R} {seq} step {s}")


def check_data_invariants(lib=None, seed: int = 3, steps: int = 12):
    """Slot bytes and byte counters on a small random trace with host data:
    every served slot holds the selected row's bytes; bytes = n_miss * row;
    hit slots keep their bytes; counters add up to k."""
    rng = np.random.default_rng(seed)
    C, R, L, k, rb = 24, 4, 200, 16, 32
    host = rng.integers(0, 256, (L + steps, rb), dtype=np.uint8)
    st = OracleStream(C, R, L + steps, rb, host=host, lib=lib)
    st.seed_window(L)
    ctx = L
    prev = rng.choice(ctx, k, replace=False)
    for s in range(steps):
        keep = rng.choice(prev, k // 2, replace=False)
        pool = np.setdiff1d(np.arange(ctx), keep)
        sel = rng.permutation(np.concatenate([keep, rng.choice(pool, k - k // 2, replace=False)]))
        before = st.slots.copy()
        r = st.resolve(sel, ctx)
        assert r.status == 0
        c = r.counters
        assert c["n_pad"] + c["n_res"] + c["n_hit"] + c["n_miss"] == k
        assert c["bytes"] == c["n_miss"] * rb
        missed = set(r.log_slot.tolist())
        for i, p in enumerate(sel):
            assert (st.slots[r.out[i]] == host[p]).all(), f"step {s}: slot of position {p}"
            if r.out[i] < C and r.out[i] not in missed:
                assert (st.slots[r.out[i]] == before[r.out[i]]).all(), "a hit changed slot bytes"
        # append one row and slide the window
        st.append(rng.integers(0, 256, rb, dtype=np.uint8), ctx)
        ctx += 1
        prev = sel


def check_validation(lib=None):
    """Invalid rows leave the state untouched and return -1 everywhere."""
    st = OracleStream(4, 1, 20, 16, lib=lib)
    r = st.resolve([3, 5], 10)
    assert r.status == 0
    snap = st.snapshot()
    for bad, ctx in (([3, 10], 10), ([3, -2], 10), ([4, 4], 10), ([1, 2], 21),
                     ([1, 2, 3, 4, 5], 10)):
        r = st.resolve(bad, ctx)
        assert r.status != 0, f"{bad} at ctx {ctx} accepted"
        assert (r.out == -1).all()
        for key, val in snap.items():
            assert (getattr(st, key) == val).all(), f"{key} changed by a rejected row"
    r = st.resolve([-1, -1], 10)
    assert r.status == 0 and r.out.tolist() == [-1, -1] and int(st.t[0]) == 2


def check_golden_multi(name: str = "multi_query_example.txt", lib=None, resolve_multi=None):
    """Hand-derived multi-query example: out per entry, status, eviction log,
    union counters, slot2pos, last_use, the clock, and the slot bytes."""
    resolve_multi = resolve_multi or _oracle_resolve_multi
    cfg, events = parse_golden(name)
    C, R, L = cfg["C"], cfg["R"], cfg["L"]
    row_bytes = 16
    host = np.zeros((L, row_bytes), np.uint8)
    for p in range(L):
        host[p] = (p * 5 + 3 * np.arange(row_bytes)) % 239
    st = OracleStream(C, R, L, row_bytes, host=host, lib=lib)
    st.seed_window(next(ev["ctx"][0] for kind, ev in events if kind == "mstep"))
    for kind, ev in events:
        assert kind == "mstep"
        where = f"{name} call at t={ev['mstep'][0]}"
        r = resolve_multi(st, np.array(ev["sel"]), ev["ctx"][0])
        assert r.status == ev["status"][0], f"{where}: status {r.status}"
        assert r.out.tolist() == ev["out"], f"{where}: out {r.out.tolist()} != {ev['out']}"
        got_log = list(zip(r.log_slot.tolist(), r.log_old.tolist()))
        assert got_log == ev["log"], f"{where}: log {got_log} != {ev['log']}"
        c = r.counters
        got = [c["n_pad"], c["n_res"], c["n_hit"], c["n_miss"], c["n_evict"]]
        assert got == ev["counts"], f"{where}: counters {got} != {ev['counts']}"
        assert st.slot2pos.tolist() == ev["slot2pos"], f"{where}: slot2pos"
        assert st.last_use.tolist() == ev["last_use"], f"{where}: last_use"
        assert int(st.t[0]) == ev["mstep"][0], f"{where}: clock {int(st.t[0])}"
        for q, row in enumerate(ev["sel"]):
            for i, p in enumerate(row):
                if p >= 0 and r.status == 0:
                    assert (st.slots[r.out[q, i]] == host[p]).all(), f"{where}: bytes of {p}"


def check_bruteforce_multi(lib=None, n_traces: int = 200, seed: int = 11, resolve_multi=None):
    """Random tiny multi-query traces (Q <= 3 queries of k <= 3 selections over
    few positions, so the queries overlap), checked against the brute-force
    entry-wise formulation: out per entry, eviction log, slot2pos and the
    distinct-position counters."""
    resolve_multi = resolve_multi or _oracle_resolve_multi
    rng = np.random.default_rng(seed)
    for n in range(n_traces):
        Q = int(rng.integers(1, 4))
        k = int(rng.integers(1, 4))
        C = Q * k + int(rng.integers(0, 3))
        R = int(rng.integers(0, 3))
        L = int(rng.integers(max(k, 3), 10))
        steps = int(rng.integers(2, 12))
        st = OracleStream(C, R, L, 16, lib=lib)
        br = BruteStream(C, R)
        for s in range(steps):
            sel = np.full((Q, k), -1, np.int32)
            for q in range(Q):
                n_sel = k if rng.random() < 0.8 else int(rng.integers(0, k + 1))
                sel[q, :n_sel] = rng.choice(L, n_sel, replace=False)
                sel[q] = rng.permutation(sel[q])
            if rng.random() < 0.03:
                sel[int(rng.integers(0, Q)), int(rng.integers(0, k))] = L + int(rng.integers(0, 2))
            where = f"multi trace {n} step {s}"
            r = resolve_multi(st, sel, L)
            b = br.resolve_multi(sel.tolist(), L)
            if b is None:
                assert r.status != 0 and (r.out == -1).all(), f"{where}: invalid call accepted"
                continue
            assert r.status == 0, f"{where}: valid call rejected"
            out, log, counts = b
            assert r.out.tolist() == out, f"{where}: out {r.out.tolist()} != {out}"
            assert list(zip(r.log_slot.tolist(), r.log_old.tolist())) == log, f"{where}: log"
            assert st.slot2pos.tolist() == br.slot2pos(), f"{where}: slot2pos"
            c = r.counters
            assert (c["n_pad"], c["n_res"], c["n_hit"], c["n_miss"]) == counts, f"{where}: counters"
