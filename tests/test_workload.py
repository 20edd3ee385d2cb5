"""The seeded input generators: traces keep their stated structure and the
row generator is deterministic, subset-consistent and N(0,1)-distributed
(no GPU)."""
import numpy as np
import pytest

from workload import WORKLOADS
from workload import rows as wrows
from workload.traces import full_trace, stream_trace, touched_positions


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_trace_structure(cfg_id):
    cfg = WORKLOADS[cfg_id]
    tr = stream_trace(cfg, 0, 0)
    assert tr.shape == (cfg.steps, cfg.k) and tr.dtype == np.int32
    for s in range(cfg.steps):
        row = tr[s]
        assert np.unique(row).size == cfg.k
        assert row.min() >= 0 and row.max() < cfg.ctx_at(s)
        if s:
            assert np.intersect1d(row, tr[s - 1]).size == cfg.n_keep
    assert np.array_equal(tr, stream_trace(cfg, 0, 0))
    assert not np.array_equal(tr, stream_trace(cfg, 1, 0))


def test_carry_counts_match_the_stated_fractions():
    assert [WORKLOADS[c].n_keep for c in (1, 2, 3, 4, 5)] == [1843, 1740, 1638, 1536, 89]


def test_shared_and_independent_layers():
    cfg4 = WORKLOADS[4].scaled(steps=3, B=2)
    t4 = full_trace(cfg4)
    assert all(np.array_equal(t4[:, 0], t4[:, l]) for l in range(cfg4.layers))
    cfg3 = WORKLOADS[3].scaled(steps=3, B=2, layers=3)
    t3 = full_trace(cfg3)
    assert not np.array_equal(t3[:, 0], t3[:, 1])


def test_zipf_replacements_favour_recent_positions():
    cfg = WORKLOADS[4].scaled(steps=8)
    tr = stream_trace(cfg, 0, 0)
    dist = cfg.L0 - tr[1:].astype(np.int64)
    # uniform would put ~1.6% of the positions within 4096 of the end; Zipf(1.0)
    # distances, thinned by the distinctness rejection, put ~40% there
    assert np.mean(dist <= 4096) > 0.3


def test_mix_replacements_are_half_uniform():
    cfg = WORKLOADS[2].scaled(steps=6)
    tr = stream_trace(cfg, 0, 0)
    far = np.mean(cfg.L0 - tr[0].astype(np.int64) > cfg.L0 // 2)
    # the uniform half lands in the older half about half the time (~25%);
    # the Zipf(1.1) half almost never does
    assert 0.15 < far < 0.35


def test_growth_workload_uses_current_context():
    cfg = WORKLOADS[3]
    assert cfg.l_cap == 131072 + 31
    assert cfg.ctx_at(31) == 131103


def test_row_fill_subset_and_append_consistency():
    n, elems = 300, 576
    full = np.zeros((n, 2 * elems), np.uint8)
    wrows.fill_range(full, elems, 0, n, 99, 3, 4)
    part = np.zeros_like(full)
    wrows.fill_rows(part, elems, [5, 77, 299], 99, 3, 4)
    for p in (5, 77, 299):
        assert np.array_equal(part[p], full[p])
        assert np.array_equal(wrows.make_row(elems, p, 99, 3, 4), full[p])
    assert not part[6].any()
    other = np.zeros_like(full)
    wrows.fill_range(other, elems, 0, n, 99, 3, 5)
    assert not np.array_equal(other, full)


def test_row_values_are_standard_normal_bf16():
    n, elems = 2000, 576
    raw = np.zeros((n, 2 * elems), np.uint8)
    wrows.fill_range(raw, elems, 0, n, 2002, 0, 0)
    x = wrows.bf16_bytes_to_f64(raw).ravel()
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1.0) < 0.01
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 0.01
    # every value is exactly representable in bf16: low 16 bits of f32 are 0
    f32 = x.astype(np.float32).view(np.uint32)
    assert not (f32 & 0xFFFF).any()


def test_touched_positions_cover_window_and_selections():
    cfg = WORKLOADS[2].scaled(steps=3)
    tr = stream_trace(cfg, 0, 0)
    pos = touched_positions(tr, cfg)
    assert set(np.unique(tr).tolist()) <= set(pos.tolist())
    assert set(range(cfg.L0 - cfg.R, cfg.L0)) <= set(pos.tolist())
