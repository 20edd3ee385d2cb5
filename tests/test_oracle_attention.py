"""Pins of the float64 sparse-MLA decode attention oracle (oracle/attention.py),
the reference the GPU attention is checked against.

The page the exactness claim comes from ("HiSparse: Scaling Sparse-Attention
Decoding with Hierarchical KV Cache Management", Abstract: only KV placement
changes, so outputs are unchanged) fixes no attention formula of its own; the
oracle is the textbook softmax attention over sparse-MLA rows (576 values:
512 latent values that are both key and value, 64 rope values that are key
only).  Pinned here against things other than itself:

  * bf16 decoding against the bfloat16 format's definition (sign, 8-bit
    exponent with bias 127, 7-bit fraction; the top half of an IEEE binary32)
    on hand-decoded bit patterns, subnormals and infinities included;
  * closed forms with two rows of different scores a and b:
    out = (e^a v1 + e^b v2) / (e^a + e^b), lse = log(e^a + e^b), with the
    score carried by a rope coordinate and, separately, by a latent one;
  * reduction to library routines: the weights equal scipy.special.softmax of
    the scaled scores and lse equals scipy.special.logsumexp, on random rows;
  * planted mistakes (natural base replaced by 2, a stray temperature, a
    score over the 512 latent values only, the wrong value slice, lse without
    its maximum, unnormalised weights, byte-swapped bf16) must each fail one
    of the above.
"""
import importlib.util
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention.py")

# (bf16 bit pattern, value), decoded by hand from the format: value =
# (-1)^sign * 2^(exp - 127) * (1 + frac/128), or 2^-126 * frac/128 when exp = 0
BF16_PINS = [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x4049, 3.140625),                   # 2^1 * (1 + 73/128)
    (0x3E80, 0.25),
    (0xBF40, -0.75),                      # -(2^-1 * (1 + 64/128))
    (0x0000, 0.0),
    (0x8000, -0.0),
    (0x0001, 2.0 ** -133),                # smallest subnormal: 2^-126 * 1/128
    (0x007F, 2.0 ** -126 * 127 / 128),    # largest subnormal
    (0x0080, 2.0 ** -126),                # smallest normal
    (0x7F7F, 2.0 ** 127 * (1 + 127 / 128)),   # largest finite
    (0x7F80, np.inf),
    (0xFF80, -np.inf),
]


def _load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _two_row_case(dim, a, b, scale, rng):
    """q = e_dim; rows whose only score-carrying value sits at `dim`, chosen so
    the scaled scores are exactly a and b; distinct latent parts."""
    q = np.zeros((1, 576))
    q[0, dim] = 1.0
    rows = rng.standard_normal((2, 576))
    rows[:, dim] = [a / scale, b / scale]
    return q, rows, rows[:, :512]   # a latent score coordinate is part of the value too


def check_bf16(mod):
    raw = np.array([p for p, _ in BF16_PINS], "<u2").view(np.uint8).reshape(-1, 2)
    got = mod.bf16_to_f64(raw).reshape(-1)
    for (pat, want), g in zip(BF16_PINS, got):
        assert g == want and np.signbit(g) == np.signbit(want), (hex(pat), g, want)
    # a 2-row array of 3 values each keeps its shape and order
    two = np.array([[0x3F80, 0xC000, 0x4049], [0x0080, 0x7F80, 0x8000]], "<u2")
    out = mod.bf16_to_f64(two.view(np.uint8))
    assert out.shape == (2, 3) and out[0, 2] == 3.140625 and out[1, 1] == np.inf


def check_closed_forms(mod):
    rng = np.random.default_rng(11)
    scale = 1.0 / 24.0
    for dim in (540, 7):                  # a rope coordinate, then a latent one
        for a, b in ((0.7, -1.3), (2.5, 2.0), (-3.0, 1.0)):
            q, rows, v = _two_row_case(dim, a, b, scale, rng)
            want = (np.exp(a) * v[0] + np.exp(b) * v[1]) / (np.exp(a) + np.exp(b))
            want_lse = np.log(np.exp(a) + np.exp(b))
            out, lse = mod.mla_decode_attention_lse(q, rows, scale)
            np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-14,
                                       err_msg=f"two-row output, dim {dim}")
            np.testing.assert_allclose(lse[0], want_lse, rtol=1e-12, err_msg="two-row lse")
            plain = mod.mla_decode_attention(q, rows, scale)
            np.testing.assert_allclose(plain[0], want, rtol=1e-12, atol=1e-14,
                                       err_msg=f"two-row output (plain), dim {dim}")


def check_library_reduction(mod):
    rng = np.random.default_rng(12)
    for n, H, scale in ((5, 3, 0.05), (64, 4, 1.0 / 24.0), (200, 2, 0.2)):
        q = rng.standard_normal((H, 576))
        rows = rng.standard_normal((n, 576))
        s = scale * q @ rows.T                       # [H, n]
        w = softmax(s, axis=1)
        want = w @ rows[:, :512]
        out, lse = mod.mla_decode_attention_lse(q, rows, scale)
        np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-13, err_msg="softmax weights")
        np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-12, err_msg="logsumexp")
        np.testing.assert_allclose(mod.mla_decode_attention(q, rows, scale), want, rtol=1e-10,
                                   atol=1e-13, err_msg="softmax weights (plain)")


def check_all(mod):
    check_bf16(mod)
    check_closed_forms(mod)
    check_library_reduction(mod)


def test_oracle_attention_passes_its_pins():
    check_all(_load(SRC, "attention_under_test"))


MUTANTS = {
    "exp_base_two_lse": ("        e = np.exp(score - m)\n", "        e = np.exp2(score - m)\n"),
    "exp_base_two_plain": ("        w = np.exp(score - score.max())\n",
                           "        w = np.exp2(score - score.max())\n"),
    "temperature_lse": ("        score = scale * (rows * q[h][None, :]).sum(axis=1)\n        m = ",
                        "        score = 0.9 * scale * (rows * q[h][None, :]).sum(axis=1)\n        m = "),
    "temperature_plain": ("        score = scale * (rows * q[h][None, :]).sum(axis=1)\n        w = ",
                          "        score = scale * scale * (rows * q[h][None, :]).sum(axis=1)\n"
                          "        w = "),
    "score_over_latent_only": (
        "        score = scale * (rows * q[h][None, :]).sum(axis=1)\n        m = ",
        "        score = scale * (rows[:, :D_LATENT] * q[h][None, :D_LATENT]).sum(axis=1)\n"
        "        m = "),
    "value_slice_shifted": ("        out[h] = ((e / z)[:, None] * rows[:, :D_LATENT]).sum(axis=0)\n",
                            "        out[h] = ((e / z)[:, None] * rows[:, 64:]).sum(axis=0)\n"),
    "lse_without_max": ("        lse[h] = m + np.log(z)\n", "        lse[h] = np.log(z)\n"),
    "weights_not_normalised": (
        "        out[h] = ((e / z)[:, None] * rows[:, :D_LATENT]).sum(axis=0)\n",
        "        out[h] = (e[:, None] * rows[:, :D_LATENT]).sum(axis=0)\n"),
    "bf16_bytes_swapped": ("    u16 = np.ascontiguousarray(raw).view(np.uint16)\n",
                           "    u16 = np.ascontiguousarray(raw).view(np.uint16).byteswap()\n"),
    "bf16_shift_wrong": ("(u16.astype(np.uint32) << 16)", "(u16.astype(np.uint32) << 15)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_attention_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / f"attention_{name}.py"
    path.write_text(src.replace(old, new))
    mod = _load(str(path), f"attention_{name}")
    with pytest.raises(AssertionError):
        check_all(mod)
