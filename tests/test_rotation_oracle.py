"""Pins of the rotation oracle (oracle/rotation.py), on the CPU.

Checked against what does not come from the oracle's own code: scipy's
Hadamard matrix, the closed form (-1)^popcount(i & j) of its entries,
orthogonality, closed-form rotations of one-hot rows, exact sums that
float64 cannot hold (a tie of fp32 that an extra 2^-80 breaks), the
invariance of attention, and the quantised bytes of a rotated one-hot
block.  Planted mistakes in the oracle must each trip at least one pin.
"""
import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import oracle.rotation as rot
import workloads as W

_rng = np.random.default_rng(2024)


def _signs(d, seed=0):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1, 1)


def pin_scipy_hadamard():
    from scipy.linalg import hadamard
    for d in (1, 2, 4, 8, 16, 64, 128, 256):
        assert np.array_equal(rot.hadamard(d), hadamard(d))


def pin_entry_closed_form():
    d = 128
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    par = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(rot.hadamard(d), np.where(par == 1, -1, 1))


def pin_orthogonal():
    for d in (16, 64, 128):
        m = rot.rotation_matrix(_signs(d, d))
        assert np.array_equal(m @ m.T, d * np.eye(d, dtype=np.int64))


def pin_one_hot_rows():
    # e_k diag(s) H = s_k H[k, :]; row 0 of H is all ones, row d-1 alternates
    # with the parity of popcount(j & (d - 1)) = popcount(j)
    d = 128
    s = _signs(d, 7)
    for k in (0, 1, d - 1):
        x = np.zeros((1, d))
        x[0, k] = 2.0
        y = rot.rotate(x, s)
        if k == 0:
            assert np.array_equal(y[0], np.full(d, 2.0 * s[0], np.float32))
        if k == d - 1:
            want = [2.0 * s[k] * (-1) ** bin(j).count("1") for j in range(d)]
            assert np.array_equal(y[0], np.asarray(want, np.float32))
        assert np.array_equal(np.abs(y[0]), np.full(d, 2.0, np.float32))


def pin_inner_products_scale_by_d():
    d = 64
    s = _signs(d, 3)
    x = _rng.integers(-8, 9, size=(5, d)).astype(np.float64)
    y = _rng.integers(-8, 9, size=(7, d)).astype(np.float64)
    rx, ry = rot.rotate(x, s).astype(np.float64), rot.rotate(y, s).astype(np.float64)
    assert np.array_equal(rx @ ry.T, d * (x @ y.T))


def pin_exact_sum_beyond_float64():
    d = 16
    s = np.ones(d, dtype=np.int64)
    x = np.zeros((1, d))
    x[0, :3] = [1.0, 2.0 ** -24, 2.0 ** -80]        # bf16 values, 80 binades apart
    y = rot.rotate(x, s)
    # column 0: 1 + 2^-24 + 2^-80 lies above the fp32 midpoint 1 + 2^-24
    assert y[0, 0] == np.float32(1.0 + 2.0 ** -23)
    # column 1: 1 - 2^-24 + 2^-80, nearest fp32 is 1 - 2^-24
    assert y[0, 1] == np.float32(1.0 - 2.0 ** -24)


def pin_bf16_rows_against_float32_of_exact():
    # bf16 rows within 38 binades: the float64 sum is exact, so numpy's
    # float64 -> float32 conversion of a plain loop sum is the RN result
    d = 128
    s = _signs(d, 11)
    bits = W.normal_bf16(77, (4, d), outliers=True)
    x = W.bf16_bits_to_f32(bits).astype(np.float64)
    h = [[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)]
    want = np.zeros((4, d), np.float32)
    for r in range(4):
        for j in range(d):
            acc = 0.0
            for i in range(d):
                acc += x[r, i] * s[i] * h[i][j]
            want[r, j] = np.float32(acc)
    assert np.array_equal(rot.rotate(x, s), want)


def pin_attention_invariant():
    B, N, H, d = 1, 9, 2, 16
    s = _signs(d, 5)
    q, k = (_rng.integers(-3, 4, size=(B, N, H, d)).astype(np.float64) for _ in range(2))
    v = _rng.standard_normal((B, N, H, d))
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, 0.25, causal=causal)
        o2, l2 = oracle.attention(rot.rotate(q, s).astype(np.float64), rot.rotate(k, s).astype(np.float64), v,
                                  0.25 / d, causal=causal)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def pin_rotated_one_hot_block():
    # every token row one-hot at coordinate 0 with value 3: every rotated
    # value is 3 s_0, so the block maximum is 3, s = fp32(3 / 448), and every
    # byte is +-448 (0x7E, or 0xFE when s_0 = -1)
    d = 64
    s = _signs(d, 1)
    s[0] = -1
    x = np.zeros((1, 130, 2, d))
    x[..., 0] = 3.0
    q, sc = rot.rotate_quantize_blocks(x, s)
    assert np.all(q == 0xFE)
    assert np.all(sc == np.float32(np.float32(3.0) / np.float32(448.0)))


def pin_zero_rows_are_positive_zero():
    # all-zero rows: every rotated value is exactly zero, stored as +0, so
    # every byte is 0x00 whatever the signs (all negative included)
    d = 64
    x = np.zeros((1, 128, 1, d))
    for s in (np.full(d, -1), _signs(d, 4)):
        y = rot.rotate(x, s)
        assert not np.any(np.signbit(y))
        q, sc = rot.rotate_quantize_blocks(x, s)
        assert np.all(q == 0) and np.all(sc == 1.0)


def pin_outlier_spread():
    # the purpose: one +-20 outlier in a row of N(0,1) values dominates the
    # row's maximum; after the rotation the maximum over the rms is small
    d = 128
    x = _rng.standard_normal((64, d))
    x[np.arange(64), _rng.integers(0, d, 64)] = 20.0
    y = rot.rotate(x, _signs(d, 9)).astype(np.float64)
    ratio = lambda a: np.max(np.abs(a), axis=1) / np.sqrt(np.mean(a * a, axis=1))
    assert np.median(ratio(x)) > 7.0 and np.median(ratio(y)) < 4.0


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---- planted mistakes -----------------------------------------------------

def _mutants():
    h0 = rot.hadamard
    return {
        "signs_after_h": ("rotation_matrix",
                          lambda s: rot.hadamard(len(s)) * np.asarray(s, np.int64)[None, :]),
        "normalised": ("rotation_matrix",
                       lambda s: np.asarray(s, np.int64)[:, None] * h0(len(s)) / np.sqrt(len(s))),
        "other_sylvester": ("hadamard",
                            lambda d: h0(d) if d < 2 else np.block([[h0(d // 2), h0(d // 2)],
                                                                   [-h0(d // 2), h0(d // 2)]])),
        "quantise_first": ("rotate_quantize_blocks",
                           lambda x, s, cu=None: oq.quantize_blocks(x, cu)),
        "double_rounding": ("_round_fraction_to_f32", lambda fr: np.float32(float(fr))),
    }


@pytest.mark.parametrize("kind", list(_mutants()))
def test_mutant_is_caught(kind, monkeypatch):
    name, fn = _mutants()[kind]
    monkeypatch.setattr(rot, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every rotation pin"


def _scattered_outliers(seed, shape, mag):
    """N(0,1) bf16 with 1 % of the entries set to +-mag at random positions."""
    g = np.random.default_rng(seed)
    x = W.bf16_bits_to_f32(W.normal_bf16(seed, shape)).astype(np.float32)
    hit = g.random(shape) < 0.01
    x = np.where(hit, np.where(g.random(shape) < 0.5, -mag, mag), x).astype(np.float32)
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("mag", [20.0, 20000.0])
def test_rotation_does_not_help_scattered_outliers(mag):
    """The reason the fp8 workload keeps the plain quantiser, from the oracle
    alone: with outliers at random positions of Q and K, exact attention on
    the plainly quantised operands is closer to exact attention on the bf16
    operands than it is on the rotated-then-quantised ones (e4m3 rounding is
    relative to each element, and the rotation makes every product of a
    score large).  Both chains use the same plainly quantised V."""
    shape = (1, 1024, 4, 128)
    q, k = _scattered_outliers(960, shape, mag), _scattered_outliers(961, shape, mag)
    qf, kf, vf = (oracle.bf16_decode(x) for x in (q, k, W.normal_bf16(962, shape)))
    scale = 1 / np.sqrt(128)
    ox, _ = oracle.attention(qf, kf, vf, scale, causal=True)
    vd = oq.dequantize_blocks(*oq.quantize_blocks(vf))
    o0, _ = oracle.attention(oq.dequantize_blocks(*oq.quantize_blocks(qf)),
                             oq.dequantize_blocks(*oq.quantize_blocks(kf)), vd, scale, causal=True)
    signs = W.random_signs(963, 128)
    o1, _ = oracle.attention(oq.dequantize_blocks(*rot.rotate_quantize_blocks(qf, signs)),
                             oq.dequantize_blocks(*rot.rotate_quantize_blocks(kf, signs)), vd, scale / 128,
                             causal=True)
    e0, e1 = np.abs(o0 - ox), np.abs(o1 - ox)
    assert e0.mean() < e1.mean() and e0.max() < e1.max()
