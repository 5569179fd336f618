"""Pins of the quantiser oracle (oracle/quantize.py), on the CPU.

The encoder is checked against facts of the OCP e4m3fn format that do not
come from the oracle itself: every finite byte decodes and re-encodes to
itself, hand-computed midpoints round to the even mantissa, values beyond the
largest finite value saturate, and in-range values agree with torch's own
float8_e4m3fn cast.  The block quantiser is checked on hand-built blocks and
on properties that hold at any size (the block maximum becomes +-448, an
all-zero block has scale 1, packed input is quantised as its documents one by
one, every document block gets its own scale slot).  Planted mistakes in the
oracle must each trip at least one of these pins.
"""
import numpy as np
import pytest

import oracle.quantize as oq
from oracle.exact import e4m3_decode

_rng = np.random.default_rng(2024)
_encode = oq.e4m3_encode


def pin_round_trip_all_bytes():
    b = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oq.e4m3_encode(e4m3_decode(b).astype(np.float32)), b)


def pin_midpoints_and_saturation():
    cases = [
        (1.0625, 0x38),          # between 1.0 (0x38) and 1.125 (0x39): even -> 1.0
        (1.1875, 0x3A),          # between 1.125 (0x39) and 1.25 (0x3A): even -> 1.25
        (1.0626, 0x39),          # just above the first midpoint
        (-1.0625, 0xB8),
        (2.0 ** -10, 0x00),      # half the smallest subnormal: even -> 0
        (3 * 2.0 ** -10, 0x02),  # between 2^-9 (0x01) and 2^-8 (0x02): even -> 2^-8
        (15 * 2.0 ** -10, 0x08), # between the largest subnormal and 2^-6: even -> 2^-6
        (416.0, 0x7D),           # exactly representable: 1.625 * 2^8
        (432.0, 0x7E),           # between 416 (0x7D) and 448 (0x7E): even -> 448
        (464.0, 0x7E),           # beyond 448: saturates
        (1.0e9, 0x7E),
        (-500.0, 0xFE),
        (0.0, 0x00),
        (-0.0, 0x80),
    ]
    x = np.array([c[0] for c in cases], dtype=np.float32)
    want = np.array([c[1] for c in cases], dtype=np.uint8)
    assert np.array_equal(oq.e4m3_encode(x), want)


def pin_matches_torch_cast():
    import torch
    y = np.concatenate([
        _rng.standard_normal(4000).astype(np.float32) * 50,
        (_rng.random(2000).astype(np.float32) - 0.5) * 2 ** -5,
        _rng.uniform(-448, 448, 2000).astype(np.float32),
    ])
    t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oq.e4m3_encode(y), t)


def pin_block_extremes():
    x = np.zeros((1, 300, 2, 8), np.float32)
    x[0, 5, 0, 3] = -7.5                       # block 0 of head 0: amax 7.5
    x[0, 40, 0, 1] = 3.0
    x[0, 200, 1, 2] = 1.0e-3                   # block 1 of head 1: amax 1e-3
    q, s = oq.quantize_blocks(x)
    assert s.shape == (1, 2, 3)
    assert s[0, 0, 0] == np.float32(np.float32(7.5) / np.float32(448.0))
    assert s[0, 1, 1] == np.float32(np.float32(1.0e-3) / np.float32(448.0))
    assert s[0, 0, 1] == 1.0 and s[0, 0, 2] == 1.0 and s[0, 1, 0] == 1.0   # all-zero blocks
    assert q[0, 5, 0, 3] == 0xFE and q[0, 200, 1, 2] == 0x7E               # block maxima -> +-448
    # 3.0 / (7.5 / 448) = 179.2 -> nearest e4m3 is 176 = 1.375 * 2^7 (0x73)
    assert q[0, 40, 0, 1] == 0x73
    assert int(np.count_nonzero(q)) == 3


def pin_block_max_is_448():
    x = (_rng.standard_normal((2, 256, 3, 16)) * _rng.uniform(1e-3, 1e3, (2, 1, 3, 1))).astype(np.float32)
    q, s = oq.quantize_blocks(x)
    v = e4m3_decode(q)
    for b in range(2):
        for h in range(3):
            for k in range(2):
                blk = v[b, 128 * k:128 * (k + 1), h]
                assert np.abs(blk).max() == 448.0


def pin_scale_slots_distinct():
    for trial in range(50):
        L = _rng.integers(1, 700, size=_rng.integers(1, 40))
        cu = np.concatenate([[0], np.cumsum(L)])
        N, B = int(cu[-1]), len(L)
        slots = [oq.scale_slot(cu, d, k) for d in range(B) for k in range(-(-int(L[d]) // 128))]
        assert len(set(slots)) == len(slots)
        assert min(slots) >= 0 and max(slots) < -(-N // 128) + B


def pin_packed_is_per_document():
    L = [5, 130, 256, 1, 300]
    cu = np.concatenate([[0], np.cumsum(L)])
    x = (_rng.standard_normal((int(cu[-1]), 2, 8)) * 3).astype(np.float32)
    q, s = oq.quantize_blocks(x, cu)
    for d, n in enumerate(L):
        qd, sd = oq.quantize_blocks(x[None, cu[d]:cu[d + 1]])
        assert np.array_equal(q[cu[d]:cu[d + 1]], qd[0])
        for k in range(sd.shape[2]):
            assert np.array_equal(s[:, oq.scale_slot(cu, d, k)], sd[0, :, k])


def pin_dequantize_error_bound():
    x = (_rng.standard_normal((1, 384, 2, 16)) * 4).astype(np.float32)
    q, s = oq.quantize_blocks(x)
    r = oq.dequantize_blocks(q, s)
    step = np.repeat(s, 128, axis=2).transpose(0, 2, 1)[:, :, :, None].astype(np.float64)
    # half an e4m3 ulp: 2^-4 relative in the normal range, 2^-10 * scale below it
    assert np.all(np.abs(r - x) <= np.maximum(np.abs(x) * 2.0 ** -4, step * 2.0 ** -10) * (1 + 1e-12))


QPINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", QPINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---- planted mistakes -----------------------------------------------------

def _enc_ties_away(y):
    y = np.asarray(y, np.float32)
    a = np.abs(y).astype(np.float64)
    hi = np.minimum(np.searchsorted(oq._POS_VALS, a), len(oq._POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    idx = np.where(oq._POS_VALS[hi] - a <= a - oq._POS_VALS[lo], hi, lo)
    return oq._POS_BYTES[idx] | (np.signbit(y).astype(np.uint8) << 7)


def _enc_truncate(y):
    y = np.asarray(y, np.float32)
    a = np.abs(y).astype(np.float64)
    idx = np.maximum(np.searchsorted(oq._POS_VALS, a, side="right") - 1, 0)
    return oq._POS_BYTES[idx] | (np.signbit(y).astype(np.uint8) << 7)


def _enc_no_sign(y):
    return _encode(np.abs(np.asarray(y, np.float32)))


def _block_447(xb):
    amax = np.float32(np.max(np.abs(xb)))
    s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(447.0))
    return _encode((xb / s).astype(np.float32)), s


def _block_signed_max(xb):
    amax = np.float32(np.max(xb))
    s = np.float32(1.0) if amax <= 0 else np.float32(amax / np.float32(448.0))
    return _encode(np.clip(xb / s, -448, 448).astype(np.float32)), s


def _block_zero_scale0(xb):
    amax = np.float32(np.max(np.abs(xb)))
    s = np.float32(amax / np.float32(448.0))
    with np.errstate(invalid="ignore", divide="ignore"):
        y = np.nan_to_num((xb / s).astype(np.float32))
    return _encode(y), s


def _slot_no_doc(cu, doc, k, block=128):
    return int(cu[doc]) // block + k


_MUTANTS = {
    "ties_away": ("e4m3_encode", _enc_ties_away),
    "truncate": ("e4m3_encode", _enc_truncate),
    "no_sign": ("e4m3_encode", _enc_no_sign),
    "scale_447": ("_quantize_block", _block_447),
    "signed_max": ("_quantize_block", _block_signed_max),
    "zero_block_scale": ("_quantize_block", _block_zero_scale0),
    "slot_without_doc": ("scale_slot", _slot_no_doc),
}


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = _MUTANTS[name]
    monkeypatch.setattr(oq, attr, fn)
    caught = []
    for pin in QPINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every quantiser pin"
