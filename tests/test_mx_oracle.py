"""Pins of the MXFP8 oracle (oracle/mx.py), on the CPU.

Checked against hand-computed blocks (the scale of a block whose maximum is
exactly a power of two, of one just below, the saturation of (448, 512), an
all-zero block, a one-element-nonzero block far below the maximum), the
exact dequantisation of values already on the e4m3 grid, the error bound of
the format, the orientation of the blocks (d for Q/K, tokens for V), the
document-local restart of the V blocks, and causality: perturbing token t
changes no Q/K scale but its own token's and no V scale outside its 32-token
block.  Planted mistakes in the oracle must each trip at least one pin.
"""
import numpy as np
import pytest

import oracle.mx as mx
import workloads as W

_rng = np.random.default_rng(31)


def pin_power_of_two_maximum():
    # amax = 256 -> e = 0: elements unchanged when on the e4m3 grid
    x = np.zeros(32)
    x[:4] = [256.0, -3.0, 0.5, 0.0]
    q, s = mx.quantize_mx_d(x[None])
    assert s[0, 0] == 127
    assert np.array_equal(mx.dequantize_mx_d(q, s)[0], x)


def pin_exponent_floor():
    # amax = 1.5 -> floor(log2) = 0 -> e = -8, byte 119; 1.5 * 256 = 384 exact
    x = np.zeros(32)
    x[7] = 1.5
    x[8] = -0.75
    q, s = mx.quantize_mx_d(x[None])
    assert s[0, 0] == 119
    assert q[0, 7] == 0x7C and q[0, 8] == 0xF4       # 384 = 1.5 * 2^8 ; -192 = -1.5 * 2^7
    # amax = 511 -> e = 0 and 511 saturates to 448; 500 too
    x = np.zeros(32)
    x[:2] = [511.0, -500.0]
    q, s = mx.quantize_mx_d(x[None])
    assert s[0, 0] == 127 and q[0, 0] == 0x7E and q[0, 1] == 0xFE


def pin_all_zero_block():
    q, s = mx.quantize_mx_d(np.zeros((3, 64)))
    assert np.all(s == 127) and np.all(q == 0)


def pin_small_elements_round_to_grid():
    # amax 256 (e = 0): 2^-10 is below the smallest e4m3 subnormal 2^-9 by half -> ties to even 0;
    # 3 * 2^-10 rounds to 2^-9 * 2 (nearest) = 2^-8
    x = np.zeros(32)
    x[:3] = [256.0, 2.0 ** -10, 3 * 2.0 ** -10]
    q, s = mx.quantize_mx_d(x[None])
    assert q[0, 1] == 0x00 and q[0, 2] == 0x02


def pin_error_bound():
    # |x - x^| <= 2^-4 |x| for |x| >= 2^(e-6) (normal e4m3 range), <= 2^(e-10)
    # below it, and values above 448 * 2^e lose at most 64 * 2^e
    x = W.bf16_bits_to_f32(W.normal_bf16(5, (8, 4, 128), outliers=True)).astype(np.float64)
    q, s = mx.quantize_mx_d(x)
    xr = mx.dequantize_mx_d(q, s)
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=-1)
    err = np.abs(x - xr)
    lim = np.maximum(2.0 ** -4 * np.abs(x), np.ldexp(1.0, e - 10))
    sat = np.abs(x) > np.ldexp(448.0, e)
    assert np.all(err[~sat] <= lim[~sat]) and np.all(err[sat] <= np.ldexp(64.0, e[sat]))
    # the block maximum is kept to within its e4m3 rounding or saturation
    amax = np.abs(x).reshape(8, 4, 4, 32).max(-1)
    assert np.all((amax >= np.ldexp(256.0, s.astype(np.int64) - 127)) &
                  (amax < np.ldexp(512.0, s.astype(np.int64) - 127)))


def pin_token_blocks_orientation():
    # V blocks run along tokens: a column whose only nonzero entry is token 5
    # gets the scale of that entry in block 0, and column 1 is independent
    B, N, H, d = 1, 70, 1, 64
    x = np.zeros((B, N, H, d))
    x[0, 5, 0, 0] = 3.0
    x[0, 40, 0, 1] = 0.25
    q, s = mx.quantize_mx_tokens(x)
    assert s.shape == (1, 1, 3, 64)
    assert s[0, 0, 0, 0] == 127 + 1 - 8 and s[0, 0, 1, 1] == 127 - 2 - 8
    assert np.all(np.delete(s[0, 0].ravel(), [0 * 64 + 0, 1 * 64 + 1]) == 127)
    assert np.array_equal(mx.dequantize_mx_tokens(q, s), x)


def pin_packed_restart():
    lengths = [5, 0, 40, 33]
    cu = [int(c) for c in W.cu_seqlens_from_lengths(lengths)]
    x = W.bf16_bits_to_f32(W.normal_bf16(9, (cu[-1], 2, 32))).astype(np.float64)
    q, s = mx.quantize_mx_tokens(x, cu)
    for doc in range(len(lengths)):
        a, b = cu[doc], cu[doc + 1]
        if b == a:
            continue
        qd, sd = mx.quantize_mx_tokens(x[None, a:b])
        assert np.array_equal(q[a:b], qd[0])
        for k in range(sd.shape[2]):
            assert np.array_equal(s[:, mx.v_scale_slot(cu, doc, k)], sd[0, :, k])


def pin_causality():
    x = W.bf16_bits_to_f32(W.normal_bf16(11, (1, 96, 2, 64))).astype(np.float64)
    x2 = x.copy()
    x2[0, 50] *= 40.0                                   # token 50 (V block 1)
    qa, sa = mx.quantize_mx_d(x)
    qb, sb = mx.quantize_mx_d(x2)
    changed = np.any(sa != sb, axis=(2, 3))[0]
    assert np.array_equal(np.nonzero(changed)[0], [50])
    va, vsa = mx.quantize_mx_tokens(x)
    vb, vsb = mx.quantize_mx_tokens(x2)
    assert np.array_equal(va[0, :32], vb[0, :32]) and np.array_equal(vsa[:, :, 0], vsb[:, :, 0])
    assert np.array_equal(va[0, 64:], vb[0, 64:]) and np.array_equal(vsa[:, :, 2], vsb[:, :, 2])
    assert np.any(vsa[:, :, 1] != vsb[:, :, 1])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---- planted mistakes -----------------------------------------------------

def _mutants():
    enc = mx.e4m3_encode
    return {
        "ceil_exponent": ("_block_exponent",
                          lambda a: 0 if a == 0 else int(np.ceil(np.log2(float(a)))) - 8),
        "emax_7": ("_block_exponent", lambda a: 0 if a == 0 else int(np.floor(np.log2(float(a)))) - 7),
        "zero_block_byte_0": ("_block_exponent",
                              lambda a: -127 if a == 0 else int(np.floor(np.log2(float(a)))) - 8),
        "scale_multiplies": ("_quantize_group",
                             lambda xg: (lambda e: (enc(np.clip(np.ldexp(xg, e), -448, 448).astype(np.float32)),
                                                    np.uint8(e + 127)))(
                                 mx._block_exponent(float(np.max(np.abs(xg))) if xg.size else 0.0))),
        "v_blocks_of_64": ("MX_BLOCK", 64),
    }


@pytest.mark.parametrize("kind", list(_mutants()))
def test_mutant_is_caught(kind, monkeypatch):
    name, fn = _mutants()[kind]
    monkeypatch.setattr(mx, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every MX pin"
