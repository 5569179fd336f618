"""GPU parity of the rotating quantiser (attn_quantize_fp8_rotated) against
the rotation oracle, byte for byte and scale for scale, and of fp8 attention
on rotated Q and K (scale / d) against the fp64 oracle on the dequantised
operands; plus what the rotation is for: when Q and K share outlier
channels, fp8 attention after the rotation lands closer to the exact bf16
attention than fp8 attention without it."""
import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import oracle.rotation as orot
import workloads as W
from parity import TOL_FP8, assert_within, errors, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


def run_rot(bits, signs, cu=None):
    import torch
    import io_aware_exact_attn_amd as ia
    if cu is not None:
        N, H, d = bits.shape
        B = len(cu) - 1
        sshape = (H, -(-N // 128) + B)
    else:
        B, N, H, d = bits.shape
        sshape = (B, H, -(-N // 128))
    y = torch.full(bits.shape, 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full(sshape, SENTINEL, dtype=torch.float32, device="cuda")
    cu_d = to_dev(np.asarray(cu, np.int32)) if cu is not None else None
    ia.attn_quantize_fp8_rotated(to_dev(bits), y, s, to_dev(signs), B, H, N, d, cu_d)
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


def _bf16(seed, shape, outliers=True, mags=(1.0, 2.0 ** -60, 2.0 ** 40, 2.0 ** -7)):
    x = W.bf16_bits_to_f32(W.normal_bf16(seed, shape, outliers=outliers)).astype(np.float64)
    for h in range(shape[-2]):
        x[..., h, :] *= mags[h % len(mags)]
    return W.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("N,d", [(1, 128), (127, 64), (128, 128), (129, 64), (300, 128), (1000, 64)])
def test_rotated_quantize_fixed_bit_exact(N, d):
    bits = _bf16(500 + N + d, (2, N, 4, d))
    signs = W.random_signs(600 + d, d)
    y, s = run_rot(bits, signs)
    yr, sr = orot.rotate_quantize_blocks(oracle.bf16_decode(bits), signs)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(y, yr)


@pytest.mark.parametrize("d", [64, 128])
def test_rotated_quantize_packed_bit_exact(d):
    lengths = [1, 127, 0, 128, 129, 300, 64, 0, 255]
    cu = W.cu_seqlens_from_lengths(lengths)
    N, B = int(cu[-1]), len(lengths)
    bits = _bf16(700 + d, (N, 3, d))
    signs = W.random_signs(800 + d, d)
    y, s = run_rot(bits, signs, cu)
    yr, sr = orot.rotate_quantize_blocks(oracle.bf16_decode(bits), signs, cu)
    used = np.zeros(-(-N // 128) + B, bool)
    for doc in range(B):
        for k in range(-(-(int(cu[doc + 1]) - int(cu[doc])) // 128)):
            used[oq.scale_slot(cu, doc, k)] = True
    assert np.array_equal(y, yr)
    assert np.array_equal(s[:, used].view(np.uint32), sr[:, used].view(np.uint32))
    assert np.all(s[:, ~used] == SENTINEL)


def test_rotated_quantize_special_rows():
    """All-zero blocks, one-hot rows (every rotated value equal in
    magnitude), all signs negative, and a row spanning 30 binades (still
    exact in fp64)."""
    d = 128
    x = np.zeros((1, 256, 2, d), np.float32)
    x[0, 128:, 0, 5] = 3.0                      # one-hot rows
    x[0, :128, 1, :] = 2.0 ** -20
    x[0, :128, 1, 0] = 2.0 ** 10                # 30 binades in one row
    x[0, 128:, 1, :] = 0.0                      # an all-zero block
    bits = W.f32_to_bf16_bits(x)
    for signs in (W.random_signs(3, d), np.full(d, -1, np.int8)):
        y, s = run_rot(bits, signs)
        yr, sr = orot.rotate_quantize_blocks(oracle.bf16_decode(bits), signs)
        assert np.array_equal(y, yr) and np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def _fp8_chain(q, k, v, scale, causal, signs=None):
    """Quantise (rotating Q and K when signs are given) and run attn_fwd_fp8;
    returns O, LSE and the dequantised operands the kernel saw."""
    import torch
    import io_aware_exact_attn_amd as ia
    B, N, H, d = q.shape
    nb = -(-N // 128)
    outs = []
    for name, x in (("q", q), ("k", k), ("v", v)):
        y = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty((B, H, nb), dtype=torch.float32, device="cuda")
        if signs is not None and name != "v":
            ia.attn_quantize_fp8_rotated(to_dev(x), y, s, to_dev(signs), B, H, N, d)
        else:
            ia.attn_quantize_fp8(to_dev(x), y, s, B, H, N, d)
        outs.append((y, s))
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    sc = scale / d if signs is not None else scale
    ia.attn_fwd_fp8(outs[0][0].view(torch.float8_e4m3fn), outs[1][0].view(torch.float8_e4m3fn),
                    outs[2][0].view(torch.float8_e4m3fn), outs[0][1], outs[1][1], outs[2][1], o, lse,
                    B, H, N, d, sc, int(causal))
    torch.cuda.synchronize()
    deq = [oq.dequantize_blocks(y.cpu().numpy(), s.cpu().numpy()) for y, s in outs]
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), deq, sc


@pytest.mark.parametrize("N,causal", [(200, True), (513, False), (1024, True)])
def test_rotated_fp8_attention_parity(N, causal):
    """The kernel on rotated operands against the oracle on the same
    dequantised operands with scale / d."""
    shape = (1, N, 2, 128)
    q, k, v = (W.normal_bf16(900 + i, shape, outliers=True) for i in range(3))
    signs = W.random_signs(901, 128)
    O, L, (qd, kd, vd), sc = _fp8_chain(q, k, v, 1 / np.sqrt(128), causal, signs)
    Or, Lr = oracle.attention(qd, kd, vd, sc, causal=causal)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)


def _channel_outliers(seed, shape, channels, mag):
    x = W.bf16_bits_to_f32(W.normal_bf16(seed, shape)).astype(np.float32)
    x[..., channels] *= mag
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("mag,nch", [(10.0, 1), (10.0, 4), (30.0, 2)])
def test_rotation_reduces_fp8_error(mag, nch):
    """Exact bf16 attention as the target; Q and K share outlier channels
    (the same coordinates scaled by mag in every token), so one product
    q_c k_c dominates each score and its e4m3 rounding is not averaged; the
    rotation spreads it over all d coordinates.  The rotated chain's mean and
    max O errors and its LSE error must all be below the plain chain's.
    (With outliers at random positions instead, the plain chain is the more
    accurate one: e4m3 rounding is relative, and mixing coordinates makes
    every product of the score large.)"""
    shape = (1, 1024, 4, 128)
    ch = np.random.default_rng(nch).choice(128, nch, replace=False)
    q, k = (_channel_outliers(950 + i, shape, ch, mag) for i in range(2))
    v = W.normal_bf16(952, shape)
    scale = 1 / np.sqrt(128)
    Ox, Lx = oracle.attention(oracle.bf16_decode(q), oracle.bf16_decode(k), oracle.bf16_decode(v), scale,
                              causal=True)
    O0, L0, _, _ = _fp8_chain(q, k, v, scale, True)
    O1, L1, _, _ = _fp8_chain(q, k, v, scale, True, W.random_signs(953, 128))
    e0, e1 = np.abs(O0 - Ox), np.abs(O1 - Ox)
    l0, l1 = np.abs(L0 - Lx).max(), np.abs(L1 - Lx).max()
    print(f"plain fp8: mean {e0.mean():.5f} max {e0.max():.4f} lse {l0:.4f}; "
          f"rotated: mean {e1.mean():.5f} max {e1.max():.4f} lse {l1:.4f}")
    assert e1.mean() < e0.mean() and e1.max() < e0.max() and l1 < l0


def test_rotated_quantize_workload_tensor():
    """The whole q tensor `bench.py --extra rotate` rotates ([2, 8192, 16,
    128] bf16, 1% +-20 outliers, its seeded signs), bit for bit."""
    shape = (2, 8192, 16, 128)
    bits = W.normal_bf16(7100, shape, True)
    signs = W.random_signs(7102, 128)
    y, s = run_rot(bits, signs)
    yr, sr = orot.rotate_quantize_blocks(oracle.bf16_decode(bits), signs)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(y, yr)
