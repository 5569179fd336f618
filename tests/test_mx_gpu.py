"""GPU parity of the MXFP8 path: the quantiser (attn_quantize_mxfp8, along d
for Q/K and along tokens for V) against the MX oracle byte for byte and
scale for scale, and MXFP8 attention (attn_fwd_mxfp8) against the fp64
oracle on the dequantised operands."""
import numpy as np
import pytest

import oracle
import oracle.mx as omx
import workloads as W
from parity import TOL_FP8, assert_within, errors, to_dev

pytestmark = pytest.mark.gpu

SENT = 0xEE


def _bf16(seed, shape, mags=(1.0, 2.0 ** -100, 2.0 ** 60, 2.0 ** -7)):
    x = W.bf16_bits_to_f32(W.normal_bf16(seed, shape, outliers=True)).astype(np.float64)
    for h in range(shape[-2]):
        x[..., h, :] *= mags[h % len(mags)]
    return W.f32_to_bf16_bits(x.astype(np.float32))


def run_mx(bits, tokens, cu=None):
    import torch
    import io_aware_exact_attn_amd as ia
    packed = cu is not None
    if packed:
        N, H, d = bits.shape
        B = len(cu) - 1
    else:
        B, N, H, d = bits.shape
    if tokens:
        sshape = (H, -(-N // 32) + B, d) if packed else (B, H, -(-N // 32), d)
    else:
        sshape = bits.shape[:-1] + (d // 32,)
    y = torch.full(bits.shape, 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full(sshape, SENT, dtype=torch.uint8, device="cuda")
    cu_d = to_dev(np.asarray(cu, np.int32)) if packed else None
    ia.attn_quantize_mxfp8(to_dev(bits), y, s, B, H, N, d, cu_d, int(tokens))
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("N,d", [(1, 128), (31, 64), (32, 128), (33, 64), (300, 128), (1000, 64)])
def test_mx_along_d_bit_exact(N, d):
    bits = _bf16(10 + N + d, (2, N, 4, d))
    y, s = run_mx(bits, False)
    yr, sr = omx.quantize_mx_d(oracle.bf16_decode(bits))
    assert np.array_equal(s, sr) and np.array_equal(y, yr)


@pytest.mark.parametrize("N,d", [(1, 128), (31, 64), (32, 128), (33, 64), (300, 128), (1000, 64)])
def test_mx_along_tokens_bit_exact(N, d):
    bits = _bf16(20 + N + d, (2, N, 4, d))
    y, s = run_mx(bits, True)
    yr, sr = omx.quantize_mx_tokens(oracle.bf16_decode(bits))
    assert np.array_equal(s, sr) and np.array_equal(y, yr)


@pytest.mark.parametrize("d", [64, 128])
def test_mx_packed_bit_exact(d):
    lengths = [1, 31, 0, 32, 33, 300, 64, 0, 95]
    cu = [int(c) for c in W.cu_seqlens_from_lengths(lengths)]
    N, B = cu[-1], len(lengths)
    bits = _bf16(30 + d, (N, 3, d))
    y, s = run_mx(bits, False, cu)
    yr, sr = omx.quantize_mx_d(oracle.bf16_decode(bits))
    assert np.array_equal(s, sr) and np.array_equal(y, yr)
    y, s = run_mx(bits, True, cu)
    yr, sr = omx.quantize_mx_tokens(oracle.bf16_decode(bits), cu)
    used = np.zeros(-(-N // 32) + B, bool)
    for doc in range(B):
        for k in range(-(-(cu[doc + 1] - cu[doc]) // 32)):
            used[omx.v_scale_slot(cu, doc, k)] = True
    assert np.array_equal(y, yr)
    assert np.array_equal(s[:, used], sr[:, used]) and np.all(s[:, ~used] == SENT)


def test_mx_special_blocks():
    """All-zero blocks, maxima of exactly 2^k and just below, values that
    saturate (amax in (448, 512) times 2^e), bf16 subnormals, and the largest
    bf16 magnitudes."""
    x = np.zeros((1, 64, 2, 128), np.float32)
    x[0, 0, 0, :32] = 256.0
    x[0, 1, 0, :32] = np.linspace(-511, 511, 32)
    x[0, 2, 0, :32] = 2.0 ** -130                      # bf16 subnormal block
    x[0, 3, 0, :32] = np.float32(3.0e38)
    x[0, 4, 0, 32:64] = 1.9921875                      # just below 2
    x[0, 5:, 1, :] = W.bf16_bits_to_f32(W.normal_bf16(3, (59, 128)))
    bits = W.f32_to_bf16_bits(x)
    for tokens in (False, True):
        y, s = run_mx(bits, tokens)
        yr, sr = (omx.quantize_mx_tokens if tokens else omx.quantize_mx_d)(oracle.bf16_decode(bits))
        assert np.array_equal(s, sr) and np.array_equal(y, yr), tokens
