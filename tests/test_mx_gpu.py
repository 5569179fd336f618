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


# ---------------------------------------------------------------------------
# MXFP8 attention
# ---------------------------------------------------------------------------

def mx_chain(q, k, v, scale, causal, cu=None):
    """Quantise on the GPU (Q, K along d; V along tokens), run attn_fwd_mxfp8;
    returns O, LSE and the dequantised operands the kernel saw."""
    import torch
    import io_aware_exact_attn_amd as ia
    packed = cu is not None
    if packed:
        N, H, d = q.shape
        B = len(cu) - 1
        lshape = (H, N)
    else:
        B, N, H, d = q.shape
        lshape = (B, H, N)
    cud = to_dev(np.asarray(cu, np.int32)) if packed else None
    ops = []
    for x, tokens in ((q, False), (k, False), (v, True)):
        y = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        if tokens:
            # 0xFF is E8M0's NaN: packed slots no block maps to keep it, and
            # the kernel must never read them
            s = torch.full((H, -(-N // 32) + B, d) if packed else (B, H, -(-N // 32), d), 0xFF, dtype=torch.uint8,
                           device="cuda")
        else:
            s = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device="cuda")
        ia.attn_quantize_mxfp8(to_dev(x), y, s, B, H, N, d, cud, int(tokens))
        ops.append((y, s))
    o = torch.full(q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full(lshape, 7.0, dtype=torch.float32, device="cuda")
    ia.attn_fwd_mxfp8(ops[0][0], ops[1][0], ops[2][0], ops[0][1], ops[1][1], ops[2][1], o, lse, B, H, N, d,
                      scale, int(causal), cud)
    torch.cuda.synchronize()
    h = [(y.cpu().numpy(), s.cpu().numpy()) for y, s in ops]
    deq = [omx.dequantize_mx_d(*h[0]), omx.dequantize_mx_d(*h[1]), omx.dequantize_mx_tokens(*h[2], cu)]
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), deq




@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 65, 200, 513, 1000])
def test_mxfp8_attention_fixed(N, causal):
    shape = (2, N, 2, 128)
    q, k = (W.normal_bf16(1200 + 3 * N + i, shape, outliers=True) for i in range(2))
    v = W.normal_bf16(1202 + 3 * N, shape)
    O, L, (qd, kd, vd) = mx_chain(q, k, v, 1 / np.sqrt(128), causal)
    Or, Lr = oracle.attention(qd, kd, vd, 1 / np.sqrt(128), causal=causal)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)


@pytest.mark.parametrize("N", [65, 200, 513, 700, 1000, 2048, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_mxfp8_attention_all_outliers(N, causal):
    """1% +-20 outliers in all of Q, K and V, at the fp8 bound."""
    shape = (2, N, 2, 128)
    q, k, v = (W.normal_bf16(1200 + 3 * N + i, shape, outliers=True) for i in range(3))
    O, L, (qd, kd, vd) = mx_chain(q, k, v, 1 / np.sqrt(128), causal)
    Or, Lr = oracle.attention(qd, kd, vd, 1 / np.sqrt(128), causal=causal)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)


@pytest.mark.parametrize("lengths", [[1, 63, 0, 64, 65, 300, 129, 31],
                                     [int(x) for x in np.random.default_rng(3).integers(0, 60, 70)]])
@pytest.mark.parametrize("causal", [False, True])
def test_mxfp8_attention_packed(lengths, causal):
    cu = [int(c) for c in W.cu_seqlens_from_lengths(lengths)]
    shape = (cu[-1], 2, 128)
    q, k = (W.normal_bf16(1300 + i, shape, outliers=True) for i in range(2))
    v = W.normal_bf16(1302, shape)
    O, L, (qd, kd, vd) = mx_chain(q, k, v, 0.088, causal, cu)
    Or, Lr = oracle.attention(qd, kd, vd, 0.088, causal=causal, cu_seqlens=cu)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)
    v = W.normal_bf16(1302, shape, outliers=True)
    O, L, (qd, kd, vd) = mx_chain(q, k, v, 0.088, causal, cu)
    Or, Lr = oracle.attention(qd, kd, vd, 0.088, causal=causal, cu_seqlens=cu)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_mxfp8_attention_scales(scale):
    shape = (1, 130, 2, 128)
    q, k, v = (W.normal_bf16(1400 + i, shape) for i in range(3))
    O, L, (qd, kd, vd) = mx_chain(q, k, v, scale, True)
    Or, Lr = oracle.attention(qd, kd, vd, scale, causal=True)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)


def test_mxfp8_causal_scale_safety():
    """Perturbing token t changes no output row before its 32-token V block
    (Q/K scales are per token; V's per 32 tokens), bit for bit."""
    shape = (1, 256, 2, 128)
    q, k, v = (W.normal_bf16(1500 + i, shape, outliers=True) for i in range(3))
    O1, L1, _ = mx_chain(q, k, v, 0.088, True)
    t = 150
    k2, v2 = k.copy(), v.copy()
    k2[0, t] = W.normal_bf16(1510, (2, 128))
    v2[0, t] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(v[0, t]) * 64)
    O2, L2, _ = mx_chain(q, k2, v2, 0.088, True)
    cut = 32 * (t // 32)
    assert np.array_equal(O1[0, :cut], O2[0, :cut]) and np.array_equal(L1[0, :, :cut], L2[0, :, :cut])
    assert not np.array_equal(O1[0, t:], O2[0, t:])


def test_mxfp8_kernel_name():
    import io_aware_exact_attn_amd as ia
    assert ia.attn_kernel_name(128, 1, 1, 0, fp8=2) == "attn_fwd_fp8_kernel<causal,packed,mx>"
    assert ia.attn_kernel_name(64, 1, 0, 0, fp8=2) == ""


def test_mxfp8_workload_sampled_rows():
    """The shape and inputs `bench.py --extra mxfp8` times: the fp8
    workload's bf16 q, k, v ([2, 8192, 16, 128], 1% +-20 outliers in all
    three) quantised to MXFP8 on the GPU, causal; sampled query rows of two
    (sequence, head) pairs against the oracle on the dequantised operands."""
    import torch
    import io_aware_exact_attn_amd as ia
    w = W.workload(5)
    B, N, H, d = w.B, w.N, w.H, w.d
    shape = (B, N, H, d)
    bits = [W.normal_bf16(W.tensor_seed(5, t), shape, True) for t in ("q", "k", "v")]
    ys = [torch.empty(shape, dtype=torch.uint8, device="cuda") for _ in range(3)]
    ss = [torch.empty((B, N, H, d // 32), dtype=torch.uint8, device="cuda") for _ in range(2)]
    ss.append(torch.empty((B, H, N // 32, d), dtype=torch.uint8, device="cuda"))
    for i in range(3):
        ia.attn_quantize_mxfp8(to_dev(bits[i]), ys[i], ss[i], B, H, N, d, None, int(i == 2))
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd_mxfp8(ys[0], ys[1], ys[2], ss[0], ss[1], ss[2], o, lse, B, H, N, d, w.scale, 1)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 127, 128, 2047, 4096, 6000, 8190, 8191])
    for b, h in ((0, 3), (1, 14)):
        qd = omx.dequantize_mx_d(ys[0][b:b + 1, :, h:h + 1].cpu().numpy(), ss[0][b:b + 1, :, h:h + 1].cpu().numpy())
        kd = omx.dequantize_mx_d(ys[1][b:b + 1, :, h:h + 1].cpu().numpy(), ss[1][b:b + 1, :, h:h + 1].cpu().numpy())
        vd = omx.dequantize_mx_tokens(ys[2][b:b + 1, :, h:h + 1].cpu().numpy(), ss[2][b:b + 1, h:h + 1].cpu().numpy())
        Or, Lr = oracle.attention_rows(qd, kd, vd, w.scale, True, 0, 0, rows)
        og = o[b, rows, h].float().cpu().numpy().astype(np.float64)
        lg = lse[b, h, rows].cpu().numpy().astype(np.float64)
        assert_within(errors(og, Or, lg, Lr), TOL_FP8)
