"""GPU parity of the e4m3 block quantiser (attn_quantize_fp8) against the
oracle quantiser, byte for byte and scale for scale, and of packed-document
fp8 attention (attn_fwd_fp8 with cu_seqlens) against the fp64 oracle run on
the dequantised documents."""
import math

import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import workloads as W
from parity import TOL_FP8, assert_within, errors, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


def bf16_input(seed, shape, zero_block=True):
    """bf16 bits: N(0,1) with 1% +-20 outliers, a different power-of-two
    magnitude per head (one head near 2^-100), and an all-zero first block in
    the first head."""
    x = W.bf16_bits_to_f32(W.normal_bf16(seed, shape, outliers=True)).astype(np.float64)
    H = shape[-2]
    mags = [1.0, 2.0 ** -100, 2.0 ** 9, 2.0 ** -7]
    for h in range(H):
        x[..., h, :] *= mags[h % len(mags)]
    if zero_block:
        x[(0,) * (len(shape) - 3) + (slice(0, 128), 0)] = 0.0
    return W.f32_to_bf16_bits(x.astype(np.float32))


def run_quant(bits, cu=None):
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
    ia.attn_quantize_fp8(to_dev(bits), y, s, B, H, N, d, cu_d)
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


def oracle_quant(bits, cu=None):
    return oq.quantize_blocks(oracle.bf16_decode(bits).astype(np.float32), cu)


def _used_slots(cu, N, B):
    used = np.zeros(-(-N // 128) + B, bool)
    for d in range(B):
        for k in range(-(-(cu[d + 1] - cu[d]) // 128)):
            used[oq.scale_slot(cu, d, k)] = True
    return used


@pytest.mark.parametrize("N,d", [(1, 128), (127, 128), (128, 64), (129, 128), (300, 64), (1000, 128)])
def test_quantize_fixed_bit_exact(N, d):
    bits = bf16_input(300 + N + d, (2, N, 4, d))
    y, s = run_quant(bits)
    yr, sr = oracle_quant(bits)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(y, yr)


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_packed_bit_exact(d):
    lengths = [1, 127, 0, 128, 129, 300, 513, 64, 0, 255]
    cu = W.cu_seqlens_from_lengths(lengths)
    N, B = int(cu[-1]), len(lengths)
    bits = bf16_input(77 + d, (N, 3, d))
    y, s = run_quant(bits, cu)
    yr, sr = oracle_quant(bits, cu)
    used = _used_slots(cu, N, B)
    assert np.array_equal(y, yr)
    assert np.array_equal(s[:, used].view(np.uint32), sr[:, used].view(np.uint32))
    assert np.all(s[:, ~used] == SENTINEL)           # slots no block maps to stay untouched


def test_quantize_many_scales_bit_exact():
    """Every (block, head) gets its own random magnitude 2^u * m (u in
    [-60, 60], m in [1, 2)), so the blocks' scales, and with them the
    quotients x / s, cover many different significands."""
    rng = np.random.default_rng(321)
    B, N, H, d = 1, 128 * 48, 8, 128
    x = W.bf16_bits_to_f32(W.normal_bf16(321, (B, N, H, d), True)).astype(np.float64)
    mag = np.exp2(rng.uniform(-60, 60, (N // 128, H))) * rng.uniform(1, 2, (N // 128, H))
    x = x * np.repeat(mag, 128, axis=0)[None, :, :, None]
    bits = W.f32_to_bf16_bits(x.astype(np.float32))
    y, s = run_quant(bits)
    yr, sr = oracle_quant(bits)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(y, yr)


def test_quantize_workload5_q_tensor():
    """The fp8 workload's shape [2, 8192, 16, 128], every block."""
    w = W.workload(5)
    bits = W.normal_bf16(W.tensor_seed(5, "q"), (w.B, w.N, w.H, w.d), True)
    y, s = run_quant(bits)
    yr, sr = oracle_quant(bits)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(y, yr)


def run_fp8_packed(q, k, v, qs, ks, vs, cu, scale, causal):
    import torch
    import io_aware_exact_attn_amd as ia
    N, H, d = q.shape
    B = len(cu) - 1
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd_fp8(to_dev(q), to_dev(k), to_dev(v), to_dev(qs), to_dev(ks), to_dev(vs), o, lse,
                    B, H, N, d, scale, int(causal), to_dev(np.asarray(cu, np.int32)))
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _packed_inputs(seed, lengths, H=2):
    cu = W.cu_seqlens_from_lengths(lengths)
    N = int(cu[-1])
    qkv = []
    for i in range(3):
        x = W.bf16_bits_to_f32(W.normal_bf16(seed * 10 + i, (N, H, 128), True))
        qkv.append(oq.quantize_blocks(x, cu))
    return cu, qkv


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("lengths", [[1, 127, 128, 129, 300, 513, 64],
                                     [700],
                                     [5] * 20 + [130, 260, 1, 0, 400] + [17] * 45])
def test_packed_fp8_attention(lengths, causal):
    cu, ((q, qs), (k, ks), (v, vs)) = _packed_inputs(11 + len(lengths) + causal, lengths)
    O, L = run_fp8_packed(q, k, v, qs, ks, vs, cu, 1 / math.sqrt(128), causal)
    deq = [oq.dequantize_blocks(a, s, cu) for a, s in ((q, qs), (k, ks), (v, vs))]
    Or, Lr = oracle.attention(*deq, 1 / math.sqrt(128), causal=bool(causal), cu_seqlens=cu)
    err = errors(O, Or, L, Lr, out="bf16")
    print(len(lengths), "documents", err)
    assert_within(err, TOL_FP8)


def test_quantize_then_packed_attention():
    """bf16 documents -> attn_quantize_fp8 -> attn_fwd_fp8 (both on the GPU)
    against the oracle quantiser, dequantisation and attention."""
    import torch
    import io_aware_exact_attn_amd as ia
    lengths = [300, 1, 129, 640, 77]
    cu = W.cu_seqlens_from_lengths(lengths)
    N, B, H, d = int(cu[-1]), len(lengths), 2, 128
    bits = [W.normal_bf16(900 + i, (N, H, d), True) for i in range(3)]
    cu_d = to_dev(np.asarray(cu, np.int32))
    nsl = -(-N // 128) + B
    ys = [torch.empty((N, H, d), dtype=torch.uint8, device="cuda") for _ in range(3)]
    ss = [torch.zeros((H, nsl), dtype=torch.float32, device="cuda") for _ in range(3)]
    for b_, y, s in zip(bits, ys, ss):
        ia.attn_quantize_fp8(to_dev(b_), y, s, B, H, N, d, cu_d)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(d)
    ia.attn_fwd_fp8(ys[0], ys[1], ys[2], ss[0], ss[1], ss[2], o, lse, B, H, N, d, scale, 1, cu_d)
    torch.cuda.synchronize()
    ref = [oracle_quant(b_, cu) for b_ in bits]
    deq = [oq.dequantize_blocks(a, s, cu) for a, s in ref]
    Or, Lr = oracle.attention(*deq, scale, causal=True, cu_seqlens=cu)
    err = errors(o.float().cpu().numpy(), Or, lse.cpu().numpy(), Lr, out="bf16")
    assert_within(err, TOL_FP8)


def test_packed_fp8_causal_scale_safety():
    """Changing one token of a document (and so its block's scales) leaves every
    other document, and every row of the same document before that block,
    bitwise unchanged."""
    lengths = [200, 450, 90]
    cu = W.cu_seqlens_from_lengths(lengths)
    N, H = int(cu[-1]), 2
    xs = [W.bf16_bits_to_f32(W.normal_bf16(40 + i, (N, H, 128), True)) for i in range(3)]
    qkv = [oq.quantize_blocks(x, cu) for x in xs]
    O1, L1 = run_fp8_packed(*[a for a, _ in qkv], *[s for _, s in qkv], cu, 0.09, True)
    t = int(cu[1]) + 300                     # document 1, its block 2 (tokens 256..383)
    for x in xs:
        x[t] *= 7.0
    qkv2 = [oq.quantize_blocks(x, cu) for x in xs]
    O2, L2 = run_fp8_packed(*[a for a, _ in qkv2], *[s for _, s in qkv2], cu, 0.09, True)
    blk = int(cu[1]) + 256
    assert np.array_equal(O1[:blk], O2[:blk]) and np.array_equal(L1[:, :blk], L2[:, :blk])
    assert np.array_equal(O1[int(cu[2]):], O2[int(cu[2]):])
    assert not np.array_equal(O1[blk:int(cu[2])], O2[blk:int(cu[2])])


def test_packed_workload_fp8_sampled():
    """The packed-document workload (26 documents, 32768 tokens, H 16, d 128)
    as `bench.py --extra fp8_packed` runs it: bf16 Q, K and V quantised by
    attn_quantize_fp8 with document-local scales, then attn_fwd_fp8 with
    cu_seqlens.  Rows of the longest and of a median-length document, in the
    first and last heads, against the oracle on the operands of the oracle's
    own quantiser, applied to each sampled document alone."""
    w = W.workload(4)
    inp = W.make_inputs(w)
    cu = [int(c) for c in inp["cu_seqlens"]]
    gpu = [run_quant(inp[t], cu) for t in ("q", "k", "v")]
    O, L = run_fp8_packed(*[y for y, _ in gpu], *[s for _, s in gpu], cu, w.scale, 1)
    lens = np.diff(cu)
    Os, Or, Ls, Lr = [], [], [], []
    for doc, h in ((int(np.argmax(lens)), 0), (int(np.argsort(lens)[len(lens) // 2]), w.H - 1)):
        # documents are independent: the oracle takes this one on its own
        a, n = cu[doc], int(lens[doc])
        one = [0, n]
        deq = [oq.dequantize_blocks(*oracle_quant(inp[t][a:a + n], one), one) for t in ("q", "k", "v")]
        local = np.unique(np.clip([0, 1, 63, 64, 127, 128, 129, n // 3, n // 2, n - 2, n - 1], 0, n - 1))
        o_ref, l_ref = oracle.attention_rows(*deq, w.scale, True, 0, h, local, cu_seqlens=one)
        Os.append(O[a + local, h]); Or.append(o_ref); Ls.append(L[h, a + local]); Lr.append(l_ref)
    err = errors(np.concatenate(Os), np.concatenate(Or), np.concatenate(Ls), np.concatenate(Lr), out="bf16")
    print("packed workload fp8", err)
    assert_within(err, TOL_FP8)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


@pytest.mark.parametrize("kind", ["fp8", "fp8_rotated", "mx_d", "mx_tokens"])
@pytest.mark.parametrize("d", [64, 128])
def test_quantizers_max_head_stride(kind, d):
    """Every quantiser at H * d = 2^24 (the boundary's limit; N = 65: one full
    128-token block row of 65 tokens, a 32-token MX block and a one-token
    tail): four seeded heads (first, second, middle, last) bit for bit
    against the oracle on those heads, and a zero head quantised to zero
    bytes under the all-zero block's scale."""
    import torch
    import io_aware_exact_attn_amd as ia
    import oracle.mx as omx
    import oracle.rotation as orot
    B, N = 1, 65
    H = (1 << 24) // d
    heads = [0, 1, H // 2, H - 1]
    zero_head = 2
    bits = bf16_input(9500 + d, (B, N, len(heads), d), zero_block=False)
    x = torch.zeros((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    for j, h in enumerate(heads):
        x[:, :, h] = to_dev(np.ascontiguousarray(bits[:, :, j]))
    y = torch.full((B, N, H, d), 0xAA, dtype=torch.uint8, device="cuda")
    signs = W.random_signs(9501, d)
    if kind in ("fp8", "fp8_rotated"):
        s = torch.full((B, H, 1), SENTINEL, dtype=torch.float32, device="cuda")
        if kind == "fp8":
            ia.attn_quantize_fp8(x, y, s, B, H, N, d, None)
        else:
            ia.attn_quantize_fp8_rotated(x, y, s, to_dev(signs), B, H, N, d, None)
    elif kind == "mx_d":
        s = torch.full((B, N, H, d // 32), 0xAA, dtype=torch.uint8, device="cuda")
        ia.attn_quantize_mxfp8(x, y, s, B, H, N, d, None, 0)
    else:
        s = torch.full((B, H, -(-N // 32), d), 0xAA, dtype=torch.uint8, device="cuda")
        ia.attn_quantize_mxfp8(x, y, s, B, H, N, d, None, 1)
    torch.cuda.synchronize()
    hidx = heads + [zero_head]
    yh = y[:, :, hidx].cpu().numpy()
    sh = (s[:, :, hidx] if kind == "mx_d" else s[:, hidx]).cpu().numpy()
    del x, y, s
    torch.cuda.empty_cache()
    xf = oracle.bf16_decode(bits).astype(np.float32)
    if kind == "fp8":
        yr, sr = oq.quantize_blocks(xf)
    elif kind == "fp8_rotated":
        yr, sr = orot.rotate_quantize_blocks(oracle.bf16_decode(bits), signs)
    elif kind == "mx_d":
        yr, sr = omx.quantize_mx_d(oracle.bf16_decode(bits))
    else:
        yr, sr = omx.quantize_mx_tokens(oracle.bf16_decode(bits))
    assert np.array_equal(yh[:, :, :4], yr)
    if kind.startswith("fp8"):
        assert np.array_equal(sh[:, :4].view(np.uint32), sr.view(np.uint32))
        assert np.all(sh[:, 4] == 1.0)                     # an all-zero block's scale
    elif kind == "mx_d":
        assert np.array_equal(sh[:, :, :4], sr)
        assert np.all(sh[:, :, 4] == 127)                  # E8M0 2^0
    else:
        assert np.array_equal(sh[:, :4], sr)
        assert np.all(sh[:, 4] == 127)
    assert np.all(yh[:, :, 4] == 0)
