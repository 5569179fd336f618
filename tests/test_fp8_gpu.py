"""GPU parity of the block-scaled fp8 path (attn_fwd_fp8) against the fp64
oracle run on the dequantised inputs, plus its causal scale-safety property."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL_FP8, assert_within, errors, run_fp8

pytestmark = pytest.mark.gpu


def _quantized(seed, shape, outliers="qkv"):
    res = []
    for i, t in enumerate("qkv"):
        x = W.bf16_bits_to_f32(W.normal_bf16(seed * 10 + i, shape, t in outliers))
        res.extend(W.quantize_e4m3_blocks(x))
    q, qs, k, ks, v, vs = res
    return q, k, v, qs, ks, vs


def _deq(q, k, v, qs, ks, vs):
    return (oracle.dequantize_e4m3_blocks(q, qs), oracle.dequantize_e4m3_blocks(k, ks),
            oracle.dequantize_e4m3_blocks(v, vs))


def test_worked_example_fp8():
    """The page's two-score example (scores 0 and ln 2, values 1 and 3) with
    unit scales: key A = 0, key B = e0 in another 128-token block, every
    other key -448 e0 (weight 2^-448 = 0); the weights 1/2 and 1 are exact
    in e4m3, so O = 7/3 exactly before the bf16 rounding of the output."""
    N, d = 256, 128
    q = np.zeros((1, N, 1, d), np.uint8)
    q[..., 0] = 0x38                       # 1.0
    k = np.zeros((1, N, 1, d), np.uint8)
    k[..., 0] = 0xFE                       # -448
    v = np.full((1, N, 1, d), 0x60, np.uint8)   # 32: irrelevant, weight 0
    k[0, 0, 0, 0] = 0x00
    v[0, 0, 0, :] = 0x38                   # value 1
    k[0, 128, 0, 0] = 0x38
    v[0, 128, 0, :] = 0x44                 # value 3
    ones = np.ones((1, 1, 2), np.float32)
    O, L = run_fp8(q, k, v, ones, ones, ones, float(np.float32(math.log(2.0))), False)
    assert np.all(O == 2.328125)
    assert np.abs(L - math.log(3.0)).max() < 2e-6


@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 255, 257, 300, 511, 513, 700, 1000, 2048])
@pytest.mark.parametrize("causal", [0, 1])
def test_small_shapes_fp8(N, causal):
    """1% +-20 outliers in all of Q, K and V (the fp8 workload's
    distribution), rows up to 2048 keys long, against the oracle on the
    dequantised operands at the fp8 bound."""
    q, k, v, qs, ks, vs = _quantized(N + 31 * causal, (2, N, 3, 128))
    O, L = run_fp8(q, k, v, qs, ks, vs, 1 / math.sqrt(128), causal)
    Or, Lr = oracle.attention(*_deq(q, k, v, qs, ks, vs), 1 / math.sqrt(128), causal=bool(causal))
    err = errors(O, Or, L, Lr, out="bf16")
    assert_within(err, TOL_FP8)



def test_noncausal_long_rows_fp8():
    """Non-causal rows over 4096 keys with +-20 outliers in Q, K and V, at
    the fp8 bound."""
    q, k, v, qs, ks, vs = _quantized(98, (1, 4096, 2, 128))
    O, L = run_fp8(q, k, v, qs, ks, vs, 1 / math.sqrt(128), False)
    Or, Lr = oracle.attention(*_deq(q, k, v, qs, ks, vs), 1 / math.sqrt(128), causal=False)
    assert_within(errors(O, Or, L, Lr), TOL_FP8)

@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5])
def test_scale_values_fp8(scale):
    q, k, v, qs, ks, vs = _quantized(55, (1, 200, 2, 128), outliers="")
    O, L = run_fp8(q, k, v, qs, ks, vs, scale, 1)
    Or, Lr = oracle.attention(*_deq(q, k, v, qs, ks, vs), scale, causal=True)
    assert_within(errors(O, Or, L, Lr, out="bf16"), TOL_FP8)


@pytest.fixture(scope="module")
def inputs5():
    return W.make_inputs(W.workload(5))


def test_workload5_sampled_rows(inputs5):
    w = W.workload(5)
    i = inputs5
    O, L = run_fp8(i["q"], i["k"], i["v"], i["q_scale"], i["k_scale"], i["v_scale"], w.scale, True)
    qd, kd, vd = _deq(i["q"], i["k"], i["v"], i["q_scale"], i["k_scale"], i["v_scale"])
    rng = np.random.default_rng(5)
    Os, Or, Ls, Lr = [], [], [], []
    for b, h in ((0, 0), (0, 9), (1, 15)):
        rows = set(range(40)) | set(range(w.N - 40, w.N)) | set(int(x) for x in rng.integers(0, w.N, 96))
        rows |= {t for blk in range(128, w.N, 128 * 9) for t in (blk - 1, blk)}
        rows = np.array(sorted(rows))
        o_ref, l_ref = oracle.attention_rows(qd, kd, vd, w.scale, True, b, h, rows)
        Os.append(O[b, rows, h]); Or.append(o_ref); Ls.append(L[b, h, rows]); Lr.append(l_ref)
    err = errors(np.concatenate(Os), np.concatenate(Or), np.concatenate(Ls), np.concatenate(Lr), out="bf16")
    print("workload 5", err)
    assert_within(err, TOL_FP8)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


def test_fp8_causal_scale_safety():
    """Changing token t (and so the scales of its 128-token block) leaves every
    output row before that block bitwise unchanged: no scale carries a later
    token's information into earlier rows."""
    shape = (1, 640, 2, 128)
    x = [W.bf16_bits_to_f32(W.normal_bf16(70 + i, shape, True)) for i in range(3)]
    qkv = [W.quantize_e4m3_blocks(t) for t in x]
    O1, L1 = run_fp8(qkv[0][0], qkv[1][0], qkv[2][0], qkv[0][1], qkv[1][1], qkv[2][1], 0.09, True)
    t = 400                                   # block 3 = tokens 384..511
    x2 = [a.copy() for a in x]
    for a in x2:
        a[0, t] *= 7.0                        # raises that block's amax and scales
    qkv2 = [W.quantize_e4m3_blocks(a) for a in x2]
    assert not np.array_equal(qkv2[1][1], qkv[1][1])
    O2, L2 = run_fp8(qkv2[0][0], qkv2[1][0], qkv2[2][0], qkv2[0][1], qkv2[1][1], qkv2[2][1], 0.09, True)
    blk = 128 * (t // 128)
    assert np.array_equal(O1[0, :blk], O2[0, :blk])
    assert np.array_equal(L1[0, :, :blk], L2[0, :, :blk])
    assert not np.array_equal(O1[0, blk:], O2[0, blk:])


def test_fp8_deterministic():
    q, k, v, qs, ks, vs = _quantized(8, (1, 700, 2, 128))
    a = run_fp8(q, k, v, qs, ks, vs, 0.1, True)
    b = run_fp8(q, k, v, qs, ks, vs, 0.1, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_max_head_stride(causal):
    """H * d at the boundary's 2^24 limit (H = 2^17 heads at d = 128): a
    64-token tile of all heads spans 2^30 bytes of e4m3.  N = 65 gives a full
    tile and a one-row tail.  Four heads (first, second, middle, last) hold
    seeded quantised inputs with outliers, the rest zeros under unit scales;
    those four are compared with the oracle on their dequantised inputs."""
    import torch
    import io_aware_exact_attn_amd as ia
    from parity import to_dev
    B, N, d = 1, 65, 128
    H = (1 << 24) // d
    heads = [0, 1, H // 2, H - 1]
    scale = 1.0 / math.sqrt(d)
    q, k, v, qs, ks, vs = _quantized(97, (B, N, len(heads), d))
    dev, sdev = [], []
    for x, s in ((q, qs), (k, ks), (v, vs)):
        t = torch.zeros((B, N, H, d), dtype=torch.uint8, device="cuda")
        st = torch.ones((B, H, s.shape[2]), dtype=torch.float32, device="cuda")
        for j, h in enumerate(heads):
            t[:, :, h] = torch.from_numpy(np.ascontiguousarray(x[:, :, j])).cuda()   # the bytes as they are
            st[:, h] = to_dev(np.ascontiguousarray(s[:, j]))
        dev.append(t.view(torch.float8_e4m3fn))
        sdev.append(st)
    o = torch.full((B, N, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd_fp8(dev[0], dev[1], dev[2], sdev[0], sdev[1], sdev[2], o, lse, B, H, N, d, scale, causal)
    torch.cuda.synchronize()
    O = o[:, :, heads].float().cpu().numpy().astype(np.float64)
    L = lse[:, heads].cpu().numpy().astype(np.float64)
    del dev, sdev, o, lse
    torch.cuda.empty_cache()
    qd, kd, vd = _deq(q, k, v, qs, ks, vs)
    Or, Lr = oracle.attention(qd, kd, vd, scale, causal=bool(causal))
    assert_within(errors(O, Or, L, Lr), TOL_FP8)
