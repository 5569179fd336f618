"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle
on the same seeded inputs (element by element at small sizes; all rows at
the multi-head causal workload; sampled rows at the long-context and packed
workloads, in the same launch configuration the benchmark times)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from parity import (TOL_BF16, TOL_BF16_WORKLOAD, TOL_F32, assert_within, errors, oracle_bf16,
                    run_bf16)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, shape, outliers=""):
    return tuple(W.normal_bf16(seed * 10 + i, shape, t in outliers) for i, t in enumerate("qkv"))


def _check(q, k, v, scale, causal, out, cu=None, tol=None):
    O, L, _ = run_bf16(q, k, v, scale, causal, out=out, cu_seqlens=cu)
    Or, Lr = oracle_bf16(q, k, v, scale, causal, cu_seqlens=cu)
    err = errors(O, Or, L, Lr, out=out)
    assert_within(err, tol or (TOL_BF16 if out == "bf16" else TOL_F32))
    return err


# ---------------------------------------------------------------------------
# the page's worked example through the ABI
# ---------------------------------------------------------------------------

def _worked_inputs(reverse):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json"), encoding="utf-8"))
    assert g["values"] == [1.0, 3.0]
    N, d = 128, 64
    # q rows = e0; key A = 0 (score 0, value 1), key B = e0 with scale fp32(ln2)
    # (score ln2, value 3), in different 64-key tiles; every other key is
    # -4096 e0, whose weight exp(-4096 ln2) is exactly 0 in fp32 and fp64.
    q = np.zeros((1, N, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, N, 1, d), np.float32)
    k[..., 0] = -4096.0
    v = np.full((1, N, 1, d), 100.0, np.float32)
    ia, ib = (64, 0) if reverse else (0, 64)
    k[0, ia, 0, 0] = 0.0
    v[0, ia, 0, :] = 1.0
    k[0, ib, 0, 0] = 1.0
    v[0, ib, 0, :] = 3.0
    return tuple(W.f32_to_bf16_bits(x) for x in (q, k, v)), float(np.float32(math.log(2.0)))


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_worked_example(reverse, out):
    (q, k, v), scale = _worked_inputs(reverse)
    O, L, _ = run_bf16(q, k, v, scale, False, out=out)
    if out == "f32":
        assert np.all(np.abs(O - 7.0 / 3.0) < 2e-6)
    else:
        assert np.all(O == 2.328125)            # bf16 round-to-nearest-even of 7/3
    assert np.all(np.abs(L - math.log(3.0)) < 2e-6)


# ---------------------------------------------------------------------------
# small shapes: several tiles and ragged tails, element by element
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 257, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_small_shapes(N, d, causal, out):
    q, k, v = _case(N * 7 + d + causal, (2, N, 3, d))
    _check(q, k, v, float(np.float32(1 / math.sqrt(d))), causal, out)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_small_varlen(d, causal, out):
    lengths = [1, 15, 16, 17, 127, 128, 129, 300]
    cu = W.cu_seqlens_from_lengths(lengths)
    q, k, v = _case(500 + d + causal, (int(cu[-1]), 2, d))
    _check(q, k, v, float(np.float32(1 / math.sqrt(d))), causal, out, cu=cu)


@pytest.mark.parametrize("n_docs", [63, 64, 65, 150])
@pytest.mark.parametrize("causal", [0, 1])
def test_many_documents(n_docs, causal):
    """The kernel orders up to 64 documents longest first (one lane ranks
    each) and keeps a plain per-XCD order beyond that: both sides of the
    limit, with lengths 1..300 including ties and empty documents."""
    rng = np.random.default_rng(900 + n_docs + causal)
    lengths = rng.integers(1, 300, n_docs)
    lengths[::7] = 64                    # ties
    lengths[3] = 0                       # an empty document
    cu = W.cu_seqlens_from_lengths(lengths)
    q, k, v = _case(910 + n_docs + causal, (int(cu[-1]), 2, 64))
    _check(q, k, v, 0.125, causal, "f32", cu=cu)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1e-3, 0.9])
def test_scale_values(scale):
    q, k, v = _case(77, (1, 200, 2, 64))
    _check(q, k, v, scale, 1, "f32")


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_large_scores_qk_outliers(causal, out):
    # the long-context workload's distribution: 1% of Q and K entries are +-20
    q, k, v = _case(78, (1, 520, 2, 128), outliers="qk")
    _check(q, k, v, 1 / math.sqrt(128), causal, out)


@pytest.mark.parametrize("d", [64, 128])
def test_noncausal_long_rows(d):
    """Non-causal rows over 4096 keys (64 tiles, no mask anywhere but the
    workgroups' own rows), with the long-context workload's 1 % +-20
    outliers in Q and K: the lazy reference maximum across many unmasked
    tiles."""
    q, k, v = _case(79 + d, (1, 4096, 2, d), outliers="qk")
    _check(q, k, v, 1 / math.sqrt(d), 0, "bf16")


@pytest.mark.parametrize("per_tile,N,d", [(80.0, 300, 128), (170.0, 200, 128), (400.0, 136, 128),
                                           (170.0, 200, 64)])
@pytest.mark.parametrize("causal", [0, 1])
def test_rising_scores(per_tile, N, d, causal):
    """Scores that rise along the keys by about `per_tile` exp2 units per
    64-key tile move every row's reference maximum on nearly every tile: by
    fewer than 120 units (the kernel rescales the weights it formed in place)
    or by more (it forms them again; at 400 units they overflow fp32 before
    the shift).  Magnitudes stay where fp32 scores are accurate to ~1e-4 in
    the exponent, so the workload tolerances apply."""
    scale = 1 / math.sqrt(d)
    c = scale / math.log(2.0)
    slope = per_tile / (64 * 4.0 * c)          # q[..., 0] = 4: 4 * slope raw score per key
    rng = np.random.default_rng(int(per_tile) * 1000 + N + d)
    q = rng.standard_normal((1, N, 2, d)).astype(np.float32) * np.float32(0.05)
    q[..., 0] = 4.0
    k = rng.standard_normal((1, N, 2, d)).astype(np.float32)
    k[..., 0] = (np.float32(slope) * np.arange(N, dtype=np.float32))[None, :, None]
    v = rng.standard_normal((1, N, 2, d)).astype(np.float32)
    q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    for out in ("bf16", "f32"):
        _check(q, k, v, scale, causal, out)


@pytest.mark.parametrize("causal", [0, 1])
def test_large_values_scale_exactly(causal):
    """Inside the stated range (N * max|v| < 2^68) the result is exact up to
    rounding at any magnitude of V: V times 2^48 gives O times 2^48, bit for
    bit (fp32 output; every product and partial sum just moves up 48
    binades), and the same LSE."""
    q, k, v = _case(81, (1, 2048, 2, 128), outliers="qk")
    O1, L1, _ = run_bf16(q, k, v, 1 / math.sqrt(128), causal, out="f32")
    v48 = W.f32_to_bf16_bits(W.bf16_bits_to_f32(v) * np.float32(2.0 ** 48))
    O2, L2, _ = run_bf16(q, k, v48, 1 / math.sqrt(128), causal, out="f32")
    assert np.all(np.isfinite(O2))
    assert np.array_equal(O2, O1 * 2.0 ** 48) and np.array_equal(L1, L2)


@pytest.mark.parametrize("causal", [0, 1])
def test_large_weights_and_values(causal):
    """Scores rising by about 50 exp2 units per 64-key tile keep weights of up
    to ~2^50 against the lazy reference, with V scaled by 2^40: still inside
    the range, and within the fp32-output tolerance relative to 2^40."""
    d, N = 128, 640
    scale = 1 / math.sqrt(d)
    c = scale / math.log(2.0)
    slope = 50.0 / (64 * 4.0 * c)
    rng = np.random.default_rng(82 + causal)
    q = rng.standard_normal((1, N, 2, d)).astype(np.float32) * np.float32(0.05)
    q[..., 0] = 4.0
    k = rng.standard_normal((1, N, 2, d)).astype(np.float32)
    k[..., 0] = (np.float32(slope) * np.arange(N, dtype=np.float32))[None, :, None]
    v = rng.standard_normal((1, N, 2, d)).astype(np.float32) * np.float32(2.0 ** 40)
    q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    O, L, _ = run_bf16(q, k, v, scale, causal, out="f32")
    Or, Lr = oracle_bf16(q, k, v, scale, causal)
    err = errors(O / 2.0 ** 40, Or / 2.0 ** 40, L, Lr, out="f32")
    assert_within(err, TOL_F32)


def test_value_outliers_bound():
    """With +-20 outliers in V as well, the bf16 rounding of P before the P.V
    contraction bounds the error by u * max|v| (u = 2^-8, the unit roundoff
    of bf16; the weights sum to 1), plus fp32 accumulation."""
    q, k, v = _case(79, (1, 520, 2, 128), outliers="qkv")
    vmax = float(np.abs(W.bf16_bits_to_f32(v)).max())
    err = _check(q, k, v, 1 / math.sqrt(128), 1, "f32",
                 tol=dict(max_raw=2.0 ** -8 * vmax + 1e-3, mean=1e-3, lse=1e-3))
    print("value outliers", vmax, err)


# ---------------------------------------------------------------------------
# the five workloads (bf16 ones here)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_max_head_stride(d, causal):
    """H * d at the boundary's 2^24 limit (H = 2^24 / d heads): one 64-token
    tile of all heads spans 2^31 bytes, the most the kernels' 32-bit tile
    offsets and buffer sizes allow.  N = 65 gives a full tile and a one-row
    tail.  Four heads (first, second, middle, last) hold seeded inputs, the
    rest zeros; those four are compared with the oracle."""
    import torch
    import io_aware_exact_attn_amd as ia
    B, N = 1, 65
    H = (1 << 24) // d
    heads = [0, 1, H // 2, H - 1]
    scale = 1.0 / math.sqrt(d)
    bits = {t: W.normal_bf16(9100 + 10 * d + i, (B, N, len(heads), d)) for i, t in enumerate("qkv")}
    dev = {}
    for t in "qkv":
        x = torch.zeros((B, N, H, d), dtype=torch.bfloat16, device="cuda")
        for j, h in enumerate(heads):
            x[:, :, h] = torch.from_numpy(np.ascontiguousarray(bits[t][:, :, j]).view(np.int16)).view(
                torch.bfloat16).cuda()
        dev[t] = x
    o = torch.full((B, N, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, B, H, N, d, scale, causal, None, ia.ATTN_BF16)
    torch.cuda.synchronize()
    O = o[:, :, heads].float().cpu().numpy().astype(np.float64)
    L = lse[:, heads].cpu().numpy().astype(np.float64)
    del dev, o, lse
    torch.cuda.empty_cache()
    Or, Lr = oracle_bf16(bits["q"], bits["k"], bits["v"], scale, causal)
    assert_within(errors(O, Or, L, Lr, out="bf16"), TOL_BF16)


def test_workload1_single_head():
    w = W.workload(1)
    inp = W.make_inputs(w)
    err = _check(inp["q"], inp["k"], inp["v"], w.scale, w.causal, w.out)
    print("workload 1", err)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_workload2_all_rows(out):
    w = W.workload(2)
    inp = W.make_inputs(w)
    err = _check(inp["q"], inp["k"], inp["v"], w.scale, w.causal, out,
                 tol=TOL_BF16_WORKLOAD if out == "bf16" else TOL_F32)
    print("workload 2", out, err)


def _sample_rows(n, rng, extra=()):
    rows = set(range(0, min(n, 48))) | set(range(max(0, n - 48), n))
    rows |= set(int(x) for x in rng.integers(0, n, 96))
    for bm in (128, 256):
        for t in range(bm, n, bm * 7):
            rows |= {t - 1, t}
    rows |= set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < n))


@pytest.fixture(scope="module")
def inputs3():
    return W.make_inputs(W.workload(3))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_workload3_sampled_rows(inputs3, out):
    w = W.workload(3)
    q, k, v = inputs3["q"], inputs3["k"], inputs3["v"]
    O, L, _ = run_bf16(q, k, v, w.scale, True, out=out)
    rng = np.random.default_rng(3)
    Os, Or, Ls, Lr = [], [], [], []
    for h in (0, 13, 31):
        rows = _sample_rows(w.N, rng)
        o_ref, l_ref = oracle.attention_rows(oracle.bf16_decode(q), oracle.bf16_decode(k),
                                             oracle.bf16_decode(v), w.scale, True, 0, h, rows)
        Os.append(O[0, rows, h]); Or.append(o_ref); Ls.append(L[0, h, rows]); Lr.append(l_ref)
    err = errors(np.concatenate(Os), np.concatenate(Or), np.concatenate(Ls), np.concatenate(Lr), out=out)
    print("workload 3", out, err)
    assert_within(err, TOL_BF16_WORKLOAD if out == "bf16" else TOL_F32)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


@pytest.fixture(scope="module")
def inputs4():
    return W.make_inputs(W.workload(4))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_workload4_packed(inputs4, out):
    w = W.workload(4)
    q, k, v, cu = inputs4["q"], inputs4["k"], inputs4["v"], inputs4["cu_seqlens"]
    O, L, _ = run_bf16(q, k, v, w.scale, True, out=out, cu_seqlens=cu)
    qd, kd, vd = (oracle.bf16_decode(x) for x in (q, k, v))
    # two heads in full
    Of, Lf = oracle.attention(qd[:, :2], kd[:, :2], vd[:, :2], w.scale, causal=True, cu_seqlens=cu)
    err_full = errors(O[:, :2], Of, L[:2], Lf, out=out)
    # every head: first, last and random rows of every document
    rng = np.random.default_rng(4)
    rows = set()
    for a, b in zip(cu[:-1], cu[1:]):
        rows |= {int(a), int(b) - 1, int(a) + (int(b) - int(a)) // 2}
        rows |= set(int(x) for x in rng.integers(a, b, 4))
    rows = np.array(sorted(rows))
    Os, Or, Ls, Lr = [], [], [], []
    for h in range(w.H):
        o_ref, l_ref = oracle.attention_rows(qd, kd, vd, w.scale, True, 0, h, rows, cu_seqlens=cu)
        Os.append(O[rows, h]); Or.append(o_ref); Ls.append(L[h, rows]); Lr.append(l_ref)
    err_rows = errors(np.concatenate(Os), np.concatenate(Or), np.concatenate(Ls), np.concatenate(Lr), out=out)
    print("workload 4", out, err_full, err_rows)
    tol = TOL_BF16_WORKLOAD if out == "bf16" else TOL_F32
    assert_within(err_full, tol)
    assert_within(err_rows, tol)
