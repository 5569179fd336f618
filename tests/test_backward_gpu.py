"""GPU parity of the attention backward (attn_bwd) against the fp64 gradient
oracle (oracle.backward), on the same seeded bf16 inputs, with O and the LSE
taken from the HIP forward (attn_fwd) as a training step would.

Tolerance, derived from the arithmetic of the kernels rather than fixed:
every input (Q, K, V, dO) is bf16 on both sides, so the kernels' errors come
from
  * P: the forward's LSE is the log of a sum of bf16-rounded probabilities
    (relative error of the sum <= 2^-9), and the backward rounds P to bf16
    before dV = P^T dO (another 2^-9): |P~ - P| <= 2^-8 P to first order;
    2^-7 P is allowed;
  * D = rowsum(dO * O) is taken from the forward's bf16 O, so
    |D~ - D| <= sum_d |dO| |O~ - O| with O~ the HIP output;
  * dS = P (dP - D) is rounded to bf16 (2^-9 |dS|) before dQ and dK;
  * the fp32 sums of d products behind S, dP and D, each within 2^-17 of its
    sum of absolute products (the worst case of a 128-term fp32 sum: 127
    roundings of at most 2^-24 each): this is what is left of dP - D when
    one key holds all the weight and the two nearly cancel, and it moves P
    by a relative |scale| 2^-17 (|q_i| . |k_j| + max_j' |q_i| . |k_j'|);
    the gradient kernels start their dP sums at D (they accumulate D - dP),
    which adds |D| <= |dO| . |O| to those sums' absolute terms;
  * the bf16 output rounding, half an ulp of the result.
Propagated without cancellation, element by element:
    |dV~ - dV| <= (2^-7 + e_S) (P^T |dO|)                + half ulp
    E = (2^-7 + e_S) P |dP - D| + P (|D~ - D| + 2^-17 (|dO| |V|^T + 2 |dO| . |O|)) + 2^-9 |dS|
    |dQ~ - dQ| <= |scale| E |K|,  |dK~ - dK| <= |scale| E^T |Q|  (+ half ulp)
That is a worst case (all errors of one sign); the Frobenius error of each
gradient relative to its norm must also stay below 2^-7, which a
systematic mistake (a dropped mask, a wrong row term) exceeds.
"""
import numpy as np
import pytest

import oracle
import oracle.backward as ob
import workloads as W
from parity import bf16_half_ulp, oracle_bf16, to_dev

pytestmark = pytest.mark.gpu

REL_P = 2.0 ** -7
REL_DS = 2.0 ** -9
REL_SUM = 2.0 ** -17
ABS_FLOOR = 1e-5


def _inputs(seed, shape):
    return tuple(W.normal_bf16(seed * 10 + i, shape) for i in range(4))   # q, k, v, dO


def run_fwd_bwd(q, k, v, do, scale, causal, cu=None):
    """Forward then backward through the C ABI.  Returns float64 arrays
    (O, dQ, dK, dV, delta) in the input layouts, delta laid out as the LSE."""
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
    tq, tk, tv, tdo = (to_dev(x) for x in (q, k, v, do))
    o = torch.full(q.shape, 77.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full(lshape, 77.0, dtype=torch.float32, device="cuda")
    cud = to_dev(np.asarray(cu, np.int32)) if packed else None
    ia.attn_fwd(tq, tk, tv, o, lse, B, H, N, d, scale, int(causal), cud, ia.ATTN_BF16)
    delta = torch.full(lshape, 77.0, dtype=torch.float32, device="cuda")
    g = [torch.full(q.shape, 77.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ia.attn_bwd(tq, tk, tv, o, tdo, lse, delta, g[0], g[1], g[2], B, H, N, d, scale, int(causal), cud)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(o), f(g[0]), f(g[1]), f(g[2]), f(delta)


def _seq_bounds(q, k, v, do, o_gpu, o_ref, scale, causal):
    """Per-element bounds of one (sequence, head), from fp64 quantities."""
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    dp = do @ v.T
    dd = (o_ref * do).sum(axis=1, keepdims=True)
    err_d = (np.abs(do) * np.abs(o_gpu - o_ref)).sum(axis=1, keepdims=True)
    ds = p * (dp - dd)
    qk = np.abs(q) @ np.abs(k).T
    rel = REL_P + abs(scale) * REL_SUM * (qk + qk.max(axis=1, keepdims=True))
    dov = np.abs(do) @ np.abs(v).T
    doo = (np.abs(do) * np.abs(o_ref)).sum(axis=1, keepdims=True)
    # the dP sums start at D: |D| <= |dO| . |O| joins their absolute terms,
    # beside D's own sum
    e = rel * p * np.abs(dp - dd) + p * (err_d + REL_SUM * (dov + 2 * doo)) + REL_DS * np.abs(ds)
    bq = abs(scale) * (e @ np.abs(k))
    bk = abs(scale) * (e.T @ np.abs(q))
    bv = (rel * p).T @ np.abs(do)
    return bq, bk, bv


def _bounds(q, k, v, do, o_gpu, o_ref, scale, causal, cu=None):
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
    if cu is not None:
        for a, b in zip(cu[:-1], cu[1:]):
            if b <= a:
                continue
            for h in range(q.shape[1]):
                r = _seq_bounds(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], o_gpu[a:b, h], o_ref[a:b, h],
                                scale, causal)
                for x, y in zip(out, r):
                    x[a:b, h] = y
        return out
    for bb in range(q.shape[0]):
        for h in range(q.shape[2]):
            r = _seq_bounds(q[bb, :, h], k[bb, :, h], v[bb, :, h], do[bb, :, h], o_gpu[bb, :, h],
                            o_ref[bb, :, h], scale, causal)
            for x, y in zip(out, r):
                x[bb, :, h] = y
    return out


def check_case(bits, scale, causal, cu=None):
    q, k, v, do = bits
    O, dq, dk, dv, delta = run_fwd_bwd(q, k, v, do, scale, causal, cu)
    return verify_case(bits, O, dq, dk, dv, delta, scale, causal, cu)


def verify_case(bits, O, dq, dk, dv, delta, scale, causal, cu=None):
    """The gradients and D the kernels returned for inputs `bits`, against
    the oracle under the bounds of this file's docstring."""
    q, k, v, do = bits
    qf, kf, vf, dof = (oracle.bf16_decode(x) for x in bits)
    Or, _ = oracle_bf16(q, k, v, scale, causal, cu_seqlens=cu)
    want = ob.attention_grads(qf, kf, vf, dof, scale, causal, cu)
    bounds = _bounds(qf, kf, vf, dof, O, Or, scale, causal, cu)
    report = {}
    for name, got, ref, bnd in zip(("dq", "dk", "dv"), (dq, dk, dv), want, bounds):
        assert np.all(np.isfinite(got)), name
        err = np.abs(got - ref)
        lim = bnd + bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref))) + ABS_FLOOR
        worst = float((err / lim).max()) if err.size else 0.0
        nref = float(np.linalg.norm(ref))
        rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
        report[name] = dict(max_abs=float(err.max()) if err.size else 0.0, worst_ratio=worst, frob_rel=rel)
        assert worst <= 1.0, (name, report)
        assert rel <= REL_P, (name, report)
    # D against rowsum(dO * O) of the O the kernel was given (fp32 sums of
    # exact bf16 products)
    dref = ob.row_dot(O, dof)
    dabs = ob.row_dot(np.abs(O), np.abs(dof))
    assert np.all(np.abs(delta - dref) <= 1e-5 * dabs + 1e-30), "delta"
    return report


FIXED = [(1, 2, 1, 128), (2, 2, 63, 64), (1, 2, 64, 128), (2, 1, 65, 64), (1, 2, 127, 128),
         (1, 2, 129, 64), (1, 2, 300, 128), (1, 1, 1000, 64), (1, 1, 1000, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", FIXED)
def test_bwd_fixed(B, H, N, d, causal):
    bits = _inputs(1000 + N + d, (B, N, H, d))
    check_case(bits, 1.0 / np.sqrt(d), causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_packed(d, causal):
    lengths = [1, 127, 0, 128, 129, 300, 513, 64, 0, 255]
    cu = W.cu_seqlens_from_lengths(lengths)
    bits = _inputs(2000 + d, (int(cu[-1]), 2, d))
    check_case(bits, 1.0 / np.sqrt(d), causal, [int(x) for x in cu])


def test_bwd_packed_many_documents():
    """More than 64 documents: the work decode's other branch."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 90, size=80)]
    cu = W.cu_seqlens_from_lengths(lengths)
    bits = _inputs(2100, (int(cu[-1]), 2, 128))
    check_case(bits, 0.088, True, [int(x) for x in cu])


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5])
def test_bwd_scales(scale):
    """A negative scale (the order of the scores flips), zero (uniform P, so
    dQ = dK = 0 exactly) and a large one (peaked P)."""
    bits = _inputs(3000, (1, 200, 2, 128))
    check_case(bits, scale, True)
    if scale == 0.0:
        q, k, v, do = bits
        _, dq, dk, _, _ = run_fwd_bwd(q, k, v, do, scale, True)
        assert np.all(dq == 0) and np.all(dk == 0)


def test_bwd_gradient_outliers():
    """Keys with +-20 outliers: peaked rows and large |dP - D|."""
    shape = (1, 257, 2, 128)
    q, k, v = (W.normal_bf16(4000 + i, shape, outliers=True) for i in range(3))
    do = W.normal_bf16(4003, shape)
    check_case((q, k, v, do), 1.0 / np.sqrt(128), True)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_noncausal_long_rows(d):
    """Non-causal rows over 4096 keys with +-20 outliers in Q and K: 64 key
    tiles per dQ workgroup and 64 query tiles per dK/dV workgroup, no mask."""
    shape = (1, 4096, 2, d)
    q, k = (W.normal_bf16(4100 + d + i, shape, outliers=True) for i in range(2))
    v, do = (W.normal_bf16(4102 + d + i, shape) for i in range(2))
    check_case((q, k, v, do), 1.0 / np.sqrt(d), False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_max_head_stride(d, causal):
    """H * d at the boundary's 2^24 limit (H = 2^24 / d heads): a 64-token
    tile of all heads spans 2^31 bytes, the most the backward kernels' 32-bit
    tile offsets and buffer sizes allow.  N = 65 gives a full tile and a
    one-row tail.  Four heads (first, second, middle, last) hold seeded q, k,
    v and dO, the rest zeros; their gradients and D are checked."""
    import torch
    import io_aware_exact_attn_amd as ia
    B, N = 1, 65
    H = (1 << 24) // d
    heads = [0, 1, H // 2, H - 1]
    scale = 1.0 / np.sqrt(d)
    bits = tuple(W.normal_bf16(9300 + 10 * d + i, (B, N, len(heads), d)) for i in range(4))   # q, k, v, dO
    dev = []
    for x in bits:
        t = torch.zeros((B, N, H, d), dtype=torch.bfloat16, device="cuda")
        for j, h in enumerate(heads):
            t[:, :, h] = torch.from_numpy(np.ascontiguousarray(x[:, :, j]).view(np.int16)).view(torch.bfloat16).cuda()
        dev.append(t)
    o = torch.full((B, N, H, d), 77.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), 77.0, dtype=torch.float32, device="cuda")
    ia.attn_fwd(dev[0], dev[1], dev[2], o, lse, B, H, N, d, scale, causal, None, ia.ATTN_BF16)
    delta = torch.full((B, H, N), 77.0, dtype=torch.float32, device="cuda")
    g = [torch.full((B, N, H, d), 77.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ia.attn_bwd(dev[0], dev[1], dev[2], o, dev[3], lse, delta, g[0], g[1], g[2], B, H, N, d, scale, causal, None)
    torch.cuda.synchronize()
    f = lambda t: t[:, :, heads].float().cpu().numpy().astype(np.float64)
    O, dq, dk, dv = f(o), f(g[0]), f(g[1]), f(g[2])
    D = delta[:, heads].cpu().numpy().astype(np.float64)
    del dev, o, lse, delta, g
    torch.cuda.empty_cache()
    verify_case(bits, O, dq, dk, dv, D, scale, bool(causal))


@pytest.fixture(scope="module")
def long_context_run():
    """The long-context causal workload (B 1, H 32, N 16384, d 128) with the
    seeded dO, run once through the forward and the single attn_bwd launch
    sequence that `bench.py --extra bwd` times; returns the inputs and the
    outputs on the host."""
    import torch
    import io_aware_exact_attn_amd as ia
    w = W.workload(3)
    inp = W.make_inputs(w)
    B, N, H, d = w.B, w.N, w.H, w.d
    shape = (B, N, H, d)
    do_bits = W.normal_bf16(W.tensor_seed(3, "q") + 500, shape)
    dev = [to_dev(inp[t]) for t in ("q", "k", "v")] + [to_dev(do_bits)]
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd(dev[0], dev[1], dev[2], o, lse, B, H, N, d, w.scale, 1, None, ia.ATTN_BF16)
    delta = torch.empty_like(lse)
    g = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ia.attn_bwd(dev[0], dev[1], dev[2], o, dev[3], lse, delta, g[0], g[1], g[2], B, H, N, d, w.scale, 1, None)
    torch.cuda.synchronize()
    host = lambda t: t.float().cpu().numpy()
    return w, inp, do_bits, host(o), [host(t) for t in g], host(delta)


def _long_context_head(run, h, rows):
    w, inp, do_bits, o, g, delta = run
    qh, kh, vh, doh = (oracle.bf16_decode(x[0, :, h]) for x in (inp["q"], inp["k"], inp["v"], do_bits))
    f64 = lambda x: x.astype(np.float64)
    _check_sampled_rows(qh, kh, vh, doh, f64(o[0, :, h]), [f64(t[0, rows, h]) for t in g],
                        f64(delta[0, h, rows]), rows, w.scale)


def test_bwd_long_context_sampled(long_context_run):
    """Long-context workload: dQ rows and dK/dV rows sampled in two heads
    (first and last rows, tile and block edges) against the row-sampled
    oracle, each element within the bound of this file's docstring."""
    rows = np.array([0, 1, 63, 64, 127, 128, 129, 4095, 8191, 12000, 16382, 16383])
    for h in (7, 30):
        _long_context_head(long_context_run, h, rows)


@pytest.mark.parametrize("h", [0, 21])
def test_bwd_long_context_all_rows(long_context_run, h):
    """Long-context workload: every row of dQ, dK and dV of head h against
    the oracle, each element within the bound of this file's docstring."""
    _long_context_head(long_context_run, h, np.arange(long_context_run[0].N))


def _check_sampled_rows(qh, kh, vh, doh, o_gpu, got, dl, rows, sc, chunk=2048):
    """dQ rows and dK/dV rows of one causal (sequence, head) at `rows`
    against the row-sampled oracle, each element within the bound of this
    file's docstring (the max over keys of |q_i| . |k_j| there bounded by
    sum_d |q_id| max_j |k_jd|); `dl` is the kernel's D at those rows.  The
    bounds are formed `chunk` rows at a time, so every row of a long
    sequence can be checked without an n x n matrix per term."""
    N = qh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    dq, dk, dv, parts = ob.grads_at(qh, kh, vh, doh, sc, True, rows, rows)
    L, D, O = parts["L"], parts["D"], parts["O"]
    err_d = (np.abs(doh) * np.abs(o_gpu - O)).sum(axis=1)
    qk_max = np.abs(qh) @ np.abs(kh).max(axis=0)
    sums_row = REL_SUM * (np.abs(doh) * np.abs(O)).sum(axis=1)
    aq, ak, av, ado = np.abs(qh), np.abs(kh), np.abs(vh), np.abs(doh)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        sl = slice(c0, c0 + len(r))
        # dQ rows: all keys
        s = sc * (qh[r] @ kh.T)
        s = np.where(np.arange(N)[None, :] > r[:, None], -np.inf, s)
        p = np.exp(s - L[r][:, None])
        dpd = doh[r] @ vh.T - D[r][:, None]
        rel = REL_P + abs(sc) * REL_SUM * (aq[r] @ ak.T + qk_max[r][:, None])
        sums = REL_SUM * (ado[r] @ av.T) + sums_row[r][:, None]
        e = rel * p * np.abs(dpd) + p * (err_d[r][:, None] + sums) + REL_DS * np.abs(p * dpd)
        bq = abs(sc) * (e @ ak)
        # dK, dV rows: all queries
        s = sc * (qh @ kh[r].T)
        s = np.where(r[None, :] > np.arange(N)[:, None], -np.inf, s)
        p = np.exp(s - L[:, None])
        dpd = doh @ vh[r].T - D[:, None]
        rel = REL_P + abs(sc) * REL_SUM * (aq @ ak[r].T + qk_max[:, None])
        sums = REL_SUM * (ado @ av[r].T) + sums_row[:, None]
        e = rel * p * np.abs(dpd) + p * (err_d[:, None] + sums) + REL_DS * np.abs(p * dpd)
        bk = abs(sc) * (e.T @ aq)
        bv = (rel * p).T @ ado
        for name, gg, ref, bnd in zip(("dq", "dk", "dv"), got, (dq, dk, dv), (bq, bk, bv)):
            gg, ref = gg[sl], ref[sl]
            lim = bnd + bf16_half_ulp(np.maximum(np.abs(gg), np.abs(ref))) + ABS_FLOOR
            ratio = float((np.abs(gg - ref) / lim).max())
            assert np.all(np.isfinite(gg)) and ratio <= 1.0, (name, int(r[0]), ratio)
    assert np.all(np.abs(dl - (o_gpu[rows] * doh[rows]).sum(axis=1)) <= 1e-5 * (np.abs(o_gpu[rows]) *
                                                                                np.abs(doh[rows])).sum(axis=1))


@pytest.mark.parametrize("cid", [2, 4])
def test_bwd_workload_rows(cid):
    """The multi-head causal (B 4, H 16, N 2048, d 128) and packed-document
    (26 documents, 32768 tokens, H 16, d 128) workloads with the seeded dO and
    the launch sequence that `bench.py --extra bwd` times; every row of dQ, dK
    and dV in two (sequence or document, head) pairs (the longest document
    and a median one when packed)."""
    import torch
    import io_aware_exact_attn_amd as ia
    w = W.workload(cid)
    inp = W.make_inputs(w)
    shape = inp["q"].shape
    do_bits = W.normal_bf16(W.tensor_seed(cid, "q") + 500, shape)
    dev = [to_dev(inp[t]) for t in ("q", "k", "v")] + [to_dev(do_bits)]
    if w.varlen:
        cu = [int(c) for c in inp["cu_seqlens"]]
        B, lse_shape, cud = len(cu) - 1, (w.H, w.N), to_dev(np.asarray(cu, np.int32))
        lens = np.diff(cu)
        docs = [int(np.argmax(lens)), int(np.argsort(lens)[len(lens) // 2])]
        picks = [((cu[j], cu[j + 1]), h) for j, h in zip(docs, (0, w.H - 1))]
    else:
        B, lse_shape, cud = w.B, (w.B, w.H, w.N), None
        picks = [(0, 0), (w.B - 1, w.H - 1)]
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    ia.attn_fwd(dev[0], dev[1], dev[2], o, lse, B, w.H, w.N, w.d, w.scale, 1, cud, ia.ATTN_BF16)
    delta = torch.empty_like(lse)
    g = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ia.attn_bwd(dev[0], dev[1], dev[2], o, dev[3], lse, delta, g[0], g[1], g[2], B, w.H, w.N, w.d, w.scale, 1,
                cud)
    torch.cuda.synchronize()

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    for seq, h in picks:
        if w.varlen:
            a, b = seq
            n = b - a
            take = [x[a:b, h] for x in (inp["q"], inp["k"], inp["v"], do_bits)]
            rows = np.arange(n)
            o_h, got = f64(o[a:b, h]), [f64(t[a + rows, h]) for t in g]
            dl = f64(delta[h, a + rows])
        else:
            take = [x[seq, :, h] for x in (inp["q"], inp["k"], inp["v"], do_bits)]
            rows = np.arange(w.N)
            o_h, got = f64(o[seq, :, h]), [f64(t[seq, rows, h]) for t in g]
            dl = f64(delta[seq, h, rows])
        qh, kh, vh, doh = (oracle.bf16_decode(x) for x in take)
        _check_sampled_rows(qh, kh, vh, doh, o_h, got, dl, rows, w.scale)
