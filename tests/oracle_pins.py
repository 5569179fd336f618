"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees.
They are run directly by ``test_oracle_pins.py`` and, against deliberately
broken copies of the oracle, by ``test_oracle_mutants.py`` (every planted
mistake must trip at least one pin).  None of them re-types the oracle's
formula: each compares against a value printed on a page, a closed form, an
independent library routine (scipy), or an explicit 50-digit brute force.
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import scipy.special

import oracle


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _num(s):
    """Parse the small exact expressions used in the golden files."""
    table = {"0": 0.0, "1": 1.0, "ln2": math.log(2.0), "3/2": 1.5, "7/2": 3.5,
             "1/3": 1.0 / 3.0, "2/3": 2.0 / 3.0, "7/3": 7.0 / 3.0}
    return table[s]


def _scores_as_qk(S):
    """Inputs whose unscaled scores are exactly the matrix S [r, n]: query i is
    the unit vector e_i and key j holds column j of S.  Needs d >= r."""
    r, n = S.shape
    q = np.eye(r)
    k = np.ascontiguousarray(S.T)                       # k[j, i] = S[i, j]
    return q, k


def _fixed(q, k, v):
    """Wrap [N, d] matrices as [B=1, N, H=1, d]."""
    return q[None, :, None, :], k[None, :, None, :], v[None, :, None, :]


# --------------------------------------------------------------------------
# the page's worked example
# --------------------------------------------------------------------------

def pin_worked_example_plain():
    g = _golden("worked_example.json")
    s = np.array([_num(x) for x in g["scores"]])
    vals = np.array(g["values"])
    # one query, d = 1: q = [1], keys = the scores, scale 1
    q, k, v = _fixed(np.ones((1, 1)), s[:, None], vals[:, None])
    # a one-row query against two keys: pad the query sequence to 2 rows
    q = np.concatenate([q, q], axis=1)
    O, L = oracle.attention(q, k, v, 1.0, causal=False)
    assert abs(O[0, 0, 0, 0] - _num(g["result"])) < 1e-15, O[0, 0, 0, 0]
    assert abs(L[0, 0, 0] - math.log(3.0)) < 1e-15, L[0, 0, 0]
    w = np.exp(s - L[0, 0, 0])
    assert np.allclose(w, [_num(x) for x in g["weights"]], rtol=0, atol=1e-15)


def pin_worked_example_states():
    g = _golden("worked_example.json")
    s = [_num(x) for x in g["scores"]]
    vals = g["values"]
    states, res = oracle.online_softmax_states(s, vals, g["forward_order"]["blocks"])
    for got, want in zip(states, g["forward_order"]["states"]):
        assert abs(got[0] - _num(want["m"])) < 1e-15
        assert abs(got[1] - _num(want["l"])) < 1e-15
        assert abs(got[2][0] - _num(want["u"])) < 1e-15
    assert abs(res[0] - _num(g["result"])) < 1e-15
    # reverse order (the page's exercise): ln2 first gives (ln2, 1, 3), then the
    # zero score enters with weight exp(0 - ln2) = 1/2: (ln2, 3/2, 7/2)
    states, res = oracle.online_softmax_states(s, vals, g["reverse_order"]["blocks"])
    assert abs(states[0][0] - math.log(2)) < 1e-15 and states[0][1] == 1.0 and states[0][2][0] == 3.0
    assert abs(states[1][1] - 1.5) < 1e-15 and abs(states[1][2][0] - 3.5) < 1e-15
    assert abs(res[0] - _num(g["reverse_order"]["result"])) < 1e-15


def pin_online_matches_plain():
    """The running-statistics recurrence, in any block order, equals the plain
    definition (exactness up to rounding order)."""
    rng = np.random.default_rng(11)
    n, d = 37, 5
    s = rng.standard_normal(n) * 4
    vals = rng.standard_normal((n, d))
    q, k = _scores_as_qk(s[None, :])
    q = np.concatenate([q, np.zeros((n - 1, 1))])        # pad to n query rows
    O, L = oracle.attention(*_fixed(q, k, vals), 1.0)
    for order in (np.arange(n), rng.permutation(n)):
        blocks = [order[i:i + 8] for i in range(0, n, 8)]
        _, res = oracle.online_softmax_states(s, vals, blocks)
        assert np.allclose(res, O[0, 0, 0], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# closed forms and library routines
# --------------------------------------------------------------------------

def pin_scipy_softmax_rows():
    """Arbitrary non-symmetric score matrices: each row equals scipy's softmax
    and logsumexp of the scaled visible scores."""
    rng = np.random.default_rng(5)
    r, n, dv = 6, 9, 4
    S = rng.standard_normal((r, n)) * 3
    q, k = _scores_as_qk(S)
    q = np.concatenate([q, np.zeros((n - r, r))])       # n query rows
    k = np.asarray(k)
    v = rng.standard_normal((n, dv))
    scale = 0.37
    for causal in (False, True):
        O, L = oracle.attention(*_fixed(q, k, v), scale, causal=causal)
        for i in range(r):
            vis = np.arange(i + 1 if causal else n)
            z = scale * S[i, vis]
            assert abs(L[0, 0, i] - scipy.special.logsumexp(z)) < 1e-13
            assert np.allclose(O[0, i, 0], scipy.special.softmax(z) @ v[vis], rtol=0, atol=1e-13)


def pin_two_key_closed_form():
    """Two keys with scores s0, s1: O = (v0 + e^D v1) / (1 + e^D), D = s1 - s0,
    LSE = s0 + ln(1 + e^D)  (generalises the page's worked example)."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        s0, s1 = rng.standard_normal(2) * 5
        v = rng.standard_normal((2, 3))
        q = np.array([[1.0], [1.0]])
        k = np.array([[s0], [s1]])
        O, L = oracle.attention(*_fixed(q, k, v), 1.0)
        D = s1 - s0
        want = (v[0] + math.exp(D) * v[1]) / (1 + math.exp(D))
        assert np.allclose(O[0, 0, 0], want, rtol=0, atol=1e-13)
        assert abs(L[0, 0, 0] - (s0 + math.log1p(math.exp(D)))) < 1e-13


def pin_uniform_scores_mean():
    """Q = 0: every visible score is 0, so O_i is the mean of the visible values
    and LSE_i = ln(number of visible keys)."""
    rng = np.random.default_rng(3)
    n, d = 13, 4
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    for causal in (False, True):
        O, L = oracle.attention(*_fixed(q, k, v), 0.9, causal=causal)
        for i in range(n):
            cnt = i + 1 if causal else n
            assert np.allclose(O[0, i, 0], v[:cnt].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(L[0, 0, i] - math.log(cnt)) < 1e-14


def pin_causal_row0():
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(4)
    n, d = 10, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    O, L = oracle.attention(*_fixed(q, k, v), 0.5, causal=True)
    assert np.array_equal(O[0, 0, 0], v[0])
    assert abs(L[0, 0, 0] - 0.5 * float(np.dot(q[0], k[0]))) < 1e-14


def pin_hard_attention():
    """Query i aligned with key pi(i) at a score >= 100 above every other key
    returns V[pi(i)] (to exp(-100))."""
    rng = np.random.default_rng(8)
    n, d = 8, 8
    perm = rng.permutation(n)
    q = np.eye(n) * 20.0
    k = np.zeros((n, d))
    k[perm, np.arange(n)] = 10.0                 # key perm[i] = 10 e_i  -> score 200 with q_i
    v = rng.standard_normal((n, 5))
    O, _ = oracle.attention(*_fixed(q, k, v), 1.0)
    for i in range(n):
        assert np.allclose(O[0, i, 0], v[perm[i]], rtol=0, atol=1e-12)


def pin_lse_merge():
    """Splitting the keys into two sets A, B and merging the partial results
    by their LSEs reproduces the whole: LSE = logaddexp(LSE_A, LSE_B),
    O = e^(LSE_A - LSE) O_A + e^(LSE_B - LSE) O_B."""
    rng = np.random.default_rng(9)
    n, d = 24, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    O, L = oracle.attention(*_fixed(q, k, v), 0.7)
    A, Bk = slice(0, 10), slice(10, n)
    # queries against half of the keys: the query count must match the key
    # count in the [B, N, H, d] layout, so pad/trim q to each half's length
    OA, LA = oracle.attention(*_fixed(q[:10], k[A], v[A]), 0.7)
    qB = q[:n - 10]
    OB, LB = oracle.attention(*_fixed(qB, k[Bk], v[Bk]), 0.7)
    for i in range(10):
        lse = np.logaddexp(LA[0, 0, i], LB[0, 0, i])
        assert abs(lse - L[0, 0, i]) < 1e-12
        o = math.exp(LA[0, 0, i] - lse) * OA[0, i, 0] + math.exp(LB[0, 0, i] - lse) * OB[0, i, 0]
        assert np.allclose(o, O[0, i, 0], rtol=0, atol=1e-12)


def pin_permutation_equivariance():
    """Non-causal: permuting keys and values together leaves O unchanged;
    permuting the queries permutes the rows of O."""
    rng = np.random.default_rng(10)
    n, d = 16, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    O, L = oracle.attention(*_fixed(q, k, v), 0.3)
    p = rng.permutation(n)
    O2, L2 = oracle.attention(*_fixed(q, k[p], v[p]), 0.3)
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(L, L2, rtol=0, atol=1e-13)
    O3, L3 = oracle.attention(*_fixed(q[p], k, v), 0.3)
    assert np.allclose(O3[0, :, 0], O[0, p, 0], rtol=0, atol=1e-13)
    assert np.allclose(L3[0, 0], L[0, 0, p], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# brute force at 50 digits
# --------------------------------------------------------------------------

def _brute(q, k, v, scale, causal, lo=0, hi=None):
    """Explicit loops in mpmath (50 digits) over one sequence [lo, hi)."""
    mpmath.mp.dps = 50
    hi = q.shape[0] if hi is None else hi
    O, L = [], []
    for i in range(lo, hi):
        js = range(lo, (i + 1) if causal else hi)
        sc = [mpmath.mpf(float(scale)) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                                     for a, b in zip(q[i], k[j])) for j in js]
        w = [mpmath.e ** x for x in sc]
        tot = mpmath.fsum(w)
        O.append([mpmath.fsum(wj * mpmath.mpf(float(v[j, c])) for wj, j in zip(w, js)) / tot
                  for c in range(v.shape[1])])
        L.append(mpmath.log(tot))
    return np.array(O, dtype=np.float64), np.array(L, dtype=np.float64)


def pin_brute_force_fixed():
    rng = np.random.default_rng(12)
    for n, d, causal in ((5, 3, False), (7, 8, True), (8, 4, True), (1, 2, False)):
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        O, L = oracle.attention(*_fixed(q, k, v), 0.6, causal=causal)
        Ob, Lb = _brute(q, k, v, 0.6, causal)
        assert np.allclose(O[0, :, 0], Ob, rtol=0, atol=1e-12), (n, d, causal)
        assert np.allclose(L[0, 0], Lb, rtol=0, atol=1e-12), (n, d, causal)


def pin_brute_force_varlen():
    """Packed documents: each query attends only within its document."""
    rng = np.random.default_rng(13)
    lengths = [3, 1, 5, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    n, H, d = int(cu[-1]), 2, 4
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    for causal in (True, False):
        O, L = oracle.attention(q, k, v, 0.8, causal=causal, cu_seqlens=cu)
        for h in range(H):
            for a, b in zip(cu[:-1], cu[1:]):
                Ob, Lb = _brute(q[:, h], k[:, h], v[:, h], 0.8, causal, a, b)
                assert np.allclose(O[a:b, h], Ob, rtol=0, atol=1e-12)
                assert np.allclose(L[h, a:b], Lb, rtol=0, atol=1e-12)
        rows = np.array([0, 2, 3, 4, 8, 10])
        Or, Lr = oracle.attention_rows(q, k, v, 0.8, causal, 0, 1, rows, cu_seqlens=cu)
        assert np.allclose(Or, O[rows, 1], rtol=0, atol=1e-14)
        assert np.allclose(Lr, L[1, rows], rtol=0, atol=1e-14)


def pin_rows_subset():
    rng = np.random.default_rng(14)
    B, n, H, d = 2, 9, 3, 4
    q, k, v = (rng.standard_normal((B, n, H, d)) for _ in range(3))
    O, L = oracle.attention(q, k, v, 0.5, causal=True)
    rows = np.array([8, 0, 4])
    Or, Lr = oracle.attention_rows(q, k, v, 0.5, True, 1, 2, rows)
    Ob, Lb = _brute(q[1, :, 2], k[1, :, 2], v[1, :, 2], 0.5, True)
    assert np.allclose(Or, Ob[rows], rtol=0, atol=1e-12)
    assert np.allclose(Lr, Lb[rows], rtol=0, atol=1e-12)
    assert np.allclose(O[1, :, 2], Ob, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def pin_e4m3_decode():
    b = np.arange(256, dtype=np.uint8)
    x = oracle.e4m3_decode(b)
    # closed-form points of the OCP E4M3 definition
    assert x[0x38] == 1.0 and x[0x7E] == 448.0 and x[0xFE] == -448.0
    assert x[0x01] == 2.0 ** -9 and x[0x08] == 2.0 ** -6 and x[0x07] == 7 * 2.0 ** -9
    assert x[0x80] == 0.0 and np.signbit(x[0x80])
    assert np.isnan(x[0x7F]) and np.isnan(x[0xFF])
    assert np.count_nonzero(np.isnan(x)) == 2
    import torch
    t = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(t)
    assert np.array_equal(np.isnan(x), ~fin)
    assert np.array_equal(x[fin], t[fin])


def pin_bf16_decode():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_decode(b)
    assert x[0x3F80] == 1.0 and x[0xC000] == -2.0 and x[0x0001] == 2.0 ** -133
    import torch
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(x), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(x[fin], t[fin])


def pin_dequantize_blocks():
    B, N, H, d = 1, 256, 2, 4
    byt = np.full((B, N, H, d), 0x38, dtype=np.uint8)    # every element 1.0
    byt[0, 130, 1, 2] = 0x7E                              # 448 in block 1 of head 1
    scales = np.array([[[0.5, 2.0], [3.0, 0.25]]], dtype=np.float32)
    x = oracle.dequantize_e4m3_blocks(byt, scales)
    assert x[0, 0, 0, 0] == 0.5 and x[0, 127, 0, 3] == 0.5 and x[0, 128, 0, 0] == 2.0
    assert x[0, 5, 1, 1] == 3.0 and x[0, 200, 1, 0] == 0.25
    assert x[0, 130, 1, 2] == 448.0 * 0.25


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
