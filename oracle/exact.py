"""Plain fp64 exact attention: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  No code is shared with the HIP kernels.

What it computes.  "Flash Attention và IO" (aihero.vn) defines attention as
comparing each query with the keys to get weights, normalising them, and
summing the values with those weights: O = softmax(Q K^T) V (diagram of the
page and its opening).  Its section "Tiling giữ công việc ở gần nơi tính"
states that the tiled method is exact: it differs from this plain result only
by floating-point evaluation order.  So the oracle is the plain definition,
not the tiled algorithm: for every visible set of keys it forms all scores of
a query row, subtracts the row maximum (the stable softmax of the section
"Softmax qua nhiều khối cần thống kê chạy"), exponentiates, normalises and
forms the weighted sum, in float64.

Conventions where the pages are silent (each is a stated reading):
  * scores are s_ij = scale * sum_c q_ic k_jc, then an additive mask of -inf;
  * causal: key j is visible to query i iff j <= i (one sequence length for
    queries and keys, aligned at the first token);
  * packed documents (cu_seqlens): a query sees only keys of its own
    document, with the causal rule applied to positions inside the document;
  * LSE_i = m_i + ln(sum_j exp(s_ij - m_i)), natural log, of the scaled and
    masked scores;
  * a row with no visible key has O = 0 and LSE = -inf (cannot occur in the
    measured workloads).

Layouts: q, k, v are [B, N, H, d] (packed: [N_total, H, d] with host
cu_seqlens of B+1 int entries); O has the same layout; LSE is [B, H, N]
(packed: [H, N_total]).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

_ROW_CHUNK = 512   # rows of scores held at once; bounds memory only


def _rows_plain(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                row_ids: np.ndarray, causal: bool):
    """Exact attention for the query rows ``q_rows`` (positions ``row_ids``)
    of one sequence with keys k [n, d] and values v [n, dv]; float64."""
    n = k.shape[0]
    s = float(scale) * (q_rows @ k.T)                      # [r, n] scores
    if causal:
        mask = np.arange(n)[None, :] > row_ids[:, None]    # future keys
        s = np.where(mask, -np.inf, s)
    m = s.max(axis=1)                                      # row maxima
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])                        # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (p @ v) / l[:, None]
        lse = m_safe + np.log(l)
    o = np.where(empty[:, None], 0.0, o)
    lse = np.where(empty, -np.inf, lse)
    return o, lse


def _sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal: bool, rows: Optional[np.ndarray] = None):
    """Exact attention of one (sequence, head): q, k [n, d], v [n, dv]."""
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, _ROW_CHUNK):
        r = rows[c0:c0 + _ROW_CHUNK]
        o[c0:c0 + r.size], lse[c0:c0 + r.size] = _rows_plain(q[r], k, v, scale, r, causal)
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False,
              cu_seqlens: Optional[Sequence[int]] = None,
              heads: Optional[Iterable[int]] = None):
    """Exact attention forward in float64.

    q, k, v: arrays convertible to float64, [B, N, H, d] or, with
    ``cu_seqlens``, [N_total, H, d].  ``heads`` restricts the computation to
    some heads (the other heads of the outputs are left as NaN).
    Returns (O, LSE): O like q (float64), LSE [B, H, N] or [H, N_total].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if cu_seqlens is not None:
        cu = [int(x) for x in cu_seqlens]
        Nt, H, _ = q.shape
        O = np.full(v.shape[:2] + (v.shape[2],), np.nan)
        L = np.full((H, Nt), np.nan)
        hs = range(H) if heads is None else heads
        for doc in range(len(cu) - 1):
            a, b = cu[doc], cu[doc + 1]
            if b <= a:
                continue
            for h in hs:
                O[a:b, h], L[h, a:b] = _sequence(q[a:b, h], k[a:b, h], v[a:b, h], scale, causal)
        return O, L
    B, N, H, _ = q.shape
    O = np.full((B, N, H, v.shape[3]), np.nan)
    L = np.full((B, H, N), np.nan)
    hs = range(H) if heads is None else heads
    for b in range(B):
        for h in hs:
            O[b, :, h], L[b, h] = _sequence(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal)
    return O, L


def attention_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows,
                   cu_seqlens: Optional[Sequence[int]] = None):
    """Exact attention for selected query rows of one (batch, head).

    Fixed length: ``rows`` are positions in sequence b.  Packed (cu_seqlens
    given, b ignored): ``rows`` are global token indices; each row attends
    within its own document.  Returns (O [len(rows), dv], LSE [len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    if cu_seqlens is None:
        qs = np.asarray(q[b, :, h], dtype=np.float64)
        ks = np.asarray(k[b, :, h], dtype=np.float64)
        vs = np.asarray(v[b, :, h], dtype=np.float64)
        return _sequence(qs, ks, vs, scale, causal, rows)
    cu = np.asarray([int(x) for x in cu_seqlens])
    O = np.empty((rows.size, v.shape[2]))
    L = np.empty(rows.size)
    doc_of = np.searchsorted(cu, rows, side="right") - 1
    for doc in np.unique(doc_of):
        sel = np.nonzero(doc_of == doc)[0]
        a, e = int(cu[doc]), int(cu[doc + 1])
        qs = np.asarray(q[a:e, h], dtype=np.float64)
        ks = np.asarray(k[a:e, h], dtype=np.float64)
        vs = np.asarray(v[a:e, h], dtype=np.float64)
        O[sel], L[sel] = _sequence(qs, ks, vs, scale, causal, rows[sel] - a)
    return O, L


def online_softmax_states(scores: Sequence[float], values: Sequence[Sequence[float]],
                          blocks: Sequence[Sequence[int]]):
    """The running-statistics softmax of "Flash Attention và IO", section
    "Softmax qua nhiều khối cần thống kê chạy", for one query row.

    State: running maximum m, normaliser l, weighted value sum u.  For each
    block with maximum m_b: m_new = max(m, m_b); the old l and u are scaled by
    exp(m - m_new); the block's scores contribute exp(s - m_new) to l and
    exp(s - m_new) * value to u.  The result is u / l.

    ``blocks`` lists the score indices of each block in processing order.
    Returns (states, result): states[t] = (m, l, u) after block t.
    Used only to reproduce the page's worked example and to cross-check the
    plain definition; never the reference for the GPU path.
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    m = -math.inf
    l = 0.0
    u = np.zeros(vals.shape[1])
    states = []
    for blk in blocks:
        blk = list(blk)
        m_b = float(np.max(s[blk]))
        m_new = max(m, m_b)
        shrink = math.exp(m - m_new) if m != -math.inf else 0.0
        coef = np.exp(s[blk] - m_new)
        l = l * shrink + float(coef.sum())
        u = u * shrink + coef @ vals[blk]
        m = m_new
        states.append((m, l, u.copy()))
    return states, u / l


# ---------------------------------------------------------------------------
# number formats, decoded from their definitions
# ---------------------------------------------------------------------------

def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  bf16 is the upper 16 bits of
    an IEEE-754 binary32: sign, 8 exponent bits (bias 127), 7 fraction bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        val = np.where(e == 0, np.ldexp(f / 128.0, -126),
                       np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int32)))
        val = np.where(e == 0xFF, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def e4m3_decode(bytes_) -> np.ndarray:
    """OCP 8-bit float E4M3 ("e4m3fn") bytes -> float64.

    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field
    0 is subnormal: (m / 8) * 2**-6.  Otherwise (1 + m / 8) * 2**(e - 7).
    There are no infinities; exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN,
    so the largest finite value is 1.75 * 2**8 = 448.
    """
    b = np.asarray(bytes_, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequantize_e4m3_blocks(bytes_, scales, block: int = 128) -> np.ndarray:
    """Block-scaled e4m3 tensor -> float64 values.

    bytes_ [B, N, H, d] uint8, scales [B, H, N // block] float32: token t of
    (b, h) is multiplied by scales[b, h, t // block].  The product of an e4m3
    value (<= 4 significant bits) and an fp32 scale (24 bits) is exact in
    float64.
    """
    x = e4m3_decode(bytes_)
    s = np.asarray(scales, dtype=np.float64)            # [B, H, nb]
    B, N, H, d = x.shape
    per_tok = np.repeat(s, block, axis=2)[:, :, :N]     # [B, H, N]
    return x * per_tok.transpose(0, 2, 1)[:, :, :, None]
