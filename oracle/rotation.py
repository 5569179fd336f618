"""Incoherent processing of Q and K before e4m3 quantisation: the oracle of
the rotating quantiser kernel.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  No code is shared with the HIP kernels.

What it computes.  The FP8 part of "FlashAttention, pelatihan multi-GPU, dan
kuantisasi bobot" (section 1, its FlashAttention-3 part) softens outliers
before quantisation by multiplying Q and K by a random orthogonal matrix.  The
page names no particular matrix.  Readings taken here:

  * the matrix is M = diag(s) H_d: the coordinates of each row are first
    multiplied by random signs s_i in {+1, -1}, then the row is multiplied by
    the Sylvester Hadamard matrix H_d (H_1 = [1], H_2n = [[H_n, H_n],
    [H_n, -H_n]]; entry (i, j) = (-1)^popcount(i & j)), the usual
    randomised Hadamard choice because it costs O(d log d) per row;
  * M is left unnormalised: M M^T = d I, so (Q M)(K M)^T = d Q K^T and the
    attention on rotated operands takes scale / d (d a power of two, so the
    change of scale is exact); the per-block scale of the quantiser absorbs
    the sqrt(d) growth of the magnitudes;
  * the rotated value is the exact product rounded once to fp32 (round to
    nearest, ties to even); a sum that is exactly zero is +0 (the exact
    value carries no sign, and its e4m3 byte is then 0x00); the block
    quantiser of oracle.quantize then
    works on those fp32 values unchanged: s = amax / 448 in fp32 and each
    byte = e4m3(RN_fp32(x / s)).

The exact product.  Every entry of M is +-1, so a rotated value is a signed
sum of d bf16 values.  A bf16 value is m 2^e with an integer |m| < 256, so
the sum is an integer multiple of 2^(min e) below 2^(max e - min e + 8 + 7)
of that unit: float64 holds it exactly when the exponents of a row's nonzero
entries span at most 38 binades, whatever order the sum takes.  Rows outside
that range are summed with Python fractions and rounded to fp32 directly.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

from .quantize import quantize_blocks


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), int64 +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs) -> np.ndarray:
    """M = diag(signs) H_d as int64."""
    s = np.asarray(signs, dtype=np.int64)
    return s[:, None] * hadamard(s.shape[0])


def _exact_in_f64(row: np.ndarray) -> bool:
    nz = row[row != 0]
    if nz.size == 0:
        return True
    _, e = np.frexp(np.abs(nz))
    return int(e.max() - e.min()) <= 38


def _round_fraction_to_f32(fr: Fraction) -> np.float32:
    """The fp32 value nearest to fr, ties to even."""
    c = np.float32(float(fr))                       # within one fp32 ulp of fr
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for x in cands:
        if not np.isfinite(x):
            continue
        dist = abs(Fraction(float(x)) - fr)
        even = (int(np.asarray(x, np.float32).view(np.uint32)) & 1) == 0
        key = (dist, not even)
        if best is None or key < best[0]:
            best = (key, x)
    return np.float32(best[1])


def rotate(x, signs) -> np.ndarray:
    """Rows of x (last axis d, values exactly representable in float64)
    times M = diag(signs) H_d, each result the exact sum rounded once to
    fp32.  Returns float32 of x's shape."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    m = rotation_matrix(signs)
    assert m.shape == (d, d)
    flat = x.reshape(-1, d)
    out = (flat @ m.astype(np.float64)).astype(np.float32)
    for r in range(flat.shape[0]):
        if not _exact_in_f64(flat[r]):
            fr = [Fraction(float(v)) for v in flat[r]]
            for j in range(d):
                out[r, j] = _round_fraction_to_f32(sum((f * int(m[i, j]) for i, f in enumerate(fr)), Fraction(0)))
    out += np.float32(0.0)                          # an exact zero is +0
    return out.reshape(x.shape)


def rotate_quantize_blocks(x, signs, cu_seqlens: Optional[Sequence[int]] = None):
    """The rotating quantiser: (bytes, scales) of quantize_blocks(rotate(x))."""
    return quantize_blocks(rotate(x, signs), cu_seqlens)
