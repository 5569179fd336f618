"""Seeded synthetic inputs for the exact attention forward.

This module only *makes inputs*: random draws, the bf16 storage rounding of
those draws, the packed-document length draw and the fp8 e4m3 block
quantisation that turns bf16 tensors into the fp8 operands of the
block-scaled path.  It holds none of the attention arithmetic (no scores, no
softmax, no weighted sums), so both the fp64 oracle and the HIP path may use
it without sharing any of the method's code.

Everything is numpy.  Random numbers come from ``numpy.random.Generator``
over ``PCG64(seed)``; tensor seed = 1000 * config id + {1: Q, 2: K, 3: V,
4: document lengths}.

Workloads (the five shapes the attention forward is measured and checked
on; FlashAttention-style exact attention as described on the page
"Flash Attention và IO" (aihero.vn) and the FlashAttention-2/3 section of
"FlashAttention, pelatihan multi-GPU, dan kuantisasi bobot"):

  1  single head, non-causal, B=1 H=1 N=256 d=64, fp32 output
  2  multi-head causal, B=4 H=16 N=2048 d=128, bf16 output
  3  long-context causal, B=1 H=32 N=16384 d=128, 1% of Q/K entries +-20
  4  packed variable-length causal, 32768 tokens, H=16 d=128
  5  fp8 e4m3 block-scaled causal, B=2 H=16 N=8192 d=128, Q/K/V 1% +-20
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "tensor_seed",
    "normal_bf16", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "e4m3_encode_rne_sat", "quantize_e4m3_blocks",
    "varlen_lengths", "cu_seqlens_from_lengths", "make_inputs",
    "E4M3_MAX", "FP8_BLOCK",
]

E4M3_MAX = 448.0        # largest finite OCP e4m3fn value (1.75 * 2**8)
FP8_BLOCK = 128         # tokens per fp8 scale block


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    H: int
    d: int
    causal: bool
    B: int = 1
    N: int = 0                 # tokens per sequence (fixed length) or total tokens (varlen)
    varlen: bool = False
    fp8: bool = False
    out: str = "bf16"          # output dtype: "bf16" or "f32"
    outliers: str = ""         # which of q/k/v carry 1% +-20 outliers

    @property
    def scale(self) -> float:
        """fp32(1/sqrt(d)): the value handed to the kernel and the oracle alike."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    1: Workload(1, "single_head_noncausal_n256_d64", B=1, H=1, N=256, d=64,
                causal=False, out="f32"),
    2: Workload(2, "multihead_causal_b4_h16_n2048_d128", B=4, H=16, N=2048, d=128,
                causal=True),
    3: Workload(3, "long_context_causal_b1_h32_n16384_d128", B=1, H=32, N=16384, d=128,
                causal=True, outliers="qk"),
    4: Workload(4, "packed_varlen_causal_t32768_h16_d128", H=16, N=32768, d=128,
                causal=True, varlen=True),
    5: Workload(5, "fp8_block_scaled_causal_b2_h16_n8192_d128", B=2, H=16, N=8192, d=128,
                causal=True, fp8=True, outliers="qkv"),
}


def workload(cid: int) -> Workload:
    return WORKLOADS[cid]


def tensor_seed(cid: int, which: str) -> int:
    return 1000 * cid + {"q": 1, "k": 2, "v": 3, "lengths": 4}[which]


# ---------------------------------------------------------------------------
# bf16 storage rounding
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; returns uint16 bit patterns.

    bf16 is the top half of an IEEE binary32; RNE adds 0x7FFF plus the lowest
    kept bit before truncating.  NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, shape, outliers: bool = False) -> np.ndarray:
    """i.i.d. N(0,1) draws in C order of ``shape``, optionally with 1% +-20 outliers,
    rounded to bf16.  Returns uint16 bit patterns.

    Outliers: after the normals, the same generator draws a uniform per entry
    (entry becomes an outlier when it is < 0.01) and then a uniform per entry
    for the sign (< 0.5 gives -20).  +-20 is exact in bf16 and in e4m3.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32)
    if outliers:
        hit = rng.random(shape, dtype=np.float32) < np.float32(0.01)
        neg = rng.random(shape, dtype=np.float32) < np.float32(0.5)
        x = np.where(hit, np.where(neg, np.float32(-20.0), np.float32(20.0)), x)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# fp8 e4m3 (OCP "e4m3fn": bias 7, no infinities, 0x7F/0xFF are NaN, max 448)
# ---------------------------------------------------------------------------

def e4m3_encode_rne_sat(y: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn byte, round-to-nearest-even, saturating to +-448.

    Normal numbers (|y| >= 2**-6) keep 3 mantissa bits; below that the
    spacing is the subnormal step 2**-9.  Values whose rounding exceeds 448
    saturate to 448.  NaN maps to 0x7F.  Sign is kept, so -0.0 -> 0x80.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    _, e = np.frexp(a)                   # a = f * 2**e, f in [0.5, 1)
    E = e.astype(np.int64) - 1           # a in [2**E, 2**(E+1))
    E = np.maximum(E, -6)                # subnormal binade shares the 2**-6 exponent
    step = np.ldexp(1.0, (E - 3).astype(np.int32))
    q = np.rint(a / step) * step         # np.rint rounds half to even
    q = np.minimum(q, E4M3_MAX)
    # encode q (exactly representable) into fields
    out = np.zeros(y.shape, dtype=np.uint8)
    nz = q > 0
    qn = q[nz]
    _, e2 = np.frexp(qn)
    E2 = e2.astype(np.int64) - 1
    normal = E2 >= -6
    mant = np.where(normal,
                    np.rint(qn / np.ldexp(1.0, (E2 - 3).astype(np.int32))) - 8,
                    np.rint(qn / 2.0 ** -9))
    expf = np.where(normal, E2 + 7, 0)
    out[nz] = (expf.astype(np.uint8) << 3) | mant.astype(np.uint8)
    out = out | sign
    nan = np.isnan(y)
    if nan.any():
        out = np.where(nan, np.uint8(0x7F), out)
    return out


def quantize_e4m3_blocks(x: np.ndarray, block: int = FP8_BLOCK):
    """Block-scale a [B, N, H, d] float32 tensor to e4m3.

    One fp32 scale per (batch, head, ``block`` consecutive tokens) over all d:
    s = amax / 448 (s = 1 when the block is all zero), x_hat = e4m3(x / s)
    with the division done in fp32.  A scale is computed from its own block's
    tokens only, so no scale mixes tokens of different blocks; a last partial
    block uses just its own tokens.

    Returns (bytes uint8 [B, N, H, d], scales float32 [B, H, ceil(N / block)]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, N, H, d = x.shape
    nb = -(-N // block)
    pad = nb * block - N
    xp = np.concatenate([x, np.zeros((B, pad, H, d), np.float32)], axis=1) if pad else x
    xb = xp.reshape(B, nb, block, H, d)
    amax = np.abs(xb).max(axis=(2, 4))                     # [B, nb, H]
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    y = (xb / s[:, :, None, :, None]).astype(np.float32)
    q = e4m3_encode_rne_sat(y).reshape(B, nb * block, H, d)[:, :N]
    scales = np.ascontiguousarray(s.transpose(0, 2, 1))    # [B, H, nb]
    return np.ascontiguousarray(q), scales


# ---------------------------------------------------------------------------
# packed documents
# ---------------------------------------------------------------------------

def varlen_lengths(seed: int, total: int = 32768, mean: int = 1024,
                   lo: int = 16, hi: int = 8192) -> np.ndarray:
    """Document lengths drawn from Geometric(p = 1/mean) on {1, 2, ...}, clipped
    to [lo, hi], appended until exactly ``total`` tokens are used.

    Each draw is capped at the remaining budget; a draw that would leave a
    remainder in (0, lo) takes the whole remainder instead (or remainder - lo
    when the whole remainder exceeds hi).  So every length is in [lo, hi] and
    the lengths sum to ``total``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    remaining = total
    while remaining > 0:
        L = int(rng.geometric(1.0 / mean))
        L = min(max(L, lo), hi)
        L = min(L, remaining)
        rest = remaining - L
        if 0 < rest < lo:
            L = remaining if remaining <= hi else remaining - lo
        out.append(L)
        remaining -= L
    return np.asarray(out, dtype=np.int64)


def random_signs(seed: int, d: int) -> np.ndarray:
    """d independent fair +-1 signs (int8), the random diagonal of a
    sign-randomised Hadamard rotation."""
    u = np.random.Generator(np.random.PCG64(seed)).integers(0, 2, size=d)
    return np.where(u == 1, -1, 1).astype(np.int8)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


# ---------------------------------------------------------------------------
# one entry point for a workload
# ---------------------------------------------------------------------------

def make_inputs(w: Workload, heads: Optional[int] = None) -> dict:
    """Inputs of workload ``w`` as numpy arrays.

    bf16 workloads: q, k, v uint16 bf16 bits, [B, N, H, d] (varlen: [N, H, d]).
    fp8 workload: q, k, v uint8 e4m3 bytes [B, N, H, d] plus q_scale, k_scale,
    v_scale float32 [B, H, N // 128].  varlen also gets ``cu_seqlens`` (int32,
    docs + 1 entries) and ``lengths``.

    ``heads`` keeps only the first ``heads`` heads (draws are made at the full
    shape first, so the kept heads are identical to those of the full tensor).
    """
    shape = (w.N, w.H, w.d) if w.varlen else (w.B, w.N, w.H, w.d)
    res = {"workload": w}
    for t in ("q", "k", "v"):
        res[t] = normal_bf16(tensor_seed(w.cid, t), shape, outliers=t in w.outliers)
    if w.varlen:
        lengths = varlen_lengths(tensor_seed(w.cid, "lengths"), total=w.N)
        res["lengths"] = lengths
        res["cu_seqlens"] = cu_seqlens_from_lengths(lengths)
    if w.fp8:
        for t in ("q", "k", "v"):
            qb, sc = quantize_e4m3_blocks(bf16_bits_to_f32(res[t]))
            res[t] = qb
            res[t + "_scale"] = sc
    if heads is not None:
        for t in ("q", "k", "v"):
            res[t] = np.ascontiguousarray(res[t][..., :heads, :])
            if w.fp8:
                res[t + "_scale"] = np.ascontiguousarray(res[t + "_scale"][:, :heads, :])
    return res
