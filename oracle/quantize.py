"""Block-scaled e4m3 quantisation: the oracle of the quantiser kernel.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  No code is shared with the HIP kernels.

What it computes.  The FP8 part of "FlashAttention, pelatihan multi-GPU, dan
kuantisasi bobot" (section 1) quantises each tile of the operands with a
scale of its own; FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel Olarak
Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat Mekanizması", sections
"Uzun Bağlamlarda Dikkat (Attention) Maliyeti ve Blackwell Mimarisi" and
"FLAMIA Mimarisi ve Temel Tasarım İlkeleri") requires that no scale mixes
tokens across the causal boundary and that packed documents need no
repacking.  Readings taken where the pages give no formula:

  * a block is 128 consecutive tokens of one (sequence, head), over all d; in
    packed input the blocks restart at every document start (document-local),
    and a document's last block may be partial;
  * the block scale is s = amax / 448 computed in fp32 (s = 1 for an all-zero
    block), 448 being the largest finite e4m3 value;
  * each element becomes e4m3(x / s), the division done in fp32 and the
    conversion rounding to the nearest e4m3 value, ties to the even mantissa,
    saturating at +-448;
  * packed scales live in an [H, ceil(N / 128) + B] fp32 array: block k of
    document d (tokens cu[d] + 128 k ...) has slot cu[d] // 128 + d + k.
    Distinct blocks get distinct slots (a document of L tokens has
    ceil(L / 128) <= floor(L / 128) + 1 blocks and the next document's first
    slot is at least floor((cu[d] + L) / 128) + d + 1), so the slot needs no
    scan over the documents; slots no block maps to are unused.

The e4m3 encoder here is the definition written out: the candidate set is the
253 finite e4m3 values, and every input goes to the nearest one.  It shares
nothing with the input generator's encoder.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .exact import e4m3_decode

E4M3_MAX = 448.0
BLOCK = 128

# the non-negative finite e4m3 values and their bytes, in increasing order
_POS_BYTES = np.array([b for b in range(0x7F)], dtype=np.uint8)     # 0x00 .. 0x7E
_POS_VALS = e4m3_decode(_POS_BYTES)                                  # 0 .. 448, increasing


def e4m3_encode(y) -> np.ndarray:
    """float32 values -> e4m3fn bytes: nearest finite e4m3 value, ties to the
    value whose mantissa (lowest bit of the byte) is even, +-448 beyond the
    range; the sign is kept (-0.0 -> 0x80).  Inputs must not be NaN."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64).ravel()
    if np.isnan(a).any():
        raise ValueError("e4m3_encode: NaN input")
    # index of the first candidate >= a (a above 448 saturates to the last)
    hi = np.searchsorted(_POS_VALS, a, side="left")
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALS[hi] - a
    d_lo = a - _POS_VALS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_BYTES[hi] % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= E4M3_MAX, len(_POS_VALS) - 1, idx)
    out = _POS_BYTES[idx]
    sign = np.signbit(y.ravel()).astype(np.uint8) << 7
    return (out | sign).reshape(y.shape)


def _quantize_block(xb: np.ndarray):
    """One block of float32 values (any shape) -> (bytes, scale)."""
    amax = np.float32(np.max(np.abs(xb))) if xb.size else np.float32(0.0)
    s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
    y = (xb.astype(np.float32) / s).astype(np.float32)
    return e4m3_encode(y), s


def quantize_blocks(x, cu_seqlens: Optional[Sequence[int]] = None, block: int = BLOCK):
    """Block-scaled e4m3 quantisation of a float32 (or bf16-valued) tensor.

    Fixed length: x [B, N, H, d] -> (bytes [B, N, H, d] uint8,
    scales [B, H, ceil(N / block)] float32).
    Packed: x [N, H, d] with host cu_seqlens (B + 1 ints) -> (bytes [N, H, d],
    scales [H, ceil(N / block) + B] float32, unused slots NaN).
    """
    x = np.asarray(x, dtype=np.float32)
    if cu_seqlens is None:
        B, N, H, d = x.shape
        nb = -(-N // block)
        q = np.zeros(x.shape, np.uint8)
        sc = np.zeros((B, H, nb), np.float32)
        for b in range(B):
            for h in range(H):
                for k in range(nb):
                    t0, t1 = k * block, min((k + 1) * block, N)
                    q[b, t0:t1, h], sc[b, h, k] = _quantize_block(x[b, t0:t1, h])
        return q, sc
    cu = [int(c) for c in cu_seqlens]
    N, H, d = x.shape
    B = len(cu) - 1
    q = np.zeros(x.shape, np.uint8)
    sc = np.full((H, -(-N // block) + B), np.nan, np.float32)
    for doc in range(B):
        s0, s1 = cu[doc], cu[doc + 1]
        for k in range(-(-(s1 - s0) // block)):
            t0, t1 = s0 + k * block, min(s0 + (k + 1) * block, s1)
            slot = scale_slot(cu, doc, k, block)
            for h in range(H):
                q[t0:t1, h], sc[h, slot] = _quantize_block(x[t0:t1, h])
    return q, sc


def scale_slot(cu_seqlens: Sequence[int], doc: int, k: int, block: int = BLOCK) -> int:
    """Slot of block k of document doc in the packed scale array."""
    return int(cu_seqlens[doc]) // block + doc + k


def dequantize_blocks(bytes_, scales, cu_seqlens: Optional[Sequence[int]] = None,
                      block: int = BLOCK) -> np.ndarray:
    """Inverse map to float64 values: e4m3 value times its block's scale (exact
    in float64).  Layouts as quantize_blocks."""
    v = e4m3_decode(bytes_)
    s = np.asarray(scales, dtype=np.float64)
    if cu_seqlens is None:
        B, N, H, d = v.shape
        per_tok = np.repeat(s, block, axis=2)[:, :, :N]           # [B, H, N]
        return v * per_tok.transpose(0, 2, 1)[:, :, :, None]
    cu = [int(c) for c in cu_seqlens]
    N, H, d = v.shape
    out = np.empty(v.shape, np.float64)
    for doc in range(len(cu) - 1):
        for t in range(cu[doc], cu[doc + 1]):
            slot = scale_slot(cu, doc, (t - cu[doc]) // block, block)
            out[t] = v[t] * s[:, slot][:, None]
    return out
