"""MXFP8: e4m3 elements with one power-of-two (E8M0) scale per block of 32
elements; the oracle of the MX quantiser kernels and of the MXFP8 attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  No code is shared with the HIP kernels.

What it computes.  FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel
Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat Mekanizması",
section "FLAMIA Mimarisi ve Temel Tasarım İlkeleri") is an attention kernel
family with an MXFP8 path, and its closing section ("Yazılım Geliştiriciler ve
AI Mühendisleri İçin Çıkarımlar") warns that block micro-scales must not carry
information from future tokens.  The pages give no formula for the format;
readings taken here:

  * the format is the microscaling one the name refers to: blocks of 32
    elements share a scale 2^e stored as a biased byte (E8M0, e + 127), and
    each element is e4m3 (OCP e4m3fn, largest 448);
  * e = floor(log2(amax)) - 8 for the block maximum amax, 8 being the
    exponent of e4m3's largest binade, so amax / 2^e lies in [256, 512); e is
    clamped to [-127, 127]; an all-zero block has e = 0 (byte 127);
  * an element becomes e4m3(x / 2^e): the quotient (exact: a power-of-two
    division of a bf16 value, or below every e4m3 value) rounded to the
    nearest e4m3 value, ties to the even mantissa, and clamped to +-448
    (values in (448, 512) saturate);
  * a block is 32 elements along the contraction each product uses: Q and K
    along d (32 coordinates of one token and head; such a scale depends on
    that token only, so it can never carry a later token's information), V
    along tokens (32 consecutive tokens of one head and coordinate, the keys
    P.V sums over).  A V block restarts at every packed document's first
    token; inside a block a later token can still change an earlier token's
    scale, as with the 128-token blocks of oracle.quantize.

Layouts.  Q/K scales: [B, N, H, d // 32] bytes beside [B, N, H, d] elements
(packed: [N, H, d // 32]).  V scales: [B, H, ceil(N / 32), d] bytes, block k of
(b, h) covering tokens 32k .. 32k + 31 (packed: [H, ceil(N / 32) + B, d],
block k of document j in slot cu[j] // 32 + j + k).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .exact import e4m3_decode
from .quantize import e4m3_encode

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def _block_exponent(amax: float) -> int:
    if amax == 0:
        return 0
    e = int(np.floor(np.log2(float(amax)))) - E4M3_EMAX
    return max(-127, min(127, e))


def _quantize_group(xg: np.ndarray):
    """One block (any shape, float64 values) -> (e4m3 bytes, E8M0 byte)."""
    e = _block_exponent(float(np.max(np.abs(xg))) if xg.size else 0.0)
    y = np.clip(np.ldexp(xg, -e), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return e4m3_encode(y), np.uint8(e + 127)


def quantize_mx_d(x):
    """Q/K: blocks of 32 along the last axis (d).  x [..., d] -> (bytes like
    x, scales [..., d // 32] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    flat = x.reshape(-1, d // MX_BLOCK, MX_BLOCK)
    q = np.zeros(flat.shape, np.uint8)
    s = np.zeros(flat.shape[:2], np.uint8)
    for r in range(flat.shape[0]):
        for g in range(flat.shape[1]):
            q[r, g], s[r, g] = _quantize_group(flat[r, g])
    return q.reshape(x.shape), s.reshape(x.shape[:-1] + (d // MX_BLOCK,))


def v_scale_slot(cu_seqlens: Sequence[int], doc: int, k: int) -> int:
    """Slot of 32-token block k of document doc in the packed V scales."""
    return int(cu_seqlens[doc]) // MX_BLOCK + doc + k


def quantize_mx_tokens(x, cu_seqlens: Optional[Sequence[int]] = None):
    """V: blocks of 32 tokens per (sequence or document, head, coordinate).
    Fixed: x [B, N, H, d] -> (bytes [B, N, H, d], scales [B, H, ceil(N/32), d]).
    Packed: x [N, H, d] -> (bytes [N, H, d], scales [H, ceil(N/32) + B, d],
    unused slots 0)."""
    x = np.asarray(x, dtype=np.float64)
    if cu_seqlens is None:
        B, N, H, d = x.shape
        nb = -(-N // MX_BLOCK)
        q = np.zeros(x.shape, np.uint8)
        s = np.zeros((B, H, nb, d), np.uint8)
        for b in range(B):
            for h in range(H):
                for k in range(nb):
                    t0, t1 = k * MX_BLOCK, min((k + 1) * MX_BLOCK, N)
                    for c in range(d):
                        q[b, t0:t1, h, c], s[b, h, k, c] = _quantize_group(x[b, t0:t1, h, c])
        return q, s
    cu = [int(c) for c in cu_seqlens]
    N, H, d = x.shape
    B = len(cu) - 1
    q = np.zeros(x.shape, np.uint8)
    s = np.zeros((H, -(-N // MX_BLOCK) + B, d), np.uint8)
    for doc in range(B):
        s0, s1 = cu[doc], cu[doc + 1]
        for k in range(-(-(s1 - s0) // MX_BLOCK)):
            t0, t1 = s0 + k * MX_BLOCK, min(s0 + (k + 1) * MX_BLOCK, s1)
            slot = v_scale_slot(cu, doc, k)
            for h in range(H):
                for c in range(d):
                    q[t0:t1, h, c], s[h, slot, c] = _quantize_group(x[t0:t1, h, c])
    return q, s


def e8m0_decode(b) -> np.ndarray:
    """E8M0 bytes -> 2^(b - 127) as float64 (255, the format's NaN, is not used)."""
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)


def dequantize_mx_d(bytes_, scales) -> np.ndarray:
    v = e4m3_decode(bytes_)
    sc = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)
    return v * sc


def dequantize_mx_tokens(bytes_, scales, cu_seqlens: Optional[Sequence[int]] = None) -> np.ndarray:
    v = e4m3_decode(bytes_)
    sc = e8m0_decode(scales)
    if cu_seqlens is None:
        B, N, H, d = v.shape
        per_tok = np.repeat(sc, MX_BLOCK, axis=2)[:, :, :N]          # [B, H, N, d]
        return v * per_tok.transpose(0, 2, 1, 3)
    cu = [int(c) for c in cu_seqlens]
    N, H, d = v.shape
    out = np.zeros(v.shape)
    for doc in range(len(cu) - 1):
        for t in range(cu[doc], cu[doc + 1]):
            slot = v_scale_slot(cu, doc, (t - cu[doc]) // MX_BLOCK)
            out[t] = v[t] * sc[:, slot, :]
    return out
