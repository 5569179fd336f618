"""GPU invariants that hold exactly (bitwise) or in closed form, whatever the
size: causal row 0, uniform scores, determinism, document independence,
packed = fixed length, output canaries."""
import math

import numpy as np
import pytest

import workloads as W
from parity import run_bf16

pytestmark = pytest.mark.gpu


def _case(seed, shape):
    return tuple(W.normal_bf16(seed * 10 + i, shape) for i in range(3))


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0(d):
    q, k, v = _case(1, (2, 300, 3, d))
    O, L, _ = run_bf16(q, k, v, 0.1, True, out="bf16")
    assert np.array_equal(O[:, 0], W.bf16_bits_to_f32(v[:, 0]).astype(np.float64))
    qf, kf = W.bf16_bits_to_f32(q).astype(np.float64), W.bf16_bits_to_f32(k).astype(np.float64)
    s00 = 0.1 * np.einsum("bhd,bhd->bh", qf[:, 0], kf[:, 0])
    assert np.allclose(L[:, :, 0], s00, rtol=0, atol=1e-5)


@pytest.mark.parametrize("causal", [0, 1])
def test_uniform_scores_mean(causal):
    B, N, H, d = 1, 333, 2, 128
    _, k, v = _case(2, (B, N, H, d))
    q = np.zeros_like(k)
    O, L, _ = run_bf16(q, k, v, 0.3, causal, out="f32")
    vf = W.bf16_bits_to_f32(v).astype(np.float64)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    want = (np.cumsum(vf, axis=1) / cnt[None, :, None, None]) if causal else np.broadcast_to(vf.mean(axis=1, keepdims=True), vf.shape)
    assert np.abs(O - want).max() < 1e-4    # every weight is exactly 1; fp32 sums
    assert np.abs(L - np.log(cnt)[None, None, :]).max() < 1e-4


def test_deterministic():
    q, k, v = _case(3, (1, 1000, 4, 128))
    O1, L1, _ = run_bf16(q, k, v, 0.088, True)
    O2, L2, _ = run_bf16(q, k, v, 0.088, True)
    O3, L3, _ = run_bf16(q, k, v, 0.088, True)
    assert np.array_equal(O1, O2) and np.array_equal(O1, O3)
    assert np.array_equal(L1, L2) and np.array_equal(L1, L3)


@pytest.mark.parametrize("causal", [0, 1])
def test_document_independence(causal):
    lengths = [100, 257, 64, 500, 3]
    cu = W.cu_seqlens_from_lengths(lengths)
    q, k, v = _case(4, (int(cu[-1]), 2, 128))
    O1, L1, _ = run_bf16(q, k, v, 0.09, causal, cu_seqlens=cu)
    # perturb document 1 entirely
    a, b = cu[1], cu[2]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rnd = W.normal_bf16(999, (b - a, 2, 128))
    q2[a:b], k2[a:b], v2[a:b] = rnd, rnd[::-1], rnd
    O2, L2, _ = run_bf16(q2, k2, v2, 0.09, causal, cu_seqlens=cu)
    keep = np.ones(int(cu[-1]), bool)
    keep[a:b] = False
    assert np.array_equal(O1[keep], O2[keep])
    assert np.array_equal(L1[:, keep], L2[:, keep])
    assert not np.array_equal(O1[a:b], O2[a:b])


@pytest.mark.parametrize("causal", [0, 1])
def test_packed_equals_fixed(causal):
    # equal documents packed == the same sequences batched (bitwise)
    B, N, H, d = 3, 200, 2, 128
    q, k, v = _case(5, (B, N, H, d))
    Of, Lf, _ = run_bf16(q, k, v, 0.1, causal)
    cu = W.cu_seqlens_from_lengths([N] * B)
    Op, Lp, _ = run_bf16(q.reshape(B * N, H, d), k.reshape(B * N, H, d), v.reshape(B * N, H, d),
                         0.1, causal, cu_seqlens=cu)
    assert np.array_equal(Of.reshape(B * N, H, d), Op)
    assert np.array_equal(Lf.transpose(1, 0, 2).reshape(H, B * N), Lp)


@pytest.mark.parametrize("packed", [False, True])
def test_output_canaries(packed):
    if packed:
        cu = W.cu_seqlens_from_lengths([5, 130, 17])
        q, k, v = _case(6, (int(cu[-1]), 3, 64))
        _, _, ex = run_bf16(q, k, v, 0.1, 1, cu_seqlens=cu, canary=True)
    else:
        q, k, v = _case(6, (2, 131, 3, 64))
        _, _, ex = run_bf16(q, k, v, 0.1, 1, canary=True)
    assert ex["canary_ok"]


def test_causal_prefix_invariance():
    # rows before a changed token are bitwise unchanged (causal)
    q, k, v = _case(7, (1, 700, 2, 128))
    O1, L1, _ = run_bf16(q, k, v, 0.1, True)
    k2, v2 = k.copy(), v.copy()
    k2[0, 450:] = W.normal_bf16(5, k2[0, 450:].shape)
    v2[0, 450:] = W.normal_bf16(6, v2[0, 450:].shape)
    O2, L2, _ = run_bf16(q, k2, v2, 0.1, True)
    assert np.array_equal(O1[0, :450], O2[0, :450])
    assert np.array_equal(L1[0, :, :450], L2[0, :, :450])
