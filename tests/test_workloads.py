"""Seeded input generators: converters against torch's CPU casts, the packed
document length rule, and the block quantiser's locality (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rne_matches_torch_random_and_ties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1_000_000) * rng.choice([1e-30, 1e-3, 1, 1e3, 1e30], 1_000_000)).astype(np.float32)
    # exact ties: bf16 value + half an ulp (lower 16 bits = 0x8000), both parities
    u = rng.integers(0, 2**31, 200_000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (x, ties, -ties):
        got = W.f32_to_bf16_bits(arr)
        want = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)


def test_bf16_roundtrip_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(b)
    fin = np.isfinite(f)
    assert np.array_equal(W.f32_to_bf16_bits(f[fin]), b[fin])


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(2_000_000) * rng.choice([1e-4, 1e-2, 1, 30, 200], 2_000_000)).astype(np.float32)
    x = x[np.abs(x) < 464]            # torch does not saturate: >= 464 becomes NaN there
    allb = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = np.unique(allb[np.isfinite(allb)])
    mids = ((fin[:-1].astype(np.float64) + fin[1:]) / 2).astype(np.float32)
    for arr in (x, fin, mids):
        got = W.e4m3_encode_rne_sat(arr)
        want = torch.from_numpy(arr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, want)


def test_e4m3_saturates():
    x = np.array([447.9, 448, 460, 464, 1e6, -1e6, np.inf, -np.inf], dtype=np.float32)
    got = W.e4m3_encode_rne_sat(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert W.e4m3_encode_rne_sat(np.array([np.nan], np.float32))[0] == 0x7F


def test_varlen_rule():
    for seed in (4004, 4, 5, 6, 123):
        L = W.varlen_lengths(seed)
        assert L.sum() == 32768 and L.min() >= 16 and L.max() <= 8192
        assert np.array_equal(L, W.varlen_lengths(seed))
    L = W.varlen_lengths(4004)
    assert len(L) == 26 and L.min() == 126 and L.max() == 4305
    cu = W.cu_seqlens_from_lengths(L)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 32768 and len(cu) == 27


def test_varlen_remainder_rule():
    # budgets that force the "remainder in (0, 16)" branch
    for total in (17, 31, 8200, 8207, 20000):
        for seed in range(20):
            L = W.varlen_lengths(seed, total=total)
            assert L.sum() == total and L.min() >= 16 and L.max() <= 8192


def test_generators_deterministic_and_outliers():
    a = W.normal_bf16(7, (64, 4, 8), outliers=True)
    b = W.normal_bf16(7, (64, 4, 8), outliers=True)
    assert np.array_equal(a, b)
    f = W.bf16_bits_to_f32(a)
    frac = np.mean(np.abs(f) == 20.0)
    assert 0.002 < frac < 0.03
    c = W.normal_bf16(7, (64, 4, 8), outliers=False)
    assert not np.any(np.abs(W.bf16_bits_to_f32(c)) == 20.0)


def test_quantize_blocks_scale_and_locality():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 384, 3, 16)).astype(np.float32)
    x[0, 5, 1, 2] = 20.0
    q, s = W.quantize_e4m3_blocks(x)
    assert q.shape == x.shape and s.shape == (2, 3, 3)
    amax = np.abs(x.reshape(2, 3, 128, 3, 16)).max(axis=(2, 4)).transpose(0, 2, 1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the block maximum maps to +-448 (0x7E / 0xFE)
    assert set(np.unique(q.reshape(2, 3, 128, 3, 16).transpose(0, 3, 1, 2, 4).reshape(2, 3, 3, -1).__and__(0x7F).max(axis=-1)).tolist()) == {0x7E}
    # changing a token changes only its own block's scale and bytes
    y = x.copy()
    y[1, 200, 2, 0] = 50.0
    q2, s2 = W.quantize_e4m3_blocks(y)
    changed = np.argwhere(s2 != s)
    assert changed.tolist() == [[1, 2, 1]]
    diff_tok = np.unique(np.argwhere(q2 != q)[:, 1])
    assert diff_tok.min() >= 128 and diff_tok.max() < 256


def test_quantize_zero_block_scale_one():
    x = np.zeros((1, 128, 1, 4), np.float32)
    q, s = W.quantize_e4m3_blocks(x)
    assert s[0, 0, 0] == 1.0 and not q.any()


@pytest.mark.parametrize("cid", [1, 2, 4])
def test_make_inputs_shapes(cid):
    w = W.workload(cid)
    inp = W.make_inputs(w, heads=2 if w.H > 2 else None)
    shp = inp["q"].shape
    if w.varlen:
        assert shp == (w.N, 2, w.d) and inp["cu_seqlens"][-1] == w.N
    else:
        assert shp[0] == w.B and shp[1] == w.N and shp[-1] == w.d
    assert inp["q"].dtype == np.uint16


def test_make_inputs_heads_subset_is_prefix():
    w = W.workload(2)
    full = W.make_inputs(w)
    sub = W.make_inputs(w, heads=3)
    assert np.array_equal(full["k"][:, :, :3], sub["k"])


def test_scale_is_fp32_rounded():
    assert W.workload(2).scale == float(np.float32(1 / np.sqrt(128)))
    assert W.workload(1).scale == 0.125


def test_quantize_partial_last_block():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 300, 2, 8)).astype(np.float32)
    q, s = W.quantize_e4m3_blocks(x)
    assert q.shape == x.shape and s.shape == (1, 2, 3)
    # the partial block (tokens 256..299) is scaled by its own amax only
    assert s[0, 1, 2] == np.float32(np.abs(x[0, 256:, 1]).max() / np.float32(448))
    q2, s2 = W.quantize_e4m3_blocks(x[:, :256])
    assert np.array_equal(q2, q[:, :256]) and np.array_equal(s2, s[:, :, :2])
