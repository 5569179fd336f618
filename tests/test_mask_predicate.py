"""Host-side check of the wave-uniform tests with which the backward kernels
skip the causal and tail mask (attn_bwd.hip), by brute force over tile
offsets, on the CPU.

Whenever a test selects the unmasked weight loop, every score that loop
keeps must be visible: both positions inside the sequence and, under the
causal mask, the key no later than the query.  In the dK/dV kernels every
query of the 32-row block feeds the key's gradient sums, so all of them
count; in the dQ kernel only the rows that are stored (inside the
sequence) do.
"""
import itertools

import pytest

BN = 64


def dkdv_unmasked(causal, q0, half, wk0, seq_len):
    """The dK/dV kernels' test (`half` is the 32-query half of the tile)."""
    return (not causal or q0 + half * 32 >= wk0 + 31) and q0 + half * 32 + 32 <= seq_len and wk0 + 32 <= seq_len


def dq_unmasked(causal, wq0, kv0, kb, seq_len):
    """The dQ kernel's test (`kb` is the 32-key half of the tile)."""
    vis_lo = min(wq0, seq_len - 1) if causal else seq_len - 1
    return vis_lo >= kv0 + kb * 32 + 31


def _visible(causal, q, k, seq_len):
    return q < seq_len and k < seq_len and (not causal or k <= q)


@pytest.mark.parametrize("causal", [False, True])
def test_dkdv_skip_is_sound(causal):
    taken = 0
    for seq_len in (1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 256, 300):
        for j, half, wk0 in itertools.product(range(-(-seq_len // BN)), (0, 1), range(0, seq_len, 32)):
            q0 = j * BN
            if not dkdv_unmasked(causal, q0, half, wk0, seq_len):
                continue
            taken += 1
            qs = range(q0 + half * 32, q0 + half * 32 + 32)
            assert all(_visible(causal, q, k, seq_len) for q in qs for k in range(wk0, wk0 + 32)), \
                (seq_len, q0, half, wk0)
    assert taken > 0


@pytest.mark.parametrize("causal", [False, True])
def test_dq_skip_is_sound(causal):
    taken = 0
    for seq_len in (1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 256, 300):
        for wq0, j, kb in itertools.product(range(0, seq_len, 32), range(-(-seq_len // BN)), (0, 1)):
            kv0 = j * BN
            if not dq_unmasked(causal, wq0, kv0, kb, seq_len):
                continue
            taken += 1
            stored = [q for q in range(wq0, wq0 + 32) if q < seq_len]
            keys = range(kv0 + kb * 32, kv0 + kb * 32 + 32)
            assert all(_visible(causal, q, k, seq_len) for q in stored for k in keys), (seq_len, wq0, kv0, kb)
    assert taken > 0


def test_interior_tiles_skip_the_mask():
    """The test is not vacuous: a tile well below the diagonal of a long
    causal sequence takes the unmasked loop in both kernels."""
    assert dkdv_unmasked(True, 1024, 0, 256, 16384)
    assert dq_unmasked(True, 1024, 256, 1, 16384)
    assert not dkdv_unmasked(True, 256, 0, 256, 16384)
    assert not dq_unmasked(True, 256, 256, 0, 16384)
