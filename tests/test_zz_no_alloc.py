"""attn_bwd_noalloc, the backward for callers that cannot allocate, against
attn_bwd (the same kernels with a caller-provided D workspace): dQ, dK and
dV must agree bit for bit, through the C ABI, on two calls in a row - the
second smaller, so a stale D left in the fixed scratch by the first call
would show - fixed length and packed documents."""
import math

import numpy as np
import pytest

import workloads as W
from parity import to_dev

pytestmark = pytest.mark.gpu


def _grads(noalloc, q, k, v, do, B, H, N, d, scale, causal, cu=None):
    import torch
    import io_aware_exact_attn_amd as ia
    packed = cu is not None
    tq, tk, tv, tdo = (to_dev(x) for x in (q, k, v, do))
    cud = to_dev(np.asarray(cu, np.int32)) if packed else None
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N) if packed else (B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd(tq, tk, tv, o, lse, B, H, N, d, scale, causal, cud, ia.ATTN_BF16)
    g = [torch.full(q.shape, 3.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    if noalloc:
        ia.attn_bwd_noalloc(tq, tk, tv, o, tdo, lse, g[0], g[1], g[2], B, H, N, d, scale, causal, cud)
    else:
        delta = torch.empty_like(lse)
        ia.attn_bwd(tq, tk, tv, o, tdo, lse, delta, g[0], g[1], g[2], B, H, N, d, scale, causal, cud)
    torch.cuda.synchronize()
    return [x.view(torch.int16).cpu().numpy() for x in g]


def _case(seed, shape):
    return [W.normal_bf16(seed + i, shape) for i in range(4)]


@pytest.mark.parametrize("order", ["large_then_small", "packed_then_fixed"])
def test_noalloc_matches_attn_bwd(order):
    calls = []
    if order == "large_then_small":
        calls.append(dict(shape=(2, 700, 3, 128), causal=1, cu=None, seed=10))
        calls.append(dict(shape=(1, 130, 2, 64), causal=0, cu=None, seed=20))
    else:
        lengths = [300, 1, 0, 129, 64, 500]
        cu = [int(c) for c in W.cu_seqlens_from_lengths(lengths)]
        calls.append(dict(shape=(cu[-1], 4, 128), causal=1, cu=cu, seed=30))
        calls.append(dict(shape=(1, 200, 2, 128), causal=1, cu=None, seed=40))
    for c in calls:
        shape, cu = c["shape"], c["cu"]
        if cu is None:
            B, N, H, d = shape
        else:
            N, H, d = shape
            B = len(cu) - 1
        q, k, v, do = _case(c["seed"], shape)
        scale = 1 / math.sqrt(d)
        ref = _grads(False, q, k, v, do, B, H, N, d, scale, c["causal"], cu)
        got = _grads(True, q, k, v, do, B, H, N, d, scale, c["causal"], cu)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert np.array_equal(a, b), (order, shape, name)


def test_noalloc_rejects_more_rows_than_its_scratch():
    import io_aware_exact_attn_amd as ia
    P = 0x10000
    st = ia.attn_bwd_noalloc(P, P, P, P, P, P, P, P, P, 1, 32, (1 << 16) + 1, 128, 0.1, 1, None, stream=0,
                             check=False)
    assert st == ia.ATTN_ERR_SCRATCH
