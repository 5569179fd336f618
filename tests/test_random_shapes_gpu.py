"""Seeded random configurations through every compute entry point, each
against the oracle at the tolerances of its own parity tests: sizes,
causal flag, packed document sets (empty and one-token documents included),
head counts and the sign of the scale drawn from one generator, so shapes
the hand-picked cases do not name still get checked."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL_BF16, TOL_FP8, assert_within, errors, oracle_bf16, run_bf16, to_dev

pytestmark = pytest.mark.gpu

CASES = 12


def _draw(i):
    g = np.random.default_rng(8800 + i)
    packed = bool(g.integers(0, 2))
    causal = bool(g.integers(0, 2))
    H = int(g.integers(1, 4))
    if packed:
        lengths = [int(x) for x in g.integers(0, 400, size=int(g.integers(1, 9)))]
        lengths[int(g.integers(0, len(lengths)))] = int(g.integers(1, 3))
        cu = [int(c) for c in W.cu_seqlens_from_lengths(lengths)]
        if cu[-1] == 0:
            cu[-1] = 1
            cu = [0] * (len(cu) - 1) + [1]
        B, N = len(cu) - 1, cu[-1]
    else:
        cu = None
        B, N = int(g.integers(1, 3)), int(g.integers(1, 700))
    scale = float(np.float32((1 if g.integers(0, 4) else -1) * g.uniform(0.02, 0.2)))
    return dict(packed=packed, causal=causal, H=H, B=B, N=N, cu=cu, scale=scale, seed=9000 + 10 * i)


def _shape(c, d):
    return (c["N"], c["H"], d) if c["packed"] else (c["B"], c["N"], c["H"], d)


@pytest.mark.parametrize("i", range(CASES))
def test_random_bf16_forward(i):
    c = _draw(i)
    for d in (64, 128):
        q, k, v = (W.normal_bf16(c["seed"] + j + d, _shape(c, d)) for j in range(3))
        O, L, _ = run_bf16(q, k, v, c["scale"], c["causal"], cu_seqlens=c["cu"])
        Or, Lr = oracle_bf16(q, k, v, c["scale"], c["causal"], cu_seqlens=c["cu"])
        assert_within(errors(O, Or, L, Lr), TOL_BF16)


@pytest.mark.parametrize("i", range(CASES))
def test_random_backward(i):
    import test_backward_gpu as T
    c = _draw(i)
    for d in (64, 128):
        bits = tuple(W.normal_bf16(c["seed"] + 5 + j + d, _shape(c, d)) for j in range(4))
        T.check_case(bits, c["scale"], c["causal"], c["cu"])


@pytest.mark.parametrize("i", range(CASES))
def test_random_fp8_and_mxfp8(i):
    """Per-128 fp8 and MXFP8 through the GPU quantisers, against the oracle
    on the dequantised operands."""
    import torch
    import io_aware_exact_attn_amd as ia
    import oracle.quantize as oq
    import test_mx_gpu as M
    c = _draw(i)
    d = 128
    # 1% +-20 outliers in all of Q, K and V, as in the fp8 workload
    q, k, v = (W.normal_bf16(c["seed"] + 20 + j, _shape(c, d), outliers=True) for j in range(3))
    O, L, deq = M.mx_chain(q, k, v, c["scale"], c["causal"], c["cu"])
    Or, Lr = oracle.attention(*deq, c["scale"], causal=c["causal"], cu_seqlens=c["cu"])
    assert_within(errors(O, Or, L, Lr), TOL_FP8)
    B, N, H = c["B"], c["N"], c["H"]
    cud = to_dev(np.asarray(c["cu"], np.int32)) if c["packed"] else None
    nsl = (H, -(-N // 128) + B) if c["packed"] else (B, H, -(-N // 128))
    ops = []
    for x in (q, k, v):
        y = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        s = torch.full(nsl, 1.0, dtype=torch.float32, device="cuda")
        ia.attn_quantize_fp8(to_dev(x), y, s, B, H, N, d, cud)
        ops.append((y, s))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N) if c["packed"] else (B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd_fp8(*(y.view(torch.float8_e4m3fn) for y, _ in ops), *(s for _, s in ops), o, lse, B, H, N, d,
                    c["scale"], int(c["causal"]), cud)
    torch.cuda.synchronize()
    deq = [oq.dequantize_blocks(y.cpu().numpy(), s.cpu().numpy(), c["cu"]) for y, s in ops]
    Or, Lr = oracle.attention(*deq, c["scale"], causal=c["causal"], cu_seqlens=c["cu"])
    assert_within(errors(o.float().cpu().numpy().astype(np.float64), Or,
                         lse.cpu().numpy().astype(np.float64), Lr), TOL_FP8)
