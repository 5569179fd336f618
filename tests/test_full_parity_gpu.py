"""Whole-tensor parity at the measured workloads' full sizes: every query row of
every (sequence or document, head), O and LSE element by element against the
fp64 oracle on the same seeded inputs, in the launch configuration the
benchmark times.  The sampled-row tests elsewhere are quicker pre-checks; these
leave no row unchecked ("Flash Attention và IO", section "Bài tập kiểm tính
đúng trước khi đo tốc độ": compare outputs at dtype-appropriate thresholds
before timing).

The oracle runs per (sequence, head) and only its errors are kept, so the host
holds one head's fp64 result at a time."""
import numpy as np
import pytest

import oracle
import oracle.mx as omx
import workloads as W
from parity import TOL_BF16_WORKLOAD, TOL_F32, TOL_FP8, assert_within, bf16_half_ulp, run_bf16, run_fp8, to_dev

pytestmark = pytest.mark.gpu


class Acc:
    """Running error statistics over many (sequence, head) slices."""

    def __init__(self, out):
        self.out, self.n, self.sum_raw, self.sum_ex = out, 0, 0.0, 0.0
        self.max_raw = self.max_ex = self.lse = 0.0
        self.nonfinite = 0

    def add(self, o, r, l, lr):
        o = np.asarray(o, np.float64)
        d = np.abs(o - r)
        self.n += d.size
        self.sum_raw += float(d.sum())
        self.max_raw = max(self.max_raw, float(d.max()))
        if self.out == "bf16":
            ex = np.maximum(0.0, d - bf16_half_ulp(np.maximum(np.abs(o), np.abs(r))))
            self.sum_ex += float(ex.sum())
            self.max_ex = max(self.max_ex, float(ex.max()))
        self.lse = max(self.lse, float(np.abs(np.asarray(l, np.float64) - lr).max()))
        self.nonfinite += int((~np.isfinite(o)).sum()) + int((~np.isfinite(l)).sum())

    def result(self):
        res = {"max_raw": self.max_raw, "mean": self.sum_raw / self.n, "lse": self.lse, "nonfinite": self.nonfinite}
        if self.out == "bf16":
            res.update(max_excess=self.max_ex, mean_excess=self.sum_ex / self.n)
        return res


def test_long_context_every_row():
    """B 1, H 32, N 16384, causal, Q/K outliers: all 32 heads, bf16 and fp32 output."""
    w = W.workload(3)
    inp = W.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    outs = {out: run_bf16(q, k, v, w.scale, True, out=out)[:2] for out in ("bf16", "f32")}
    qd, kd, vd = (oracle.bf16_decode(x) for x in (q, k, v))
    acc = {out: Acc(out) for out in outs}
    for h in range(w.H):
        o_ref, l_ref = oracle.attention(qd[:, :, h:h + 1], kd[:, :, h:h + 1], vd[:, :, h:h + 1], w.scale, causal=True)
        for out, (O, L) in outs.items():
            acc[out].add(O[:, :, h], o_ref[:, :, 0], L[:, h], l_ref[:, 0])
    for out in outs:
        err = acc[out].result()
        print("long-context every row", out, err)
        assert_within(err, TOL_BF16_WORKLOAD if out == "bf16" else TOL_F32)


def test_packed_documents_every_row():
    """32768 packed tokens (26 documents), H 16, document-local causal mask."""
    w = W.workload(4)
    inp = W.make_inputs(w)
    q, k, v, cu = inp["q"], inp["k"], inp["v"], inp["cu_seqlens"]
    outs = {out: run_bf16(q, k, v, w.scale, True, out=out, cu_seqlens=cu)[:2] for out in ("bf16", "f32")}
    qd, kd, vd = (oracle.bf16_decode(x) for x in (q, k, v))
    acc = {out: Acc(out) for out in outs}
    for h in range(w.H):
        o_ref, l_ref = oracle.attention(qd[:, h:h + 1], kd[:, h:h + 1], vd[:, h:h + 1], w.scale, causal=True,
                                        cu_seqlens=cu)
        for out, (O, L) in outs.items():
            acc[out].add(O[:, h], o_ref[:, 0], L[h], l_ref[0])
    for out in outs:
        err = acc[out].result()
        print("packed every row", out, err)
        assert_within(err, TOL_BF16_WORKLOAD if out == "bf16" else TOL_F32)


def test_fp8_every_row():
    """B 2, H 16, N 8192, causal, e4m3 with 128-token block scales, 1% +-20
    outliers in Q, K and V: all 32 (sequence, head) pairs against the oracle
    on the dequantised operands."""
    w = W.workload(5)
    i = W.make_inputs(w)
    O, L = run_fp8(i["q"], i["k"], i["v"], i["q_scale"], i["k_scale"], i["v_scale"], w.scale, True)
    qd, kd, vd = (oracle.dequantize_e4m3_blocks(i[t], i[t + "_scale"]) for t in "qkv")
    acc = Acc("bf16")
    for b in range(w.B):
        for h in range(w.H):
            o_ref, l_ref = oracle.attention(qd[b:b + 1, :, h:h + 1], kd[b:b + 1, :, h:h + 1],
                                            vd[b:b + 1, :, h:h + 1], w.scale, causal=True)
            acc.add(O[b, :, h], o_ref[0, :, 0], L[b, h], l_ref[0, 0])
    err = acc.result()
    print("fp8 every row", err)
    assert_within(err, TOL_FP8)


def test_mxfp8_every_row():
    """The MXFP8 run `bench.py --extra mxfp8` times: the fp8 workload's bf16
    Q, K, V (1% +-20 outliers in all three) quantised to MXFP8 on the GPU,
    causal; all 32 (sequence, head) pairs against the oracle on the
    dequantised operands."""
    import torch
    import io_aware_exact_attn_amd as ia
    w = W.workload(5)
    B, N, H, d = w.B, w.N, w.H, w.d
    shape = (B, N, H, d)
    bits = [W.normal_bf16(W.tensor_seed(5, t), shape, True) for t in ("q", "k", "v")]
    ys = [torch.empty(shape, dtype=torch.uint8, device="cuda") for _ in range(3)]
    ss = [torch.empty((B, N, H, d // 32), dtype=torch.uint8, device="cuda") for _ in range(2)]
    ss.append(torch.empty((B, H, N // 32, d), dtype=torch.uint8, device="cuda"))
    for t in range(3):
        ia.attn_quantize_mxfp8(to_dev(bits[t]), ys[t], ss[t], B, H, N, d, None, int(t == 2))
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ia.attn_fwd_mxfp8(ys[0], ys[1], ys[2], ss[0], ss[1], ss[2], o, lse, B, H, N, d, w.scale, 1)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    yh = [y.cpu().numpy() for y in ys]
    sh = [s.cpu().numpy() for s in ss]
    qd = omx.dequantize_mx_d(yh[0], sh[0])
    kd = omx.dequantize_mx_d(yh[1], sh[1])
    vd = omx.dequantize_mx_tokens(yh[2], sh[2])
    acc = Acc("bf16")
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = oracle.attention(qd[b:b + 1, :, h:h + 1], kd[b:b + 1, :, h:h + 1],
                                            vd[b:b + 1, :, h:h + 1], w.scale, causal=True)
            acc.add(O[b, :, h], o_ref[0, :, 0], L[b, h], l_ref[0, 0])
    err = acc.result()
    print("mxfp8 every row", err)
    assert_within(err, TOL_FP8)
