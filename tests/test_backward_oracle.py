"""Pins of the backward oracle (oracle/backward.py), on the CPU.

The gradients are checked against things that do not come from the oracle's
own formulas: central finite differences of the loss sum(dO * O) with the
forward oracle, torch's autograd through a plain float64 attention, closed
forms (all scores equal, a single key), the identity rowsum(P * dP) =
rowsum(dO * O), and the invariance of softmax to shifting every key by one
vector (so the key gradients of a sequence sum to zero).  Planted mistakes in
the oracle must each trip at least one pin.
"""
import numpy as np
import pytest

import oracle
import oracle.backward as ob

_rng = np.random.default_rng(99)


def _rand(shape):
    return _rng.standard_normal(shape)


def _fd_grads(q, k, v, do, scale, causal, cu=None, eps=1e-6):
    """Central differences of L = sum(dO * O) with respect to every input."""
    out = []
    for which in range(3):
        args = [q, k, v]
        x = args[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            for sgn in (1, -1):
                xp = x.copy()
                xp[idx] += sgn * eps
                a = list(args)
                a[which] = xp
                O, _ = oracle.attention(*a, scale, causal=causal, cu_seqlens=cu)
                g[idx] += sgn * np.nansum(do * O) / (2 * eps)
        out.append(g)
    return out


def pin_finite_differences_fixed():
    for causal in (False, True):
        q, k, v, do = _rand((1, 5, 2, 3)), _rand((1, 5, 2, 3)), _rand((1, 5, 2, 4)), _rand((1, 5, 2, 4))
        got = ob.attention_grads(q, k, v, do, 0.7, causal)
        want = _fd_grads(q, k, v, do, 0.7, causal)
        for g, w in zip(got, want):
            assert np.allclose(g, w, rtol=1e-6, atol=1e-8)


def pin_finite_differences_packed():
    cu = [0, 3, 4, 7]
    q, k, v, do = _rand((7, 2, 3)), _rand((7, 2, 3)), _rand((7, 2, 3)), _rand((7, 2, 3))
    got = ob.attention_grads(q, k, v, do, 1.3, True, cu)
    want = _fd_grads(q, k, v, do, 1.3, True, cu)
    for g, w in zip(got, want):
        assert np.allclose(g, w, rtol=1e-6, atol=1e-8)


def pin_torch_autograd():
    import torch
    for causal in (False, True):
        q, k, v, do = _rand((2, 9, 3, 8)), _rand((2, 9, 3, 8)), _rand((2, 9, 3, 8)), _rand((2, 9, 3, 8))
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        s = 0.4 * torch.einsum("bihd,bjhd->bhij", tq, tk)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(9, 9, dtype=torch.bool), 1), float("-inf"))
        o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
        (o * torch.tensor(do)).sum().backward()
        got = ob.attention_grads(q, k, v, do, 0.4, causal)
        for g, t in zip(got, (tq, tk, tv)):
            assert np.allclose(g, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_equal_scores():
    # q = 0: every visible key weighs 1/n, so dV_j is the mean of dO over the
    # rows that see j, and dK = scale dS^T Q = 0
    n = 6
    q = np.zeros((1, n, 1, 4))
    k, v, do = _rand((1, n, 1, 4)), _rand((1, n, 1, 4)), _rand((1, n, 1, 4))
    dq, dk, dv = ob.attention_grads(q, k, v, do, 0.5, False)
    assert np.allclose(dv[0, :, 0], np.repeat(do[0, :, 0].mean(axis=0, keepdims=True), n, axis=0))
    assert np.all(dk == 0)
    dq, dk, dv = ob.attention_grads(q, k, v, do, 0.5, True)
    want = np.array([sum(do[0, i, 0] / (i + 1) for i in range(j, n)) for j in range(n)])
    assert np.allclose(dv[0, :, 0], want)


def pin_single_key():
    q, k, v, do = _rand((1, 1, 2, 5)), _rand((1, 1, 2, 5)), _rand((1, 1, 2, 5)), _rand((1, 1, 2, 5))
    dq, dk, dv = ob.attention_grads(q, k, v, do, 0.3, True)
    assert np.array_equal(dv, do) and np.allclose(dq, 0) and np.allclose(dk, 0)


def pin_row_dot_identity():
    q, k, v, do = _rand((2, 11, 2, 6)), _rand((2, 11, 2, 6)), _rand((2, 11, 2, 6)), _rand((2, 11, 2, 6))
    O, _ = oracle.attention(q, k, v, 0.6, causal=True)
    D = ob.row_dot(O, do)
    # rowsum(P * dP) from scratch for one (b, h)
    b, h = 1, 0
    s = 0.6 * q[b, :, h] @ k[b, :, h].T
    s = np.where(np.triu(np.ones((11, 11), bool), 1), -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(D[b, h], (p * (do[b, :, h] @ v[b, :, h].T)).sum(axis=1))


def pin_key_shift_invariance():
    q, k, v, do = _rand((1, 13, 2, 4)), _rand((1, 13, 2, 4)), _rand((1, 13, 2, 4)), _rand((1, 13, 2, 4))
    for causal in (False, True):
        _, dk, _ = ob.attention_grads(q, k, v, do, 0.9, causal)
        assert np.allclose(dk.sum(axis=1), 0, atol=1e-12)


def pin_sampled_rows_torch_autograd():
    # grads_at against torch autograd (float64) at chosen rows, with a chunk
    # smaller than the sequence so that the row-chunked pass is exercised
    import torch
    n, d = 37, 8
    q, k, v, do = _rand((n, d)), _rand((n, d)), _rand((n, 5)), _rand((n, 5))
    rows = [0, 1, 17, 36]
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        s = 0.3 * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        (torch.softmax(s, dim=-1) @ tv * torch.tensor(do)).sum().backward()
        dq, dk, dv, parts = ob.grads_at(q, k, v, do, 0.3, causal, rows, rows, chunk=8)
        assert np.allclose(dq, tq.grad.numpy()[rows], rtol=1e-11, atol=1e-12)
        assert np.allclose(dk, tk.grad.numpy()[rows], rtol=1e-11, atol=1e-12)
        assert np.allclose(dv, tv.grad.numpy()[rows], rtol=1e-11, atol=1e-12)
        assert np.allclose(parts["L"], torch.logsumexp(s, dim=-1).detach().numpy(), atol=1e-12)


BPINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", BPINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---- planted mistakes -----------------------------------------------------

def test_grads_at_matches_full_oracle():
    """The row-sampled form equals attention_grads on the same sequence."""
    n, d = 50, 6
    q, k, v, do = _rand((n, d)), _rand((n, d)), _rand((n, d)), _rand((n, d))
    rows = [0, 13, 49]
    for causal in (False, True):
        fq, fk, fv = ob._sequence_grads(q, k, v, do, 0.5, causal)
        dq, dk, dv, _ = ob.grads_at(q, k, v, do, 0.5, causal, rows, rows, chunk=16)
        assert np.allclose(dq, fq[rows]) and np.allclose(dk, fk[rows]) and np.allclose(dv, fv[rows])


def _mutant(kind):
    def grads(q, k, v, do, scale, causal):
        n = q.shape[0]
        s = float(scale) * (q @ k.T)
        if causal:
            sel = (np.arange(n)[None, :] >= np.arange(n)[:, None]) if kind == "mask_offbyone" else \
                  (np.arange(n)[None, :] > np.arange(n)[:, None])
            s = np.where(sel, -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        p = np.divide(p, l, out=np.zeros_like(p), where=l > 0)
        dv = (p @ do) if kind == "dv_no_transpose" else p.T @ do
        dp = do @ v.T
        dd = (p * dp).sum(axis=1, keepdims=True)
        ds = p * dp if kind == "no_row_term" else p * (dp - dd)
        dq = (ds @ k) if kind == "dq_no_scale" else float(scale) * (ds @ k)
        dk = float(scale) * ((ds @ q) if kind == "dk_no_transpose" else (ds.T @ q))
        return dq, dk, dv
    return grads


_KINDS = ["mask_offbyone", "dv_no_transpose", "no_row_term", "dq_no_scale", "dk_no_transpose"]


@pytest.mark.parametrize("kind", _KINDS)
def test_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ob, "_sequence_grads", _mutant(kind))
    caught = []
    for pin in BPINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every backward pin"
