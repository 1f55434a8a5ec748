"""Pins of the oracle's sparse-attention backward (CPU): torch autograd in
float64 on a dense masked formulation written here independently, finite
differences of the oracle's own forward, and closed forms."""
import numpy as np
import pytest
import torch

import oracle.msa_oracle as om
from oracle import sparse_attention, sparse_attention_backward
from synthetic.gen import to_bf16_bits


def _case(seed, qo, kv, Hq, Hkv, k, B=16, dtype_bits=True):
    rng = np.random.default_rng(seed)
    T = sum(qo)
    nbs = [-(-L // B) for L in kv]
    N = sum(nbs) + 2
    kvi = rng.permutation(N)[:sum(nbs)].astype(np.int32)
    q = to_bf16_bits(rng.standard_normal((T, Hq, 32)).astype(np.float32))
    kp = to_bf16_bits(rng.standard_normal((N, Hkv, B, 32)).astype(np.float32))
    vp = to_bf16_bits(rng.standard_normal((N, Hkv, B, 32)).astype(np.float32))
    dout = to_bf16_bits(rng.standard_normal((T, Hq, 32)).astype(np.float32))
    sel = np.full((T, Hkv, k), -1, np.int32)
    lay = om.Layout(qo, kv, B)
    for r in range(T):
        loc = lay.local(r)
        for g in range(Hkv):
            others = rng.permutation(loc)[:min(k - 1, loc)]
            sel[r, g, :others.size + 1] = np.sort(np.concatenate([others, [loc]]))
    return q, kp, vp, kvi, sel, dout, lay


def _bits_to_t(b):
    return torch.from_numpy((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


@pytest.mark.parametrize("qo,kv,Hq,Hkv,k", [([40], [40], 4, 2, 2), ([20, 33], [50, 33], 4, 1, 3), ([17], [64], 2, 2, 1)])
def test_backward_matches_torch_autograd_dense_masked(qo, kv, Hq, Hkv, k):
    """dq, dk, dv equal torch autograd of sum(out * dout), where out is
    softmax attention over a dense key axis with the selection-and-causal
    mask, keys taken from the pools by the page table."""
    B = 16
    q, kp, vp, kvi, sel, dout, lay = _case(3, qo, kv, Hq, Hkv, k, B)
    scale = 0.3
    dq, dk, dv = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, scale, dout)
    Kt, Vt = _bits_to_t(kp).requires_grad_(), _bits_to_t(vp).requires_grad_()
    Qt = _bits_to_t(q).requires_grad_()
    loss = 0
    G = Hq // Hkv
    for s in range(len(kv)):
        L = kv[s]
        j = torch.arange(L)
        pages = torch.from_numpy(kvi[lay.page_start[s]:lay.page_start[s + 1]].astype(np.int64))[j // B]
        for r in range(lay.row_start[s], lay.row_start[s + 1]):
            pos = lay.pos(r)
            for h in range(Hq):
                g = h // G
                blocks = [int(b) for b in sel[r, g] if b >= 0]
                mask = torch.tensor([(int(x) // B in blocks) and int(x) <= pos for x in j])
                Ks, Vs = Kt[pages, g, j % B], Vt[pages, g, j % B]
                sc = (Ks @ Qt[r, h]) * scale
                sc = torch.where(mask, sc, torch.tensor(float("-inf"), dtype=torch.float64))
                o = torch.softmax(sc, 0) @ Vs
                loss = loss + (o * _bits_to_t(dout[r, h])).sum()
    loss.backward()
    assert np.allclose(dq, Qt.grad.numpy(), atol=1e-10, rtol=1e-9)
    assert np.allclose(dk, Kt.grad.numpy(), atol=1e-10, rtol=1e-9)
    assert np.allclose(dv, Vt.grad.numpy(), atol=1e-10, rtol=1e-9)


def test_backward_matches_finite_differences_of_the_forward():
    """Directional derivatives of sum(out * dout) through the oracle forward."""
    B = 16
    qo, kv = [30], [30]
    q, kp, vp, kvi, sel, dout, lay = _case(5, qo, kv, 4, 2, 2, B)
    scale = 0.25
    dq, dk, dv = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, scale, dout)
    do = (dout.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def loss(qf, kf, vf):
        # forward on float values: patch the oracle's bf16 decoding to identity
        orig = om.bf16_to_f64
        om.bf16_to_f64 = lambda x: np.asarray(x, dtype=np.float64)
        try:
            out, _ = sparse_attention(qf, kf, vf, kvi, sel, qo, kv, B, scale)
        finally:
            om.bf16_to_f64 = orig
        return float((out * do).sum())
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q, K, V = f(q), f(kp), f(vp)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for X, g, which in ((Q, dq, 0), (K, dk, 1), (V, dv, 2)):
        dirn = rng.standard_normal(X.shape)
        args_p = [Q, K, V]
        args_m = [Q, K, V]
        args_p[which] = X + eps * dirn
        args_m[which] = X - eps * dirn
        fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert abs(fd - (g * dirn).sum()) <= 1e-6 * max(1.0, abs(fd)), which


def test_backward_closed_forms():
    """A row that attends to one key only: dq = dk = 0 for it, dv = dout."""
    B = 16
    qo, kv = [1], [1]
    q, kp, vp, kvi, sel, dout, lay = _case(7, qo, kv, 2, 1, 1, B)
    dq, dk, dv = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.5, dout)
    do = (dout.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    assert np.allclose(dv[kvi[0], 0, 0], do[0, 0] + do[0, 1])


def test_backward_row_and_group_restrictions_are_sums_of_parts():
    """Visiting a subset of rows or groups only drops the other terms: the
    restricted results add up to the unrestricted ones."""
    B = 16
    qo, kv = [20, 33], [50, 33]
    q, kp, vp, kvi, sel, dout, lay = _case(11, qo, kv, 4, 2, 3, B)
    full = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.3, dout)
    T = sum(qo)
    half = np.arange(0, T, 2)
    rest = np.arange(1, T, 2)
    a = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.3, dout, rows=half)
    b = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.3, dout, rows=rest)
    g0 = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.3, dout, groups=[0])
    g1 = sparse_attention_backward(q, kp, vp, kvi, sel, qo, kv, B, 0.3, dout, groups=[1])
    for i in range(3):
        assert np.allclose(a[i] + b[i], full[i], atol=1e-12)
        assert np.allclose(g0[i] + g1[i], full[i], atol=1e-12)
    assert np.abs(g0[0][:, 2:]).max() == 0 and np.abs(g0[1][:, 1]).max() == 0
    assert np.array_equal(a[0][half], full[0][half]) and np.abs(a[0][rest]).max() == 0
