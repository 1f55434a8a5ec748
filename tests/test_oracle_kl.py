"""Pins of the oracle's proxy distillation gradient (CPU): torch autograd of
KL(p_main || softmax(z)) on a dense masked formulation written here, finite
differences of the oracle's own KL values, a closed form (proxy equal to the
main attention gives zero loss and zero gradient) and the invariant that the
proxy-K gradient of every (sequence, head) sums to zero over its keys."""
import numpy as np
import pytest
import torch

import oracle.msa_oracle as om
from oracle import proxy_kl_backward
from synthetic.gen import to_bf16_bits


def _case(seed, qo, kv, Hq, Hkv, k, B=16, d=32):
    rng = np.random.default_rng(seed)
    T = sum(qo)
    nbs = [-(-L // B) for L in kv]
    N = sum(nbs) + 2
    kvi = rng.permutation(N)[:sum(nbs)].astype(np.int32)
    bits = lambda *shape: to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q, kp = bits(T, Hq, d), bits(N, Hkv, B, d)
    pq, pk = bits(T, Hkv, d), bits(N, Hkv, B, d)
    sel = np.full((T, Hkv, k), -1, np.int32)
    lay = om.Layout(qo, kv, B)
    for r in range(T):
        loc = lay.local(r)
        for g in range(Hkv):
            others = rng.permutation(loc)[:min(k - 1, loc)]
            sel[r, g, :others.size + 1] = np.sort(np.concatenate([others, [loc]]))
    return q, kp, pq, pk, kvi, sel, lay


def _t(b):
    return torch.from_numpy((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


@pytest.mark.parametrize("qo,kv,Hq,Hkv,k", [([40], [40], 4, 2, 2), ([20, 33], [50, 33], 4, 1, 3), ([17], [64], 2, 2, 1)])
def test_kl_gradient_matches_torch_autograd(qo, kv, Hq, Hkv, k):
    B = 16
    q, kp, pq, pk, kvi, sel, lay = _case(3, qo, kv, Hq, Hkv, k, B)
    scale, pscale, gs = 0.3, 0.2, 0.7
    dpq, dpk, kl, _ = proxy_kl_backward(pq, pk, q, kp, kvi, sel, qo, kv, B, scale, pscale, grad_scale=gs)
    PQ, PK = _t(pq).requires_grad_(), _t(pk).requires_grad_()
    Q, K = _t(q), _t(kp)
    G = Hq // Hkv
    loss = 0
    for s in range(len(kv)):
        L = kv[s]
        j = torch.arange(L)
        pages = torch.from_numpy(kvi[lay.page_start[s]:lay.page_start[s + 1]].astype(np.int64))[j // B]
        for r in range(lay.row_start[s], lay.row_start[s + 1]):
            pos = lay.pos(r)
            visible = j <= pos
            for g in range(Hkv):
                blocks = [int(b) for b in sel[r, g] if b >= 0]
                chosen = visible & torch.tensor([int(x) // B in blocks for x in j])
                target = 0
                for h in range(g * G, (g + 1) * G):
                    sc = (K[pages, g, j % B] @ Q[r, h]) * scale
                    target = target + torch.softmax(sc.masked_fill(~chosen, float("-inf")), 0) / G
                z = (PK[pages, g, j % B] @ PQ[r, g]) * pscale
                logp = torch.log_softmax(z.masked_fill(~visible, float("-inf")), 0)
                term = torch.where(target > 0, target * (torch.log(target) - logp), torch.zeros(()))
                assert abs(float(term.detach().sum()) - kl[r, g]) < 1e-10
                loss = loss + gs * term.sum()
    loss.backward()
    assert np.allclose(dpq, PQ.grad.numpy(), atol=1e-10, rtol=1e-9)
    assert np.allclose(dpk, PK.grad.numpy(), atol=1e-10, rtol=1e-9)


def test_kl_gradient_matches_finite_differences_of_the_loss():
    B = 16
    qo, kv = [30], [30]
    q, kp, pq, pk, kvi, sel, lay = _case(5, qo, kv, 4, 2, 2, B)
    scale, pscale = 0.25, 0.3
    dpq, dpk, _, _ = proxy_kl_backward(pq, pk, q, kp, kvi, sel, qo, kv, B, scale, pscale)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def loss(pqf, pkf):
        orig = om.bf16_to_f64
        om.bf16_to_f64 = lambda x: np.asarray(x, dtype=np.float64)
        try:
            _, _, kl, _ = proxy_kl_backward(pqf, pkf, f(q), f(kp), kvi, sel, qo, kv, B, scale, pscale)
        finally:
            om.bf16_to_f64 = orig
        return float(kl.sum())
    PQ, PK = f(pq), f(pk)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for which, X, g in ((0, PQ, dpq), (1, PK, dpk)):
        dirn = rng.standard_normal(X.shape)
        a = [PQ, PK]
        b = [PQ, PK]
        a[which] = X + eps * dirn
        b[which] = X - eps * dirn
        fd = (loss(*a) - loss(*b)) / (2 * eps)
        assert abs(fd - (g * dirn).sum()) <= 1e-6 * max(1.0, abs(fd)), which


def test_kl_vanishes_when_the_proxy_is_the_main_attention():
    """One head per group, the proxy pair equal to the main q and K, the same
    scale and every visible block selected: p_proxy = p_main."""
    B = 16
    qo, kv = [25], [40]
    nb = 3
    q, kp, _, _, kvi, _, lay = _case(7, qo, kv, 2, 2, nb, B)
    sel = np.full((25, 2, nb), -1, np.int32)
    for r in range(25):
        loc = lay.local(r)
        sel[r, :, :loc + 1] = np.arange(loc + 1)
    dpq, dpk, kl, plse = proxy_kl_backward(q, kp, q, kp, kvi, sel, qo, kv, B, 0.4, 0.4)
    assert np.abs(kl).max() < 1e-12
    assert np.abs(dpq).max() < 1e-12 and np.abs(dpk).max() < 1e-12
    # the proxy's log-sum-exp is then the main attention's, from the oracle forward
    _, lse = om.sparse_attention(q, kp, kp, kvi, sel, qo, kv, B, 0.4)
    assert np.allclose(plse, lse, atol=1e-12)


def test_kl_proxy_k_gradient_sums_to_zero_per_sequence_and_head():
    """Both distributions sum to one, so the proxy-score gradients of a row sum
    to zero and shifting every proxy K row of a sequence changes nothing."""
    B = 16
    qo, kv = [20, 33], [50, 33]
    q, kp, pq, pk, kvi, sel, lay = _case(11, qo, kv, 4, 2, 3, B)
    _, dpk, kl, _ = proxy_kl_backward(pq, pk, q, kp, kvi, sel, qo, kv, B, 0.3, 0.3)
    assert (kl >= -1e-12).all()
    for s in range(2):
        pages = kvi[lay.page_start[s]:lay.page_start[s + 1]]
        tot = dpk[pages].sum(axis=(0, 2))                      # [heads, d]
        assert np.abs(tot).max() < 1e-10
