"""Pins of the oracle's block-sparse attention (O3) and decode (O4).

  * with every block selected it must equal dense causal GQA attention, as
    computed by torch's scaled_dot_product_attention in float64 with the KV
    heads repeated and an explicit bottom-right causal mask;
  * with only the local block it must equal SDPA under a block-diagonal
    causal mask;
  * closed forms: the first key of a sequence alone gives o = v_0; constant V
    gives that constant; zero queries give the plain mean of the visible
    selected values and lse = log(#keys);
  * invariants: page-table permutation, GQA -> MHA replication, -1 padding.
"""
import math

import numpy as np
import pytest
import torch

from oracle import sparse_attention, sparse_decode, bf16_to_f64, e4m3fn_to_f64, FP8
from synthetic.gen import to_e4m3fn_bits
from tests._build import page_table, paged_bits, bf16, rand_bf16


def _case(seed, qo, kv, Hq, Hkv, B, d=32, perm=True):
    rng = np.random.default_rng(seed)
    T = sum(qo)
    q = rand_bf16(rng, (T, Hq, d))
    krows = [rand_bf16(rng, (L, Hkv, d)) for L in kv]
    vrows = [rand_bf16(rng, (L, Hkv, d)) for L in kv]
    nbs = [-(-L // B) for L in kv]
    kvi, N = page_table(nbs, seed if perm else None, extra=2)
    nan = np.uint16(0x7FC0)
    kp = paged_bits(krows, B, kvi, N, fill=nan)
    vp = paged_bits(vrows, B, kvi, N, fill=nan)
    return q, krows, vrows, kp, vp, kvi


def _all_blocks(qo, kv, Hkv, B, k):
    rows = []
    for qo_s, kv_s in zip(qo, kv):
        for i in range(qo_s):
            loc = (kv_s - qo_s + i) // B
            sel = list(range(loc + 1))[-k:] if k < loc + 1 else list(range(loc + 1))
            rows.append([sel + [-1] * (k - len(sel))] * Hkv)
    return np.array(rows, np.int32)


def _local_only(qo, kv, Hkv, B, k):
    rows = []
    for qo_s, kv_s in zip(qo, kv):
        for i in range(qo_s):
            loc = (kv_s - qo_s + i) // B
            rows.append([[loc] + [-1] * (k - 1)] * Hkv)
    return np.array(rows, np.int32)


def _sdpa(q, krows, vrows, qo, kv, Hq, Hkv, scale, mask_fn):
    G = Hq // Hkv
    outs = []
    r0 = 0
    for s, (qo_s, kv_s) in enumerate(zip(qo, kv)):
        Q = torch.from_numpy(bf16_to_f64(q[r0:r0 + qo_s])).permute(1, 0, 2)[None]          # [1, Hq, qo, d]
        K = torch.from_numpy(bf16_to_f64(krows[s])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        V = torch.from_numpy(bf16_to_f64(vrows[s])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        i = np.arange(qo_s)[:, None]
        j = np.arange(kv_s)[None, :]
        pos = kv_s - qo_s + i
        m = torch.from_numpy(mask_fn(pos, j))
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=m, scale=scale)
        outs.append(o[0].permute(1, 0, 2).numpy())
        r0 += qo_s
    return np.concatenate(outs, 0)


@pytest.mark.parametrize("qo,kv,B,Hq,Hkv", [
    ([200], [200], 32, 4, 2),
    ([37, 1, 64], [100, 1, 300], 32, 8, 2),     # varlen, prefix rows, a single-token sequence
    ([130], [130], 128, 2, 1),                  # ragged 128-blocks
])
def test_all_blocks_selected_equals_dense_causal_gqa(qo, kv, B, Hq, Hkv):
    q, kr, vr, kp, vp, kvi = _case(1, qo, kv, Hq, Hkv, B)
    k = max(-(-L // B) for L in kv) + 1
    sel = _all_blocks(qo, kv, Hkv, B, k)
    sc = 1.0 / math.sqrt(32)
    out, lse = sparse_attention(q, kp, vp, kvi, sel, qo, kv, B, sc)
    ref = _sdpa(q, kr, vr, qo, kv, Hq, Hkv, sc, lambda pos, j: j <= pos)
    assert np.abs(out - ref).max() < 1e-12


def test_local_block_only_equals_block_diagonal_causal():
    qo, kv, B, Hq, Hkv = [150, 90], [150, 200], 32, 4, 1
    q, kr, vr, kp, vp, kvi = _case(2, qo, kv, Hq, Hkv, B)
    sel = _local_only(qo, kv, Hkv, B, 3)
    sc = 0.2
    out, _ = sparse_attention(q, kp, vp, kvi, sel, qo, kv, B, sc)
    ref = _sdpa(q, kr, vr, qo, kv, Hq, Hkv, sc, lambda pos, j: (j <= pos) & (j // B == pos // B))
    assert np.abs(out - ref).max() < 1e-12


def test_arbitrary_selection_equals_masked_sdpa():
    qo, kv, B, Hq, Hkv = [160], [160], 16, 4, 2
    q, kr, vr, kp, vp, kvi = _case(3, qo, kv, Hq, Hkv, B)
    rng = np.random.default_rng(3)
    k = 4
    sel = np.full((160, Hkv, k), -1, np.int32)
    for i in range(160):
        loc = i // B
        for g in range(Hkv):
            c = rng.choice(loc, size=min(k - 1, loc), replace=False) if loc else []
            v = sorted(list(c) + [loc])
            sel[i, g, :len(v)] = v
    out, _ = sparse_attention(q, kp, vp, kvi, sel, qo, kv, B, 0.3)
    # group-by-group SDPA with the selection written as a key mask
    G = Hq // Hkv
    for g in range(Hkv):
        sub = np.zeros((160, 160), bool)
        for i in range(160):
            for b in sel[i, g]:
                if b >= 0:
                    sub[i, b * B:(b + 1) * B] = True
        sub &= np.arange(160)[None, :] <= np.arange(160)[:, None]
        Q = torch.from_numpy(bf16_to_f64(q[:, g * G:(g + 1) * G])).permute(1, 0, 2)[None]
        K = torch.from_numpy(bf16_to_f64(kr[0][:, g:g + 1])).permute(1, 0, 2)[None]
        V = torch.from_numpy(bf16_to_f64(vr[0][:, g:g + 1])).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(sub), scale=0.3)
        assert np.abs(out[:, g * G:(g + 1) * G] - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


def test_closed_forms():
    qo, kv, B, Hq, Hkv = [70], [70], 32, 2, 1
    q, kr, vr, kp, vp, kvi = _case(4, qo, kv, Hq, Hkv, B)
    sel = _all_blocks(qo, kv, Hkv, B, 3)
    out, lse = sparse_attention(q, kp, vp, kvi, sel, qo, kv, B, 0.7)
    v0 = bf16_to_f64(vr[0][0, 0])
    # row 0 sees key 0 only
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)
    k0 = bf16_to_f64(kr[0][0, 0])
    assert abs(lse[0, 0] - 0.7 * float(bf16_to_f64(q[0, 0]) @ k0)) < 1e-12
    # constant V rows -> output is that constant
    cv = np.full((70, 1, 32), 1.5, np.float32)
    vconst = paged_bits([bf16(cv)], B, kvi, kp.shape[0], fill=np.uint16(0x7FC0))
    o2, _ = sparse_attention(q, kp, vconst, kvi, sel, qo, kv, B, 0.7)
    assert np.abs(o2 - 1.5).max() < 1e-12
    # zero queries -> plain mean of visible values; lse = log(number of keys)
    o3, l3 = sparse_attention(np.zeros_like(q), kp, vp, kvi, sel, qo, kv, B, 0.7)
    V = bf16_to_f64(vr[0][:, 0])
    for i in (0, 31, 32, 33, 69):
        assert np.abs(o3[i, 0] - V[:i + 1].mean(0)).max() < 1e-12
        assert abs(l3[i, 1] - math.log(i + 1)) < 1e-12


def test_invariances():
    qo, kv, B, Hq, Hkv = [100], [100], 16, 4, 2
    q, kr, vr, kp, vp, kvi = _case(5, qo, kv, Hq, Hkv, B, perm=False)
    rng = np.random.default_rng(5)
    sel = np.full((100, Hkv, 3), -1, np.int32)
    for i in range(100):
        loc = i // B
        for g in range(Hkv):
            c = rng.choice(loc, size=min(2, loc), replace=False) if loc else []
            v = sorted(list(c) + [loc])
            sel[i, g, :len(v)] = v
    base, lb = sparse_attention(q, kp, vp, kvi, sel, qo, kv, B, 0.25)
    # permuted page table
    kvi2, N2 = page_table([7], 99, extra=3)
    kp2 = paged_bits(kr, B, kvi2, N2, fill=np.uint16(0x7FC0))
    vp2 = paged_bits(vr, B, kvi2, N2, fill=np.uint16(0x7FC0))
    o2, l2 = sparse_attention(q, kp2, vp2, kvi2, sel, qo, kv, B, 0.25)
    assert np.array_equal(o2, base) and np.array_equal(l2, lb)
    # GQA -> MHA: repeat each KV head G times and the selection with it
    G = Hq // Hkv
    kp3 = np.repeat(kp, G, axis=1)
    vp3 = np.repeat(vp, G, axis=1)
    sel3 = np.repeat(sel, G, axis=1)
    o3, l3 = sparse_attention(q, kp3, vp3, kvi, sel3, qo, kv, B, 0.25)
    assert np.array_equal(o3, base) and np.array_equal(l3, lb)
    # extra -1 padding changes nothing
    sel4 = np.concatenate([sel, np.full((100, Hkv, 2), -1, np.int32)], axis=2)
    o4, _ = sparse_attention(q, kp, vp, kvi, sel4, qo, kv, B, 0.25)
    assert np.array_equal(o4, base)


def test_decode_all_blocks_equals_dense_and_last_prefill_row():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d = 16, 8, 2, 32
    kv = [50, 16, 33]
    T = len(kv)
    x = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in kv]
    y = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in kv]
    allk, ks = to_e4m3fn_bits(np.concatenate(x), 1)
    allv, vs = to_e4m3fn_bits(np.concatenate(y), 1)
    split = np.cumsum(kv)[:-1]
    kr, vr = np.split(allk, split), np.split(allv, split)
    nbs = [-(-L // B) for L in kv]
    kvi, N = page_table(nbs, 6, extra=1)
    kp = paged_bits(kr, B, kvi, N, fill=np.uint8(0x7F))
    vp = paged_bits(vr, B, kvi, N, fill=np.uint8(0x7F))
    q = rand_bf16(rng, (T, Hq, d))
    k = 5
    sel = np.full((T, Hkv, k), -1, np.int32)
    for s, nb in enumerate(nbs):
        sel[s, :, :nb] = np.arange(nb)
    out, lse = sparse_decode(q, kp, vp, kvi, sel, kv, B, 0.2, FP8, ks, vs)
    G = Hq // Hkv
    for s in range(T):
        K = e4m3fn_to_f64(kr[s]) * ks.astype(np.float64)[None, :, None]
        V = e4m3fn_to_f64(vr[s]) * vs.astype(np.float64)[None, :, None]
        Qt = torch.from_numpy(bf16_to_f64(q[s:s + 1])).permute(1, 0, 2)[None]
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, scale=0.2)[0].permute(1, 0, 2).numpy()
        assert np.abs(out[s] - ref[0]).max() < 1e-12
    # fp8 V scale multiplies the output
    out2, _ = sparse_decode(q, kp, vp, kvi, sel, kv, B, 0.2, FP8, ks, vs * 2)
    assert np.abs(out2 - 2 * out).max() < 1e-12


def test_mxfp4_kv_equals_bf16_path_on_the_same_values():
    """Attention over MXFP4 K/V records equals the bf16 path bit for bit on
    values both formats hold exactly (E2M1 x 2^X)."""
    from oracle import MXFP4, E2M1_TABLE, Layout
    from synthetic.gen import to_mxfp4_rows, mxfp4_pool_to_records, to_bf16_bits
    rng = np.random.default_rng(21)
    qo, kv, B, Hq, Hkv, k = [200, 1], [300, 500], 128, 4, 2, 3
    T = sum(qo)
    nbs = [-(-L // B) for L in kv]
    N = sum(nbs)
    kvi = rng.permutation(N).astype(np.int32)

    def mx_values(shape):
        codes = rng.integers(0, 16, size=shape + (128,))
        codes[..., ::32] = rng.choice([6, 7, 14, 15], size=shape + (4,))
        X = rng.integers(-4, 1, size=shape + (4,))
        return E2M1_TABLE[codes] * np.repeat(np.ldexp(1.0, X), 32, axis=-1)
    kvals, vvals = mx_values((N, Hkv, B)), mx_values((N, Hkv, B))
    q = to_bf16_bits(rng.standard_normal((T, Hq, 128)).astype(np.float32))
    sel = np.full((T, Hkv, k), -1, np.int32)
    lay = Layout(qo, kv, B)
    for r in range(T):
        loc = lay.local(r)
        for g in range(Hkv):
            pick = np.sort(rng.choice(loc + 1, size=min(k, loc + 1), replace=False))
            if loc not in pick:
                pick[-1] = loc
                pick = np.sort(pick)
            sel[r, g, :pick.size] = pick
    krec = mxfp4_pool_to_records(to_mxfp4_rows(kvals.astype(np.float32)))
    vrec = mxfp4_pool_to_records(to_mxfp4_rows(vvals.astype(np.float32)))
    a, la = sparse_attention(q, krec, vrec, kvi, sel, qo, kv, B, 0.1, MXFP4)
    b, lb = sparse_attention(q, to_bf16_bits(kvals.astype(np.float32)), to_bf16_bits(vvals.astype(np.float32)), kvi,
                             sel, qo, kv, B, 0.1)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
