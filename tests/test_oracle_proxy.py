"""Pins of the oracle's proxy block max score (O1) by closed forms and
invariants that do not retype its formula.

Construction used for the closed forms: proxy head p reads coordinates
(2p, 2p+1) only (its query is (1, 256) there and zero elsewhere), and key j of
the head stores (j mod 256, j div 256) there, so the proxy logit of key j is
exactly j (even heads) or -j (odd heads, by negating the query).  The block
max is then the last (even) or first (odd) visible key of the block, times the
scale, which follows from causality and the block partition alone.
"""
import math

import numpy as np
import pytest

from oracle import proxy_block_maxscore, BF16, FP8
from synthetic.gen import to_e4m3fn_bits
from tests._build import page_table, paged_bits, bf16


def _positional_case(qo_lens, kv_lens, P, Pk, B, perm_seed, d=128, noise_seed=1):
    rng = np.random.default_rng(noise_seed)
    T = sum(qo_lens)
    pq = np.zeros((T, P, d), np.float32)
    for p in range(P):
        sgn = 1.0 if p % 2 == 0 else -1.0
        pq[:, p, 2 * p] = sgn
        pq[:, p, 2 * p + 1] = sgn * 256.0
    rows = []
    for L in kv_lens:
        k = rng.standard_normal((L, Pk, d)).astype(np.float32)
        j = np.arange(L)
        for p in range(P):
            ph = p if Pk == P else 0
            k[:, ph, 2 * p] = j % 256
            k[:, ph, 2 * p + 1] = j // 256
        rows.append(bf16(k))
    nbs = [-(-L // B) for L in kv_lens]
    kv_indices, N = page_table(nbs, perm_seed, extra=2)
    pool = paged_bits(rows, B, kv_indices, N, fill=np.uint16(0x7FC0))   # NaN in unused pages and tails
    return bf16(pq), pool, kv_indices


def _expected_positional(qo_lens, kv_lens, P, B, scale):
    out = []
    for qo, kv in zip(qo_lens, kv_lens):
        nb = -(-kv // B)
        for i in range(qo):
            pos = kv - qo + i
            e = np.full((P, nb), np.nan)
            for b in range(pos // B + 1):
                last = min(pos, (b + 1) * B - 1)
                first = b * B
                for p in range(P):
                    e[p, b] = scale * (last if p % 2 == 0 else -first)
            out.append(e)
    return out


@pytest.mark.parametrize("qo_lens,kv_lens,B,Pk", [
    ([300], [300], 16, 2),            # many small blocks, ragged tail
    ([256], [256], 128, 2),           # two full 128-blocks
    ([5, 40, 131], [5, 70, 300], 32, 1),  # varlen, prefix (qo < kv), shared proxy-K head
    ([1, 1], [129, 1000], 128, 2),    # decode-like rows
])
def test_positional_closed_form(qo_lens, kv_lens, B, Pk):
    P = 2 if Pk in (1, 2) else Pk
    scale = 1.0 / math.sqrt(128)
    pq, pool, kvi = _positional_case(qo_lens, kv_lens, P, Pk, B, perm_seed=7)
    ms = proxy_block_maxscore(pq, pool, kvi, qo_lens, kv_lens, B, scale)
    exp = _expected_positional(qo_lens, kv_lens, P, B, scale)
    for r, e in enumerate(exp):
        nb = e.shape[1]
        got = ms[r, :, :nb]
        assert np.array_equal(np.isnan(got), np.isnan(e)), r
        m = ~np.isnan(e)
        assert np.allclose(got[m], e[m], rtol=0, atol=1e-12), (r, got[m], e[m])


def test_page_table_permutation_invariance():
    rng = np.random.default_rng(3)
    qo, kv, B, P = [200, 77], [200, 300], 32, 3
    rows = [bf16(rng.standard_normal((L, P, 64))) for L in kv]
    pq = bf16(rng.standard_normal((sum(qo), P, 64)))
    nbs = [-(-L // B) for L in kv]
    outs = []
    for seed in (None, 11, 12):
        kvi, N = page_table(nbs, seed, extra=3)
        pool = paged_bits(rows, B, kvi, N, fill=np.uint16(0x7FC0))
        outs.append(proxy_block_maxscore(pq, pool, kvi, qo, kv, B, 0.125))
    for o in outs[1:]:
        assert np.array_equal(np.isnan(o), np.isnan(outs[0]))
        assert np.array_equal(o[~np.isnan(o)], outs[0][~np.isnan(o)])


def test_local_block_bounds_the_diagonal_score_and_all_visible_scores():
    rng = np.random.default_rng(5)
    qo, kv, B, P = [64], [160], 32, 2
    k = rng.standard_normal((kv[0], P, 32)).astype(np.float32)
    q = rng.standard_normal((qo[0], P, 32)).astype(np.float32)
    kvi, N = page_table([5], 1)
    pool = paged_bits([bf16(k)], B, kvi, N)
    s = 0.3
    ms = proxy_block_maxscore(bf16(q), pool, kvi, qo, kv, B, s)
    qf = bf16(q).astype(np.uint32) << 16
    kf = bf16(k).astype(np.uint32) << 16
    qd = qf.view(np.float32).astype(np.float64)
    kd = kf.view(np.float32).astype(np.float64)
    for i in range(qo[0]):
        pos = kv[0] - qo[0] + i
        for p in range(P):
            # each visible key's score is <= its block's max, and each block's
            # max is attained by one of its visible keys
            for b in range(pos // B + 1):
                keys = range(b * B, min(pos, (b + 1) * B - 1) + 1)
                vals = [s * float(np.dot(qd[i, p], kd[j, p])) for j in keys]
                assert ms[i, p, b] >= max(vals) - 1e-12
                assert min(abs(ms[i, p, b] - v) for v in vals) < 1e-12


def test_shared_proxy_k_head_equals_replicated_heads():
    rng = np.random.default_rng(9)
    qo, kv, B, P = [100], [100], 16, 4
    k1 = rng.standard_normal((kv[0], 1, 32)).astype(np.float32)
    q = bf16(rng.standard_normal((qo[0], P, 32)))
    kvi, N = page_table([7], 2)
    pool1 = paged_bits([bf16(k1)], B, kvi, N)
    poolP = paged_bits([bf16(np.repeat(k1, P, axis=1))], B, kvi, N)
    a = proxy_block_maxscore(q, pool1, kvi, qo, kv, B, 0.2)
    b = proxy_block_maxscore(q, poolP, kvi, qo, kv, B, 0.2)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_fp8_scales_multiply_the_scores():
    rng = np.random.default_rng(4)
    qo, kv, B, P = [90], [90], 16, 2
    q8, _ = to_e4m3fn_bits(rng.standard_normal((qo[0], P, 32)).astype(np.float32), 1)
    k8, _ = to_e4m3fn_bits(rng.standard_normal((kv[0], P, 32)).astype(np.float32), 1)
    kvi, N = page_table([6], 3)
    pool = paged_bits([k8], B, kvi, N)
    one = np.ones(P, np.float32)
    sq = np.array([0.5, 0.03125], np.float32)
    sk = np.array([4.0, 0.25], np.float32)
    base = proxy_block_maxscore(q8, pool, kvi, qo, kv, B, 1.0, FP8, one, one)
    scaled = proxy_block_maxscore(q8, pool, kvi, qo, kv, B, 1.0, FP8, sq, sk)
    m = ~np.isnan(base)
    fac = (sq * sk).astype(np.float64)[None, :, None] * np.ones_like(base)
    assert np.array_equal(scaled[m], base[m] * fac[m])    # powers of two: exact


def test_rows_subset_matches_full():
    rng = np.random.default_rng(8)
    qo, kv, B, P = [50, 60], [80, 60], 16, 2
    rows = [bf16(rng.standard_normal((L, P, 16))) for L in kv]
    nbs = [-(-L // B) for L in kv]
    kvi, N = page_table(nbs, 4)
    pool = paged_bits(rows, B, kvi, N)
    pq = bf16(rng.standard_normal((sum(qo), P, 16)))
    full = proxy_block_maxscore(pq, pool, kvi, qo, kv, B, 0.25)
    sub = [0, 49, 50, 51, 109]
    part = proxy_block_maxscore(pq, pool, kvi, qo, kv, B, 0.25, rows=sub)
    assert np.array_equal(np.nan_to_num(part, nan=7.0), np.nan_to_num(full[sub], nan=7.0))


def test_mxfp4_proxy_k_equals_bf16_path_on_the_same_values():
    """With an MXFP4 proxy K the oracle decodes the records and scores with an
    fp8 proxy q; on values that bf16 and e4m3 hold exactly (E2M1 x 2^X, e4m3
    codes with unit scale) the result must equal the bf16 path bit for bit."""
    from oracle import MXFP4, E2M1_TABLE
    from synthetic.gen import to_mxfp4_rows, mxfp4_pool_to_records, to_bf16_bits
    rng = np.random.default_rng(11)
    qo, kv, B, P, Pk = [1, 3], [700, 300], 128, 2, 1
    T = sum(qo)
    nbs = [-(-L // B) for L in kv]
    N = sum(nbs) + 1
    kvi = rng.permutation(N)[:sum(nbs)].astype(np.int32)
    codes = rng.integers(0, 16, size=(N, Pk, B, 128))
    codes[..., ::32] = rng.choice([6, 7, 14, 15], size=(N, Pk, B, 4))
    X = rng.integers(-3, 3, size=(N, Pk, B, 4))
    kvals = E2M1_TABLE[codes] * np.repeat(np.ldexp(1.0, X), 32, axis=-1)
    rec = mxfp4_pool_to_records(to_mxfp4_rows(kvals.astype(np.float32)))
    q8 = rng.integers(0, 256, size=(T, P, 128)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x10                       # no NaN codes
    one = np.ones(P, np.float32)
    from oracle import e4m3fn_to_f64
    qbits = to_bf16_bits(e4m3fn_to_f64(q8).astype(np.float32))
    kbits = to_bf16_bits(kvals.astype(np.float32))
    a = proxy_block_maxscore(q8, rec, kvi, qo, kv, B, 0.125, MXFP4, one, None)
    b = proxy_block_maxscore(qbits, kbits, kvi, qo, kv, B, 0.125, BF16)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_mxfp4_q_and_k_equal_bf16_path_on_the_same_values():
    """MXFP4 proxy q rows and MXFP4 K records decode to values bf16 holds
    exactly; the scores must equal the bf16 path's bit for bit."""
    from oracle import MXFP4_QK, E2M1_TABLE
    from synthetic.gen import to_mxfp4_rows, mxfp4_pool_to_records, to_bf16_bits
    rng = np.random.default_rng(12)
    qo, kv, B, P, Pk = [130, 1], [300, 700], 128, 2, 2
    T = sum(qo)
    nbs = [-(-L // B) for L in kv]
    N = sum(nbs)
    kvi = rng.permutation(N).astype(np.int32)

    def mx_values(shape):
        codes = rng.integers(0, 16, size=shape + (128,))
        codes[..., ::32] = rng.choice([6, 7, 14, 15], size=shape + (4,))
        X = rng.integers(-3, 3, size=shape + (4,))
        return E2M1_TABLE[codes] * np.repeat(np.ldexp(1.0, X), 32, axis=-1)
    kvals = mx_values((N, Pk, B))
    qvals = mx_values((T, P))
    rec = mxfp4_pool_to_records(to_mxfp4_rows(kvals.astype(np.float32)))
    qrows = to_mxfp4_rows(qvals.astype(np.float32))
    a = proxy_block_maxscore(qrows, rec, kvi, qo, kv, B, 0.125, MXFP4_QK)
    b = proxy_block_maxscore(to_bf16_bits(qvals.astype(np.float32)), to_bf16_bits(kvals.astype(np.float32)), kvi, qo,
                             kv, B, 0.125, BF16)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
