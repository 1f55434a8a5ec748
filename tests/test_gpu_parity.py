"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs small enough for the oracle, spanning several tiles and ragged
tails: each stage is checked in turn (max scores, selection, attention), and
the attention is checked on the selection the GPU produced so that near-ties
cannot move the output.

Tolerances: max scores |gpu - oracle| <= 1e-4 + 1e-5 |oracle| (fp32
accumulation of exact bf16 products), plus, for low-precision proxy scores
(fp8, fp8 x MXFP4, MXFP4 x MXFP4 on the scaled matrix cores, which do not sum
products exactly), the library's error bound coef * scale * max|q| * max|k|;
selections by the 1e-3 band rule against the oracle's exact scores -- for
low-precision proxies this is the fused call's claim (its undecided
boundary blocks are re-scored exactly), while the separate top-k call is
exact on the scores it is given; outputs max-abs <= 2e-2 and cosine >= 0.999
(bf16 K/V) or <= 6e-2 and >= 0.99 (fp8 K/V)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs, workload, seed_of, to_bf16_bits, FP8, BF16, MXFP4, MXFP4_QK
from tests._gpu import (device_inputs, plan_for, bf16_out_to_f64, oracle_scores, check_max_score, check_selection,
                        check_output, lowp_score_bound, BF16_ATOL, BF16_COS, FP8_ATOL, FP8_COS, LOW_PRECISION_PROXY)

pytestmark = pytest.mark.gpu


def _msa():
    from block_sparse_top_amd import msa
    return msa


PREFILL_CASES = {
    "cfg1": (workload(1), seed_of(1), 0),
    "cfg1_shared_proxy_k": (workload(1, num_proxy_kv_heads=1, name="cfg1b"), seed_of(1), 0),
    "varlen_ragged_prefix": (Workload("ragged", [300, 77, 1, 513], [300, 200, 1, 700], 16, 4, 4, 4, topk=5,
                                      extra_pages=0.25, poison_tail=True), 11, 0),
    "gqa8": (Workload("gqa8", [640], [640], 16, 2, 2, 2, topk=3), 12, 0),
    "gqa1_gqa16": (Workload("g1", [384], [384], 2, 2, 2, 2, topk=2), 13, 0),
    "gqa16": (Workload("g16", [260], [400], 32, 2, 2, 2, topk=3, poison_tail=True), 14, 0),
    "fp8_proxy": (Workload("fp8p", [700], [700], 8, 2, 2, 2, topk=4, proxy_dtype=FP8), 15, 0),
    "lowrank": (Workload("lr", [512, 1024], [512, 1024], 16, 2, 2, 2, topk=4, lowrank=8), 16, 0),
    "chunked_calls": (Workload("chunk", [900, 333], [900, 400], 8, 2, 2, 2, topk=6, poison_tail=True), 17, 200),
    "topk_exceeds_blocks": (Workload("bigk", [500], [500], 8, 2, 2, 2, topk=9), 18, 0),
    "topk1_local_only": (Workload("k1", [450], [450], 8, 2, 2, 2, topk=1), 19, 0),
    # one query row per sequence (a decode step's indexer pass; the one-row proxy kernel)
    "onerow_fp8_shared_proxy_k": (Workload("row1a", [1] * 6, [1000, 128, 129, 2000, 5000, 131], 16, 2, 2, 1, topk=17,
                                           proxy_dtype=FP8, extra_pages=0.1, poison_tail=True), 26, 0),
    "onerow_bf16_per_head_proxy_k": (Workload("row1b", [1] * 5, [300, 7000, 256, 1, 4000], 8, 2, 2, 2, topk=5,
                                              poison_tail=True), 27, 0),
    # MXFP4 proxy K (fp8 proxy q): NaN scale bytes in spare pages and page tails
    "onerow_mxfp4_shared_proxy_k": (Workload("row1c", [1] * 6, [1000, 128, 129, 2000, 5000, 131], 16, 2, 2, 1,
                                             topk=17, proxy_dtype=MXFP4, extra_pages=0.1, poison_tail=True), 28, 0),
    "onerow_mxfp4_per_head_proxy_k": (Workload("row1d", [1] * 5, [300, 7000, 256, 1, 4000], 8, 2, 2, 2, topk=5,
                                               proxy_dtype=MXFP4, lowrank=8, poison_tail=True), 29, 0),
    "onerow_mxfp4_qk": (Workload("row1e", [1] * 4, [3000, 129, 700, 12000], 16, 2, 2, 1, topk=17,
                                 proxy_dtype=MXFP4_QK, lowrank=8, poison_tail=True), 30, 0),
    # multi-row prefill with MXFP4 proxies (several row tiles, ragged, prefix rows)
    "mxfp4_proxy_k_prefill": (Workload("mxk", [700, 77, 1], [700, 300, 1], 8, 2, 2, 1, topk=6, proxy_dtype=MXFP4,
                                       extra_pages=0.2, poison_tail=True), 31, 0),
    "mxfp4_qk_prefill": (Workload("mxqk", [600, 513], [900, 513], 16, 2, 2, 2, topk=5, proxy_dtype=MXFP4_QK,
                                  lowrank=8, poison_tail=True), 32, 200),
    # fp8 and MXFP4 K/V pages in the sparse prefill attention
    "fp8_kv_prefill": (Workload("kv8", [700, 77, 1], [700, 300, 1], 16, 4, 4, 4, topk=5, kv_dtype=FP8,
                                extra_pages=0.2, poison_tail=True), 33, 0),
    "mxfp4_kv_prefill": (Workload("kv4", [513, 300], [513, 900], 16, 2, 2, 2, topk=6, kv_dtype=MXFP4,
                                  proxy_dtype=MXFP4_QK, extra_pages=0.2, poison_tail=True), 34, 0),
}


def run_prefill_stages(msa, inp, max_rows):
    w = inp.w
    d = device_inputs(inp)
    plan = plan_for(msa, inp, max_rows_per_call=max_rows)
    T = w.total_rows
    R = plan.max_rows_per_call
    ms_all = []
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    ms = msa.max_score_buffer(plan)
    for r0 in range(0, T, R):
        n = min(R, T - r0)
        ms.fill_(float("nan"))
        msa.msa_proxy_block_maxscore(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                                     d["kv_indices"], r0, n, ms)
        msa.msa_topk_select(plan, ms, r0, n, sel)
        ms_all.append(msa.max_score_rows(ms, plan, n).cpu().numpy().copy())
    out = torch.full((T, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse,
                                d["k_scale"], d["v_scale"])
    torch.cuda.synchronize()
    return np.concatenate(ms_all, axis=2), sel.cpu().numpy(), bf16_out_to_f64(out), lse.cpu().numpy()


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_stages_match_oracle(case):
    msa = _msa()
    w, seed, max_rows = PREFILL_CASES[case]
    inp = make_inputs(w, seed)
    print(f"[parity] prefill case={case} T={w.total_rows} seed={seed}", flush=True)
    gms, gsel, gout, glse = run_prefill_stages(msa, inp, max_rows)
    ref_ms = oracle_scores(inp)
    lowp = w.proxy_dtype in LOW_PRECISION_PROXY
    extra = lowp_score_bound(inp, np.arange(w.total_rows), w.proxy_sm_scale) if lowp else None
    check_max_score(gms, ref_ms, case, extra)
    lay = O.Layout(w.qo_lens, w.kv_lens, w.page_size)
    locals_ = np.array([lay.local(r) for r in range(w.total_rows)])
    if lowp:
        # the separate top-k call is exact on the (low-precision) scores it is given
        g = np.transpose(gms, (2, 0, 1)).astype(np.float64)
        for r in range(w.total_rows):
            for p in range(w.num_kv_heads):
                exp = O.topk_select_row(g[r, p], int(locals_[r]), w.topk)
                assert np.array_equal(gsel[r, p], exp), (case, r, p, gsel[r, p], exp)
    else:
        check_selection(gsel, ref_ms, locals_, w.topk, case)
    ref_out, ref_lse = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, gsel, w.qo_lens,
                                          w.kv_lens, w.page_size, w.sm_scale, w.kv_dtype, inp.k_scale, inp.v_scale)
    check_output(gout, ref_out, BF16_ATOL, BF16_COS, case)
    assert np.abs(glse - ref_lse).max() < 1e-3, case


@pytest.mark.parametrize("G", [4, 8, 16])
def test_prefill_windows_cut_record_tiles(G):
    """Attention windows of 204 rows over three sequences of ragged lengths:
    neither a window nor a sequence's first row falls on a multiple of a
    merge workgroup's 128 / G rows, so the partial records' row tiles are
    cut short at the end of the record index and workgroups straddle two
    tiles.  Output and LSE against the oracle on the selection made."""
    msa = _msa()
    w = Workload(f"win{G}", [700, 77, 333], [700, 300, 400], 2 * G, 2, 2, 2, topk=5, poison_tail=True)
    inp = make_inputs(w, 70 + G)
    print(f"[parity] prefill windows of 204 rows G={G} T={w.total_rows}", flush=True)
    d = device_inputs(inp)
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, attn_window_rows=204)
    T = w.total_rows
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, T, sel)
    out = torch.full((T, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse,
                                d["k_scale"], d["v_scale"])
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    ref_out, ref_lse = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, gsel, w.qo_lens,
                                          w.kv_lens, w.page_size, w.sm_scale, w.kv_dtype, inp.k_scale, inp.v_scale)
    check_output(bf16_out_to_f64(out), ref_out, BF16_ATOL, BF16_COS, f"win{G}")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3, G


def test_prefill_one_nonlocal_key_carries_each_row():
    """The stored partials' precision at its limit: every row of blocks 1..7
    selects block 0 besides its own block, and one key of block 0 takes most
    of every row's softmax (score about 12 against about 0 for the rest),
    with a value row of magnitudes between 2 and 4.  Each output row is then
    mostly that slot's partial as stored (block floating point, a step of
    about 2^-6 at these magnitudes; off the bf16 grid, as the other keys mix
    in) and rounded to bf16: the two roundings together must still meet the
    output tolerance against the oracle (8-bit fields would not: 0.0235)."""
    msa = _msa()
    w = Workload("peak", [1024], [1024], 8, 2, 2, 2, topk=2)
    inp = make_inputs(w, 90)
    g = np.random.default_rng(90)
    widen = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    u = g.standard_normal(128).astype(np.float32)
    u /= np.linalg.norm(u)
    q = 0.3 * widen(inp.q) + 4.0 * u            # every row and head leans on u
    k_pages = widen(inp.k_pages).copy()
    v_pages = widen(inp.v_pages).copy()
    page0 = int(inp.kv_indices[0])
    k_pages[page0, :, 5, :] = 34.0 * u          # key 5 of block 0: q.k / sqrt(128) ~ 12
    mag = g.uniform(2.0, 4.0, size=(w.num_kv_heads, 128))
    v_pages[page0, :, 5, :] = (mag * np.where(g.random(mag.shape) < 0.5, -1.0, 1.0)).astype(np.float32)
    inp = dataclasses.replace(inp, q=to_bf16_bits(q), k_pages=to_bf16_bits(k_pages), v_pages=to_bf16_bits(v_pages))
    T = w.total_rows
    blk = np.arange(T) // 128
    sel = np.full((T, w.num_kv_heads, 2), -1, np.int32)
    sel[:, :, 0] = 0
    sel[blk > 0, :, 1] = blk[blk > 0, None]
    print("[parity] prefill with one dominant non-local key per row", flush=True)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    out = torch.full((T, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"],
                                torch.from_numpy(sel).cuda(), out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, w.qo_lens,
                                          w.kv_lens, w.page_size, w.sm_scale)
    gout = bf16_out_to_f64(out)
    # the premise: rows past block 0 are carried by the one key (|out| near 2..4)
    assert np.abs(ref_out[128:]).min() > 1.5
    err, c = check_output(gout, ref_out, BF16_ATOL, BF16_COS, "dominant key")
    print(f"[parity] dominant key: max|err| {err:.4g}, cos {c:.7f}", flush=True)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_fused_proxy_topk_selection(case):
    """msa_proxy_topk_select: with a bf16 proxy it gives, bit for bit, the
    selection of msa_proxy_block_maxscore + msa_topk_select (same fp32
    scores, same tie rule); with a low-precision proxy its selection must be
    exact under the band rule against the oracle's exact scores on every
    row.  A sub-range call writes exactly its rows, equal to the whole call."""
    msa = _msa()
    w, seed, max_rows = PREFILL_CASES[case]
    inp = make_inputs(w, seed)
    print(f"[parity] fused proxy+topk case={case} T={w.total_rows} seed={seed}", flush=True)
    gms, gsel, _, _ = run_prefill_stages(msa, inp, max_rows)
    d = device_inputs(inp)
    plan = plan_for(msa, inp, max_rows_per_call=max_rows)
    T = w.total_rows
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, T, sel)
    fsel = sel.cpu().numpy()
    if w.proxy_dtype in LOW_PRECISION_PROXY:
        lay = O.Layout(w.qo_lens, w.kv_lens, w.page_size)
        ref_ms = oracle_scores(inp)
        check_selection(fsel, ref_ms, np.array([lay.local(r) for r in range(T)]), w.topk, case)
        print(f"[parity] {case}: fused exact selection differs from the low-precision top-k in "
              f"{int((fsel != gsel).any(axis=2).sum())} (row, group) pairs", flush=True)
        gsel = fsel
    else:
        assert np.array_equal(fsel, gsel), f"{case}: {int((fsel != gsel).any(axis=2).sum())} (row, group) differ"
    # a sub-range writes only its rows
    if T > 3:
        r0, n = T // 3, max(1, T // 3)
        sel2 = torch.full_like(sel, -7)
        msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                                  d["kv_indices"], r0, n, sel2)
        s2 = sel2.cpu().numpy()
        assert np.array_equal(s2[r0:r0 + n], gsel[r0:r0 + n]), case
        assert (s2[:r0] == -7).all() and (s2[r0 + n:] == -7).all(), case


def test_row_range_attention_equals_whole_call():
    """msa_sparse_attn_prefill_rows over consecutive row ranges (ragged, one
    of them a single row, some crossing sequence boundaries) writes exactly
    those rows, and together they give the whole call's output bit for bit."""
    msa = _msa()
    w, seed, _ = PREFILL_CASES["varlen_ragged_prefix"]
    inp = make_inputs(w, seed)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    T = w.total_rows
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, T, sel)
    ref = torch.full((T, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.full((T, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, ref, ref_lse)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    bounds = [0, 150, 151, 377, 600, T]
    for r0, r1 in zip(bounds[:-1], bounds[1:]):
        msa.msa_sparse_attn_prefill_rows(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, r0,
                                         r1 - r0, lse)
        torch.cuda.synchronize()
        assert torch.isnan(out[r1:].float()).all() and torch.isnan(lse[r1:]).all(), (r0, r1)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


TIE_CASES = {
    # many query rows per sequence: the thread-per-row kernel
    "multi_row": (Workload("ties", [1500, 40], [1500, 300], 8, 2, 2, 2, topk=6), 5),
    # one query row per sequence, rows up to 2048 blocks: the wave-per-row kernel
    "one_row_k17": (Workload("ties1", [1] * 6, [262144, 70000, 5000, 129, 128, 1], 8, 2, 2, 2, topk=17), 6),
    "one_row_k64": (Workload("ties2", [1] * 3, [200000, 9000, 8193], 8, 2, 2, 2, topk=64), 7),
}


@pytest.mark.parametrize("case", list(TIE_CASES))
def test_topk_exact_on_given_scores_with_ties(case):
    """The top-k kernel on fp32 scores with many exact ties (and some -inf)
    must equal the oracle's selection bit for bit (same fp32 values, lower id
    wins)."""
    msa = _msa()
    w, seed = TIE_CASES[case]
    T = w.total_rows
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, 8, 2, 2, 2, topk=w.topk, max_rows_per_call=T)
    rng = np.random.default_rng(seed)
    scores = rng.integers(-3, 4, size=(2, plan.nb_max, T)).astype(np.float32)     # heavy ties
    scores[:, :, ::7] = rng.standard_normal((2, plan.nb_max, len(range(0, T, 7)))).astype(np.float32)
    scores[rng.random(scores.shape) < 0.01] = -np.inf
    ms = torch.from_numpy(scores).cuda()
    sel = torch.full((T, 2, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_topk_select(plan, ms, 0, T, sel)
    got = sel.cpu().numpy()
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    for r in range(T):
        for p in range(2):
            exp = O.topk_select_row(scores[p, :, r].astype(np.float64), lay.local(r), w.topk)
            assert np.array_equal(got[r, p], exp), (case, r, p, got[r, p], exp)


DECODE_CASES = {
    "fp8_g8": (Workload("dec", [1] * 4, [1000, 128, 2000, 5000], 16, 2, topk=17, kv_dtype=FP8, mode="decode",
                        extra_pages=0.2, poison_tail=True), 21),
    "bf16_g8": (Workload("decb", [1] * 3, [129, 4000, 777], 16, 2, topk=9, kv_dtype=BF16, mode="decode",
                         poison_tail=True), 22),
    "fp8_g16": (Workload("dec16", [1] * 2, [3000, 300], 32, 2, topk=5, kv_dtype=FP8, mode="decode"), 23),
    "fp8_g4_local_only": (Workload("dec1", [1] * 5, [50, 128, 129, 255, 1000], 8, 2, topk=1, kv_dtype=FP8,
                                   mode="decode", poison_tail=True), 24),
    "fp8_g1": (Workload("decg1", [1] * 2, [640, 1500], 4, 4, topk=3, kv_dtype=FP8, mode="decode"), 25),
}


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_matches_oracle(case):
    msa = _msa()
    w, seed = DECODE_CASES[case]
    inp = make_inputs(w, seed)
    print(f"[parity] decode case={case} B={w.num_seqs} seed={seed}", flush=True)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    out = torch.full((w.num_seqs, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.num_seqs, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_decode(plan, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"],
                               d["kv_indices"], d["kv_block_indexes"], out, lse)
    torch.cuda.synchronize()
    ref, ref_lse = O.sparse_decode(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, inp.kv_block_indexes, w.kv_lens,
                                   w.page_size, w.sm_scale, w.kv_dtype, inp.k_scale, inp.v_scale)
    atol, cmin = (FP8_ATOL, FP8_COS) if w.kv_dtype == FP8 else (BF16_ATOL, BF16_COS)
    check_output(bf16_out_to_f64(out), ref, atol, cmin, case)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3, case
