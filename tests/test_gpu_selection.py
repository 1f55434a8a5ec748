"""Exact block selection with low-precision proxies (fp8, fp8 x MXFP4,
MXFP4 x MXFP4), through the fused call msa_proxy_topk_select.

The selection rule of the pages (README "Usage": `sparse_topk_select` keeps
the `topk` best blocks by proxy score; Flash-MSA article: the local block is
always kept) is applied to the exact scores of the stored operands: the
selected set must equal the oracle's whenever the oracle's (k-1)-th and k-th
competing scores differ by more than 1e-3 (band rule), on every row.  The
matrix cores' low-precision scores are off by up to ~2^-10.7 of
scale * max|q| * max|k|, so the library re-scores the blocks near the
boundary exactly; these tests check the result on whole workloads, on exact
ties that overflow the fused pass's candidate list, and on one-query-row
plans."""
import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs, FP8, MXFP4, MXFP4_QK
from tests._gpu import device_inputs, plan_for, check_selection, oracle_scores

pytestmark = pytest.mark.gpu


def _msa():
    from block_sparse_top_amd import msa
    return msa


@pytest.mark.parametrize("dt", [FP8, MXFP4, MXFP4_QK])
def test_lowp_fused_selection_every_row(dt):
    """8192 tokens, 8 groups, topk 16: every (row, group) selection passes the
    band rule against the oracle; the number of pairs whose exact selection
    differs from the plain low-precision top-k is reported."""
    msa = _msa()
    w = Workload(f"sel8k_{dt}", [8192], [8192], 32, 8, 8, 8, topk=16, proxy_dtype=dt)
    print(f"[selection] full rows workload={w.name}", flush=True)
    inp = make_inputs(w, 4100)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    T = w.total_rows
    sel = torch.full((T, 8, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, T, sel)
    ms = msa.max_score_buffer(plan)
    low = torch.full_like(sel, -7)
    msa.msa_proxy_block_maxscore(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                                 d["kv_indices"], 0, T, ms)
    msa.msa_topk_select(plan, ms, 0, T, low)
    torch.cuda.synchronize()
    fsel, lsel = sel.cpu().numpy(), low.cpu().numpy()
    ref = oracle_scores(inp)
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    check_selection(fsel, ref, np.array([lay.local(r) for r in range(T)]), 16, w.name)
    print(f"[selection] {w.name}: {int((fsel != lsel).any(axis=2).sum())} of {T * 8} pairs differ from the "
          f"low-precision top-k", flush=True)


def _tied_inputs(dt, seed):
    """A prefill whose proxy-K blocks 0..29 are one block repeated: for late
    rows more than 24 blocks tie exactly at the top, overflowing the fused
    pass's candidate list (so every competing block is re-scored)."""
    w = Workload(f"ties_{dt}", [4096, 1000], [4096, 1000], 8, 2, 2, 2, topk=6, proxy_dtype=dt)
    inp = make_inputs(w, seed)
    pk = inp.proxy_k_pages
    src = int(inp.kv_indices[5])
    for b in range(30):
        pk[int(inp.kv_indices[b])] = pk[src]
    return w, inp


@pytest.mark.parametrize("dt", [FP8, MXFP4])
def test_lowp_fused_selection_exact_ties(dt):
    """Exact ties among 30 blocks: the selection must equal the oracle's
    bit for bit (the tied blocks have identical exact scores in both, and
    the lower block wins)."""
    msa = _msa()
    w, inp = _tied_inputs(dt, 4200)
    print(f"[selection] exact ties workload={w.name}", flush=True)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    T = w.total_rows
    sel = torch.full((T, 2, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, T, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    ref = oracle_scores(inp)
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    tied_rows = 0
    for r in range(T):
        loc = lay.local(r)
        for p in range(2):
            exp = O.topk_select_row(ref[r, p], loc, w.topk)
            assert np.array_equal(got[r, p], exp), (r, p, got[r, p], exp)
            tied_rows += int(loc > 30 and r < 4096)
    assert tied_rows > 0


@pytest.mark.parametrize("dt", [FP8, MXFP4, MXFP4_QK])
def test_lowp_onerow_selection_with_ties(dt):
    """One query row per sequence (the decode-step indexer's plan): the exact
    selection over every block of the row, with 40 exactly tied blocks in one
    sequence, against the oracle bit for bit where ties are exact and by the
    band rule elsewhere."""
    msa = _msa()
    w = Workload(f"row_ties_{dt}", [1] * 5, [9000, 128, 700, 20000, 129], 16, 2, 2, 1, topk=17, proxy_dtype=dt,
                 lowrank=8 if dt != FP8 else 0, poison_tail=True)
    inp = make_inputs(w, 4300)
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    start = lay.page_start[3]
    src = int(inp.kv_indices[start + 11])
    for b in range(40):
        inp.proxy_k_pages[int(inp.kv_indices[start + 50 + b])] = inp.proxy_k_pages[src]
    print(f"[selection] one-row workload={w.name}", flush=True)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    S = w.total_rows
    sel = torch.full((S, 2, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, S, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    ref = oracle_scores(inp)
    check_selection(got, ref, np.array([lay.local(r) for r in range(S)]), w.topk, w.name)
    for p in range(2):
        exp = O.topk_select_row(ref[3, p], lay.local(3), w.topk)
        cs = np.sort(ref[3, p, :lay.local(3)])[::-1]
        if cs[15] - cs[16] > 1e-3 or cs[15] == cs[16]:
            assert np.array_equal(got[3, p], exp), (p, got[3, p], exp)
