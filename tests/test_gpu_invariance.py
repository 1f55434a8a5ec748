"""Invariances of the HIP path that hold without any reference output:

* the page table is only an address map: permuting the pool (same logical
  keys) leaves every output bit-identical, for prefill and decode;
* the whole forward is deterministic: two runs are bit-identical;
* GQA -> MHA: repeating each KV head (and its proxy head) G times over a
  plan with G = 1 gives the same outputs;
* the decode's split count (1, 2, 4, 17 workgroups per (sequence, group),
  merged by log-sum-exp) changes only fp32 rounding;
* two plans sharing one workspace, called alternately, give the results of
  their own workspaces (the plan metadata is copied again when the
  workspace last held another plan's);
* a one-query-row plan with 64 proxy heads sharing one proxy-K head (two
  32-column groups of the one-row kernel) matches the oracle.
Inputs are seeded and small (several tiles, ragged tails)."""
import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs, FP8, BF16
from tests._gpu import (device_inputs, plan_for, bf16_out_to_f64, check_output, check_selection, oracle_scores,
                        check_max_score, lowp_score_bound, BF16_ATOL, BF16_COS, FP8_ATOL, FP8_COS)

pytestmark = pytest.mark.gpu


def _msa():
    from block_sparse_top_amd import msa
    return msa


def _forward(msa, plan, d, w):
    T = w.total_rows
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    out = torch.full((T, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, w.num_qo_heads), float("nan"), device="cuda")
    msa.run_prefill(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"], d["q"],
                    d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse, k_scale=d["k_scale"],
                    v_scale=d["v_scale"])
    torch.cuda.synchronize()
    return sel, out, lse


W_PREFILL = Workload("inv", [700, 300, 129], [700, 500, 129], 16, 4, 4, 4, topk=5, poison_tail=True)


@pytest.mark.parametrize("proxy", [BF16, FP8])
def test_page_permutation_and_run_twice(proxy):
    msa = _msa()
    import dataclasses
    w = dataclasses.replace(W_PREFILL, proxy_dtype=proxy, page_table="identity")
    print(f"[invariance] page permutation proxy={proxy}", flush=True)
    inp = make_inputs(w, 51)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    sel, out, lse = _forward(msa, plan, d, w)
    sel2, out2, lse2 = _forward(msa, plan, d, w)
    assert torch.equal(sel, sel2) and torch.equal(out, out2) and torch.equal(lse, lse2), "run twice"
    # the same logical keys in a permuted pool
    N = inp.k_pages.shape[0]
    perm = np.random.default_rng(52).permutation(N)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(N)
    dp = dict(d)
    for name in ("k_pages", "v_pages", "proxy_k_pages"):
        t = d[name]
        pt = torch.empty_like(t)
        pt[torch.from_numpy(perm).cuda()] = t
        dp[name] = pt
    dp["kv_indices"] = torch.from_numpy(perm[inp.kv_indices].astype(np.int32)).cuda()
    sel3, out3, lse3 = _forward(msa, plan, dp, w)
    assert torch.equal(sel, sel3), "selection depends on the page table"
    assert torch.equal(out, out3) and torch.equal(lse, lse3), "output depends on the page table"
    ref, _ = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel.cpu().numpy(), w.qo_lens,
                                w.kv_lens, 128, w.sm_scale)
    check_output(bf16_out_to_f64(out), ref, BF16_ATOL, BF16_COS, "permutation")


def test_gqa_equals_replicated_mha():
    """G = 4 against a plan with 16 KV heads holding each group's K/V (and
    proxy) head 4 times: same selections per head, same outputs."""
    msa = _msa()
    w = W_PREFILL
    print("[invariance] GQA -> MHA replication", flush=True)
    inp = make_inputs(w, 53)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    sel, out, lse = _forward(msa, plan, d, w)
    G = w.num_qo_heads // w.num_kv_heads
    import dataclasses
    wm = dataclasses.replace(w, num_kv_heads=w.num_qo_heads, num_proxy_heads=w.num_qo_heads,
                             num_proxy_kv_heads=w.num_qo_heads)
    dm = dict(d)
    for name in ("k_pages", "v_pages", "proxy_k_pages"):
        dm[name] = d[name].repeat_interleave(G, dim=1).contiguous()
    dm["proxy_q"] = d["proxy_q"].repeat_interleave(G, dim=1).contiguous()
    pm = msa.msa_plan(wm.qo_lens, wm.kv_lens, wm.num_qo_heads, wm.num_kv_heads, wm.num_proxy_heads,
                      wm.num_proxy_kv_heads, topk=wm.topk)
    selm, outm, lsem = _forward(msa, pm, dm, wm)
    assert torch.equal(selm, sel.repeat_interleave(G, dim=1)), "replicated groups select differently"
    err = (outm.float() - out.float()).abs().max().item()
    lerr = (lsem - lse).abs().max().item()
    print(f"[invariance] MHA vs GQA: max|out diff| {err:.3g}, bit-equal {torch.equal(outm, out)}, "
          f"max|lse diff| {lerr:.3g}", flush=True)
    assert err <= 2.0 ** -8 and lerr <= 1e-5


@pytest.mark.parametrize("kv", [FP8, BF16])
def test_decode_split_counts_agree(kv):
    msa = _msa()
    w = Workload("dsplit", [1] * 3, [5000, 129, 2000], 16, 2, topk=17, kv_dtype=kv, mode="decode", poison_tail=True)
    print(f"[invariance] decode splits kv={kv}", flush=True)
    inp = make_inputs(w, 54)
    d = device_inputs(inp)
    outs = {}
    for ns in (1, 2, 4, 17):
        plan = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype=kv, mode="decode",
                            decode_splits=ns)
        out = torch.full((3, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((3, 16), float("nan"), device="cuda")
        msa.msa_sparse_attn_decode(plan, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"],
                                   d["kv_indices"], d["kv_block_indexes"], out, lse)
        torch.cuda.synchronize()
        outs[ns] = (out.float(), lse)
    for ns in (2, 4, 17):
        e = (outs[ns][0] - outs[1][0]).abs().max().item()
        le = (outs[ns][1] - outs[1][1]).abs().max().item()
        assert e <= 2.0 ** -7 and le <= 1e-5, (ns, e, le)
    ref, _ = O.sparse_decode(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, inp.kv_block_indexes, w.kv_lens, 128,
                             w.sm_scale, kv, inp.k_scale, inp.v_scale)
    atol, cmin = (FP8_ATOL, FP8_COS) if kv == FP8 else (BF16_ATOL, BF16_COS)
    for ns in (1, 17):
        check_output(outs[ns][0].cpu().numpy().astype(np.float64), ref, atol, cmin, f"splits {ns}")


def test_two_plans_share_one_workspace():
    msa = _msa()
    wa = Workload("wsa", [600, 200], [600, 300], 8, 2, 2, 2, topk=4)
    wb = Workload("wsb", [1000], [1000], 8, 2, 2, 2, topk=6)
    print("[invariance] two plans, one workspace", flush=True)
    ia, ib = make_inputs(wa, 55), make_inputs(wb, 56)
    da, db = device_inputs(ia), device_inputs(ib)
    pa, pb = plan_for(msa, ia), plan_for(msa, ib)
    ref_a = _forward(msa, pa, da, wa)
    ref_b = _forward(msa, pb, db, wb)
    shared = torch.empty(max(pa.workspace_bytes, pb.workspace_bytes), dtype=torch.uint8, device="cuda")
    pa.workspace = shared
    pb.workspace = shared
    for it in range(2):
        got_a = _forward(msa, pa, da, wa)
        got_b = _forward(msa, pb, db, wb)
        for x, y in zip(got_a, ref_a):
            assert torch.equal(x, y), f"plan A after plan B (iteration {it})"
        for x, y in zip(got_b, ref_b):
            assert torch.equal(x, y), f"plan B after plan A (iteration {it})"


@pytest.mark.parametrize("dt", [BF16, FP8])
def test_onerow_64_proxy_heads_one_proxy_k_head(dt):
    msa = _msa()
    w = Workload(f"row64_{dt}", [1] * 4, [3000, 129, 700, 128], 64, 64, 64, 1, topk=5, proxy_dtype=dt,
                 poison_tail=True)
    print(f"[invariance] one-row plan, 64 proxy heads on one proxy-K head, {dt}", flush=True)
    inp = make_inputs(w, 57)
    d = device_inputs(inp)
    plan = plan_for(msa, inp)
    S = w.total_rows
    ms = msa.max_score_buffer(plan)
    ms.fill_(float("nan"))
    msa.msa_proxy_block_maxscore(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                                 d["kv_indices"], 0, S, ms)
    sel = torch.full((S, 64, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                              d["kv_indices"], 0, S, sel)
    torch.cuda.synchronize()
    ref = oracle_scores(inp)
    extra = lowp_score_bound(inp, np.arange(S), w.proxy_sm_scale) if dt == FP8 else None
    check_max_score(msa.max_score_rows(ms, plan, S).cpu().numpy(), ref, w.name, extra)
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    check_selection(sel.cpu().numpy(), ref, np.array([lay.local(r) for r in range(S)]), w.topk, w.name)


@pytest.mark.parametrize("hkv", [8, 2])
def test_xcd_pinned_work_items_match(hkv):
    """MSA_XCD_PIN=1 (read when a plan is made) deals a KV group's attention
    work items to one XCD (Hkv >= 8) or to 8 / Hkv XCDs (Hkv < 8): the same
    items in another order, so every output is bit-identical; with small
    attention windows (several launches)."""
    import os
    msa = _msa()
    w = Workload(f"pin{hkv}", [700, 300, 129], [700, 500, 129], 2 * hkv, hkv, hkv, hkv, topk=5, poison_tail=True)
    print(f"[invariance] XCD pinning Hkv={hkv}", flush=True)
    inp = make_inputs(w, 58)
    d = device_inputs(inp)
    res = []
    old = os.environ.get("MSA_XCD_PIN")
    try:
        for pin in ("0", "1"):
            os.environ["MSA_XCD_PIN"] = pin
            plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                                w.num_proxy_kv_heads, topk=w.topk, attn_window_rows=256)
            res.append(_forward(msa, plan, d, w))
    finally:
        if old is None:
            os.environ.pop("MSA_XCD_PIN", None)
        else:
            os.environ["MSA_XCD_PIN"] = old
    for x, y in zip(*res):
        assert torch.equal(x, y), "pinned work items give other results"
    ref, _ = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, res[1][0].cpu().numpy(), w.qo_lens,
                                w.kv_lens, 128, w.sm_scale)
    check_output(bf16_out_to_f64(res[1][1]), ref, BF16_ATOL, BF16_COS, "pinned")
