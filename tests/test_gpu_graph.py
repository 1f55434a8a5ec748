"""The decode step (indexer pass on a one-query-row plan with an fp8 proxy,
then the fp8 sparse decode on its selection) captured once in a HIP graph:
every replay, with unrelated eager work and synchronizations between
replays, must reproduce the eager step's selection and output bit for bit.
The benchmark times decode steps replayed this way."""
import numpy as np
import pytest
import torch

from synthetic.gen import Workload, make_inputs, FP8
from tests._gpu import device_inputs

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    from block_sparse_top_amd import msa
    w = Workload("graph_step", [1] * 6, [9000, 128, 700, 20000, 129, 4000], 16, 2, 2, 1, topk=9, kv_dtype=FP8,
                 proxy_dtype=FP8, lowrank=8, poison_tail=True, mode="decode")
    print("[graph] decode step capture", flush=True)
    inp = make_inputs(w, 71)
    d = device_inputs(inp)
    S = w.num_seqs
    ip = msa.msa_plan([1] * S, w.kv_lens, w.num_qo_heads, w.num_kv_heads, 2, 1, topk=w.topk, proxy_dtype="fp8")
    dp = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    sel = torch.full((S, 2, w.topk), -7, dtype=torch.int32, device="cuda")
    out = torch.full((S, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")

    def step():
        msa.msa_proxy_topk_select(ip, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"],
                                  d["kv_indices"], 0, S, sel)
        msa.msa_sparse_attn_decode(dp, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"],
                                   d["kv_indices"], sel, out)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref_sel, ref_out = sel.clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    other = torch.randn(4096, 4096, device="cuda")
    for rep in range(4):
        sel.fill_(-7)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel), f"replay {rep}: selection"
        assert torch.equal(out, ref_out), f"replay {rep}: output"
        other = other @ other.T * 1e-4       # unrelated eager work between replays
        torch.cuda.synchronize()
    assert np.isfinite(out.float().cpu().numpy()).all()
