"""msa_sparse_attn_decode_noalloc (the allocation-free decode entry point,
for callers that cannot allocate device memory) against
msa_sparse_attn_decode on the same inputs, through the C ABI: two calls in a
row, the second on a smaller batch (another plan, so the static scratch's
metadata is replaced), each equal to the workspace entry point's output bit
for bit and within the fp8 bar of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs, FP8
from tests._gpu import device_inputs, bf16_out_to_f64, check_output, FP8_ATOL, FP8_COS

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _case(msa, w, seed):
    inp = make_inputs(w, seed)
    d = device_inputs(inp)
    S = w.num_seqs
    plan = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    ref = torch.full((S, w.num_qo_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.full((S, w.num_qo_heads), float("nan"), device="cuda")
    msa.msa_sparse_attn_decode(plan, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"],
                               d["kv_indices"], d["kv_block_indexes"], ref, ref_lse)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    st = msa.lib().msa_sparse_attn_decode_noalloc(
        plan.handle, _ptr(d["q"]), _ptr(d["k_pages"]), _ptr(d["v_pages"]), _ptr(d["k_scale"]), _ptr(d["v_scale"]),
        _ptr(d["kv_indices"]), _ptr(d["kv_block_indexes"]), _ptr(out), _ptr(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == msa.MSA_OK, msa.lib().msa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse), w.name
    oref, olse = O.sparse_decode(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, inp.kv_block_indexes, w.kv_lens, 128,
                                 w.sm_scale, FP8, inp.k_scale, inp.v_scale)
    check_output(bf16_out_to_f64(out), oref, FP8_ATOL, FP8_COS, w.name)
    assert np.abs(lse.cpu().numpy() - olse).max() < 1e-3


def test_noalloc_decode_equals_workspace_decode():
    from block_sparse_top_amd import msa
    print("[no-alloc] decode, two calls (4 then 2 sequences)", flush=True)
    # few (sequence, group) pairs: split partials in the scratch, merged
    _case(msa, Workload("noalloc_a", [1] * 4, [3000, 129, 5000, 700], 16, 2, topk=9, kv_dtype=FP8, mode="decode",
                        extra_pages=0.1, poison_tail=True), 61)
    _case(msa, Workload("noalloc_b", [1] * 2, [1500, 300], 8, 2, topk=5, kv_dtype=FP8, mode="decode",
                        poison_tail=True), 62)


def test_noalloc_decode_rejects_plans_beyond_the_scratch():
    from block_sparse_top_amd import msa
    # 65536 sequences of one block: metadata alone exceeds 16 MiB
    plan = msa.msa_plan(None, [128] * 65536 * 17, 16, 2, topk=2, kv_dtype="fp8", mode="decode", allocate=False)
    assert plan.workspace_bytes > 16 << 20
    a = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = _ptr(a)
    st = msa.lib().msa_sparse_attn_decode_noalloc(plan.handle, p, p, p, p, p, p, p, p, None, None)
    assert st == msa.MSA_ERR_INVALID_ARG and b"16777216" in msa.lib().msa_last_error()
