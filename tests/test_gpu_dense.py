"""GPU parity of the warm-up mode (dense main attention, msa_dense_attn_prefill
and msa_dense_attn_prefill_backward) against the fp64 oracle given every
visible block as the selection (the dense case of the sparse definitions,
itself pinned against torch's scaled_dot_product_attention on the CPU).

Tolerances as for the sparse path: outputs max-abs 2e-2 and cosine >= 0.999,
lse within 1e-3; gradients cosine >= 0.999 and max |err| <= 1e-2 x max
|oracle|.  The main gradients with and without the proxy term are equal bit
for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs
from tests._gpu import device_inputs, check_output, bf16_out_to_f64
from tests.test_gpu_backward import _check

pytestmark = pytest.mark.gpu

CASES = {
    "gqa4_ragged_prefix": (Workload("dn4", [300, 77, 1, 513], [300, 200, 1, 700], 16, 4, 4, 4, topk=5,
                                    extra_pages=0.25, poison_tail=True), 61, 0.5),
    "gqa1": (Workload("dn1", [384], [384], 2, 2, 2, 2, topk=2), 62, 1.0),
    "gqa16": (Workload("dn16", [260], [400], 32, 2, 2, 2, topk=3, poison_tail=True), 63, -1.5),
    "gqa8_two_tiles": (Workload("dn8", [700], [700], 16, 2, 2, 2, topk=4, poison_tail=True), 64, 1.0),
}


def _all_blocks(w):
    lay = O.Layout(w.qo_lens, w.kv_lens, w.page_size)
    nbm = max(lay.nb)
    sel = np.full((w.total_rows, w.num_kv_heads, nbm), -1, np.int32)
    for r in range(w.total_rows):
        loc = lay.local(r)
        sel[r, :, :loc + 1] = np.arange(loc + 1)
    return sel


@pytest.mark.parametrize("case", list(CASES))
def test_dense_forward_and_backward_match_oracle(case):
    from block_sparse_top_amd import msa
    w, seed, gs = CASES[case]
    inp = make_inputs(w, seed)
    print(f"[dense] case={case} T={w.total_rows} seed={seed}", flush=True)
    d = device_inputs(inp)
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk)
    T, Hq, Hkv, N = w.total_rows, w.num_qo_heads, w.num_kv_heads, inp.num_pages
    nan = float("nan")
    out = torch.full((T, Hq, 128), nan, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, Hq), nan, dtype=torch.float32, device="cuda")
    msa.msa_dense_attn_prefill(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], out, lse)
    torch.cuda.synchronize()
    sel = _all_blocks(w)
    ref, ref_lse = O.sparse_attention(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, w.qo_lens, w.kv_lens,
                                      w.page_size, w.sm_scale)
    check_output(bf16_out_to_f64(out), ref, 2e-2, 0.999, case)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3

    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dout = torch.randn((T, Hq, 128), generator=g).to(torch.bfloat16).cuda()
    grads = [torch.full((T, Hq, 128), nan, device="cuda"), torch.full((N, Hkv, 128, 128), nan, device="cuda"),
             torch.full((N, Hkv, 128, 128), nan, device="cuda")]
    plain = [torch.full_like(x, nan) for x in grads]
    dpq = torch.full((T, Hkv, 128), nan, device="cuda")
    dpk = torch.full((N, Hkv, 128, 128), nan, device="cuda")
    plse = torch.full((T, Hkv), nan, device="cuda")
    msa.msa_dense_attn_prefill_backward(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], out, lse, dout,
                                        *grads, d["proxy_q"], d["proxy_k_pages"], gs, dpq, dpk, plse)
    msa.msa_dense_attn_prefill_backward(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], out, lse, dout,
                                        *plain)
    torch.cuda.synchronize()
    used = torch.from_numpy(np.asarray(inp.kv_indices, dtype=np.int64)).cuda()
    from tests.test_gpu_backward import assert_same_main_grads
    for name, a, b in zip(("dq", "dk", "dv"), grads, plain):
        if name != "dq":
            a, b = a[used], b[used]
        assert_same_main_grads(case, name, a, b)
    dout_bits = dout.cpu().view(torch.int16).numpy().view(np.uint16)
    rq, rk, rv = O.sparse_attention_backward(inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, w.qo_lens,
                                             w.kv_lens, w.page_size, w.sm_scale, dout_bits)
    ui = np.asarray(inp.kv_indices, dtype=np.int64)
    _check(f"{case} dq", grads[0].cpu().numpy().astype(np.float64), rq)
    _check(f"{case} dk", grads[1].cpu().numpy()[ui].astype(np.float64), rk[ui])
    _check(f"{case} dv", grads[2].cpu().numpy()[ui].astype(np.float64), rv[ui])
    pq, pk, _, pl = O.proxy_kl_backward(inp.proxy_q, inp.proxy_k_pages, inp.q, inp.k_pages, inp.kv_indices, sel,
                                        w.qo_lens, w.kv_lens, w.page_size, w.sm_scale, w.proxy_sm_scale,
                                        grad_scale=gs)
    assert np.abs(plse.cpu().numpy() - pl).max() < 1e-3
    _check(f"{case} dproxy_q", dpq.cpu().numpy().astype(np.float64), pq)
    _check(f"{case} dproxy_k", dpk.cpu().numpy()[ui].astype(np.float64), pk[ui])
