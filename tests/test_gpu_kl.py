"""GPU parity of the fused main + proxy-distillation backward
(msa_sparse_attn_prefill_backward_kl) against the fp64 oracle, on the GPU's
own forward selection, output and log-sum-exp.

The main gradients must equal those of msa_sparse_attn_prefill_backward bit
for bit (same kernels, the proxy term only adds products).  The proxy
gradients follow the same rounding as the main ones (bf16 P before the matrix
products, bf16 per-slot partials of the sparse term), so each tensor must
reach cosine >= 0.999 with the oracle and max |err| <= 1e-2 x max |oracle|;
the proxy log-sum-exp (fp32 accumulation of exact-rounded bf16 products)
within 1e-3."""
import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import Workload, make_inputs
from tests._gpu import device_inputs
from tests.test_gpu_backward import _check

pytestmark = pytest.mark.gpu

CASES = {
    "gqa4_ragged": (Workload("kl4", [300, 77, 1, 513], [300, 200, 1, 700], 16, 4, 4, 4, topk=5, extra_pages=0.25,
                             poison_tail=True), 51, 0, 0.75),
    "gqa1": (Workload("kl1", [384], [384], 2, 2, 2, 2, topk=2), 52, 0, 1.0),
    "gqa16": (Workload("kl16", [260], [400], 32, 2, 2, 2, topk=3, poison_tail=True), 53, 0, -2.0),
    "gqa8_windows": (Workload("klw", [900, 333], [900, 400], 16, 2, 2, 2, topk=6, poison_tail=True), 54, 256, 1.0),
    "all_blocks": (Workload("kla", [640], [640], 8, 2, 2, 2, topk=9), 55, 0, 1.0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_kl_backward_matches_oracle(case):
    from block_sparse_top_amd import msa
    w, seed, window, gs = CASES[case]
    inp = make_inputs(w, seed)
    print(f"[kl] case={case} T={w.total_rows} seed={seed}", flush=True)
    d = device_inputs(inp)
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, attn_window_rows=window)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    sel = torch.full((T, Hkv, w.topk), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    msa.run_prefill(plan, d["proxy_q"], d["proxy_k_pages"], d["proxy_q_scale"], d["proxy_k_scale"], d["q"],
                    d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dout = torch.randn((T, Hq, 128), generator=g).to(torch.bfloat16).cuda()
    N = inp.num_pages
    nan = float("nan")
    grads = [torch.full((T, Hq, 128), nan, device="cuda"), torch.full((N, Hkv, 128, 128), nan, device="cuda"),
             torch.full((N, Hkv, 128, 128), nan, device="cuda")]
    ref_main = [torch.full_like(x, nan) for x in grads]
    dpq = torch.full((T, Hkv, 128), nan, device="cuda")
    dpk = torch.full((N, Hkv, 128, 128), nan, device="cuda")
    plse = torch.full((T, Hkv), nan, device="cuda")
    msa.msa_sparse_attn_prefill_backward_kl(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse,
                                            dout, d["proxy_q"], d["proxy_k_pages"], gs, *grads, dpq, dpk, plse)
    msa.msa_sparse_attn_prefill_backward(plan, d["q"], d["k_pages"], d["v_pages"], d["kv_indices"], sel, out, lse,
                                         dout, *ref_main)
    torch.cuda.synchronize()
    used = torch.from_numpy(np.asarray(inp.kv_indices, dtype=np.int64)).cuda()
    from tests.test_gpu_backward import assert_same_main_grads
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref_main):
        if name != "dq":
            a, b = a[used], b[used]
        assert_same_main_grads(case, name, a, b)
    rq, rk, _, rl = O.proxy_kl_backward(inp.proxy_q, inp.proxy_k_pages, inp.q, inp.k_pages, inp.kv_indices,
                                        sel.cpu().numpy(), w.qo_lens, w.kv_lens, w.page_size, w.sm_scale,
                                        w.proxy_sm_scale, grad_scale=gs)
    ui = np.asarray(inp.kv_indices, dtype=np.int64)
    assert np.abs(plse.cpu().numpy() - rl).max() < 1e-3, case
    _check(f"{case} dproxy_q", dpq.cpu().numpy().astype(np.float64), rq)
    _check(f"{case} dproxy_k", dpk.cpu().numpy()[ui].astype(np.float64), rk[ui])


@pytest.mark.parametrize("pk,proxy_dtype", [(1, "bf16"), (2, "fp8")])
def test_fused_kl_backward_rejects_a_plan_without_its_proxy_shape(pk, proxy_dtype):
    """A shared proxy-K head or a low-precision proxy: the plan has no room
    for the proxy term and the call is refused before any launch."""
    from block_sparse_top_amd import msa
    plan = msa.msa_plan([256], [256], 8, 2, 2, pk, topk=2, proxy_dtype=proxy_dtype)
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_attn_prefill_backward_kl(plan, *([x] * 10), 1.0, *([x] * 6))
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED
