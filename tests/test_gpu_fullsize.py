"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (default plan: 32768-row proxy/top-k chunks and attention
windows).  The oracle computes sampled rows one by one: evenly spaced rows
plus the edge rows of every sequence (first, last, and the rows around the
first 128- and 1920-key boundaries).  The decode workload is checked on every
output.  Inputs come from the seeded device generator (the same recipe as the
CPU generator, drawn on the GPU).

Tolerances as in test_gpu_parity: max scores 1e-4 + 1e-5|x| (plus the fp8
accumulation bound for fp8 proxy scores), the 1e-3 band
rule for selections, outputs max-abs 2e-2 / cosine 0.999 (bf16 K/V) or
6e-2 / 0.99 (fp8 K/V)."""
import numpy as np
import pytest
import torch

import oracle as O
from synthetic.gen import workload, seed_of, FP8
from synthetic.device_gen import make_inputs_device, to_host
from tests._gpu import (bf16_out_to_f64, check_max_score, check_selection, check_output, lowp_score_bound, LOW_PRECISION_PROXY,
                        BF16_ATOL, BF16_COS, FP8_ATOL, FP8_COS)

pytestmark = pytest.mark.gpu


def _sample_rows(w, n_even, seed, n_random=8):
    T = w.total_rows
    rows = set(np.linspace(0, T - 1, n_even).astype(np.int64).tolist())
    r0 = 0
    for qo in w.qo_lens:
        for i in (0, 1, 127, 128, 129, 1919, 1920, qo - 1):
            if 0 <= i < qo:
                rows.add(r0 + i)
        r0 += qo
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, T, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _prefill_case(n_cfg, n_even, n_random=8):
    from block_sparse_top_amd import msa
    w = workload(n_cfg)
    print(f"[fullsize] prefill workload={w.name} T={w.total_rows}", flush=True)
    inp = make_inputs_device(w, seed_of(n_cfg))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, kv_dtype=w.kv_dtype, proxy_dtype=w.proxy_dtype)
    T, R = w.total_rows, plan.max_rows_per_call
    lowp = w.proxy_dtype in LOW_PRECISION_PROXY
    rows = _sample_rows(w, n_even, seed_of(n_cfg), n_random)
    sel = torch.full((T, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    ms = msa.max_score_buffer(plan)
    got_ms = np.full((w.num_proxy_heads, plan.nb_max, rows.size), np.nan, np.float32)
    for r0 in range(0, T, R):
        n = min(R, T - r0)
        msa.msa_proxy_block_maxscore(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale,
                                     inp.kv_indices, r0, n, ms)
        msa.msa_topk_select(plan, ms, r0, n, sel)
        here = np.nonzero((rows >= r0) & (rows < r0 + n))[0]
        if here.size:
            got_ms[:, :, here] = msa.max_score_rows(ms, plan, n)[:, :, torch.from_numpy(rows[here] - r0).cuda()].cpu().numpy()
    low_sel = None
    if w.topk <= 17:
        # the fused pass (what run_prefill uses): with a bf16 proxy the same
        # blocks as the separate calls, every row; with a low-precision proxy
        # the exact selection, which the checks below use
        fsel = torch.full_like(sel, -7)
        msa.msa_proxy_topk_select(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale,
                                  inp.kv_indices, 0, T, fsel)
        if lowp:
            ndiff = int((fsel != sel).any(dim=2).sum())
            print(f"[fullsize] {w.name}: exact selection differs from the low-precision top-k in {ndiff} of "
                  f"{T * w.num_kv_heads} (row, group) pairs", flush=True)
            low_sel = sel[torch.from_numpy(rows).cuda()].cpu().numpy()
            sel = fsel
        else:
            assert torch.equal(fsel, sel), f"{w.name}: fused selection differs in {int((fsel != sel).any(dim=2).sum())} rows"
            del fsel
    out = torch.empty((T, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, w.num_qo_heads), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, lse)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    gout = bf16_out_to_f64(out[torch.from_numpy(rows).cuda()])
    glse = lse[torch.from_numpy(rows).cuda()].cpu().numpy()
    del out, lse, ms
    h = {k: to_host(getattr(inp, k)) for k in ("q", "k_pages", "v_pages", "kv_indices", "proxy_q", "proxy_k_pages",
                                                "proxy_q_scale", "proxy_k_scale")}
    del inp
    torch.cuda.empty_cache()
    ref_ms = O.proxy_block_maxscore(h["proxy_q"], h["proxy_k_pages"], h["kv_indices"], w.qo_lens, w.kv_lens, 128,
                                    w.proxy_sm_scale, w.proxy_dtype, h["proxy_q_scale"], h["proxy_k_scale"], rows=rows)
    extra = None
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    if lowp:
        from synthetic.gen import Inputs
        hi = Inputs(w, h["kv_indices"], h["q"], h["k_pages"], h["v_pages"], proxy_q=h["proxy_q"],
                    proxy_k_pages=h["proxy_k_pages"], proxy_q_scale=h["proxy_q_scale"],
                    proxy_k_scale=h["proxy_k_scale"])
        extra = lowp_score_bound(hi, rows, w.proxy_sm_scale)
        # the separate top-k call is exact on the low-precision scores it was given
        g = np.transpose(got_ms, (2, 0, 1)).astype(np.float64)
        for i, r in enumerate(rows):
            for p in range(w.num_kv_heads):
                exp = O.topk_select_row(g[i, p], lay.local(int(r)), w.topk)
                assert np.array_equal(low_sel[i, p], exp), (int(r), p)
    check_max_score(got_ms, ref_ms, w.name, extra)
    locs = np.array([lay.local(int(r)) for r in rows])
    check_selection(gsel[rows], ref_ms, locs, w.topk, w.name)
    # gaps at the boundary of the checked rows: how many sat in the band or
    # just above it (where an inexact score could have moved the set)
    gaps = []
    for i in range(rows.size):
        R = min(w.topk - 1, int(locs[i]))
        if 0 < R < locs[i]:
            cs = -np.sort(-ref_ms[i, :, :locs[i]], axis=1)
            gaps.append(cs[:, R - 1] - cs[:, R])
    if gaps:
        gp = np.concatenate(gaps)
        print(f"[fullsize] {w.name}: {gp.size} checked (row, group) pairs with a boundary; oracle gap <= 1e-3: "
              f"{int((gp <= 1e-3).sum())}, in (1e-3, 1e-2]: {int(((gp > 1e-3) & (gp <= 1e-2)).sum())}", flush=True)
    # every row: local block present, ascending, valid padding
    loc_all = np.concatenate([(np.arange(kv - qo, kv) // 128) for qo, kv in zip(w.qo_lens, w.kv_lens)])
    valid = gsel >= 0
    assert np.all(valid[:, :, 0]), "every row selects at least its local block"
    last = np.where(valid, gsel, -1).max(axis=2)
    assert np.array_equal(last, np.broadcast_to(loc_all[:, None], last.shape)), "local block missing somewhere"
    ref_out, ref_lse = O.sparse_attention(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], gsel, w.qo_lens,
                                          w.kv_lens, 128, w.sm_scale, rows=rows)
    err, cos = check_output(gout, ref_out, BF16_ATOL, BF16_COS, w.name)
    lse_err = np.abs(glse - ref_lse).max()
    print(f"[fullsize] {w.name}: output max|err| {err:.4g} (tol {BF16_ATOL}), cos {cos:.7f}, lse max|err| "
          f"{lse_err:.3g}", flush=True)
    assert lse_err < 1e-3, w.name


def _backward_case(n_cfg, n_even):
    """The training backward at full size, in the launch configuration the
    benchmark times: dq on sampled rows against the oracle; dk and dv of two
    (group, block) pairs exactly (the oracle visits every row that selected
    the block); and over every sequence and group the identity
    sum_j dv_j = sum of that group's dout rows (each row's P sums to 1)."""
    from block_sparse_top_amd import msa
    w = workload(n_cfg)
    print(f"[fullsize] backward workload={w.name}", flush=True)
    inp = make_inputs_device(w, seed_of(n_cfg))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, proxy_dtype=w.proxy_dtype)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    sel = torch.empty((T, Hkv, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    msa.run_prefill(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale, inp.q, inp.k_pages,
                    inp.v_pages, inp.kv_indices, sel, out, lse)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(n_cfg) + 77)
    dout = torch.randn((T, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty((T, Hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.zeros((inp.k_pages.shape[0], Hkv, 128, 128), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    msa.msa_sparse_attn_prefill_backward(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, lse, dout,
                                         dq, dk, dv)
    torch.cuda.synchronize()
    from tests.test_gpu_backward import _check
    h = {k: to_host(getattr(inp, k)) for k in ("q", "k_pages", "v_pages", "kv_indices")}
    gsel = sel.cpu().numpy()
    dob = to_host(dout)
    rows = _sample_rows(w, n_even, seed_of(n_cfg))
    print(f"[fullsize] oracle dq on {rows.size} rows", flush=True)
    rq, _, _ = O.sparse_attention_backward(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], gsel, w.qo_lens,
                                           w.kv_lens, 128, w.sm_scale, dob, rows=rows)
    _check(f"{w.name} dq (sampled rows)", dq[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64), rq[rows])
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    rng = np.random.default_rng(seed_of(n_cfg))
    # late blocks of the first sequence: few rows select them, so the oracle stays cheap
    nb0 = lay.nb[0]
    for gg, b in ((0, nb0 - 2), (int(rng.integers(Hkv)), int(rng.integers(nb0 - 12, nb0 - 2)))):
        sel_rows = np.nonzero((gsel[:, gg, :] == b).any(axis=1) & (np.arange(T) < lay.row_start[1]))[0]
        print(f"[fullsize] oracle dk, dv of group {gg} block {b}: {sel_rows.size} rows", flush=True)
        _, rk, rv = O.sparse_attention_backward(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], gsel, w.qo_lens,
                                                w.kv_lens, 128, w.sm_scale, dob, rows=sel_rows, groups=[gg])
        page = int(h["kv_indices"][lay.page_start[0] + b])
        _check(f"{w.name} dk (group {gg}, block {b})", dk[page, gg].cpu().numpy().astype(np.float64), rk[page, gg])
        _check(f"{w.name} dv (group {gg}, block {b})", dv[page, gg].cpu().numpy().astype(np.float64), rv[page, gg])
    G = Hq // Hkv
    kvi = torch.from_numpy(h["kv_indices"].astype(np.int64)).cuda()
    for si in range(len(w.kv_lens)):
        pages = kvi[int(lay.page_start[si]):int(lay.page_start[si + 1])]
        r0, r1 = int(lay.row_start[si]), int(lay.row_start[si + 1])
        for gg in range(Hkv):
            got = dv[pages, gg].double().sum(dim=(0, 1))
            ref = dout[r0:r1, gg * G:(gg + 1) * G].double().sum(dim=(0, 1))
            scale = dout[r0:r1, gg * G:(gg + 1) * G].double().abs().sum(dim=(0, 1))
            assert ((got - ref).abs() <= 2.0 ** -7 * scale + 1e-6).all(), (si, gg)


def test_prefill_32k_backward():
    _backward_case(2, 48)


def test_prefill_varlen_128k_backward():
    """Four sequences, G = 8 and four 32768-row attention windows: dk and dv
    accumulate across windows."""
    _backward_case(3, 24)


def _check_sum_zero(name, grad, kvi, lay, scale):
    """Per sequence and head, the gradient rows of a sequence's keys sum to
    zero (up to fp32 accumulation, relative to the sum of magnitudes)."""
    for si in range(len(lay.kv)):
        pages = kvi[int(lay.page_start[si]):int(lay.page_start[si + 1])]
        got = grad[pages].double().sum(dim=(0, 2))              # [heads, d]
        mag = grad[pages].double().abs().sum(dim=(0, 2))
        assert ((got.abs() <= 1e-3 * mag + 1e-6 * scale)).all(), (name, si)


def _late_blocks(lay, rng, Hkv):
    """Two (group, block) pairs among the first sequence's last blocks: few
    rows see them, so the oracle, which must visit every one, stays quick."""
    nb0 = lay.nb[0]
    return ((0, nb0 - 2), (int(rng.integers(1, Hkv)), nb0 - 3))


def test_prefill_32k_backward_kl():
    """The fused distillation backward at 32K in the benchmark's launch
    configuration: main gradients equal the main-only backward bit for bit;
    dproxy_q and the proxy lse on sampled rows and two groups; dproxy_k of two
    (group, late block) pairs exactly (the oracle visits every row that sees
    the block: the dense proxy term reaches all of them); every (sequence,
    head)'s dproxy_k sums to zero."""
    from block_sparse_top_amd import msa
    w = workload(2)
    print(f"[fullsize] fused distillation backward workload={w.name}", flush=True)
    inp = make_inputs_device(w, seed_of(2))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, proxy_dtype=w.proxy_dtype)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    N = inp.k_pages.shape[0]
    sel = torch.empty((T, Hkv, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    msa.run_prefill(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale, inp.q, inp.k_pages,
                    inp.v_pages, inp.kv_indices, sel, out, lse)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(2) + 79)
    dout = torch.randn((T, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    main = [torch.empty((T, Hq, 128), device="cuda"), torch.zeros((N, Hkv, 128, 128), device="cuda"),
            torch.zeros((N, Hkv, 128, 128), device="cuda")]
    ref_main = [torch.empty_like(main[0]), torch.zeros_like(main[1]), torch.zeros_like(main[2])]
    dpq = torch.empty((T, Hkv, 128), device="cuda")
    dpk = torch.zeros((N, Hkv, 128, 128), device="cuda")
    plse = torch.empty((T, Hkv), device="cuda")
    msa.msa_sparse_attn_prefill_backward_kl(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, lse, dout,
                                            inp.proxy_q, inp.proxy_k_pages, 1.0, *main, dpq, dpk, plse)
    msa.msa_sparse_attn_prefill_backward(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, lse, dout,
                                         *ref_main)
    torch.cuda.synchronize()
    from tests.test_gpu_backward import _check, assert_same_main_grads
    for name, a, b in zip(("dq", "dk", "dv"), main, ref_main):
        assert_same_main_grads(w.name, name, a, b)
    h = {k: to_host(getattr(inp, k)) for k in ("q", "k_pages", "proxy_q", "proxy_k_pages", "kv_indices")}
    gsel = sel.cpu().numpy()
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    rng = np.random.default_rng(seed_of(2) + 5)
    rows = _sample_rows(w, 8, seed_of(2))
    groups = sorted(set(rng.integers(Hkv, size=2).tolist()))
    print(f"[fullsize] oracle dproxy_q on {rows.size} rows, groups {groups}", flush=True)
    rq, _, _, rl = O.proxy_kl_backward(h["proxy_q"], h["proxy_k_pages"], h["q"], h["k_pages"], h["kv_indices"], gsel,
                                       w.qo_lens, w.kv_lens, 128, w.sm_scale, w.proxy_sm_scale, rows=rows,
                                       groups=groups)
    got = dpq[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    _check(f"{w.name} dproxy_q (sampled rows)", got[:, groups], rq[rows][:, groups])
    assert np.abs(plse.cpu().numpy()[rows][:, groups] - rl[rows][:, groups]).max() < 1e-3
    for gg, b in _late_blocks(lay, rng, Hkv):
        see = np.nonzero((np.arange(T) < lay.row_start[1]) &
                         (np.array([lay.pos(int(r)) for r in range(T)]) >= 128 * b))[0]
        print(f"[fullsize] oracle dproxy_k of group {gg} block {b}: {see.size} rows", flush=True)
        _, rk, _, _ = O.proxy_kl_backward(h["proxy_q"], h["proxy_k_pages"], h["q"], h["k_pages"], h["kv_indices"],
                                          gsel, w.qo_lens, w.kv_lens, 128, w.sm_scale, w.proxy_sm_scale, rows=see,
                                          groups=[gg])
        page = int(h["kv_indices"][lay.page_start[0] + b])
        _check(f"{w.name} dproxy_k (group {gg}, block {b})", dpk[page, gg].cpu().numpy().astype(np.float64),
               rk[page, gg])
    kvi = torch.from_numpy(h["kv_indices"].astype(np.int64)).cuda()
    _check_sum_zero("dproxy_k", dpk, kvi, lay, float(dpk.abs().max()))


def test_warmup_32k():
    """The warm-up mode at 32K: the dense forward on sampled rows; dq and
    dproxy_q on sampled rows and two groups; dk, dv and dproxy_k of two
    (group, late block) pairs exactly; per sequence and group sum_j dv_j =
    the group's dout sum and sum_j dk_j = 0, and dproxy_k sums to zero."""
    from block_sparse_top_amd import msa
    from tests.test_gpu_backward import _check
    w = workload(2)
    print(f"[fullsize] warm-up workload={w.name}", flush=True)
    inp = make_inputs_device(w, seed_of(2))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, proxy_dtype=w.proxy_dtype)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    N = inp.k_pages.shape[0]
    G = Hq // Hkv
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    msa.msa_dense_attn_prefill(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, out, lse)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(2) + 80)
    dout = torch.randn((T, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty((T, Hq, 128), device="cuda")
    dk = torch.zeros((N, Hkv, 128, 128), device="cuda")
    dv = torch.zeros_like(dk)
    dpq = torch.empty((T, Hkv, 128), device="cuda")
    dpk = torch.zeros_like(dk)
    plse = torch.empty((T, Hkv), device="cuda")
    msa.msa_dense_attn_prefill_backward(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, out, lse, dout, dq, dk,
                                        dv, inp.proxy_q, inp.proxy_k_pages, 1.0, dpq, dpk, plse)
    torch.cuda.synchronize()
    h = {k: to_host(getattr(inp, k)) for k in ("q", "k_pages", "v_pages", "proxy_q", "proxy_k_pages", "kv_indices")}
    lay = O.Layout(w.qo_lens, w.kv_lens, 128)
    allsel = np.full((T, Hkv, max(lay.nb)), -1, np.int32)
    for r in range(T):
        allsel[r, :, :lay.local(r) + 1] = np.arange(lay.local(r) + 1)
    rng = np.random.default_rng(seed_of(2) + 6)
    rows = _sample_rows(w, 4, seed_of(2))
    print(f"[fullsize] oracle dense forward on {rows.size} rows", flush=True)
    ref, ref_lse = O.sparse_attention(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], allsel, w.qo_lens,
                                      w.kv_lens, 128, w.sm_scale, rows=rows)
    tr = torch.from_numpy(rows).cuda()
    check_output(bf16_out_to_f64(out[tr]), ref, BF16_ATOL, BF16_COS, w.name + " warm-up forward")
    assert np.abs(lse[tr].cpu().numpy() - ref_lse).max() < 1e-3
    groups = sorted(set(rng.integers(Hkv, size=2).tolist()))
    heads = [hh for gg in groups for hh in range(gg * G, (gg + 1) * G)]
    dob = to_host(dout)
    print(f"[fullsize] oracle dq, dproxy_q on {rows.size} rows, groups {groups}", flush=True)
    rq, _, _ = O.sparse_attention_backward(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], allsel, w.qo_lens,
                                           w.kv_lens, 128, w.sm_scale, dob, rows=rows, groups=groups)
    _check(f"{w.name} warm-up dq", dq[tr].cpu().numpy().astype(np.float64)[:, heads], rq[rows][:, heads])
    rpq, _, _, rpl = O.proxy_kl_backward(h["proxy_q"], h["proxy_k_pages"], h["q"], h["k_pages"], h["kv_indices"],
                                         allsel, w.qo_lens, w.kv_lens, 128, w.sm_scale, w.proxy_sm_scale, rows=rows,
                                         groups=groups)
    _check(f"{w.name} warm-up dproxy_q", dpq[tr].cpu().numpy().astype(np.float64)[:, groups], rpq[rows][:, groups])
    assert np.abs(plse[tr].cpu().numpy()[:, groups] - rpl[rows][:, groups]).max() < 1e-3
    # every visible row reaches a block here (dense), so the checked blocks are
    # the last (the diagonal block alone) and the one before it
    nb0 = lay.nb[0]
    for gg, b in ((0, nb0 - 1), (int(rng.integers(1, Hkv)), nb0 - 2)):
        see = np.nonzero((np.arange(T) < lay.row_start[1]) &
                         (np.array([lay.pos(int(r)) for r in range(T)]) >= 128 * b))[0]
        print(f"[fullsize] oracle dk, dv, dproxy_k of group {gg} block {b}: {see.size} rows", flush=True)
        _, rk, rv = O.sparse_attention_backward(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], allsel,
                                                w.qo_lens, w.kv_lens, 128, w.sm_scale, dob, rows=see, groups=[gg])
        _, rpk, _, _ = O.proxy_kl_backward(h["proxy_q"], h["proxy_k_pages"], h["q"], h["k_pages"], h["kv_indices"],
                                           allsel, w.qo_lens, w.kv_lens, 128, w.sm_scale, w.proxy_sm_scale,
                                           rows=see, groups=[gg])
        page = int(h["kv_indices"][lay.page_start[0] + b])
        for name, got_t, want in (("dk", dk, rk), ("dv", dv, rv), ("dproxy_k", dpk, rpk)):
            _check(f"{w.name} warm-up {name} (group {gg}, block {b})",
                   got_t[page, gg].cpu().numpy().astype(np.float64), want[page, gg])
    kvi = torch.from_numpy(h["kv_indices"].astype(np.int64)).cuda()
    for si in range(len(w.kv_lens)):
        pages = kvi[int(lay.page_start[si]):int(lay.page_start[si + 1])]
        r0, r1 = int(lay.row_start[si]), int(lay.row_start[si + 1])
        for gg in range(Hkv):
            got = dv[pages, gg].double().sum(dim=(0, 1))
            ref_sum = dout[r0:r1, gg * G:(gg + 1) * G].double().sum(dim=(0, 1))
            scale = dout[r0:r1, gg * G:(gg + 1) * G].double().abs().sum(dim=(0, 1))
            assert ((got - ref_sum).abs() <= 2.0 ** -7 * scale + 1e-6).all(), (si, gg)
    _check_sum_zero("dk", dk, kvi, lay, float(dk.abs().max()))
    _check_sum_zero("dproxy_k", dpk, kvi, lay, float(dpk.abs().max()))


def test_prefill_32k_sampled_rows():
    _prefill_case(2, 1024)


def test_prefill_varlen_128k_sampled_rows():
    _prefill_case(3, 1024)


@pytest.mark.slow
def test_prefill_1m_fp8_proxy_sampled_rows():
    """256 seeded rows (evenly spaced) plus the edge rows and 8 random rows."""
    _prefill_case(5, 256)


def test_decode_fp8_b32_131k_all_outputs():
    from block_sparse_top_amd import msa
    w = workload(4)
    print(f"[fullsize] decode workload={w.name}", flush=True)
    inp = make_inputs_device(w, seed_of(4))
    plan = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    out = torch.empty((w.num_seqs, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.num_seqs, w.num_qo_heads), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_decode(plan, inp.q, inp.k_pages, inp.v_pages, inp.k_scale, inp.v_scale, inp.kv_indices,
                               inp.kv_block_indexes, out, lse)
    torch.cuda.synchronize()
    # the oracle only needs the selected pages: gather them (a plain copy) and renumber
    sel = to_host(inp.kv_block_indexes)
    kvi = to_host(inp.kv_indices)
    lay = O.Layout([1] * w.num_seqs, w.kv_lens, 128)
    need = sorted({int(kvi[lay.page_start[s] + b]) for s in range(w.num_seqs) for b in sel[s].ravel() if b >= 0})
    remap = np.full(inp.k_pages.shape[0], -1, np.int64)
    remap[need] = np.arange(len(need))
    idx = torch.tensor(need, device="cuda")
    kp = to_host(inp.k_pages[idx])
    vp = to_host(inp.v_pages[idx])
    kvi2 = np.where(remap[kvi] >= 0, remap[kvi], 0).astype(np.int32)
    ref, ref_lse = O.sparse_decode(to_host(inp.q), kp, vp, kvi2, sel, w.kv_lens, 128, w.sm_scale, FP8,
                                   to_host(inp.k_scale), to_host(inp.v_scale))
    check_output(bf16_out_to_f64(out), ref, FP8_ATOL, FP8_COS, w.name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3


@pytest.mark.parametrize("wn", [6, 7])
def test_decode_step_indexer_and_decode_b32_131k(wn):
    """A whole decode step at 32 x 131072: the indexer pass (8 fp8 proxy
    heads sharing one fp8 or MXFP4 proxy-K head, on a one-query-row plan) selects 16 + 1
    blocks per (sequence, group), then the fp8 sparse decode runs on that
    selection.  Fused and separate indexer calls agree bit for bit; block
    scores, selections and outputs are checked against the oracle for every
    sequence."""
    from block_sparse_top_amd import msa
    from synthetic.gen import Inputs
    w = workload(wn)
    S = w.num_seqs
    print(f"[fullsize] decode step workload={w.name}", flush=True)
    inp = make_inputs_device(w, seed_of(wn))
    ip = msa.msa_plan([1] * S, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads, w.num_proxy_kv_heads,
                      topk=w.topk, proxy_dtype=w.proxy_dtype)
    dp = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    sel = torch.full((S, w.num_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_proxy_topk_select(ip, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale,
                              inp.kv_indices, 0, S, sel)
    ms = msa.max_score_buffer(ip)
    sel2 = torch.full_like(sel, -7)
    msa.msa_proxy_block_maxscore(ip, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale,
                                 inp.kv_indices, 0, S, ms)
    msa.msa_topk_select(ip, ms, 0, S, sel2)
    out = torch.empty((S, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, w.num_qo_heads), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_decode(dp, inp.q, inp.k_pages, inp.v_pages, inp.k_scale, inp.v_scale, inp.kv_indices, sel,
                               out, lse)
    torch.cuda.synchronize()
    gms = msa.max_score_rows(ms, ip, S).cpu().numpy()
    gsel = sel.cpu().numpy()
    rows = np.arange(S)
    # the separate top-k call is exact on the low-precision scores it was given;
    # the fused call's selection is the exact one (checked against the oracle below)
    g = np.transpose(gms, (2, 0, 1)).astype(np.float64)
    lsel = sel2.cpu().numpy()
    for s_ in range(S):
        for p in range(w.num_kv_heads):
            loc = (w.kv_lens[s_] - 1) // 128
            assert np.array_equal(lsel[s_, p], O.topk_select_row(g[s_, p], loc, w.topk)), (s_, p)
    print(f"[fullsize] {w.name}: exact selection differs from the low-precision top-k in "
          f"{int((gsel != lsel).any(axis=2).sum())} of {S * w.num_kv_heads} pairs", flush=True)
    h = {k: to_host(getattr(inp, k)) for k in ("q", "kv_indices", "proxy_q", "proxy_k_pages", "proxy_q_scale",
                                                "proxy_k_scale", "k_scale", "v_scale")}
    ref_ms = O.proxy_block_maxscore(h["proxy_q"], h["proxy_k_pages"], h["kv_indices"], [1] * S, w.kv_lens, 128,
                                    w.proxy_sm_scale, w.proxy_dtype, h["proxy_q_scale"], h["proxy_k_scale"])
    hi = Inputs(w, h["kv_indices"], h["q"], None, None, proxy_q=h["proxy_q"], proxy_k_pages=h["proxy_k_pages"],
                proxy_q_scale=h["proxy_q_scale"], proxy_k_scale=h["proxy_k_scale"])
    check_max_score(gms, ref_ms, w.name, lowp_score_bound(hi, rows, w.proxy_sm_scale))
    lay = O.Layout([1] * S, w.kv_lens, 128)
    check_selection(gsel, ref_ms, np.array([lay.local(int(r)) for r in rows]), w.topk, w.name)
    # the decode on the indexer's selection: the oracle reads only the selected pages
    kvi = h["kv_indices"]
    need = sorted({int(kvi[lay.page_start[s] + b]) for s in range(S) for b in gsel[s].ravel() if b >= 0})
    remap = np.full(inp.k_pages.shape[0], -1, np.int64)
    remap[need] = np.arange(len(need))
    idx = torch.tensor(need, device="cuda")
    kp = to_host(inp.k_pages[idx])
    vp = to_host(inp.v_pages[idx])
    kvi2 = np.where(remap[kvi] >= 0, remap[kvi], 0).astype(np.int32)
    ref, ref_lse = O.sparse_decode(h["q"], kp, vp, kvi2, gsel, w.kv_lens, 128, w.sm_scale, FP8, h["k_scale"],
                                   h["v_scale"])
    check_output(bf16_out_to_f64(out), ref, FP8_ATOL, FP8_COS, w.name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3
