"""Helpers for the GPU parity tests: move synthetic inputs to the device, run
the HIP path through the binding, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synthetic.gen import Inputs, BF16, FP8, MXFP4, MXFP4_QK

BAND = 1e-3          # selection tie band on block scores
MS_ATOL, MS_RTOL = 1e-4, 1e-5
BF16_ATOL, BF16_COS = 2e-2, 0.999
FP8_ATOL, FP8_COS = 6e-2, 0.99


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def device_inputs(inp: Inputs, device="cuda") -> dict:
    d = dict(q=dev(inp.q), k_pages=dev(inp.k_pages), v_pages=dev(inp.v_pages), kv_indices=dev(inp.kv_indices))
    for name in ("k_scale", "v_scale", "proxy_q", "proxy_k_pages", "proxy_q_scale", "proxy_k_scale",
                 "kv_block_indexes"):
        v = getattr(inp, name)
        d[name] = dev(v) if v is not None else None
    return d


def plan_for(msa, inp: Inputs, max_rows_per_call=0, topk=None):
    w = inp.w
    if w.mode == "decode":
        return msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=topk or w.topk,
                            kv_dtype=w.kv_dtype, mode="decode")
    return msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=topk or w.topk, kv_dtype=w.kv_dtype, proxy_dtype=w.proxy_dtype,
                        max_rows_per_call=max_rows_per_call)


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.ravel()
    b = b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def oracle_scores(inp: Inputs, rows=None):
    w = inp.w
    return O.proxy_block_maxscore(inp.proxy_q, inp.proxy_k_pages, inp.kv_indices, w.qo_lens, w.kv_lens,
                                  w.page_size, w.proxy_sm_scale, w.proxy_dtype, inp.proxy_q_scale,
                                  inp.proxy_k_scale, rows=rows)


# The fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, also for fp8 x
# MXFP4) do not sum products exactly: a product far below the largest of its
# group loses low bits.  Measured through the proxy kernels on eight operand
# distributions (Gaussian, Student-t, log-uniform, sparse spikes, low-rank,
# one dominant dim, cancelling halves, equal magnitudes): |error| <= 2^-10.7
# (fp8 x fp8), 2^-11.3 (fp8 x FP4), 2^-19.7 (FP4 x FP4) of
# proxy_sm_scale * max|q_d| * max|k_jd|.  The library's selection bound uses
# 2^-9 (2^-17 for FP4 x FP4) times the same product; the exported low-precision
# scores are checked against that bound (with max|k| over the row's visible
# keys, which is at most the library's).
LOWP_COEF = {FP8: 2.0 ** -9, MXFP4: 2.0 ** -9, MXFP4_QK: 2.0 ** -17}
LOW_PRECISION_PROXY = (FP8, MXFP4, MXFP4_QK)


def lowp_score_bound(inp, rows, scale):
    """Per (row, head, block): the error bound of a low-precision proxy score,
    coef * scale * max_d |q_d| * max |k| over the row's visible keys."""
    w = inp.w
    lay = O.Layout(w.qo_lens, w.kv_lens, w.page_size)
    P, Pk = w.num_proxy_heads, w.num_proxy_kv_heads
    rows = np.asarray(rows)
    out = np.zeros((len(rows), P, max(lay.nb)))
    coef = LOWP_COEF[w.proxy_dtype]
    for s in range(len(lay.kv)):
        idx = [i for i, r in enumerate(rows) if lay.row_start[s] <= r < lay.row_start[s + 1]]
        if not idx:
            continue
        L = lay.kv[s]
        pos = np.array([lay.pos(int(rows[i])) for i in idx])
        kcache = {}
        for p in range(P):
            ph = p if Pk == P else 0
            if ph not in kcache:
                K = np.abs(O.gather_rows(inp.proxy_k_pages, w.proxy_dtype, inp.proxy_k_scale, inp.kv_indices,
                                         lay, s, ph, np.arange(L)))
                kcache[ph] = np.maximum.accumulate(K.max(axis=1))      # max |k| over keys 0..j
            qs = None if inp.proxy_q_scale is None else inp.proxy_q_scale[p:p + 1]
            q = np.abs(O.dequant_proxy_q(inp.proxy_q[rows[idx], p:p + 1, :], w.proxy_dtype, qs))[:, 0].max(axis=1)
            kvis = kcache[ph][np.minimum(pos, L - 1)]
            out[idx, p, :] = (coef * scale * q * kvis)[:, None]
    return out


def check_max_score(gpu_ms: np.ndarray, ref: np.ndarray, what="", extra_tol=None):
    """gpu_ms [P, nb_max, n] vs ref [n, P, nb_max]; compare defined entries."""
    g = np.transpose(gpu_ms, (2, 0, 1)).astype(np.float64)
    m = ~np.isnan(ref)
    fin = m & np.isfinite(ref)
    # -inf entries must match exactly
    assert np.array_equal(np.isneginf(g[m & ~fin]), np.ones(int((m & ~fin).sum()), bool)), what
    err = np.abs(g[fin] - ref[fin])
    tol = MS_ATOL + MS_RTOL * np.abs(ref[fin])
    if extra_tol is not None:
        tol = tol + extra_tol[fin]
    bad = ~(err <= tol)           # a NaN where the oracle has a value is an error too
    assert not bad.any(), f"{what}: {int(bad.sum())} max_score entries off (worst {np.nanmax(err):.3g}, " \
                          f"{int(np.isnan(err).sum())} NaN)"


def check_selection(sel: np.ndarray, scores: np.ndarray, locals_: np.ndarray, k: int, what=""):
    """sel [n, P, k] (GPU) against fp64 oracle scores [n, P, nb]."""
    n, P, _ = sel.shape
    bad = []
    ties = 0
    for i in range(n):
        for p in range(P):
            ok, why = O.check_selection_row(sel[i, p], scores[i, p], int(locals_[i]), k, BAND)
            if not ok:
                bad.append((i, p, why))
    assert not bad, f"{what}: {len(bad)} selections rejected, first {bad[:3]}"
    return ties


def check_output(out: np.ndarray, ref: np.ndarray, atol: float, cos_min: float, what=""):
    err = np.abs(out - ref).max()
    c = cosine(out, ref)
    assert err <= atol and c >= cos_min, f"{what}: max|err| {err:.4g} (tol {atol}), cos {c:.6f} (min {cos_min})"
    return err, c
