"""Python binding of the MSA C ABI (include/msa.h).

Argument marshalling only: every step of the path runs in libmsa.so's HIP
kernels.  Tensors are torch tensors on the current HIP device; bf16 tensors
may be torch.bfloat16 or raw uint16/int16 bits, fp8 tensors
torch.float8_e4m3fn or raw uint8 bits.  Every call is enqueued on torch's
current stream.  If libmsa.so has not been built this module raises at import.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE_TOO_SMALL, MSA_ERR_HIP = range(5)
MSA_BF16, MSA_FP8_E4M3, MSA_MXFP4, MSA_MXFP4_QK = 0, 1, 2, 3
MSA_PREFILL, MSA_DECODE = 0, 1

ENTRY_POINTS = ("msa_plan", "msa_plan_destroy", "msa_plan_info", "msa_proxy_block_maxscore", "msa_topk_select",
                "msa_proxy_topk_select", "msa_sparse_attn_prefill", "msa_sparse_attn_prefill_rows",
                "msa_sparse_attn_prefill_backward", "msa_sparse_attn_prefill_backward_kl",
                "msa_dense_attn_prefill", "msa_dense_attn_prefill_backward",
                "msa_sparse_attn_decode", "msa_sparse_attn_decode_noalloc", "msa_workspace_reset", "msa_last_error", "msa_profile_kernel",
                "msa_profile_read", "msa_diag_mfma_rate")


class MsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[msa status {status}] {msg}")
        self.status = status


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("qo_lens_host", ctypes.POINTER(ctypes.c_int32)),
        ("kv_lens_host", ctypes.POINTER(ctypes.c_int32)),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_proxy_heads", ctypes.c_int32),
        ("num_proxy_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
        ("proxy_dtype", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("proxy_sm_scale", ctypes.c_float),
        ("mode", ctypes.c_int),
        ("max_rows_per_call", ctypes.c_int64),
        ("attn_window_rows", ctypes.c_int64),
        ("decode_splits", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "(or python block_sparse_top_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, VP, FP, IP = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p)
    lib.msa_plan.argtypes = [ctypes.POINTER(PlanDesc), ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_plan_destroy.argtypes = [P]
    lib.msa_plan_info.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int64)]
    lib.msa_proxy_block_maxscore.argtypes = [P, VP, VP, FP, FP, IP, I64, I64, FP, VP, SZ, P]
    lib.msa_topk_select.argtypes = [P, FP, I64, I64, IP, VP, SZ, P]
    lib.msa_proxy_topk_select.argtypes = [P, VP, VP, FP, FP, IP, I64, I64, IP, VP, SZ, P]
    lib.msa_sparse_attn_prefill.argtypes = [P, VP, VP, VP, FP, FP, IP, IP, VP, FP, VP, SZ, P]
    lib.msa_sparse_attn_prefill_rows.argtypes = [P, VP, VP, VP, FP, FP, IP, IP, VP, FP, I64, I64, VP, SZ, P]
    lib.msa_sparse_attn_prefill_backward.argtypes = [P, VP, VP, VP, IP, IP, VP, FP, VP, FP, FP, FP, VP, SZ, P]
    lib.msa_sparse_attn_prefill_backward_kl.argtypes = [P, VP, VP, VP, IP, IP, VP, FP, VP, VP, VP, ctypes.c_float, FP,
                                                        FP, FP, FP, FP, FP, VP, SZ, P]
    lib.msa_dense_attn_prefill.argtypes = [P, VP, VP, VP, IP, VP, FP, VP, SZ, P]
    lib.msa_dense_attn_prefill_backward.argtypes = [P, VP, VP, VP, IP, VP, FP, VP, VP, VP, ctypes.c_float, FP, FP, FP,
                                                    FP, FP, FP, VP, SZ, P]
    lib.msa_sparse_attn_decode.argtypes = [P, VP, VP, VP, FP, FP, IP, IP, VP, FP, VP, SZ, P]
    lib.msa_sparse_attn_decode_noalloc.argtypes = [P, VP, VP, VP, FP, FP, IP, IP, VP, FP, P]
    lib.msa_workspace_reset.argtypes = [VP, SZ]
    lib.msa_profile_kernel.argtypes = [P, ctypes.c_char_p]
    lib.msa_diag_mfma_rate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    lib.msa_profile_read.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.msa_last_error.restype = ctypes.c_char_p
    for name in ENTRY_POINTS:
        if name != "msa_last_error":
            getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int):
    if status != MSA_OK:
        raise MsaError(status, _lib.msa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MSA library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(name: str) -> int:
    return {"bf16": MSA_BF16, "fp8": MSA_FP8_E4M3, "mxfp4": MSA_MXFP4, "mxfp4_qk": MSA_MXFP4_QK}[name]


class Plan:
    """An msa_plan_t plus the device workspace it is bound to."""

    def __init__(self, desc: PlanDesc, qo, kv, device=None, allocate=True):
        self._keep = (qo, kv)
        self.one_row = qo is not None and len(qo) > 0 and all(int(x) == 1 for x in qo)  # one query row per sequence
        h = ctypes.c_void_p()
        nbytes = ctypes.c_size_t()
        _check(_lib.msa_plan(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(nbytes)))
        self.handle = h
        self.desc = desc
        self.workspace_bytes = int(nbytes.value)
        T, nbm, mr = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
        _check(_lib.msa_plan_info(h, ctypes.byref(T), ctypes.byref(nbm), ctypes.byref(mr)))
        self.total_rows, self.nb_max, self.max_rows_per_call = int(T.value), int(nbm.value), int(mr.value)
        self._workspace = None
        if allocate:
            self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device or "cuda")

    @property
    def workspace(self):
        return self._workspace

    @workspace.setter
    def workspace(self, t: Optional[torch.Tensor]):
        # memory from torch's caching allocator may have held anything
        # (another plan's metadata included): the library must copy this
        # plan's metadata into it again on first use
        if t is not None:
            _check(_lib.msa_workspace_reset(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()))
        self._workspace = t

    def __del__(self):
        h = getattr(self, "handle", None)
        lib_ = _lib  # None once the interpreter has torn the module down
        if h is not None and h.value and lib_ is not None:
            lib_.msa_plan_destroy(h)
            self.handle = None


def msa_plan(qo_lens: Sequence[int], kv_lens: Sequence[int], num_qo_heads: int, num_kv_heads: int,
             num_proxy_heads: int = 0, num_proxy_kv_heads: int = 0, topk: int = 16, kv_dtype: str = "bf16",
             proxy_dtype: str = "bf16", sm_scale: Optional[float] = None, proxy_sm_scale: Optional[float] = None,
             mode: str = "prefill", max_rows_per_call: int = 0, head_dim: int = 128, page_size: int = 128,
             device=None, allocate: bool = True, attn_window_rows: int = 0, decode_splits: int = 0) -> Plan:
    n = len(kv_lens)
    qo = (ctypes.c_int32 * n)(*[int(x) for x in qo_lens]) if qo_lens is not None else None
    kv = (ctypes.c_int32 * n)(*[int(x) for x in kv_lens])
    d = PlanDesc()
    d.batch = n
    d.qo_lens_host = ctypes.cast(qo, ctypes.POINTER(ctypes.c_int32)) if qo is not None else None
    d.kv_lens_host = ctypes.cast(kv, ctypes.POINTER(ctypes.c_int32))
    d.num_qo_heads, d.num_kv_heads = num_qo_heads, num_kv_heads
    d.num_proxy_heads, d.num_proxy_kv_heads = num_proxy_heads, num_proxy_kv_heads
    d.head_dim, d.page_size, d.topk = head_dim, page_size, topk
    d.kv_dtype, d.proxy_dtype = _dtype_code(kv_dtype), _dtype_code(proxy_dtype)
    d.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim)
    d.proxy_sm_scale = proxy_sm_scale if proxy_sm_scale is not None else 1.0 / math.sqrt(head_dim)
    d.mode = {"prefill": MSA_PREFILL, "decode": MSA_DECODE}[mode]
    d.max_rows_per_call = max_rows_per_call
    d.attn_window_rows = attn_window_rows
    d.decode_splits = decode_splits
    return Plan(d, qo, kv, device=device, allocate=allocate)


def msa_proxy_block_maxscore(plan: Plan, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale, kv_indices,
                             row_begin: int, row_count: int, max_score: torch.Tensor) -> torch.Tensor:
    _check(_lib.msa_proxy_block_maxscore(plan.handle, _ptr(proxy_q), _ptr(proxy_k_pages), _ptr(proxy_q_scale),
                                         _ptr(proxy_k_scale), _ptr(kv_indices), row_begin, row_count,
                                         _ptr(max_score), _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return max_score


def msa_topk_select(plan: Plan, max_score, row_begin: int, row_count: int, kv_block_indexes) -> torch.Tensor:
    _check(_lib.msa_topk_select(plan.handle, _ptr(max_score), row_begin, row_count, _ptr(kv_block_indexes),
                                _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return kv_block_indexes


def msa_proxy_topk_select(plan: Plan, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale, kv_indices,
                          row_begin: int, row_count: int, kv_block_indexes) -> torch.Tensor:
    _check(_lib.msa_proxy_topk_select(plan.handle, _ptr(proxy_q), _ptr(proxy_k_pages), _ptr(proxy_q_scale),
                                      _ptr(proxy_k_scale), _ptr(kv_indices), row_begin, row_count,
                                      _ptr(kv_block_indexes), _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return kv_block_indexes


def msa_sparse_attn_prefill(plan: Plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, lse=None,
                            k_scale=None, v_scale=None):
    _check(_lib.msa_sparse_attn_prefill(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                        _ptr(v_scale), _ptr(kv_indices), _ptr(kv_block_indexes), _ptr(out),
                                        _ptr(lse), _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return out, lse


def msa_sparse_attn_prefill_rows(plan: Plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, row_begin,
                                 row_count, lse=None, k_scale=None, v_scale=None):
    _check(_lib.msa_sparse_attn_prefill_rows(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                             _ptr(v_scale), _ptr(kv_indices), _ptr(kv_block_indexes), _ptr(out),
                                             _ptr(lse), row_begin, row_count, _ptr(plan.workspace),
                                             plan.workspace_bytes, _stream()))
    return out, lse


def msa_sparse_attn_prefill_backward(plan: Plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, lse, dout,
                                     dq, dk_pages, dv_pages):
    _check(_lib.msa_sparse_attn_prefill_backward(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_indices),
                                                 _ptr(kv_block_indexes), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                                 _ptr(dk_pages), _ptr(dv_pages), _ptr(plan.workspace),
                                                 plan.workspace_bytes, _stream()))
    return dq, dk_pages, dv_pages


def msa_sparse_attn_prefill_backward_kl(plan: Plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, lse, dout,
                                        proxy_q, proxy_k_pages, kl_grad_scale, dq, dk_pages, dv_pages, dproxy_q,
                                        dproxy_k_pages, proxy_lse):
    _check(_lib.msa_sparse_attn_prefill_backward_kl(
        plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_indices), _ptr(kv_block_indexes), _ptr(out),
        _ptr(lse), _ptr(dout), _ptr(proxy_q), _ptr(proxy_k_pages), float(kl_grad_scale), _ptr(dq), _ptr(dk_pages),
        _ptr(dv_pages), _ptr(dproxy_q), _ptr(dproxy_k_pages), _ptr(proxy_lse), _ptr(plan.workspace),
        plan.workspace_bytes, _stream()))
    return dq, dk_pages, dv_pages, dproxy_q, dproxy_k_pages, proxy_lse


def msa_dense_attn_prefill(plan: Plan, q, k_pages, v_pages, kv_indices, out, lse):
    _check(_lib.msa_dense_attn_prefill(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_indices), _ptr(out),
                                       _ptr(lse), _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return out, lse


def msa_dense_attn_prefill_backward(plan: Plan, q, k_pages, v_pages, kv_indices, out, lse, dout, dq, dk_pages,
                                    dv_pages, proxy_q=None, proxy_k_pages=None, kl_grad_scale=1.0, dproxy_q=None,
                                    dproxy_k_pages=None, proxy_lse=None):
    _check(_lib.msa_dense_attn_prefill_backward(
        plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_indices), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(proxy_q), _ptr(proxy_k_pages), float(kl_grad_scale), _ptr(dq), _ptr(dk_pages), _ptr(dv_pages),
        _ptr(dproxy_q), _ptr(dproxy_k_pages), _ptr(proxy_lse), _ptr(plan.workspace), plan.workspace_bytes,
        _stream()))
    return dq, dk_pages, dv_pages, dproxy_q, dproxy_k_pages, proxy_lse


def msa_sparse_attn_decode(plan: Plan, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out,
                           lse=None):
    _check(_lib.msa_sparse_attn_decode(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(kv_indices), _ptr(kv_block_indexes), _ptr(out),
                                       _ptr(lse), _ptr(plan.workspace), plan.workspace_bytes, _stream()))
    return out, lse


def msa_sparse_attn_decode_noalloc(plan: Plan, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes,
                                   out, lse=None):
    """msa_sparse_attn_decode with the library's static per-device scratch
    instead of the plan's workspace (no allocation; calls on one device must
    not overlap)."""
    _check(_lib.msa_sparse_attn_decode_noalloc(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                               _ptr(v_scale), _ptr(kv_indices), _ptr(kv_block_indexes), _ptr(out),
                                               _ptr(lse), _stream()))
    return out, lse


def msa_profile_kernel(plan: Plan, kernel: Optional[str]):
    """Bracket every later launch of one internal kernel with HIP events."""
    _check(_lib.msa_profile_kernel(plan.handle, kernel.encode() if kernel else None))


def msa_profile_read(plan: Plan):
    """(summed milliseconds, launches) of the profiled kernel since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(_lib.msa_profile_read(plan.handle, ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def msa_diag_mfma_rate(dtype: str, iters: int = 20000) -> float:
    """Dense matrix-core TFLOP/s this device sustains (diagnostic)."""
    t = ctypes.c_double()
    _check(_lib.msa_diag_mfma_rate(_dtype_code(dtype), iters, ctypes.byref(t)))
    return float(t.value)


def max_score_buffer(plan: Plan, device=None) -> torch.Tensor:
    """fp32 [P, nb_max, max_rows_per_call] buffer for the proxy/top-k chunks."""
    P = plan.desc.num_proxy_heads
    return torch.empty((P, plan.nb_max, plan.max_rows_per_call), dtype=torch.float32, device=device or "cuda")


def max_score_rows(max_score: torch.Tensor, plan: Plan, row_count: int) -> torch.Tensor:
    """The [P, nb_max, row_count] result of a proxy call over row_count rows:
    the call writes it densely at the start of the buffer (row stride =
    row_count), so a shorter last chunk is not a slice of the full buffer."""
    P = plan.desc.num_proxy_heads
    return max_score.view(-1)[:P * plan.nb_max * row_count].view(P, plan.nb_max, row_count)


def run_prefill(plan: Plan, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale, q, k_pages, v_pages, kv_indices,
                kv_block_indexes, out, lse=None, max_score=None, fused=None, k_scale=None, v_scale=None):
    """The whole prefill path: the block selection (the fused proxy + top-k
    pass when topk <= 17, else proxy max scores and top-k chunk by chunk of
    rows), then the sparse attention."""
    T, R = plan.total_rows, plan.max_rows_per_call
    if fused is None:
        fused = plan.desc.topk <= 17
    if not fused and plan.desc.proxy_dtype != MSA_BF16 and not plan.one_row:
        # the separate top-k ranks the fp32 scores it is given; only the fused
        # call re-scores the fp8 / MXFP4 proxies' boundary blocks exactly
        raise ValueError("run_prefill: fp8 / MXFP4 proxies select exactly only through the fused call (topk <= 17)")
    if fused:
        msa_proxy_topk_select(plan, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale, kv_indices, 0, T,
                              kv_block_indexes)
        msa_sparse_attn_prefill(plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, lse, k_scale, v_scale)
        return out, lse
    if max_score is None:
        max_score = max_score_buffer(plan, q.device)
    for r0 in range(0, T, R):
        n = min(R, T - r0)
        msa_proxy_block_maxscore(plan, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale, kv_indices, r0, n,
                                 max_score)
        msa_topk_select(plan, max_score, r0, n, kv_block_indexes)
    msa_sparse_attn_prefill(plan, q, k_pages, v_pages, kv_indices, kv_block_indexes, out, lse, k_scale, v_scale)
    return out, lse
