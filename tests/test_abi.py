"""The C-ABI library loads, exports every entry point include/msa.h declares,
and rejects bad arguments on the host (no GPU needed: no call here reaches
a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

LIB = os.path.join(ROOT, "block_sparse_top_amd", "libmsa.so")
if not os.path.exists(LIB):
    pytest.skip("libmsa.so not built", allow_module_level=True)
# a built library must load (an unresolved symbol is a build defect, not a skip)
from block_sparse_top_amd import msa  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"msa_plan", "msa_plan_destroy", "msa_proxy_block_maxscore", "msa_topk_select",
            "msa_sparse_attn_prefill", "msa_sparse_attn_decode", "msa_last_error"} <= set(names)
    lib = ctypes.CDLL(msa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _plan(**kw):
    args = dict(qo_lens=[300, 5], kv_lens=[300, 900], num_qo_heads=8, num_kv_heads=2, num_proxy_heads=2,
                num_proxy_kv_heads=2, topk=4, allocate=False)
    args.update(kw)
    return msa.msa_plan(**args)


def test_plan_info_and_workspace():
    p = _plan()
    assert p.total_rows == 305 and p.nb_max == 8 and p.max_rows_per_call == 305
    assert p.workspace_bytes > 0
    p2 = _plan(max_rows_per_call=100)
    assert p2.max_rows_per_call == 100
    p3 = _plan(attn_window_rows=100)          # attention partials scale with the window
    assert p3.workspace_bytes < p.workspace_bytes
    d = msa.msa_plan(None, [1000] * 4, 16, 2, topk=17, kv_dtype="fp8", mode="decode", allocate=False)
    assert d.total_rows == 4 and d.nb_max == 8


def test_window_capped_to_32bit_planes():
    # a plane of partial records (32 bytes each, rows x heads x topk plus 256
    # spare records) stays under 2^32 bytes: 64 heads, topk 64 -> 32767 rows
    def ws(w):
        return msa.msa_plan([40000], [40000], 64, 8, 8, 8, topk=64, attn_window_rows=w,
                            allocate=False).workspace_bytes
    cap = ((1 << 27) - 256) // (64 * 64)
    assert cap == 32767
    assert ws(40000) == ws(cap) > ws(cap - 1)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(page_size=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_qo_heads=6, num_kv_heads=2), msa.MSA_ERR_UNSUPPORTED),        # G = 3
    (dict(num_qo_heads=7, num_kv_heads=2), msa.MSA_ERR_INVALID_ARG),
    (dict(topk=0), msa.MSA_ERR_INVALID_ARG),
    (dict(topk=65), msa.MSA_ERR_INVALID_ARG),
    (dict(qo_lens=[300, 901]), msa.MSA_ERR_INVALID_ARG),                     # qo > kv
    (dict(qo_lens=[0, 5]), msa.MSA_ERR_INVALID_ARG),
    (dict(num_proxy_heads=1), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_proxy_kv_heads=3), msa.MSA_ERR_INVALID_ARG),
    (dict(kv_dtype="mxfp4", mode="decode", qo_lens=None), msa.MSA_ERR_UNSUPPORTED),  # MXFP4 K/V decode not built
    (dict(sm_scale=-1.0), msa.MSA_ERR_INVALID_ARG),
    (dict(attn_window_rows=-1), msa.MSA_ERR_INVALID_ARG),
])
def test_plan_validation(kw, status):
    with pytest.raises(msa.MsaError) as e:
        _plan(**kw)
    assert e.value.status == status
    assert msa.lib().msa_last_error().decode()


def test_decode_plan_needs_single_query_rows():
    with pytest.raises(msa.MsaError) as e:
        msa.msa_plan([2, 1], [100, 100], 8, 2, topk=4, mode="decode", allocate=False)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG


class _Fake:
    """Stands in for a device tensor: an aligned, never-dereferenced address."""

    def __init__(self, addr):
        self.addr = addr

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self.addr


def _call(fn, *args):
    return getattr(msa.lib(), fn)(*args)


def test_compute_calls_validate_before_touching_the_device():
    p = _plan()
    L = msa.lib()
    a = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x20000)
    none = None
    nb = p.workspace_bytes
    # null pointer
    st = L.msa_proxy_block_maxscore(p.handle, none, a, none, none, a, 0, 10, a, ws, nb, none)
    assert st == msa.MSA_ERR_INVALID_ARG and b"proxy_q" in L.msa_last_error()
    # misaligned pointer
    st = L.msa_proxy_block_maxscore(p.handle, ctypes.c_void_p(0x10004), a, none, none, a, 0, 10, a, ws, nb, none)
    assert st == msa.MSA_ERR_INVALID_ARG
    # row range outside [0, T) and empty range
    assert L.msa_proxy_block_maxscore(p.handle, a, a, none, none, a, 300, 10, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_topk_select(p.handle, a, 0, 0, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    # scales given for bf16
    assert L.msa_proxy_block_maxscore(p.handle, a, a, a, a, a, 0, 10, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    # workspace too small / missing / misaligned
    assert L.msa_topk_select(p.handle, a, 0, 10, a, ws, nb - 1, none) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert L.msa_topk_select(p.handle, a, 0, 10, a, none, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_topk_select(p.handle, a, 0, 10, a, ctypes.c_void_p(0x20010), nb, none) == msa.MSA_ERR_INVALID_ARG
    # wrong mode
    assert L.msa_sparse_attn_decode(p.handle, a, a, a, none, none, a, a, a, none, ws, nb, none) == msa.MSA_ERR_UNSUPPORTED
    # bf16 prefill takes no scales; fp8 prefill needs both; MXFP4 none
    assert L.msa_sparse_attn_prefill(p.handle, a, a, a, a, a, a, a, a, none, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    p8 = _plan(kv_dtype="fp8")
    assert L.msa_sparse_attn_prefill(p8.handle, a, a, a, a, none, a, a, a, none, ws, p8.workspace_bytes, none) == \
        msa.MSA_ERR_INVALID_ARG
    p4 = _plan(kv_dtype="mxfp4")
    assert L.msa_sparse_attn_prefill(p4.handle, a, a, a, a, a, a, a, a, none, ws, p4.workspace_bytes, none) == \
        msa.MSA_ERR_INVALID_ARG
    d = msa.msa_plan(None, [1000] * 4, 16, 2, topk=17, kv_dtype="fp8", mode="decode", allocate=False)
    # fp8 decode needs both scales
    assert L.msa_sparse_attn_decode(d.handle, a, a, a, a, none, a, a, a, none, ws, d.workspace_bytes, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_proxy_block_maxscore(d.handle, a, a, none, none, a, 0, 1, a, ws, d.workspace_bytes, none) == msa.MSA_ERR_UNSUPPORTED
    # fused proxy + top-k: the same checks, no row-chunk bound, topk <= 17
    T = p.total_rows
    assert L.msa_proxy_topk_select(p.handle, a, a, none, none, a, 0, 10, none, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_proxy_topk_select(p.handle, a, a, none, none, a, T - 5, 10, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_proxy_topk_select(p.handle, a, a, a, a, a, 0, 10, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_proxy_topk_select(p.handle, a, a, none, none, a, 0, 10, a, ws, nb - 1, none) == \
        msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert L.msa_proxy_topk_select(d.handle, a, a, none, none, a, 0, 1, a, ws, d.workspace_bytes, none) == \
        msa.MSA_ERR_UNSUPPORTED
    big = msa.msa_plan([100], [100], 8, 2, 2, 2, topk=18, allocate=False)
    assert L.msa_proxy_topk_select(big.handle, a, a, none, none, a, 0, 10, a, ws, big.workspace_bytes, none) == \
        msa.MSA_ERR_UNSUPPORTED and b"topk" in L.msa_last_error()
    # row-range attention: the range must lie in [0, T) and be non-empty
    assert L.msa_sparse_attn_prefill_rows(p.handle, a, a, a, none, none, a, a, a, none, T - 5, 10, ws, nb, none) == \
        msa.MSA_ERR_INVALID_ARG
    assert L.msa_sparse_attn_prefill_rows(p.handle, a, a, a, none, none, a, a, a, none, 0, 0, ws, nb, none) == \
        msa.MSA_ERR_INVALID_ARG
    assert L.msa_sparse_attn_prefill_rows(d.handle, a, a, a, none, none, a, a, a, none, 0, 1, ws, nb, none) == \
        msa.MSA_ERR_UNSUPPORTED
    assert L.msa_plan_destroy(None) == msa.MSA_OK


def test_mxfp4_proxy_rules():
    """MXFP4 proxies: fp8 q carries its per-head scales (MXFP4), MXFP4 q and
    K carry none (their block scales are in the data); any plan shape."""
    L = msa.lib()
    a, ws, none = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), None
    for qo in ([1, 1], [300, 5]):
        p = msa.msa_plan(qo, [300, 900], 8, 2, 2, 1, topk=4, proxy_dtype="mxfp4", allocate=False)
        pqk = msa.msa_plan(qo, [300, 900], 8, 2, 2, 2, topk=4, proxy_dtype="mxfp4_qk", allocate=False)
        for fn in ("msa_proxy_block_maxscore", "msa_proxy_topk_select"):
            f = getattr(L, fn)
            nb = p.workspace_bytes
            assert f(p.handle, a, a, none, none, a, 0, 2, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG   # q scale missing
            assert f(p.handle, a, a, a, a, a, 0, 2, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG         # k scale given
            assert f(p.handle, a, a, a, none, a, 0, 2, a, ws, nb - 1, none) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
            nb = pqk.workspace_bytes
            assert f(pqk.handle, a, a, a, none, a, 0, 2, a, ws, nb, none) == msa.MSA_ERR_INVALID_ARG   # q scale given
            assert f(pqk.handle, a, a, none, none, a, 0, 2, a, ws, nb - 1, none) == msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_training_entry_points_validate_before_touching_the_device():
    """The backward, the fused distillation backward and the warm-up calls
    reject bad arguments and unsupported plans before any launch."""
    L = msa.lib()
    a = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x20000)
    none = None
    p = _plan()
    nb = p.workspace_bytes
    f = ctypes.c_float
    # main backward: null dout, decode plan, fp8 K/V
    assert L.msa_sparse_attn_prefill_backward(p.handle, a, a, a, a, a, a, a, none, a, a, a, ws, nb, none) == \
        msa.MSA_ERR_INVALID_ARG and b"dout" in L.msa_last_error()
    d = msa.msa_plan(None, [1000] * 4, 16, 2, topk=17, kv_dtype="fp8", mode="decode", allocate=False)
    assert L.msa_sparse_attn_prefill_backward(d.handle, a, a, a, a, a, a, a, a, a, a, a, ws, d.workspace_bytes,
                                              none) == msa.MSA_ERR_UNSUPPORTED
    p8 = _plan(kv_dtype="fp8")
    assert L.msa_sparse_attn_prefill_backward(p8.handle, a, a, a, a, a, a, a, a, a, a, a, ws, p8.workspace_bytes,
                                              none) == msa.MSA_ERR_UNSUPPORTED
    # fused distillation backward: proxy shape, finite scale, every pointer
    args = lambda plan, gs, last=a: (plan.handle, a, a, a, a, a, a, a, a, a, a, f(gs), a, a, a, a, a, last, ws,
                                     plan.workspace_bytes, none)
    assert L.msa_sparse_attn_prefill_backward_kl(*args(p, float("nan"))) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_sparse_attn_prefill_backward_kl(*args(p, 1.0, none)) == msa.MSA_ERR_INVALID_ARG
    pf8 = msa.msa_plan([300], [300], 8, 2, 2, 2, topk=4, proxy_dtype="fp8", allocate=False)
    assert L.msa_sparse_attn_prefill_backward_kl(*args(pf8, 1.0)) == msa.MSA_ERR_UNSUPPORTED
    shared = msa.msa_plan([300], [300], 8, 2, 2, 1, topk=4, allocate=False)
    assert L.msa_sparse_attn_prefill_backward_kl(*args(shared, 1.0)) == msa.MSA_ERR_UNSUPPORTED
    # warm-up forward and backward
    assert L.msa_dense_attn_prefill(p.handle, a, a, a, a, a, none, ws, nb, none) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_dense_attn_prefill(d.handle, a, a, a, a, a, a, ws, d.workspace_bytes, none) == \
        msa.MSA_ERR_UNSUPPORTED
    assert L.msa_dense_attn_prefill(p8.handle, a, a, a, a, a, a, ws, p8.workspace_bytes, none) == \
        msa.MSA_ERR_UNSUPPORTED
    dense = lambda plan, pq, gs=1.0: (plan.handle, a, a, a, a, a, a, a, pq, pq, f(gs), a, a, a, a, a, a, ws,
                                      plan.workspace_bytes, none)
    assert L.msa_dense_attn_prefill_backward(*dense(pf8, a)) == msa.MSA_ERR_UNSUPPORTED
    assert L.msa_dense_attn_prefill_backward(*dense(shared, a)) == msa.MSA_ERR_UNSUPPORTED
    assert L.msa_dense_attn_prefill_backward(*dense(p, a, float("inf"))) == msa.MSA_ERR_INVALID_ARG
    # an attention window too short to hold D of every row
    tiny = msa.msa_plan([4096], [4096], 8, 2, 2, 2, topk=1, attn_window_rows=32, allocate=False)
    assert L.msa_dense_attn_prefill_backward(*dense(tiny, none)) == msa.MSA_ERR_UNSUPPORTED and \
        b"window" in L.msa_last_error()


def test_plan_limits_and_workspace_reset():
    """Sequences beyond 65536 blocks are refused; the one-row low-precision
    fused selection is bounded at 2048 blocks per sequence; the workspace
    record reset is host only and rejects NULL."""
    L = msa.lib()
    with pytest.raises(msa.MsaError) as e:
        msa.msa_plan([1], [65536 * 128 + 1], 8, 2, 2, 2, topk=4, allocate=False)
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED and "65536" in str(e.value)
    ok = msa.msa_plan([1], [65536 * 128], 8, 2, 2, 2, topk=4, allocate=False)
    assert ok.nb_max == 65536
    a = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x20000)
    none = None
    long_row = msa.msa_plan([1, 1], [2049 * 128, 300], 8, 2, 2, 1, topk=17, proxy_dtype="fp8", allocate=False)
    assert L.msa_proxy_topk_select(long_row.handle, a, a, a, a, a, 0, 2, a, ws, long_row.workspace_bytes, none) == \
        msa.MSA_ERR_UNSUPPORTED and b"2048" in L.msa_last_error()
    # one-row plans take topk above 17 (the wave-per-row selection)
    k30 = msa.msa_plan([1, 1], [5000, 300], 8, 2, 2, 1, topk=30, allocate=False)
    assert k30.nb_max == 40
    assert L.msa_workspace_reset(none, 16) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_workspace_reset(ws, 1 << 20) == msa.MSA_OK


def test_lowp_plans_reserve_the_refine_queue():
    """A multi-row plan with a low-precision proxy reserves 64 bytes per
    (row, group) for the exact re-scoring queue; a bf16 one does not."""
    b = msa.msa_plan([4096], [4096], 32, 8, 8, 1, topk=16, allocate=False)
    f = msa.msa_plan([4096], [4096], 32, 8, 8, 1, topk=16, proxy_dtype="fp8", allocate=False)
    assert f.workspace_bytes - b.workspace_bytes >= 4096 * 8 * 64


def test_run_prefill_refuses_inexact_low_precision_selection():
    """fp8 / MXFP4 proxies select exactly only through the fused call (the
    separate top-k ranks the matrix-core scores as given): run_prefill
    refuses the separate path for them on multi-row plans (before any
    device call)."""
    for dt in ("fp8", "mxfp4", "mxfp4_qk"):
        p = msa.msa_plan([300], [300], 8, 2, 2, 2, topk=18, proxy_dtype=dt, allocate=False)
        with pytest.raises(ValueError, match="fused"):
            msa.run_prefill(p, *([None] * 9), None, None)
    # bf16 proxies and one-query-row plans are not refused by this check
    assert msa.msa_plan([1, 1], [3000, 300], 8, 2, 2, 1, topk=18, proxy_dtype="fp8", allocate=False).one_row
