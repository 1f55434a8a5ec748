"""Plain fp64 CPU oracle of the MSA (MiniMax Sparse Attention) forward path.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path
in block_sparse_top_amd/ and neither side imports the other.

Everything is written as the plain definition, in float64, from the exact
stored bytes (bf16 bits -> float; fp8 e4m3fn bits -> table value x fp32
per-head scale; MXFP4 records -> E2M1 table value x E8M0 block scale).  Sources (the pages):

  [README]  "MiniMax-AI/MSA" README (pigsec.cn mirror), section "Usage": a
            dense proxy pass over a cheap query slice returns a per-block max
            score; `sparse_topk_select` turns the scores into KV block indexes
            (`topk` of them, bounded by the number of valid pages); the sparse
            plan uses the same `topk` as its `kv_block_num`; attention then
            runs on the selected blocks of the paged K/V.  k_pages.shape[1] is
            the number of KV heads, so pages are [page, head, slot, dim].
  [NEWS]    "MSA; MiniMax sparse attention kernels for SM100 GPUs"
            (news.ditty.ir), the paragraph on the three-step flow: the cheap
            pass computes the highest score of each block.
  [FLASH]   "Flash-MSA: open kernels for training sparse-attention models on
            millions of tokens" (iitog.ru), the paragraph comparing MSA with
            DSA (128-token blocks picked by max-pooling proxy scores; GQA main
            attention; each proxy head picks its own blocks for its group) and
            the paragraph on the forward kernels (each token's local block is
            always visible, like a sliding window).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * a "score" is the scaled proxy logit proxy_sm_scale * q.k (no softmax);
  * `topk` counts slots including the forced local block;
  * ties go to the lower block index; output ascending, padded with -1;
  * a query row i of a sequence sits at position kv_len - qo_len + i
    (bottom-right causal alignment); key j is visible iff j <= pos and
    j < kv_len (the diagonal key counts);
  * proxy head p drives KV group p; with one proxy-K head it is shared.

Parity pins live in tests/test_oracle_*.py.  Parity unpinned: the absolute
scale of the exported max scores beyond the scaled-logit reading (only the
selection is invariant to it) and the 16-versus-17-slot reading of the decode
workload.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP8 = "fp8"
# Proxy pair with an MXFP4 proxy K (the low-precision block-score indexer of
# the README's "Stacks" / package list, in the microscaling FP4 format that
# gfx950 matrix cores consume): proxy q is fp8 e4m3fn with per-head scales,
# proxy K pages hold MXFP4 records (see mxfp4_record_rows).
MXFP4 = "mxfp4"
# Proxy pair with both proxy q and proxy K in MXFP4 (q rows of 64 code bytes
# then 4 scale bytes, see mxfp4_q_rows).
MXFP4_QK = "mxfp4_qk"


# ----------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the bf16 value is the float32
    whose top 16 bits are these and whose low 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3fn_value(byte: int) -> float:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities), from its definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; max finite 448."""
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (-6)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(bits, dtype=np.uint8)]


def _e2m1_value(code: int) -> float:
    """OCP MX 4-bit float E2M1, from its definition: 1 sign bit (bit 3), 2
    exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal
    (m/2 * 2^0); no infinities or NaN; largest magnitude 6."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * (m / 2.0)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP MX shared scale E8M0: an unsigned biased exponent, 2^(code - 127);
    code 255 is NaN."""
    b = np.asarray(bits, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


MXFP4_BLOCK = 32            # elements sharing one E8M0 scale


def mxfp4_record_rows(rec: np.ndarray, slots) -> np.ndarray:
    """Decode key rows from MXFP4 page records (one record per page and head).

    A record of a 128-slot page with head dim d holds first 128 * d/2 bytes of
    E2M1 codes, slot-major, element 2i of a row in the low nibble of its byte
    i and element 2i+1 in the high nibble; then 128 * d/32 E8M0 scale bytes,
    slot-major, byte c scaling elements 32c .. 32c+31 of that slot.  rec is
    uint8 [n, record bytes] (one record per requested slot), slots [n];
    returns float64 [n, d]: code value x 2^(scale - 127)."""
    rec = np.asarray(rec, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    n = rec.shape[0]
    d = rec.shape[1] * 32 // (128 * 17)           # record = 128 * (d/2 + d/32) bytes
    cb, sb = d // 2, d // MXFP4_BLOCK
    codes = rec[:, :128 * cb].reshape(n, 128, cb)[np.arange(n), slots]          # [n, d/2]
    scales = rec[:, 128 * cb:128 * (cb + sb)].reshape(n, 128, sb)[np.arange(n), slots]  # [n, d/32]
    nib = np.empty((n, d), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    return E2M1_TABLE[nib] * np.repeat(e8m0_to_f64(scales), MXFP4_BLOCK, axis=1)


def mxfp4_q_rows(rows: np.ndarray) -> np.ndarray:
    """Decode MXFP4 proxy q rows: uint8 [..., d/2 + d/32] (the d/2 code bytes,
    element 2i in the low nibble of byte i, then the d/32 E8M0 scale bytes,
    byte c scaling elements 32c .. 32c+31) -> float64 [..., d]."""
    rows = np.asarray(rows, dtype=np.uint8)
    d = rows.shape[-1] * 32 // 17
    cb = d // 2
    codes, scales = rows[..., :cb], rows[..., cb:]
    nib = np.empty(rows.shape[:-1] + (d,), dtype=np.uint8)
    nib[..., 0::2] = codes & 0xF
    nib[..., 1::2] = codes >> 4
    return E2M1_TABLE[nib] * np.repeat(e8m0_to_f64(scales), MXFP4_BLOCK, axis=-1)


def dequant_proxy_q(bits: np.ndarray, proxy_dtype: str, scale=None) -> np.ndarray:
    """Proxy q [..., P, ...] stored bits -> float64 values for each proxy pair
    dtype (the MXFP4 pair's q is fp8; MXFP4_QK's q is MXFP4 rows)."""
    if proxy_dtype == MXFP4_QK:
        return mxfp4_q_rows(bits)
    return dequant(bits, FP8 if proxy_dtype == MXFP4 else proxy_dtype, scale, head_axis=1)


def dequant(bits: np.ndarray, dtype: str, scale=None, head_axis: int = 1) -> np.ndarray:
    """Stored bits -> float64 values; fp8 values are multiplied by the fp32
    per-head scale (in float64)."""
    if dtype == BF16:
        return bf16_to_f64(bits)
    if dtype == FP8:
        v = e4m3fn_to_f64(bits)
        shape = [1] * v.ndim
        shape[head_axis] = -1
        return v * np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(shape)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Sequence layout (re-derived here; the HIP path has its own planner)
# ----------------------------------------------------------------------------
class Layout:
    """Row and page bookkeeping of a varlen batch.

    Rows of all sequences are concatenated (sequence s owns rows
    row_start[s] .. row_start[s] + qo_len[s]); sequence s owns the
    ceil(kv_len / page_size) entries of the flat page table that start at
    page_start[s] ([README] "Usage": the page table is one flat list and the
    plan is built from the per-sequence lengths)."""

    def __init__(self, qo_lens, kv_lens, page_size: int):
        self.qo = [int(x) for x in qo_lens]
        self.kv = [int(x) for x in kv_lens]
        self.B = int(page_size)
        self.nb = [-(-L // self.B) for L in self.kv]
        self.row_start = np.concatenate([[0], np.cumsum(self.qo)]).astype(np.int64)
        self.page_start = np.concatenate([[0], np.cumsum(self.nb)]).astype(np.int64)
        self.T = int(self.row_start[-1])

    def seq_of_row(self, r: int) -> int:
        return int(np.searchsorted(self.row_start, r, side="right") - 1)

    def pos(self, r: int) -> int:
        """Absolute KV position of query row r (bottom-right alignment)."""
        s = self.seq_of_row(r)
        i = r - int(self.row_start[s])
        return self.kv[s] - self.qo[s] + i

    def local(self, r: int) -> int:
        return self.pos(r) // self.B


def gather_rows(pages_bits, dtype, scale, kv_indices, lay: Layout, s: int, head: int, key_idx) -> np.ndarray:
    """Logical key rows `key_idx` of sequence s, KV head `head` -> float64 [n, d].
    Key j lives in page kv_indices[page_start[s] + j // B], slot j % B."""
    key_idx = np.asarray(key_idx, dtype=np.int64)
    pages = np.asarray(kv_indices, dtype=np.int64)[lay.page_start[s] + key_idx // lay.B]
    if dtype in (MXFP4, MXFP4_QK):      # pool [N, heads, record bytes]; no per-head scale
        return mxfp4_record_rows(pages_bits[pages, head], key_idx % lay.B)
    raw = pages_bits[pages, head, key_idx % lay.B, :]
    if dtype == BF16:
        return bf16_to_f64(raw)
    if dtype == FP8:
        return e4m3fn_to_f64(raw) * np.float64(np.float32(np.asarray(scale)[head]))
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# O1: proxy block max scores
# ----------------------------------------------------------------------------
def proxy_block_maxscore(proxy_q, proxy_k_pages, kv_indices, qo_lens, kv_lens, page_size, proxy_sm_scale,
                         proxy_dtype=BF16, proxy_q_scale=None, proxy_k_scale=None, rows=None):
    """Per-block max of the scaled proxy logits ([NEWS] three-step flow;
    [README] "Usage", `output_maxscore`; [FLASH] max-pooling over proxy scores).

      ms[r, p, b] = max over keys j of block b with j <= pos(r), j < kv_len of
                    proxy_sm_scale * <pq[r, p], pk[j, pk_head(p)]>

    pk_head(p) = p when there are as many proxy-K heads as proxy heads, else 0.
    Blocks with no visible key give -inf; blocks after the row's local block
    are not defined and returned as NaN.  With proxy_dtype MXFP4 the proxy q
    is fp8 (scaled by proxy_q_scale) and the proxy K rows are decoded from
    MXFP4 records (proxy_k_scale unused); with MXFP4_QK the proxy q rows are
    MXFP4 too (no per-head scales).

    Returns float64 [len(rows), P, nb_max].
    """
    lay = Layout(qo_lens, kv_lens, page_size)
    rows = np.arange(lay.T) if rows is None else np.asarray(rows, dtype=np.int64)
    T, P, d = proxy_q.shape
    Pk = proxy_k_pages.shape[1]
    B = lay.B
    nb_max = max(lay.nb)
    out = np.full((rows.size, P, nb_max), np.nan)
    pq_all = None
    for s in range(len(lay.kv)):
        sel = np.nonzero((rows >= lay.row_start[s]) & (rows < lay.row_start[s + 1]))[0]
        if sel.size == 0:
            continue
        L = lay.kv[s]
        keys = np.arange(L)
        for p in range(P):
            ph = p if Pk == P else 0
            K = gather_rows(proxy_k_pages, proxy_dtype, proxy_k_scale, kv_indices, lay, s, ph, keys)  # [L, d]
            for c0 in range(0, sel.size, 256):
                idx = sel[c0:c0 + 256]
                r = rows[idx]
                qv = dequant_proxy_q(proxy_q[r, p:p + 1, :], proxy_dtype,
                                     None if proxy_q_scale is None else np.asarray(proxy_q_scale)[p:p + 1])[:, 0, :]
                S = proxy_sm_scale * (qv @ K.T)                               # [n, L]
                pos = np.array([lay.pos(int(x)) for x in r])
                S[keys[None, :] > pos[:, None]] = -np.inf
                nbs = lay.nb[s]
                Sp = np.full((idx.size, nbs * B), -np.inf)
                Sp[:, :L] = S
                ms = Sp.reshape(idx.size, nbs, B).max(axis=2)                 # [n, nb_s]
                loc = pos // B
                ms[np.arange(nbs)[None, :] > loc[:, None]] = np.nan
                out[idx, p, :nbs] = ms
    return out


# ----------------------------------------------------------------------------
# O2: top-k block selection
# ----------------------------------------------------------------------------
def topk_select_row(scores: np.ndarray, local: int, k: int) -> np.ndarray:
    """Selection for one (row, group) ([README] "Usage", `sparse_topk_select`
    with `topk` slots; [FLASH] forward-kernel paragraph: the local block is
    always kept).

    Competing blocks are the fully visible ones before the local block.  The
    k - 1 best of them by score (ties: lower block index first) join the
    local block.  Output ascending, padded with -1 to k entries.
    """
    cand = np.arange(local)
    R = min(k - 1, local)
    if R > 0:
        order = np.lexsort((cand, -scores[:local]))     # primary: score desc, then index asc
        chosen = cand[order[:R]]
    else:
        chosen = np.zeros(0, dtype=np.int64)
    sel = np.sort(np.concatenate([chosen, [local]]))
    out = np.full(k, -1, dtype=np.int32)
    out[:sel.size] = sel
    return out


def topk_select(max_score, qo_lens, kv_lens, page_size, topk, rows=None):
    """Apply topk_select_row to every (row, group).  max_score is indexed
    [i, p, b] for the i-th entry of `rows` (all rows by default).
    Returns int32 [len(rows), P, topk]."""
    lay = Layout(qo_lens, kv_lens, page_size)
    rows = np.arange(lay.T) if rows is None else np.asarray(rows, dtype=np.int64)
    n, P, _ = max_score.shape
    out = np.empty((n, P, topk), dtype=np.int32)
    for i, r in enumerate(rows):
        loc = lay.local(int(r))
        for p in range(P):
            out[i, p] = topk_select_row(max_score[i, p], loc, topk)
    return out


# ----------------------------------------------------------------------------
# O3 / O4: block-sparse GQA attention (prefill and decode)
# ----------------------------------------------------------------------------
def sparse_attention(q, k_pages, v_pages, kv_indices, kv_block_indexes, qo_lens, kv_lens, page_size, sm_scale,
                     kv_dtype=BF16, k_scale=None, v_scale=None, rows=None):
    """Softmax attention of each query row over the keys of its group's
    selected blocks ([README] "Usage": attention over the selected blocks of
    the paged K/V; [FLASH] GQA main attention, one block set per group).

    For row r, query head h, group g = h // (H_q / H_kv):
      K(r, g) = { j : j // B in S(r, g), j <= pos(r), j < kv_len }
      s_j = sm_scale * <q[r, h], k[j, g]>
      o   = sum_j exp(s_j - M) v[j, g] / sum_j exp(s_j - M),   M = max_j s_j
      lse = M + log sum_j exp(s_j - M)
    S(r, g) is kv_block_indexes[r, g, :] with -1 entries ignored.  A decode
    step is the case qo_len = 1.

    Returns (out float64 [len(rows), H_q, d], lse float64 [len(rows), H_q]).
    """
    lay = Layout(qo_lens, kv_lens, page_size)
    rows = np.arange(lay.T) if rows is None else np.asarray(rows, dtype=np.int64)
    T, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    B = lay.B
    out = np.zeros((rows.size, Hq, d))
    lse = np.zeros((rows.size, Hq))
    for i, r in enumerate(rows):
        r = int(r)
        s = lay.seq_of_row(r)
        pos = lay.pos(r)
        L = lay.kv[s]
        qv = bf16_to_f64(q[r])                                             # [H_q, d]
        for g in range(Hkv):
            blocks = sorted(set(int(b) for b in kv_block_indexes[r, g] if b >= 0))
            keys = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks]) if blocks else np.zeros(0, np.int64)
            keys = keys[(keys <= pos) & (keys < L)]
            K = gather_rows(k_pages, kv_dtype, k_scale, kv_indices, lay, s, g, keys)
            V = gather_rows(v_pages, kv_dtype, v_scale, kv_indices, lay, s, g, keys)
            for h in range(g * G, (g + 1) * G):
                sc = sm_scale * (K @ qv[h])
                M = sc.max()
                w = np.exp(sc - M)
                out[i, h] = (w @ V) / w.sum()
                lse[i, h] = M + np.log(w.sum())
    return out, lse


def sparse_attention_backward(q, k_pages, v_pages, kv_indices, kv_block_indexes, qo_lens, kv_lens, page_size, sm_scale,
                              dout, rows=None, groups=None):
    """Gradients of the block-sparse attention above ([FLASH] the training
    kernels: the selection is computed once in the forward pass and reused,
    so the backward runs over the same cached blocks) for bf16 q, K, V and an
    upstream gradient dout [T, H_q, d] (bf16 bits).

    For row r, head h, group g and the keys K(r, g) of the forward:
      p_j  = softmax_j(s_j),  s_j = sm_scale <q[r,h], k_j>,  o = sum_j p_j v_j
      dv_j += p_j dout[r,h]
      dp_j  = <dout[r,h], v_j>,   D = <dout[r,h], o>
      ds_j  = p_j (dp_j - D)
      dq[r,h] = sm_scale sum_j ds_j k_j
      dk_j   += sm_scale ds_j q[r,h]
    dk and dv are accumulated per (page, KV head, slot) of the paged pools.

    Returns (dq float64 [T, H_q, d], dk float64, dv float64 shaped like the
    page pools); pool slots no row attends to stay 0.  With `rows`, only those
    rows are visited: their dq rows are exact, dk and dv then hold only their
    contributions.  With `groups`, only those KV groups (and their G query
    heads) are visited; the other heads' dq and the other groups' dk, dv stay 0.
    """
    lay = Layout(qo_lens, kv_lens, page_size)
    T, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    B = lay.B
    dq = np.zeros((T, Hq, d))
    dk = np.zeros(k_pages.shape[:2] + (B, d))
    dv = np.zeros(v_pages.shape[:2] + (B, d))
    kvi = np.asarray(kv_indices, dtype=np.int64)
    for r in (range(T) if rows is None else [int(x) for x in rows]):
        s = lay.seq_of_row(r)
        pos = lay.pos(r)
        L = lay.kv[s]
        qv = bf16_to_f64(q[r])
        dov = bf16_to_f64(dout[r])
        for g in (range(Hkv) if groups is None else [int(x) for x in groups]):
            blocks = sorted(set(int(b) for b in kv_block_indexes[r, g] if b >= 0))
            keys = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks]) if blocks else np.zeros(0, np.int64)
            keys = keys[(keys <= pos) & (keys < L)]
            K = gather_rows(k_pages, BF16, None, kv_indices, lay, s, g, keys)
            V = gather_rows(v_pages, BF16, None, kv_indices, lay, s, g, keys)
            pages = kvi[lay.page_start[s] + keys // B]
            slots = keys % B
            for h in range(g * G, (g + 1) * G):
                sc = sm_scale * (K @ qv[h])
                w = np.exp(sc - sc.max())
                p = w / w.sum()
                o = p @ V
                dp = V @ dov[h]
                ds = p * (dp - dov[h] @ o)
                dq[r, h] = sm_scale * (ds @ K)
                np.add.at(dv, (pages, g, slots), p[:, None] * dov[h][None, :])
                np.add.at(dk, (pages, g, slots), sm_scale * ds[:, None] * qv[h][None, :])
    return dq, dk, dv


def proxy_kl_backward(proxy_q, proxy_k_pages, q, k_pages, kv_indices, kv_block_indexes, qo_lens, kv_lens, page_size,
                      sm_scale, proxy_sm_scale, grad_scale=1.0, rows=None, groups=None):
    """Gradient of the proxy's distillation loss with respect to the bf16
    proxy q and proxy K ([FLASH] the backward paragraph: the KL divergence
    between the proxy's and the main attention's distributions, whose gradient
    with respect to a proxy score is the proxy probability minus the main
    probability).

    Readings where the pages are silent: for row r and group g (driven by
    proxy head g, as in the forward)
      p_proxy_j = softmax over the row's visible keys j (j <= pos, j < kv_len)
                  of z_j = proxy_sm_scale <pq[r, g], pk[j, g]>   (dense proxy)
      p_main_j  = mean over the group's G heads h of the main attention
                  probability softmax_j(sm_scale <q[r, h], k[j, g]>) over the
                  selected visible keys K(r, g), and 0 on every other key
      loss      = grad_scale * sum over (r, g) of KL(p_main || p_proxy),
    with p_main a fixed target (no gradient flows into the main attention).
    Then dloss/dz_j = grad_scale (p_proxy_j - p_main_j) and
      dpq[r, g]  = proxy_sm_scale sum_j dz_j pk[j, g]
      dpk[j, g] += proxy_sm_scale dz_j pq[r, g].

    Needs one proxy head and one proxy-K head per KV group.  Returns (dpq
    float64 [T, P, d], dpk float64 shaped like the proxy pool, kl float64 [T, P]
    (each (row, group)'s KL, without grad_scale), plse float64 [T, P] (natural
    log-sum-exp of z over the row's visible keys)).  `rows` and `groups` visit
    a subset as in sparse_attention_backward.
    """
    lay = Layout(qo_lens, kv_lens, page_size)
    T, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    P, Pk = proxy_q.shape[1], proxy_k_pages.shape[1]
    if P != Hkv or Pk != P:
        raise ValueError("one proxy head and one proxy-K head per KV group")
    B = lay.B
    dpq = np.zeros((T, P, d))
    dpk = np.zeros(proxy_k_pages.shape[:2] + (B, d))
    kl = np.zeros((T, P))
    plse = np.zeros((T, P))
    kvi = np.asarray(kv_indices, dtype=np.int64)
    for r in (range(T) if rows is None else [int(x) for x in rows]):
        s = lay.seq_of_row(r)
        pos = lay.pos(r)
        L = lay.kv[s]
        vis = np.arange(min(pos + 1, L))                      # the row's visible keys
        pages = kvi[lay.page_start[s] + vis // B]
        slots = vis % B
        qv = bf16_to_f64(q[r])
        for g in (range(Hkv) if groups is None else [int(x) for x in groups]):
            pq = bf16_to_f64(proxy_q[r, g])
            PK = gather_rows(proxy_k_pages, BF16, None, kv_indices, lay, s, g, vis)
            z = proxy_sm_scale * (PK @ pq)
            plse[r, g] = z.max() + np.log(np.sum(np.exp(z - z.max())))
            logpp = z - plse[r, g]
            pp = np.exp(logpp)
            blocks = set(int(b) for b in kv_block_indexes[r, g] if b >= 0)
            chosen = np.array([int(j) // B in blocks for j in vis], dtype=bool)
            K = gather_rows(k_pages, BF16, None, kv_indices, lay, s, g, vis[chosen])
            pm = np.zeros(vis.size)
            for h in range(g * G, (g + 1) * G):
                sc = sm_scale * (K @ qv[h])
                w = np.exp(sc - sc.max())
                pm[chosen] += w / w.sum() / G
            dz = grad_scale * (pp - pm)
            dpq[r, g] = proxy_sm_scale * (dz @ PK)
            np.add.at(dpk, (pages, g, slots), proxy_sm_scale * dz[:, None] * pq[None, :])
            on = pm > 0
            kl[r, g] = float(np.sum(pm[on] * (np.log(pm[on]) - logpp[on])))
    return dpq, dpk, kl, plse


def sparse_decode(q, k_pages, v_pages, kv_indices, kv_block_indexes, kv_lens, page_size, sm_scale,
                  kv_dtype=FP8, k_scale=None, v_scale=None, rows=None):
    """Paged sparse decode ([README] "Stacks": paged FP8 decode wrapper): one
    new query row per sequence, already in the cache, so pos = kv_len - 1."""
    return sparse_attention(q, k_pages, v_pages, kv_indices, kv_block_indexes, [1] * len(kv_lens), kv_lens,
                            page_size, sm_scale, kv_dtype, k_scale, v_scale, rows)


# ----------------------------------------------------------------------------
# Acceptance rule for a selection produced elsewhere
# ----------------------------------------------------------------------------
def check_selection_row(sel: np.ndarray, scores: np.ndarray, local: int, k: int, band: float = 1e-3):
    """Is `sel` an acceptable selection for a row whose fp64 block scores are
    `scores`?  Returns (ok, reason).

    The local block must be present, the set size must be min(k, local + 1),
    ids ascending, unique, <= local, -1 padded.  Let s_1 >= s_2 >= ... be the
    scores of the competing blocks and R = min(k - 1, local).  If
    s_R - s_{R+1} > band the competing part must equal the oracle's choice;
    otherwise every chosen competing block must score >= s_R - band.
    """
    sel = np.asarray(sel)
    valid = sel[sel >= 0]
    n = min(k, local + 1)
    if valid.size != n or np.any(sel[n:] != -1):
        return False, f"size {valid.size} != {n} or bad padding"
    if np.any(np.diff(valid) <= 0):
        return False, "not strictly ascending"
    if valid[-1] != local:
        return False, "local block missing"
    comp = valid[:-1]
    R = min(k - 1, local)
    if R == 0:
        return True, ""
    cs = np.sort(scores[:local])[::-1]
    sR = cs[R - 1]
    if R < local and cs[R - 1] - cs[R] > band:
        ref = topk_select_row(scores, local, k)
        if not np.array_equal(ref, sel):
            return False, "clear gap but different set"
        return True, ""
    if np.any(scores[comp] < sR - band):
        return False, "a chosen block scores below the band"
    return True, ""
