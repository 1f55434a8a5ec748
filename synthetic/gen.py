"""Seeded synthetic inputs for the MSA forward path.

This module only draws random numbers, rounds them to the storage formats
(bf16, OCP fp8 e4m3fn with a per-head scale) and scatters token rows into a
paged pool.  It holds none of the method's arithmetic (no scores, no
selection, no attention), so both the fp64 oracle and the HIP path can take
their inputs from it.

Recipe (the same for every workload):
  * RNG: numpy PCG64 seeded with SeedSequence([seed, stream]); one stream per
    tensor so that tensors do not depend on each other's sizes.
  * values are float32 standard normals drawn in logical order
    [sequence, token, head, dim]; only afterwards are K/V rows scattered into
    pages, so the values do not depend on the page table.
  * bf16: round-to-nearest-even from float32.
  * fp8 e4m3fn: per-head scale = amax|x| / 448 over that head's whole tensor,
    round-to-nearest-even, saturate at +-448.
  * MXFP4 (proxy K of the "mxfp4" proxy pair; its proxy q is fp8): per key row
    and run of 32 dims a shared E8M0 exponent X = floor(log2 amax) - 2 (2 is
    the largest E2M1 exponent), elements x / 2^X rounded to the nearest E2M1
    value (ties to the even code), saturating at +-6 -- the conversion the
    OCP microscaling specification gives.  Stored per (page, head) as one
    record: 128 rows of packed codes (even element in the low nibble), then
    128 rows of scale bytes.
  * the page table is a seeded permutation of the pool (or the identity);
    pool pages not used by any sequence, and page slots past kv_len in a
    sequence's last page, can be filled with NaN to catch stray reads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_PQ, STREAM_PK, STREAM_PAGES, STREAM_LOWRANK, STREAM_PICKS = range(8)

BF16 = "bf16"
FP8 = "fp8"
MXFP4 = "mxfp4"          # proxy pair: fp8 q, MXFP4 K
MXFP4_QK = "mxfp4_qk"    # proxy pair: MXFP4 q (68-byte rows), MXFP4 K


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_bits(x: np.ndarray, head_axis: int) -> tuple[np.ndarray, np.ndarray]:
    """float32 -> (OCP e4m3fn bit patterns uint8, per-head float32 scales).

    scale[h] = amax over head h / 448; values are divided by the scale, clamped
    to +-448 and rounded to nearest even.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    axes = tuple(a for a in range(x.ndim) if a != head_axis)
    amax = np.abs(x).max(axis=axes) if x.size else np.zeros(x.shape[head_axis], np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    y = np.clip(x / scale.reshape(shape), -448.0, 448.0).astype(np.float32)
    bits = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return bits, scale


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)   # codes 0..7


def to_mxfp4_rows(x: np.ndarray) -> np.ndarray:
    """float32 [..., d] -> uint8 [..., d/2 + d/32]: d/2 bytes of packed E2M1
    codes (element 2i in the low nibble of byte i), then d/32 E8M0 scales."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    blk = x.reshape(x.shape[:-1] + (d // 32, 32)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    e = np.frexp(amax)[1].astype(np.int64)           # amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
    X = np.clip(np.where(amax > 0, e - 1 - 2, 0), -127, 127)
    y = blk / np.ldexp(1.0, X)[..., None]
    mag = np.abs(y)
    lo = np.clip(np.searchsorted(E2M1_MAGNITUDES, mag, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo = mag - E2M1_MAGNITUDES[lo]
    dhi = E2M1_MAGNITUDES[hi] - mag
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = np.where(mag >= 6.0, 7, code).astype(np.uint8)
    code |= ((y < 0) & (code != 0)).astype(np.uint8) << 3
    code = code.reshape(x.shape[:-1] + (d,))
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return np.concatenate([packed, (X + 127).astype(np.uint8)], axis=-1)


def mxfp4_pool_to_records(pool: np.ndarray) -> np.ndarray:
    """[N, H, B, d/2 + d/32] per-row MXFP4 bytes -> [N, H, B*(d/2) + B*(d/32)]
    page records: all rows' codes, then all rows' scales."""
    N, H, B, w = pool.shape
    cb = w * 16 // 17
    return np.concatenate([pool[..., :cb].reshape(N, H, B * cb), pool[..., cb:].reshape(N, H, B * (w - cb))], axis=-1)


def store(x: np.ndarray, dtype: str, head_axis: int):
    if dtype == BF16:
        return to_bf16_bits(x), None
    if dtype == FP8:
        return to_e4m3fn_bits(x, head_axis)
    raise ValueError(dtype)


NAN_BF16 = np.uint16(0x7FC0)
NAN_E4M3 = np.uint8(0x7F)
NAN_MXFP4 = np.uint8(0xFF)         # as a scale byte: E8M0 NaN


@dataclasses.dataclass
class Workload:
    """Shape of one synthetic MSA workload."""
    name: str
    qo_lens: list
    kv_lens: list
    num_qo_heads: int
    num_kv_heads: int
    num_proxy_heads: int = 0          # = num_kv_heads for prefill; 0 for decode
    num_proxy_kv_heads: int = 0       # 1 or num_proxy_heads
    head_dim: int = 128
    page_size: int = 128
    topk: int = 16                    # slots per (row, group), local block included
    kv_dtype: str = BF16
    proxy_dtype: str = BF16
    page_table: str = "perm"          # "perm" | "identity"
    lowrank: int = 0                  # rank of the additive proxy component (0 = none)
    lowrank_c: float = 2.0 * math.sqrt(2.0)
    extra_pages: float = 0.0          # fraction of NaN-filled spare pool pages
    poison_tail: bool = False         # NaN in page slots past kv_len
    mode: str = "prefill"             # "prefill" | "decode"

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def proxy_sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def num_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def total_rows(self) -> int:
        return int(sum(self.qo_lens))

    def pages_per_seq(self) -> list:
        return [-(-int(L) // self.page_size) for L in self.kv_lens]


# The workloads the benchmark and the parity tests are built on (1-5: the
# configurations the measurements are quoted on; 6, 7: a decode step with its
# indexer pass, fp8 or MXFP4 proxy K; 8: the 32K prefill in MXFP4).
def workload(n: int, **over) -> Workload:
    if n == 1:
        w = Workload("prefill_1k_gqa4", [1024], [1024], 8, 2, 2, 2, topk=4, page_table="identity")
    elif n == 2:
        w = Workload("prefill_32k_gqa4", [32768], [32768], 32, 8, 8, 8, topk=16)
    elif n == 3:
        lens = [16384, 32768, 49152, 32768]
        w = Workload("prefill_varlen_128k_gqa8", lens, list(lens), 64, 8, 8, 8, topk=16, lowrank=8)
    elif n == 4:
        w = Workload("decode_fp8_b32_131k", [1] * 32, [131072] * 32, 64, 8, 0, 0, topk=17,
                     kv_dtype=FP8, mode="decode")
    elif n == 5:
        w = Workload("prefill_1m_fp8proxy", [1048576], [1048576], 32, 8, 8, 8, topk=16, proxy_dtype=FP8)
    elif n == 6:
        # a whole decode step: the 32 x 131072 fp8 decode plus its own indexer
        # pass (8 proxy heads, one shared fp8 proxy-K head, low-rank component
        # for a clear top-k)
        w = Workload("decode_step_b32_131k", [1] * 32, [131072] * 32, 64, 8, 8, 1, topk=17, kv_dtype=FP8,
                     proxy_dtype=FP8, lowrank=8, mode="decode")
    elif n == 7:
        # the same decode step with an MXFP4 proxy K (fp8 proxy q)
        w = Workload("decode_step_mxfp4_b32_131k", [1] * 32, [131072] * 32, 64, 8, 8, 1, topk=17, kv_dtype=FP8,
                     proxy_dtype=MXFP4, lowrank=8, mode="decode")
    elif n == 8:
        # the 32K prefill in MXFP4: proxy q and K, and the K/V pages
        w = Workload("prefill_32k_gqa4_mxfp4", [32768], [32768], 32, 8, 8, 8, topk=16, kv_dtype=MXFP4,
                     proxy_dtype=MXFP4_QK)
    else:
        raise ValueError(n)
    return dataclasses.replace(w, **over)


def seed_of(n: int) -> int:
    return 1000 + n


@dataclasses.dataclass
class Inputs:
    w: Workload
    kv_indices: np.ndarray                      # int32 [sum nb_s]
    q: np.ndarray                               # uint16 [T, H_q, d]
    k_pages: np.ndarray                         # uint16/uint8 [N, H_kv, B, d]
    v_pages: np.ndarray
    k_scale: Optional[np.ndarray] = None        # float32 [H_kv] (fp8)
    v_scale: Optional[np.ndarray] = None
    proxy_q: Optional[np.ndarray] = None        # [T, P, d]; MXFP4_QK: [T, P, d/2 + d/32] bytes
    proxy_k_pages: Optional[np.ndarray] = None  # [N, P_k, B, d]; MXFP4: [N, P_k, record bytes]
    proxy_q_scale: Optional[np.ndarray] = None  # float32 [P]
    proxy_k_scale: Optional[np.ndarray] = None  # float32 [P_k]
    kv_block_indexes: Optional[np.ndarray] = None  # int32 [T, H_kv, k] (decode picks)

    @property
    def num_pages(self) -> int:
        return self.k_pages.shape[0]


def _normals(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def _page_table(w: Workload, seed: int):
    nbs = w.pages_per_seq()
    used = int(sum(nbs))
    total = used + int(math.ceil(used * w.extra_pages))
    if w.page_table == "identity":
        perm = np.arange(total, dtype=np.int64)
    else:
        perm = rng(seed, STREAM_PAGES).permutation(total)
    return perm[:used].astype(np.int32), total


def _scatter_pages(rows_by_seq, w: Workload, kv_indices: np.ndarray, num_pages: int, nan_value, dtype_np):
    """rows_by_seq[s]: [kv_len_s, H, d] storage bits -> pool [N, H, B, d]."""
    H, d, B = rows_by_seq[0].shape[1], rows_by_seq[0].shape[2], w.page_size
    pool = np.full((num_pages, H, B, d), nan_value, dtype=dtype_np)
    off = 0
    for s, rows in enumerate(rows_by_seq):
        L = rows.shape[0]
        nb = -(-L // B)
        for b in range(nb):
            page = kv_indices[off + b]
            chunk = rows[b * B:min(L, (b + 1) * B)]
            pool[page, :, :chunk.shape[0], :] = chunk.transpose(1, 0, 2)
            if chunk.shape[0] < B and not w.poison_tail:
                pool[page, :, chunk.shape[0]:, :] = 0
        off += nb
    return pool


def make_inputs(w: Workload, seed: int) -> Inputs:
    """Build every input tensor of workload `w` from `seed` (see module doc)."""
    d, B = w.head_dim, w.page_size
    T = w.total_rows
    kv_indices, num_pages = _page_table(w, seed)
    nbs = w.pages_per_seq()

    q32 = _normals(rng(seed, STREAM_Q), (T, w.num_qo_heads, d))
    q = to_bf16_bits(q32)
    del q32

    def kv_rows(stream, H):
        g = rng(seed, stream)
        return [_normals(g, (int(L), H, d)) for L in w.kv_lens]

    def paged(stream, H, dtype):
        rows = kv_rows(stream, H)
        if dtype == MXFP4:
            bits = [to_mxfp4_rows(r) for r in rows]
            pool = _scatter_pages(bits, w, kv_indices, num_pages, NAN_MXFP4, np.uint8)
            return mxfp4_pool_to_records(pool), None
        if dtype == BF16:
            bits = [to_bf16_bits(r) for r in rows]
            scale = None
            nanv, npdt = NAN_BF16, np.uint16
        else:
            allr = np.concatenate(rows, axis=0) if len(rows) > 1 else rows[0]
            allbits, scale = to_e4m3fn_bits(allr, head_axis=1)
            splits = np.cumsum([r.shape[0] for r in rows])[:-1]
            bits = np.split(allbits, splits, axis=0)
            nanv, npdt = NAN_E4M3, np.uint8
        return _scatter_pages(bits, w, kv_indices, num_pages, nanv, npdt), scale

    k_pages, k_scale = paged(STREAM_K, w.num_kv_heads, w.kv_dtype)
    v_pages, v_scale = paged(STREAM_V, w.num_kv_heads, w.kv_dtype)
    inp = Inputs(w, kv_indices, q, k_pages, v_pages, k_scale, v_scale)

    if w.num_proxy_heads > 0:  # prefill, or a decode step that runs its own indexer pass
        P, Pk = w.num_proxy_heads, w.num_proxy_kv_heads
        pq32 = _normals(rng(seed, STREAM_PQ), (T, P, d))
        pk_rows = kv_rows(STREAM_PK, Pk)
        if w.lowrank:
            # Additive rank-r component: per proxy head an orthonormal basis
            # V_p (d x r); one latent per KV block for proxy_k and one latent
            # per token for proxy_q.  Gives block scores a clear top-k.
            g = rng(seed, STREAM_LOWRANK)
            basis = np.stack([np.linalg.qr(g.standard_normal((d, w.lowrank)))[0] for _ in range(P)]).astype(np.float32)
            c = np.float32(w.lowrank_c)
            u = g.standard_normal((T, P, w.lowrank), dtype=np.float32)
            pq32 += c * np.einsum("pdr,tpr->tpd", basis, u)
            for s, L in enumerate(w.kv_lens):
                wb = g.standard_normal((nbs[s], Pk, w.lowrank), dtype=np.float32)
                comp = c * np.einsum("pdr,bpr->bpd", basis[:Pk], wb)          # [nb, Pk, d]
                tok = np.repeat(comp, B, axis=0)[:int(L)]                      # [L, Pk, d]
                pk_rows[s] += tok
        if w.proxy_dtype == MXFP4_QK:
            pq_bits, pq_scale = to_mxfp4_rows(pq32), None
        else:
            pq_bits, pq_scale = store(pq32, FP8 if w.proxy_dtype == MXFP4 else w.proxy_dtype, head_axis=1)
        del pq32
        if w.proxy_dtype in (MXFP4, MXFP4_QK):
            pk_bits = [to_mxfp4_rows(r) for r in pk_rows]
            pk_scale, nanv, npdt = None, NAN_MXFP4, np.uint8
        elif w.proxy_dtype == BF16:
            pk_bits = [to_bf16_bits(r) for r in pk_rows]
            pk_scale, nanv, npdt = None, NAN_BF16, np.uint16
        else:
            allr = np.concatenate(pk_rows, axis=0) if len(pk_rows) > 1 else pk_rows[0]
            allbits, pk_scale = to_e4m3fn_bits(allr, head_axis=1)
            splits = np.cumsum([r.shape[0] for r in pk_rows])[:-1]
            pk_bits = np.split(allbits, splits, axis=0)
            nanv, npdt = NAN_E4M3, np.uint8
        inp.proxy_q, inp.proxy_q_scale = pq_bits, pq_scale
        inp.proxy_k_pages = _scatter_pages(pk_bits, w, kv_indices, num_pages, nanv, npdt)
        if w.proxy_dtype in (MXFP4, MXFP4_QK):
            inp.proxy_k_pages = mxfp4_pool_to_records(inp.proxy_k_pages)
        inp.proxy_k_scale = pk_scale
    if w.mode == "decode":
        inp.kv_block_indexes = decode_picks(w, seed)
    return inp


def decode_picks(w: Workload, seed: int) -> np.ndarray:
    """Seeded block picks for decode: per (sequence, KV head) `topk - 1` distinct
    blocks drawn from the ones before the last, plus the last (local) block,
    ascending.  int32 [batch, H_kv, topk]; -1 pads when too few blocks exist."""
    g = rng(seed, STREAM_PICKS)
    k = w.topk
    out = np.full((w.num_seqs, w.num_kv_heads, k), -1, dtype=np.int32)
    for s, nb in enumerate(w.pages_per_seq()):
        for h in range(w.num_kv_heads):
            n = min(k - 1, nb - 1)
            picks = np.sort(g.choice(nb - 1, size=n, replace=False)) if n > 0 else np.zeros(0, np.int64)
            sel = np.concatenate([picks, [nb - 1]]).astype(np.int32)
            out[s, h, :sel.size] = sel
    return out
