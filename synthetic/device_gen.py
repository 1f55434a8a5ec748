"""Seeded synthetic inputs generated on the GPU, for the full-size workloads
(the 1M-token prefill and the 32 x 131072 decode pool do not fit a CPU-side
generator's time budget).  Same recipe as synthetic.gen - standard normals
in logical [sequence, token, head, dim] order, bf16 round-to-nearest-even or
per-head e4m3fn with scale amax/448, scattered into a seeded permutation of
the page pool, low-rank proxy component - but drawn with torch's device
generator, so the values differ from the CPU generator's for the same seed.
No method arithmetic here.  Returns device tensors; `.to_host()` gives the
numpy view the oracle reads."""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from .gen import (Workload, STREAM_Q, STREAM_K, STREAM_V, STREAM_PQ, STREAM_PK, STREAM_LOWRANK, BF16, FP8, MXFP4, MXFP4_QK,
                  E2M1_MAGNITUDES,
                  rng as np_rng, decode_picks, _page_table)

CHUNK = 1 << 24  # elements per generation chunk


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, stream, 7]).generate_state(1)[0]))
    return g


@dataclasses.dataclass
class DeviceInputs:
    w: Workload
    kv_indices: torch.Tensor
    q: torch.Tensor
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    proxy_q: Optional[torch.Tensor] = None
    proxy_k_pages: Optional[torch.Tensor] = None
    proxy_q_scale: Optional[torch.Tensor] = None
    proxy_k_scale: Optional[torch.Tensor] = None
    kv_block_indexes: Optional[torch.Tensor] = None

    def as_dict(self):
        return {f.name: getattr(self, f.name) for f in dataclasses.fields(self) if f.name != "w"}


def _randn_rows(g, rows: int, H: int, d: int, device, extra=None):
    """float32 normals [rows, H, d] in chunks of rows; `extra(r0, x)` may add to a chunk."""
    per = max(1, CHUNK // (H * d))
    for r0 in range(0, rows, per):
        n = min(per, rows - r0)
        x = torch.randn((n, H, d), generator=g, device=device, dtype=torch.float32)
        if extra is not None:
            extra(r0, x)
        yield r0, x


def _store_rows(w: Workload, seed: int, stream: int, H: int, dtype: str, device, rows_per_seq, extra=None):
    """Draw the logical rows of every sequence and return ([rows per seq as storage], scale)."""
    d = w.head_dim
    if dtype == BF16:
        out = []
        g = _gen(seed, stream, device)
        for s, L in enumerate(rows_per_seq):
            t = torch.empty((L, H, d), dtype=torch.bfloat16, device=device)
            for r0, x in _randn_rows(g, L, H, d, device, None if extra is None else (lambda r0, x, s=s: extra(s, r0, x))):
                t[r0:r0 + x.shape[0]] = x.to(torch.bfloat16)
            out.append(t)
        return out, None
    # fp8: pass 1 per-head amax over every sequence, pass 2 quantise (same draws)
    amax = torch.zeros(H, dtype=torch.float32, device=device)
    g = _gen(seed, stream, device)
    for s, L in enumerate(rows_per_seq):
        for r0, x in _randn_rows(g, L, H, d, device, None if extra is None else (lambda r0, x, s=s: extra(s, r0, x))):
            amax = torch.maximum(amax, x.abs().amax(dim=(0, 2)))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    g = _gen(seed, stream, device)
    out = []
    for s, L in enumerate(rows_per_seq):
        t = torch.empty((L, H, d), dtype=torch.uint8, device=device)
        for r0, x in _randn_rows(g, L, H, d, device, None if extra is None else (lambda r0, x, s=s: extra(s, r0, x))):
            y = torch.clamp(x / scale[None, :, None], -448.0, 448.0)
            t[r0:r0 + x.shape[0]] = y.to(torch.float8_e4m3fn).view(torch.uint8)
        out.append(t)
    return out, scale


def _mxfp4_rows(x: torch.Tensor) -> torch.Tensor:
    """float32 [n, H, d] -> uint8 [n, H, d/2 + d/32], the MXFP4 row format of
    synthetic.gen.to_mxfp4_rows (same conversion, on the device)."""
    n, H, d = x.shape
    blk = x.reshape(n, H, d // 32, 32)
    amax = blk.abs().amax(dim=-1)
    X = torch.where(amax > 0, torch.frexp(amax)[1].to(torch.int32) - 3, torch.zeros_like(amax, dtype=torch.int32))
    X = X.clamp(-127, 127)
    y = torch.ldexp(blk, (-X).to(torch.float32)[..., None])
    mag = y.abs()
    grid = torch.tensor(E2M1_MAGNITUDES, dtype=torch.float32, device=x.device)
    lo = (torch.searchsorted(grid, mag.contiguous(), right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    dlo = mag - grid[lo]
    dhi = grid[hi] - mag
    code = torch.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = torch.where(mag >= 6.0, torch.full_like(code, 7), code)
    code = code | (((y < 0) & (code != 0)).to(code.dtype) << 3)
    code = code.to(torch.uint8).reshape(n, H, d)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return torch.cat([packed, (X + 127).to(torch.uint8)], dim=-1)


def _store_mxfp4_rows(w: Workload, seed: int, stream: int, H: int, device, rows_per_seq, extra=None):
    d = w.head_dim
    g = _gen(seed, stream, device)
    out = []
    for s, L in enumerate(rows_per_seq):
        t = torch.empty((L, H, d // 2 + d // 32), dtype=torch.uint8, device=device)
        for r0, x in _randn_rows(g, L, H, d, device, None if extra is None else (lambda r0, x, s=s: extra(s, r0, x))):
            t[r0:r0 + x.shape[0]] = _mxfp4_rows(x)
        out.append(t)
    return out


def _records(pool: torch.Tensor) -> torch.Tensor:
    """[N, H, B, d/2 + d/32] per-row MXFP4 bytes -> [N, H, record bytes] page
    records (all rows' codes, then all rows' scales)."""
    N, H, B, wd = pool.shape
    cb = wd * 16 // 17
    return torch.cat([pool[..., :cb].reshape(N, H, B * cb), pool[..., cb:].reshape(N, H, B * (wd - cb))],
                     dim=-1).contiguous()


def _scatter(rows, w: Workload, kv_indices: torch.Tensor, num_pages: int, device):
    H, d = rows[0].shape[1], rows[0].shape[2]
    B = w.page_size
    pool = torch.zeros((num_pages, H, B, d), dtype=rows[0].dtype, device=device)
    off = 0
    for t in rows:
        L = t.shape[0]
        nb = -(-L // B)
        full = L // B
        if full:
            pool[kv_indices[off:off + full].long()] = t[:full * B].view(full, B, H, d).permute(0, 2, 1, 3)
        if nb > full:
            tail = t[full * B:]
            pool[int(kv_indices[off + full]), :, :tail.shape[0]] = tail.permute(1, 0, 2)
        off += nb
    return pool


def make_inputs_device(w: Workload, seed: int, device="cuda", picks_sets: int = 1) -> DeviceInputs:
    d, B = w.head_dim, w.page_size
    kv_np, num_pages = _page_table(w, seed)
    kv_indices = torch.from_numpy(kv_np).to(device)
    T = w.total_rows
    gq = _gen(seed, STREAM_Q, device)
    q = torch.empty((T, w.num_qo_heads, d), dtype=torch.bfloat16, device=device)
    for r0, x in _randn_rows(gq, T, w.num_qo_heads, d, device):
        q[r0:r0 + x.shape[0]] = x.to(torch.bfloat16)
    lens = [int(L) for L in w.kv_lens]

    def paged(stream):
        if w.kv_dtype == MXFP4:
            rows = _store_mxfp4_rows(w, seed, stream, w.num_kv_heads, device, lens)
            return _records(_scatter(rows, w, kv_indices, num_pages, device)), None
        rows, sc = _store_rows(w, seed, stream, w.num_kv_heads, w.kv_dtype, device, lens)
        return _scatter(rows, w, kv_indices, num_pages, device), sc
    k_pages, ks = paged(STREAM_K)
    v_pages, vs = paged(STREAM_V)
    inp = DeviceInputs(w, kv_indices, q, k_pages, v_pages, ks, vs)
    if w.num_proxy_heads > 0:  # prefill, or a decode step that runs its own indexer pass
        P, Pk = w.num_proxy_heads, w.num_proxy_kv_heads
        add_q = add_k = None
        if w.lowrank:
            g = np_rng(seed, STREAM_LOWRANK)
            basis = torch.from_numpy(np.stack([np.linalg.qr(g.standard_normal((d, w.lowrank)))[0]
                                               for _ in range(P)]).astype(np.float32)).to(device)   # [P, d, r]
            c = float(w.lowrank_c)
            gl = _gen(seed, STREAM_LOWRANK, device)
            u = torch.randn((T, P, w.lowrank), generator=gl, device=device)
            wb = [torch.randn((-(-L // B), Pk, w.lowrank), generator=gl, device=device) for L in lens]

            def add_q(s, r0, x):
                n = x.shape[0]
                x += c * torch.einsum("pdr,tpr->tpd", basis, u[r0:r0 + n])

            def add_k(s, r0, x):
                n = x.shape[0]
                blk = (torch.arange(r0, r0 + n, device=device) // B)
                x += c * torch.einsum("pdr,tpr->tpd", basis[:Pk], wb[s][blk])
        if w.proxy_dtype == MXFP4_QK:
            pq_rows, pqs = _store_mxfp4_rows(w, seed, STREAM_PQ, P, device, [T], add_q), None
        else:
            pq_rows, pqs = _store_rows(w, seed, STREAM_PQ, P, FP8 if w.proxy_dtype == MXFP4 else w.proxy_dtype,
                                       device, [T], add_q)
        inp.proxy_q, inp.proxy_q_scale = pq_rows[0], pqs
        if w.proxy_dtype in (MXFP4, MXFP4_QK):
            pk_rows = _store_mxfp4_rows(w, seed, STREAM_PK, Pk, device, lens, add_k)
            inp.proxy_k_pages = _records(_scatter(pk_rows, w, kv_indices, num_pages, device))
            pks = None
        else:
            pk_rows, pks = _store_rows(w, seed, STREAM_PK, Pk, w.proxy_dtype, device, lens, add_k)
            inp.proxy_k_pages = _scatter(pk_rows, w, kv_indices, num_pages, device)
        inp.proxy_k_scale = pks
    if w.mode == "decode":
        inp.kv_block_indexes = torch.from_numpy(decode_picks(w, seed)).to(device)
    return inp


def to_host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Device tensor -> the numpy bit view the oracle reads (bf16 -> uint16, fp8 -> uint8)."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
