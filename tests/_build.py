"""Test helpers: build paged inputs from explicit float rows (no method arithmetic)."""
from __future__ import annotations

import numpy as np

from synthetic.gen import to_bf16_bits


def page_table(nbs, perm_seed=None, extra=0):
    used = int(sum(nbs))
    total = used + extra
    if perm_seed is None:
        perm = np.arange(total)
    else:
        perm = np.random.default_rng(perm_seed).permutation(total)
    return perm[:used].astype(np.int32), total


def paged_bits(rows_by_seq, page_size, kv_indices, num_pages, fill=0):
    """rows_by_seq[s]: uint16/uint8 bits [L_s, H, d] -> pool [N, H, B, d]."""
    H, d = rows_by_seq[0].shape[1:]
    pool = np.full((num_pages, H, page_size, d), fill, dtype=rows_by_seq[0].dtype)
    off = 0
    for rows in rows_by_seq:
        L = rows.shape[0]
        nb = -(-L // page_size)
        for b in range(nb):
            c = rows[b * page_size:min(L, (b + 1) * page_size)]
            pool[kv_indices[off + b], :, :c.shape[0]] = c.transpose(1, 0, 2)
        off += nb
    return pool


def bf16(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def rand_bf16(rng, shape, scale=1.0):
    return bf16(rng.standard_normal(shape).astype(np.float32) * scale)
