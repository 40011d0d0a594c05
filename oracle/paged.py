"""Attention over a paged key/value cache in float64 -- test infrastructure, not product code.

"ML-Triton, A Multi-Level Compilation and Language Extension to Triton GPU Programming",
section 3.2 (the paged-attention kernels of Figures 8 and 9) and section 4.3: a
request's key/value cache is cut into fixed-size blocks that need not be contiguous in
memory; a block table maps the request's logical blocks to physical ones, and the
attention itself is unchanged.  The pages fix no layout, block size or table format,
so this module takes these readings (each is listed in the design notes):

  * a pool holds ``num_blocks`` physical blocks, laid out ``[num_blocks, H, bs, d]``
    (every block holds ``bs`` consecutive keys of every head);
  * sequence b owns keys ``j = 0 .. seq_lens[b]-1``; key j lives in physical block
    ``block_table[b, j // bs]`` at row ``j % bs`` (for K and for V alike);
  * every query row of sequence b attends to all of its keys (no mask), with the
    plain definition of :mod:`oracle.attention`;
  * a sequence with no keys gives ``O = 0`` (the empty weighted sum) and
    ``lse = log 0 = -inf``.

Inputs are float64 arrays (decode encoded tensors with :func:`oracle.decode` first).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import _rows_one_head

__all__ = ["gather_keys", "paged_attention_forward"]


def gather_keys(pool: np.ndarray, block_table: np.ndarray, b: int, h: int, n_keys: int,
                block_size: int) -> np.ndarray:
    """Rows ``[n_keys, d]`` of head h of sequence b, key j from block
    ``block_table[b, j // block_size]``, row ``j % block_size``."""
    j = np.arange(n_keys)
    blocks = np.asarray(block_table)[b, j // block_size]
    return pool[blocks, h, j % block_size]


def paged_attention_forward(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                            block_table: np.ndarray, seq_lens: np.ndarray, *, scale: float
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """``q [B,H,Nq,d]`` against paged ``k_pool, v_pool [num_blocks,H,bs,d]``.

    ``block_table [B, max_blocks]`` int, ``seq_lens [B]`` int with
    ``0 <= seq_lens[b] <= max_blocks * bs`` and every used entry in
    ``[0, num_blocks)``.  Returns ``(O [B,H,Nq,d], lse [B,H,Nq])`` in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_pool = np.asarray(k_pool, dtype=np.float64)
    v_pool = np.asarray(v_pool, dtype=np.float64)
    block_table = np.asarray(block_table, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B, H, Nq, d = q.shape
    nb, Hp, bs, dk = k_pool.shape
    if Hp != H or dk != d or v_pool.shape[:3] != k_pool.shape[:3]:
        raise ValueError("pool shapes do not match q")
    if block_table.ndim != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block table or sequence lengths do not match the batch")
    o = np.zeros((B, H, Nq, v_pool.shape[3]), dtype=np.float64)
    lse = np.full((B, H, Nq), -np.inf, dtype=np.float64)
    rows = np.arange(Nq)
    for b in range(B):
        n_keys = int(seq_lens[b])
        if not 0 <= n_keys <= block_table.shape[1] * bs:
            raise ValueError(f"sequence {b}: {n_keys} keys do not fit its block table")
        if n_keys == 0:
            continue
        used = block_table[b, :(n_keys + bs - 1) // bs]
        if used.min() < 0 or used.max() >= nb:
            raise ValueError(f"sequence {b}: block table entry outside the pool")
        for h in range(H):
            kh = gather_keys(k_pool, block_table, b, h, n_keys, bs)
            vh = gather_keys(v_pool, block_table, b, h, n_keys, bs)
            o[b, h], lse[b, h] = _rows_one_head(q[b, h], kh, vh, rows, False, scale)
    return o, lse
