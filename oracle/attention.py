"""Two-pass softmax attention in float64 -- test infrastructure, not product code.

What is computed (per batch b, head h, query row i), following the definition of
attention as a softmax-weighted sum of value rows in "Triton学习" (lorn3.bearblog.dev),
Puzzle 9 "Simple FlashAttention", problem statement, and the output that Algorithm 1
("FlashAttention-2 forward") of "ML-Triton, A Multi-Level Compilation and Language
Extension to Triton GPU Programming", section 2.5, produces:

    s_ij   = scale * sum_c q_ic * k_jc                    (scaled logits)
    Vis(i) = {j : j <= i} if causal else all keys         (key j visible to query i)
    m_i    = max_{j in Vis(i)} s_ij                       (row max, for stability:
                                                           "Triton学习", Puzzle 8)
    l_i    = sum_{j in Vis(i)} exp(s_ij - m_i)
    O_i    = sum_{j in Vis(i)} exp(s_ij - m_i) * v_j / l_i
    lse_i  = m_i + ln(l_i)                                (natural log)

Readings where the pages are silent (each is listed in the design notes):
  * the pages' algorithm has no scale factor; ``scale`` multiplies Q.K^T inside the
    softmax and the workloads use 1/sqrt(d);
  * the causal rule is "key j visible to query i iff j <= i" with equal query and
    key lengths, so every row sees at least one key;
  * the pages keep the running max and sum but output no logsumexp; ``lse`` here is
    over the scaled logits, natural log;
  * keys outside the visible set contribute exactly zero weight (logit -inf), not
    the zero-padded logit the blog's puzzles use for out-of-range tiles.

Inputs are the exact values of the encoded tensors: float32 arrays, or bfloat16 bit
patterns stored as uint16 (decoded exactly by :func:`decode`).
"""
from __future__ import annotations

import concurrent.futures as _cf
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = ["decode", "attention_forward", "attention_rows"]

_ROW_CHUNK = 1024


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an encoded tensor.

    ``dtype == "bf16"``: ``x`` holds bfloat16 bit patterns (uint16); a bf16 value is
    the float32 whose upper 16 bits are the pattern and lower 16 bits are zero.
    ``dtype == "f16"``: ``x`` holds IEEE binary16 bit patterns (uint16): sign bit,
    5-bit exponent e (bias 15) and 10-bit fraction f; the value is
    (-1)^sign * 2^(e-15) * (1 + f/1024) for 0 < e < 31 and (-1)^sign * 2^-14 * f/1024
    for e = 0 (e = 31, inf/NaN, does not occur in the draws and decodes as inf/NaN).
    ``dtype == "f32"``: ``x`` holds float32 values.  ``dtype == "f64"``: as is.
    """
    if dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        u = np.ascontiguousarray(x, dtype=np.uint16).astype(np.int64)
        sign = np.where(u >> 15, -1.0, 1.0)
        e = (u >> 10) & 0x1F
        f = (u & 0x3FF).astype(np.float64)
        normal = sign * np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
        sub = sign * np.ldexp(f / 1024.0, -14)
        special = np.where(f == 0, sign * np.inf, np.nan)
        return np.where(e == 0, sub, np.where(e == 31, special, normal))
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rows_one_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   causal: bool, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """O and lse for query rows ``rows`` of one (batch, head), float64.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv]; rows: int array of query indices.
    """
    s = scale * (q[rows] @ k.T)                      # [R, Nk] scaled logits
    if causal:
        key_idx = np.arange(k.shape[0])[None, :]
        s = np.where(key_idx <= rows[:, None], s, -np.inf)
    m = s.max(axis=1)                                # finite: every row sees key 0
    p = np.exp(s - m[:, None])                       # masked entries -> exp(-inf) = 0
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                      scale: float, threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of float64 ``q [B,H,Nq,d]``, ``k [B,H,Nk,d]``, ``v [B,H,Nk,dv]``.

    Returns ``(O [B,H,Nq,dv], lse [B,H,Nq])`` in float64.  Causal masking requires
    ``Nq == Nk``.  Rows are processed in chunks of at most 1024 to bound memory;
    ``threads > 1`` runs independent (batch, head, chunk) items on a thread pool.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape[:2] != (B, H) or k.shape[3] != d or v.shape[2] != k.shape[2]:
        raise ValueError("shape mismatch between q, k, v")
    Nk = k.shape[2]
    if causal and Nq != Nk:
        raise ValueError("causal attention needs equal query and key lengths")
    if Nk < 1:
        raise ValueError("need at least one key")
    o = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)

    def work(item):
        b, h, r0 = item
        rows = np.arange(r0, min(r0 + _ROW_CHUNK, Nq))
        o[b, h, rows], lse[b, h, rows] = _rows_one_head(q[b, h], k[b, h], v[b, h], rows, causal, scale)

    items = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, Nq, _ROW_CHUNK)]
    if threads <= 1:
        for it in items:
            work(it)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, items))
    return o, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool, scale: float,
                   picks: Sequence[Tuple[int, int, int]], dtype: str = "f64"
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """O and lse for selected ``(b, h, i)`` query rows only.

    ``q, k, v`` may be encoded (``dtype`` "bf16" / "f16" / "f32") full-size tensors; only the
    heads that are picked are decoded.  Returns ``(O [P, dv], lse [P])`` float64 in
    the order of ``picks``.  Used to check outputs of workloads too large to
    evaluate whole on the CPU.
    """
    picks = [tuple(int(t) for t in p) for p in picks]
    out_o = np.empty((len(picks), v.shape[3]), dtype=np.float64)
    out_l = np.empty((len(picks),), dtype=np.float64)
    by_head = {}
    for n, (b, h, i) in enumerate(picks):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), lst in by_head.items():
        qh, kh, vh = decode(q[b, h], dtype), decode(k[b, h], dtype), decode(v[b, h], dtype)
        if causal and qh.shape[0] != kh.shape[0]:
            raise ValueError("causal attention needs equal query and key lengths")
        rows = np.array([i for _, i in lst], dtype=np.int64)
        o, l = _rows_one_head(qh, kh, vh, rows, causal, scale)
        for r, (n, _) in enumerate(lst):
            out_o[n] = o[r]
            out_l[n] = l[r]
    return out_o, out_l
