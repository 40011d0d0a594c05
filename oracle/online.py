"""Tiled online-softmax attention in float64 -- test infrastructure, not product code.

This follows the steps of Algorithm 1 ("FlashAttention-2 forward") in "ML-Triton, A
Multi-Level Compilation and Language Extension to Triton GPU Programming", section 2.5:
Q is taken one row block at a time; for each key/value block j the block of scores
Q.K_j^T is formed, the online softmax updates the running row max m and row sum l,
and the output accumulator gains P.V_j.  The running-sum update is the one derived
for "Long Softmax" (Puzzle 8 of "Triton学习", lorn3.bearblog.dev):

    sum' = sum * exp(m_old - m_new) + sum_j exp(x_j - m_new)

Readings of the parts the listing leaves open:
  * the blank step inside the loop is the output rescale ``O <- O * exp(m_old - m_new)``
    before adding ``P.V_j``; the division by ``l`` happens once after the loop
    (deferred normalisation).  ``normalize_each_step=True`` instead keeps the output
    normalised after every block, as the recurrence of Puzzle 9 "Simple
    FlashAttention" of the same blog does: ``z' = z * exp(m_old - m_new) * l_old / l_new
    + sum_j exp(s_j - m_new) / l_new * v_j``.  Both give the same function;
  * a key block in which some row sees no key (possible for causal blocks on the
    diagonal) leaves that row's max at -inf; the exponent's subtrahend is then taken
    as 0 and the rescale factor as 1 so that -inf - (-inf) never occurs;
  * with a causal mask, key blocks entirely after the last query of the row block are
    not visited at all.

Its purpose is to check, on the CPU, that this recurrence reproduces the plain
definition in :mod:`oracle.attention` at any block shape, ragged tails included.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["attention_forward_tiled"]


def attention_forward_tiled(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                            scale: float, block_m: int, block_n: int,
                            normalize_each_step: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Online-softmax attention over row blocks of ``block_m`` queries and key blocks of
    ``block_n`` keys, float64.  Same arguments and results as
    :func:`oracle.attention.attention_forward`."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if causal and Nq != Nk:
        raise ValueError("causal attention needs equal query and key lengths")
    o_all = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    lse_all = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for q0 in range(0, Nq, block_m):
                q1 = min(q0 + block_m, Nq)
                qi = np.arange(q0, q1)
                Qb = q[b, h, q0:q1]                                   # "Load Q"
                m = np.full(q1 - q0, -np.inf)
                l = np.zeros(q1 - q0)
                acc = np.zeros((q1 - q0, v.shape[3]))
                kv_end = min(Nk, q1) if causal else Nk
                for k0 in range(0, kv_end, block_n):
                    k1 = min(k0 + block_n, Nk)
                    kj = np.arange(k0, k1)
                    s = scale * (Qb @ k[b, h, k0:k1].T)               # "Compute QK"
                    if causal:
                        s = np.where(kj[None, :] <= qi[:, None], s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))              # running rowmax
                    sub = np.where(np.isneginf(m_new), 0.0, m_new)
                    p = np.exp(s - sub[:, None])
                    alpha = np.where(np.isneginf(m_new), 1.0, np.exp(m - sub))
                    l_new = alpha * l + p.sum(axis=1)                 # running rowsum
                    pv = p @ v[b, h, k0:k1]                           # "O += P*V_j"
                    if normalize_each_step:
                        with np.errstate(invalid="ignore", divide="ignore"):
                            ratio = np.where(l_new > 0, alpha * l / np.where(l_new > 0, l_new, 1.0), 0.0)
                            inv = np.where(l_new > 0, 1.0 / np.where(l_new > 0, l_new, 1.0), 0.0)
                        acc = acc * ratio[:, None] + pv * inv[:, None]
                    else:
                        acc = acc * alpha[:, None] + pv
                    m, l = m_new, l_new
                if normalize_each_step:
                    o_all[b, h, q0:q1] = acc
                else:
                    o_all[b, h, q0:q1] = acc / l[:, None]             # deferred 1/l
                lse_all[b, h, q0:q1] = m + np.log(l)
    return o_all, lse_all
