"""CPU model of the fused kernel's lazy exponent offset (the reading of the online softmax
that the kernel implements; "Triton学习", Puzzle 8 "Long Softmax" running max and sum;
"ML-Triton ...", section 2.5, Algorithm 1 loop), checked against the float64 oracle.

The model follows the kernel's per-tile steps in float32 for one query row: the first
tile sets the offset to its row max; later tiles exponentiate against the current
offset, and only when a lane's sum of those exponentials (each lane holds every other
group of 8 keys of a 32-key slab) exceeds the bound are the tile's scores taken again,
the offset moved to max(offset, tile max), O and l rescaled, and the tile exponentiated
again.  The output O / l and logsumexp offset + ln l must not depend on when (or whether)
the offset moved.  Inputs include logits that jump far above the offset (exp overflows to
inf in float32) and rows whose later keys are all far below it (exp underflows to 0)."""
import numpy as np
import pytest

import oracle

LOG2E = np.float32(1.4426950408889634)


def _lane_sums(p):
    # keys of a 32-key slab: lane half G holds keys 16(r>>3) + 8G + (r&7)
    idx = np.arange(p.size)
    half = (idx % 16) // 8
    return np.float32(p[half == 0].sum(dtype=np.float32)), np.float32(p[half == 1].sum(dtype=np.float32))


def lazy_offset_row(s, v, tile, limit):
    """One row: raw scores s [Nk] (float32, -inf where masked), values v [Nk, d]."""
    c2 = LOG2E   # scale folded into s already
    m = np.float32(-np.inf)
    acc = np.zeros(v.shape[1], np.float32)
    l = np.float32(0.0)
    moves = 0
    for t0 in range(0, s.size, tile):
        st = s[t0:t0 + tile].astype(np.float32)
        vt = v[t0:t0 + tile].astype(np.float32)

        def rebase():
            nonlocal m, acc, l
            m_new = np.float32(max(m, st.max()))
            alpha = np.float32(np.exp2((m - m_new) * c2)) if np.isfinite(m) else np.float32(0.0)
            acc = acc * alpha
            l = l * alpha
            m = m_new

        if not np.isfinite(m):
            rebase()
        with np.errstate(over="ignore"):
            p = np.exp2(st * c2 - m * c2).astype(np.float32)
        if max(_lane_sums(p)) > limit:            # a lane's sum is too large (or inf)
            rebase()
            moves += 1
            p = np.exp2(st * c2 - m * c2).astype(np.float32)
        l = l + p.sum(dtype=np.float32)
        acc = acc + (p[:, None] * vt).sum(axis=0, dtype=np.float32)
    return acc / l, float(m) + float(np.log(l)), moves


@pytest.mark.parametrize("limit", [2.0 ** 24, 2.0 ** 15, 2.0 ** 4])
@pytest.mark.parametrize("kind", ["normal", "climbing", "spikes", "falling"])
def test_lazy_offset_matches_the_oracle(kind, limit):
    rng = np.random.default_rng(["normal", "climbing", "spikes", "falling"].index(kind) * 100 + int(np.log2(limit)))
    n, d = 700, 64
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.uniform(-1, 1, (1, 1, n, d))
    if kind == "climbing":
        k *= (1 + 6 * np.arange(n) / n)[None, None, :, None]
        q = np.abs(q)
        k = np.abs(k)
    elif kind == "spikes":
        for j, g in ((50, 40.0), (300, 120.0), (650, 400.0)):
            k[0, 0, j] = g * q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0])   # logit q.k = g
    elif kind == "falling":
        k[0, 0, :32] = 200.0 * q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0])   # first tile far above the rest
    q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
    scale = 1.0
    s = (q32[0, 0, 0] @ k32[0, 0].T).astype(np.float32) * np.float32(scale)
    o, lse, moves = lazy_offset_row(s, v32[0, 0], 32, np.float32(limit))
    o_ref, l_ref = oracle.attention_forward(q32.astype(np.float64), k32.astype(np.float64),
                                            v32.astype(np.float64), causal=False, scale=scale)
    assert np.all(np.isfinite(o)) and np.isfinite(lse)
    # float32 arithmetic on logits of size up to ~|lse|: a few ulps of the logit
    tol = 1e-5 * max(1.0, abs(l_ref[0, 0, 0]))
    assert abs(lse - l_ref[0, 0, 0]) <= 4 * tol, (kind, limit, moves)
    assert np.max(np.abs(o - o_ref[0, 0, 0])) <= 1e-5, (kind, limit, moves)
    if kind == "spikes":
        assert moves >= 1          # the offset had to move (exp overflowed before it did)


def test_offset_never_moves_for_ordinary_rows():
    """With N(0,1) logits the first tile's max is never exceeded by 2^24 in exp2 units, so
    the offset set on the first tile stays (no tile is formed twice)."""
    rng = np.random.default_rng(5)
    s = rng.standard_normal(4096).astype(np.float32)
    v = rng.uniform(-1, 1, (4096, 64)).astype(np.float32)
    _, _, moves = lazy_offset_row(s, v, 32, np.float32(2.0 ** 24))
    assert moves == 0
