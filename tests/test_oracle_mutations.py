"""Plant plausible mistakes in the oracle's arithmetic, on the CPU, and check that the
pins reject each of them.  This shows the pins are strong enough to notice a dropped
term, a wrong sign or index, a transposed operand or a wrong mask."""
import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import pins


def _mutant(kind):
    def rows_one_head(q, k, v, rows, causal, scale):
        sc = 1.0 if kind == "no_scale" else scale
        if kind == "transposed_scores":
            # s_ij taken as <k_i, q_j> instead of <q_i, k_j>
            s = sc * (k @ q.T)[rows] if len(k) == len(q) else sc * (q[rows] @ k.T)
        elif kind == "key_offset":
            s = sc * (q[rows] @ np.roll(k, 1, axis=0).T)
        else:
            s = sc * (q[rows] @ k.T)
        if causal:
            kj = np.arange(k.shape[0])[None, :]
            keep = {"mask_strict": kj < rows[:, None], "mask_flipped": kj >= rows[:, None]}.get(
                kind, kj <= rows[:, None])
            if kind == "mask_strict":
                keep = keep | (rows[:, None] == 0) & (kj == 0)   # keep row 0 finite
            fill = 0.0 if kind == "mask_zero_logit" else -np.inf
            s = np.where(keep, s, fill)
        m = s.max(axis=1)
        if kind == "no_max":
            m = np.zeros_like(m)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        vv = np.roll(v, 1, axis=0) if kind == "value_offset" else v
        o = p @ vv
        if kind != "no_normalise":
            o = o / l[:, None]
        if kind == "lse_no_max":
            lse = np.log(l)
        elif kind == "lse_log2":
            lse = m + np.log2(l)
        elif kind == "lse_unscaled_max":
            lse = m / sc + np.log(l)
        else:
            lse = m + np.log(l)
        if kind == "sign":
            o = -o
        return o, lse

    return rows_one_head


MUTANTS = ["no_scale", "transposed_scores", "key_offset", "mask_strict", "mask_flipped",
           "mask_zero_logit", "no_max", "value_offset", "no_normalise", "lse_no_max",
           "lse_log2", "lse_unscaled_max", "sign"]


def _fn(q, k, v, causal, scale):
    return oracle.attention_forward(q, k, v, causal=causal, scale=scale)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutant(kind, monkeypatch):
    monkeypatch.setattr(oa, "_rows_one_head", _mutant(kind))
    caught = []
    for check in (pins.check_golden, pins.check_invariants, pins.check_library, pins.check_bruteforce):
        try:
            with np.errstate(all="ignore"):
                check(_fn)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutation {kind!r} passed every pin"


def test_unmutated_passes(monkeypatch):
    # the harness itself: the real implementation passes all four checks
    for check in (pins.check_golden, pins.check_invariants):
        check(_fn)
