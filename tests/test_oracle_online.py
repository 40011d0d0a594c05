"""The tiled online-softmax recurrence (Algorithm 1 of the ML-Triton paper, section 2.5,
with the running-sum update of the blog's Long Softmax puzzle) reproduces the plain
definition at every block shape, including ragged tails and causal diagonal blocks.
CPU only."""
import math

import numpy as np
import pytest

import oracle
from tests import pins

SHAPES = [(1, 1), (2, 3), (16, 16), (128, 64), (64, 128), (5, 7)]


@pytest.mark.parametrize("bm,bn", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("normalize_each_step", [False, True])
def test_tiled_matches_definition(bm, bn, causal, normalize_each_step):
    B, H, N, d = 1, 2, 203, 8
    q, k, v = pins.rand_qkv(11, B, H, N, d, sigma=2.5)
    o_ref, l_ref = oracle.attention_forward(q, k, v, causal=causal, scale=1 / math.sqrt(d))
    o, l = oracle.attention_forward_tiled(q, k, v, causal=causal, scale=1 / math.sqrt(d),
                                          block_m=bm, block_n=bn,
                                          normalize_each_step=normalize_each_step)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(l - l_ref)) <= 1e-12


def test_tiled_passes_pins():
    fn = lambda q, k, v, causal, scale: oracle.attention_forward_tiled(
        q, k, v, causal=causal, scale=scale, block_m=4, block_n=3)
    pins.check_golden(fn)
    pins.check_invariants(fn)


def test_puzzle9_walkthrough():
    """The blog's Simple FlashAttention walk-through: scalar q, k, v (d = 1), key tiles of
    two.  After tile 1 the running values are m1, l1 and z1; after tile 2 the update
    l2 = l1*exp(m1-m2) + sum exp(s-m2) and z' = z*exp(m1-m2)*l1/l2 + sum exp(s-m2)/l2*v
    must equal the softmax over all four keys."""
    q = np.array([[[[0.5], [-1.0]]]])
    k = np.array([[[[1.0], [2.0], [4.0], [-3.0]]]])
    v = np.array([[[[1.0], [-2.0], [3.0], [0.5]]]])
    s = (q[0, 0] @ k[0, 0].T)                     # [2, 4]
    m1 = s[:, :2].max(1); l1 = np.exp(s[:, :2] - m1[:, None]).sum(1)
    z1 = (np.exp(s[:, :2] - m1[:, None]) @ v[0, 0, :2]) / l1[:, None]
    m2 = np.maximum(m1, s[:, 2:].max(1))
    l2 = l1 * np.exp(m1 - m2) + np.exp(s[:, 2:] - m2[:, None]).sum(1)
    z2 = z1 * (np.exp(m1 - m2) * l1 / l2)[:, None] + (np.exp(s[:, 2:] - m2[:, None]) @ v[0, 0, 2:]) / l2[:, None]
    o, l = oracle.attention_forward_tiled(q, k, v, causal=False, scale=1.0, block_m=2, block_n=2,
                                          normalize_each_step=True)
    assert np.max(np.abs(o[0, 0] - z2)) <= 1e-15
    assert np.max(np.abs(l[0, 0] - (m2 + np.log(l2)))) <= 1e-15
    w = np.exp(s - s.max(1, keepdims=True)); w /= w.sum(1, keepdims=True)
    assert np.max(np.abs(z2 - w @ v[0, 0])) <= 1e-15
