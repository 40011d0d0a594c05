"""The CPU oracle against facts other than itself (brute force, a library routine,
closed forms, invariants).  CPU only."""
import numpy as np
import pytest

import oracle
from tests import pins


def _oracle(q, k, v, causal, scale):
    return oracle.attention_forward(q, k, v, causal=causal, scale=scale)


def test_bruteforce_decimal():
    pins.check_bruteforce(_oracle)


def test_library_sdpa_float64():
    pins.check_library(_oracle)


def test_golden_closed_forms():
    pins.check_golden(_oracle)


def test_invariants():
    pins.check_invariants(_oracle)


def test_threaded_equals_serial():
    q, k, v = pins.rand_qkv(5, 2, 3, 2100, 8)
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, causal=causal, scale=0.3)
        o2, l2 = oracle.attention_forward(q, k, v, causal=causal, scale=0.3, threads=4)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rows_match_full():
    q, k, v = pins.rand_qkv(6, 2, 2, 300, 16)
    picks = [(0, 0, 0), (1, 1, 299), (0, 1, 150), (1, 0, 7)]
    for causal in (False, True):
        o, l = oracle.attention_forward(q, k, v, causal=causal, scale=0.25)
        po, pl = oracle.attention_rows(q, k, v, causal=causal, scale=0.25, picks=picks)
        for n, (b, h, i) in enumerate(picks):
            assert np.max(np.abs(po[n] - o[b, h, i])) <= 1e-13
            assert abs(pl[n] - l[b, h, i]) <= 1e-13


def test_decode_bf16_exact():
    # bf16 patterns: sign | 8-bit exponent | 7-bit mantissa; 0x3F80 = 1.0, 0xC040 = -3.0,
    # 0x0001 = smallest subnormal 2^-133, 0x7F7F = largest finite (2 - 2^-7) * 2^127
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = np.array([1.0, -3.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0])
    got = oracle.decode(bits, "bf16")
    assert np.array_equal(got, want) and np.signbit(got[5])


def test_causal_requires_square():
    q, k, v = pins.rand_qkv(1, 1, 1, 4, 4, Nk=5)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v, causal=True, scale=1.0)
