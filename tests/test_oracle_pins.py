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


def test_decode_f16_exact():
    # binary16 patterns: sign | 5-bit exponent (bias 15) | 10-bit fraction; 0x3C00 = 1.0,
    # 0xC000 = -2.0, 0x0001 = smallest subnormal 2^-24, 0x03FF = largest subnormal
    # 1023 * 2^-24, 0x0400 = smallest normal 2^-14, 0x7BFF = largest finite 65504,
    # 0x3555 = 1365/4096 (the float16 nearest 1/3)
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3555, 0x8000], dtype=np.uint16)
    want = np.array([1.0, -2.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 65504.0, 1365 / 4096, -0.0])
    got = oracle.decode(bits, "f16")
    assert np.array_equal(got, want) and np.signbit(got[7])
    # every finite pattern agrees with the IEEE conversion of a library (numpy's float16)
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((allbits >> 10) & 0x1F) != 31
    assert np.array_equal(oracle.decode(allbits[finite], "f16"),
                          allbits[finite].view(np.float16).astype(np.float64))


def test_bruteforce_decimal_on_f16_inputs():
    # float16-encoded inputs go through the same definition: decode exactly, then compare
    # with the 40-digit decimal evaluation of the definition
    rng = np.random.default_rng(11)
    bits = [rng.standard_normal((1, 2, 9, 5)).astype(np.float16).view(np.uint16) for _ in range(3)]
    q, k, v = (oracle.decode(b, "f16") for b in bits)
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal=causal, scale=0.7)
        o_ref, lse_ref = pins.decimal_attention(q, k, v, causal, 0.7)
        assert np.max(np.abs(o - o_ref)) <= 1e-12 and np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_causal_requires_square():
    q, k, v = pins.rand_qkv(1, 1, 1, 4, 4, Nk=5)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v, causal=True, scale=1.0)


def test_bruteforce_decimal_nonsquare():
    # fewer query rows than keys (split-KV decoding): the definition over all keys
    for n, (B, H, Nq, Nk, d) in enumerate([(1, 1, 1, 9, 4), (1, 2, 3, 17, 5), (2, 1, 2, 1, 3)]):
        q, k, v = pins.rand_qkv(300 + n, B, H, Nq, d, sigma=1.5, Nk=Nk)
        O, L = oracle.attention_forward(q, k, v, causal=False, scale=0.6)
        Ob, Lb = pins.decimal_attention(q, k, v, False, 0.6)
        assert np.max(np.abs(O - Ob)) <= 1e-12 and np.max(np.abs(L - Lb)) <= 1e-12


def test_nonsquare_closed_forms():
    # Q = 0: every key has weight 1/Nk, so O is the mean of V and lse = ln Nk
    q, k, v = pins.rand_qkv(7, 2, 3, 4, 8, Nk=300)
    O, L = oracle.attention_forward(np.zeros_like(q), k, v, causal=False, scale=0.3)
    assert np.max(np.abs(O - v.mean(axis=2, keepdims=True))) <= 1e-12
    assert np.max(np.abs(L - np.log(300))) <= 1e-12


def test_split_merge_identity():
    # Partial results over disjoint key ranges merge exactly into the full result:
    # lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s (the split-KV merge)
    q, k, v = pins.rand_qkv(8, 2, 2, 3, 16, sigma=2.0, Nk=1000)
    O, L = oracle.attention_forward(q, k, v, causal=False, scale=0.4)
    for bounds in ([0, 1000], [0, 1, 1000], [0, 64, 500, 999, 1000], list(range(0, 1001, 125))):
        parts = [oracle.attention_forward(q, k[:, :, a:b], v[:, :, a:b], causal=False, scale=0.4)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        lse_s = np.stack([p_[1] for p_ in parts])
        m = lse_s.max(axis=0)
        lse = m + np.log(np.exp(lse_s - m).sum(axis=0))
        om = sum(np.exp(p_[1] - lse)[..., None] * p_[0] for p_ in parts)
        assert np.max(np.abs(lse - L)) <= 1e-12 and np.max(np.abs(om - O)) <= 1e-12
