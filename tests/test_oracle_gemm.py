"""Pins of the GEMM oracle (oracle.matmul) against facts fixed outside it:

  * brute force: every element as an exact sum of exact products of integers or of
    binary fractions (Python integers / fractions, no floating point);
  * closed forms: all-ones operands, identity and permutation matrices, rank-one
    products;
  * the error bound: it covers float32 accumulation in several orders followed by one
    rounding (simulated on the CPU), and it is not vacuous;
  * planted mistakes (transposed operand, dropped or shifted k term, sign) are caught.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.matmul as og


def _exact(a, b):
    """Element by element with exact rational arithmetic."""
    M, K = a.shape
    N = b.shape[1]
    out = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            out[i, j] = float(sum((Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K)),
                                  Fraction(0)))
    return out


def check_bruteforce(fn):
    rng = np.random.default_rng(3)
    for (M, K, N) in ((1, 1, 1), (3, 5, 4), (7, 16, 2), (2, 33, 5)):
        # binary fractions with few significant bits: every product and partial sum is
        # exact in float64 too, so the comparison is exact
        a = rng.integers(-64, 65, size=(M, K)) / 8.0
        b = rng.integers(-64, 65, size=(K, N)) / 16.0
        np.testing.assert_array_equal(fn(a, b), _exact(a, b))
    a = rng.standard_normal((4, 9))
    b = rng.standard_normal((9, 3))
    np.testing.assert_allclose(fn(a, b), _exact(a, b), rtol=1e-15, atol=1e-15)


def check_closed_forms(fn):
    for (M, K, N) in ((2, 3, 4), (5, 1, 7), (16, 64, 8)):
        np.testing.assert_array_equal(fn(np.ones((M, K)), np.ones((K, N))), np.full((M, N), float(K)))
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 6))
    np.testing.assert_array_equal(fn(x, np.eye(6)), x)
    np.testing.assert_array_equal(fn(np.eye(6), x), x)
    p = np.eye(6)[[3, 0, 5, 1, 4, 2]]              # row i of p picks row perm[i]
    np.testing.assert_array_equal(fn(p, x), x[[3, 0, 5, 1, 4, 2]])
    np.testing.assert_array_equal(fn(x, p.T), x[:, [3, 0, 5, 1, 4, 2]])
    u = np.arange(1, 6, dtype=np.float64)[:, None]
    v = np.arange(1, 4, dtype=np.float64)[None, :]
    np.testing.assert_array_equal(fn(u, v), np.array([[i * j for j in range(1, 4)] for i in range(1, 6)], float))
    # a non-square case where a transposed operand or a shifted k index changes the result
    a = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    b = np.array([[1.0, 0.0], [0.0, 10.0], [100.0, 0.0]])
    np.testing.assert_array_equal(fn(a, b), np.array([[301.0, 20.0], [604.0, 50.0]]))


def _simulated(a, b, out_dtype, order):
    """float32 accumulation in the given k order, then one rounding to out_dtype."""
    a32, b32 = a.astype(np.float32), b.astype(np.float32)
    acc = np.zeros((a.shape[0], b.shape[1]), dtype=np.float32)
    for k in order:
        acc = (acc + np.outer(a32[:, k], b32[k, :]).astype(np.float32)).astype(np.float32)
    if out_dtype == "bf16":
        u = acc.view(np.uint32)
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
        return r.view(np.float32).astype(np.float64)
    return acc.astype(np.float16).astype(np.float64)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_error_bound_covers_float32_accumulation(out_dtype):
    rng = np.random.default_rng(5)
    M, K, N = 8, 512, 8
    # operands exactly representable in bf16 and fp16 (8 significant bits, small range)
    a = np.round(rng.standard_normal((M, K)) * 16) / 16
    b = np.round(rng.standard_normal((K, N)) * 16) / 16
    exact = _exact(a, b)
    bound = og.gemm_error_bound(a, b, out_dtype)
    for order in (range(K), range(K - 1, -1, -1), rng.permutation(K)):
        err = np.abs(_simulated(a, b, out_dtype, order) - exact)
        assert np.all(err <= bound)
    # not vacuous: well under 1 % of |A||B| per element
    assert np.all(bound <= 1e-2 * (np.abs(a) @ np.abs(b)) + 1e-6)


def test_bruteforce():
    check_bruteforce(oracle.gemm)


def test_closed_forms():
    check_closed_forms(oracle.gemm)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.gemm(np.ones((2, 3)), np.ones((4, 2)))


def _mutant(kind):
    def gemm(a, b):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        if kind == "transposed_b" and b.shape[0] == b.shape[1]:
            return a @ b.T
        if kind == "transposed_b":
            return (b.T @ a.T).T[:, ::-1]
        if kind == "drop_last_k":
            return a[:, :-1] @ b[:-1, :]
        if kind == "shifted_k":
            return a @ np.roll(b, 1, axis=0)
        if kind == "sign":
            return -(a @ b)
        if kind == "float32":
            return (a.astype(np.float32) @ b.astype(np.float32)).astype(np.float64)
        return a @ b
    return gemm


@pytest.mark.parametrize("kind", ["transposed_b", "drop_last_k", "shifted_k", "sign", "float32"])
def test_pins_reject_mutant(kind):
    fn = _mutant(kind)
    caught = False
    for check in (check_bruteforce, check_closed_forms):
        try:
            check(fn)
        except AssertionError:
            caught = True
    assert caught, kind


def test_unmutated_passes():
    for check in (check_bruteforce, check_closed_forms):
        check(_mutant("none"))
