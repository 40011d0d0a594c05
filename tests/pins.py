"""Independent checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` function takes an attention function with the oracle's signature
``fn(q, k, v, causal=..., scale=...) -> (O, lse)`` (float64 ``[B,H,N,d]`` arrays)
and raises ``AssertionError`` on a mismatch.  The oracle tests call them with the
oracle; the mutation test calls them with deliberately broken copies of it to show
that every plausible mistake is caught by at least one check.

The references used here are:
  * brute force: the definition evaluated element by element in 40-digit decimal
    arithmetic (``decimal`` module, its own exp and ln);
  * a library routine: PyTorch's ``scaled_dot_product_attention`` in float64 on the
    CPU for O, and ``torch.logsumexp`` of the masked logits for lse;
  * closed forms and invariants of softmax attention.
"""
from __future__ import annotations

import ast
import json
import math
import os
from decimal import Decimal, getcontext
from typing import Callable

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

Fn = Callable[..., tuple]


# ----------------------------------------------------------------------------- brute force
def decimal_attention(q, k, v, causal: bool, scale: float, digits: int = 40):
    """The definition, element by element, in ``digits``-digit decimal arithmetic."""
    ctx = getcontext()
    ctx.prec = digits
    B, H, Nq, d = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    sc = Decimal(float(scale))
    O = np.zeros((B, H, Nq, dv))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            K = [[Decimal(float(x)) for x in k[b, h, j]] for j in range(Nk)]
            V = [[Decimal(float(x)) for x in v[b, h, j]] for j in range(Nk)]
            for i in range(Nq):
                Q = [Decimal(float(x)) for x in q[b, h, i]]
                vis = [j for j in range(Nk) if (not causal or j <= i)]
                s = {j: sc * sum((Q[c] * K[j][c] for c in range(d)), Decimal(0)) for j in vis}
                m = max(s.values())
                w = {j: (s[j] - m).exp() for j in vis}
                l = sum(w.values(), Decimal(0))
                for c in range(dv):
                    O[b, h, i, c] = float(sum((w[j] * V[j][c] for j in vis), Decimal(0)) / l)
                L[b, h, i] = float(m + l.ln())
    return O, L


def rand_qkv(seed, B, H, N, d, sigma=1.0, dv=None, Nk=None):
    rng = np.random.default_rng(seed)
    Nk = N if Nk is None else Nk
    dv = d if dv is None else dv
    q = rng.standard_normal((B, H, N, d)) * sigma
    k = rng.standard_normal((B, H, Nk, d)) * sigma
    v = rng.standard_normal((B, H, Nk, dv))
    return q, k, v


def check_bruteforce(fn: Fn, tol=1e-12):
    cases = [(1, 1, 1, 1), (1, 1, 2, 4), (1, 2, 3, 4), (2, 1, 5, 8), (1, 1, 8, 1), (1, 1, 17, 4)]
    for n, (B, H, N, d) in enumerate(cases):
        q, k, v = rand_qkv(100 + n, B, H, N, d, sigma=1.5)
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d) if n % 2 else 0.7
            O, L = fn(q, k, v, causal=causal, scale=scale)
            Ob, Lb = decimal_attention(q, k, v, causal, scale)
            assert np.max(np.abs(O - Ob)) <= tol, ("O", B, H, N, d, causal)
            assert np.max(np.abs(L - Lb)) <= tol, ("lse", B, H, N, d, causal)


# ----------------------------------------------------------------------------- library
def torch_reference(q, k, v, causal: bool, scale: float):
    import torch

    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        N = s.shape[-1]
        mask = torch.ones(N, N, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    L = torch.logsumexp(s, dim=-1)
    return O.numpy(), L.numpy()


def check_library(fn: Fn, tol=1e-12):
    for n, (B, H, N, d, sigma) in enumerate([(2, 3, 64, 16, 1.0), (1, 2, 130, 64, 1.0), (1, 1, 97, 8, 4.0)]):
        q, k, v = rand_qkv(200 + n, B, H, N, d, sigma=sigma)
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            O, L = fn(q, k, v, causal=causal, scale=scale)
            Ot, Lt = torch_reference(q, k, v, causal, scale)
            assert np.max(np.abs(O - Ot)) <= tol, ("O", B, H, N, d, causal)
            assert np.max(np.abs(L - Lt)) <= tol * max(1.0, np.max(np.abs(Lt))), ("lse", B, H, N, d, causal)


# ----------------------------------------------------------------------------- closed forms
def _eval_expr(text: str) -> float:
    """Evaluate a golden-file expression: numbers, + - * /, unary -, ln(), exp(), e."""
    funcs = {"ln": math.log, "exp": math.exp}

    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.Name) and node.id == "e":
            return math.e
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            ops = {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b}
            if isinstance(node.op, ast.Div):
                return a / b
            return ops[type(node.op)]
        if isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id in funcs:
            return funcs[node.func.id](*[ev(a) for a in node.args])
        raise ValueError(f"unsupported expression: {text!r}")

    return ev(ast.parse(text, mode="eval"))


def golden_cases():
    with open(os.path.join(GOLDEN, "closed_forms.json"), encoding="utf-8") as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        arr = lambda rows: np.array([[_eval_expr(x) for x in r] for r in rows])[None, None]
        out.append(dict(id=c["id"], scale=_eval_expr(c["scale"]), causal=c["causal"], q=arr(c["q"]),
                        k=arr(c["k"]), v=arr(c["v"]), O=arr(c["O"]),
                        lse=np.array([_eval_expr(x) for x in c["lse"]])[None, None]))
    return out


def check_golden(fn: Fn, tol=1e-12):
    for c in golden_cases():
        O, L = fn(c["q"], c["k"], c["v"], causal=c["causal"], scale=c["scale"])
        rel = max(1.0, float(np.max(np.abs(c["lse"]))))
        assert np.max(np.abs(O - c["O"])) <= tol * 10, (c["id"], "O", O, c["O"])
        assert np.max(np.abs(L - c["lse"])) <= tol * rel, (c["id"], "lse", L, c["lse"])


# ----------------------------------------------------------------------------- invariants
def check_invariants(fn: Fn, tol=1e-12):
    B, H, N, d = 2, 2, 37, 8
    q, k, v = rand_qkv(300, B, H, N, d, sigma=2.0)
    scale = 1.0 / math.sqrt(d)
    counts = np.arange(1, N + 1, dtype=np.float64)
    for causal in (False, True):
        O, L = fn(q, k, v, causal=causal, scale=scale)
        # V = ones -> O = ones (softmax rows sum to one)
        O1, _ = fn(q, k, np.ones_like(v), causal=causal, scale=scale)
        assert np.max(np.abs(O1 - 1.0)) <= tol, "V=1"
        # affine in V: O(a V + b) = a O(V) + b
        Oa, La = fn(q, k, 2.5 * v - 0.75, causal=causal, scale=scale)
        assert np.max(np.abs(Oa - (2.5 * O - 0.75))) <= 10 * tol, "affine V"
        assert np.max(np.abs(La - L)) <= tol, "lse independent of V"
        # Q = 0 (or K = 0): uniform weights over the visible keys
        for zq, zk in ((np.zeros_like(q), k), (q, np.zeros_like(k))):
            Oz, Lz = fn(zq, zk, v, causal=causal, scale=scale)
            if causal:
                mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
                lse = np.broadcast_to(np.log(counts), Lz.shape)
            else:
                mean = np.broadcast_to(v.mean(axis=2, keepdims=True), Oz.shape)
                lse = np.full(Lz.shape, math.log(N))
            assert np.max(np.abs(Oz - mean)) <= tol, "zero logits -> mean of visible V"
            assert np.max(np.abs(Lz - lse)) <= tol, "zero logits -> lse = ln(#visible)"
        # shifting every key by the same vector u shifts row i's logits by scale*q_i.u
        u = np.linspace(-1.0, 2.0, d)
        Os, Ls = fn(q, k + u, v, causal=causal, scale=scale)
        assert np.max(np.abs(Os - O)) <= 100 * tol, "key shift leaves O unchanged"
        assert np.max(np.abs(Ls - (L + scale * (q @ u)))) <= 100 * tol, "key shift moves lse by scale*q.u"
        # the first causal row sees only key 0
        if causal:
            assert np.max(np.abs(O[:, :, 0] - v[:, :, 0])) <= tol, "causal row 0 -> v_0"
            l0 = scale * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
            assert np.max(np.abs(L[:, :, 0] - l0)) <= tol, "causal row 0 lse = scale q0.k0"
        # a single key: O = v_0 exactly
        O1k, L1k = fn(q[:, :, :1], k[:, :, :1], v[:, :, :1], causal=causal, scale=scale)
        assert np.max(np.abs(O1k - v[:, :, :1])) <= tol, "N=1"
    # non-causal: a joint permutation of the key/value rows changes nothing
    O, L = fn(q, k, v, causal=False, scale=scale)
    perm = np.random.default_rng(7).permutation(N)
    Op, Lp = fn(q, k[:, :, perm], v[:, :, perm], causal=False, scale=scale)
    assert np.max(np.abs(Op - O)) <= 10 * tol and np.max(np.abs(Lp - L)) <= 10 * tol, "key permutation"
    # heads and batches are independent: permuting heads permutes outputs
    hp = [1, 0]
    Oh, Lh = fn(q[:, hp], k[:, hp], v[:, hp], causal=True, scale=scale)
    Oc, Lc = fn(q, k, v, causal=True, scale=scale)
    assert np.max(np.abs(Oh - Oc[:, hp])) <= tol and np.max(np.abs(Lh - Lc[:, hp])) <= tol, "head order"
    # one dominant logit: the row copies that key's value
    qd = np.zeros((1, 1, 3, 2)); qd[..., 0] = 1.0
    kd = np.zeros((1, 1, 3, 2)); kd[0, 0, 1, 0] = 60.0
    vd = np.arange(6, dtype=np.float64).reshape(1, 1, 3, 2)
    Od, _ = fn(qd, kd, vd, causal=False, scale=1.0)
    assert np.max(np.abs(Od - vd[:, :, 1:2])) <= tol, "dominant key"
    # softmax rows sum to one: P = exp(s - lse) recovered from lse sums to 1 per row
    for causal in (False, True):
        _, L = fn(q, k, v, causal=causal, scale=scale)
        s = scale * np.einsum("bhic,bhjc->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        P = np.exp(s - L[..., None])
        assert np.max(np.abs(P.sum(axis=-1) - 1.0)) <= 10 * tol, "rows of P sum to 1"
