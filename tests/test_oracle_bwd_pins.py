"""Pins for the fp64 C oracle's backward pass (CPU only).

The gradients are checked against things other than the oracle's own formulas:

* central finite differences of the *forward* oracle (a separate C routine), on
  tiny inputs, for every element of Q, K and V and every causal mode: this checks
  the calculus, not only the code;
* exact rational arithmetic on the blog's worked example (s = ln 2 makes every
  softmax weight a power of two over a sum of powers of two), from the definition;
* the closed form for Q = 0 (uniform weights over the valid keys);
* invariants: the key gradients of a slice sum to zero, dV sums to the dO of the
  rows that see a key, shifting every key or every value by one vector leaves the
  gradients unchanged;
* torch.autograd through a plain fp64 CPU attention (a library routine);
* slices are independent.

``test_planted_bwd_mistakes_are_caught`` plants plausible mistakes into a copy of
the oracle source and checks that these pins catch each one.
"""
import json
import math
import os
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

LN2 = math.log(2.0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bwd(lib=None):
    return lambda *a, **kw: oracle.attention_bwd(*a, lib=lib, **kw)


def _fwd_loss(q, k, v, g, scale, causal, align):
    o, _ = oracle.attention_fwd(q, k, v, scale, causal, align=align)
    return float((o * g).sum())


# --- finite differences of the forward oracle ------------------------------------------------

def pin_bwd_finite_differences(bwd):
    rng = np.random.default_rng(1)
    for causal, align, nq, nk in ((False, "top-left", 5, 7), (True, "top-left", 6, 6),
                                  (True, "bottom-right", 4, 7), (True, "bottom-right", 7, 4)):
        q = rng.standard_normal((2, nq, 3))
        k = rng.standard_normal((2, nk, 3))
        v = rng.standard_normal((2, nk, 3))
        g = rng.standard_normal((2, nq, 3))
        scale = 0.8
        dq, dk, dv = bwd(q, k, v, g, scale, causal, align=align)
        h = 1e-6
        for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(t)
            for idx in np.ndindex(t.shape):
                tp = t.copy(); tp[idx] += h
                tm = t.copy(); tm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}; args_p[name] = tp
                args_m = {"q": q, "k": k, "v": v}; args_m[name] = tm
                num[idx] = (_fwd_loss(args_p["q"], args_p["k"], args_p["v"], g, scale, causal, align)
                            - _fwd_loss(args_m["q"], args_m["k"], args_m["v"], g, scale, causal, align)) / (2 * h)
            np.testing.assert_allclose(grad, num, rtol=0, atol=2e-7,
                                       err_msg=f"d{name} vs finite differences ({align}, causal={causal})")


# --- exact rationals on the worked example ---------------------------------------------------

def _frac_matrix(entry):
    return [[Fraction(x) for x in row] for row in entry["value"]]


def _exact_grads(Q, K, V, dO, causal):
    """Gradients over ln 2 (dq, dk) and dv, exactly, for s = ln 2 and integer scores:
    exp(s x) = 2^x, so every weight is rational."""
    nq, nk, d = len(Q), len(K), len(Q[0])
    dq = [[Fraction(0)] * d for _ in range(nq)]
    dk = [[Fraction(0)] * d for _ in range(nk)]
    dv = [[Fraction(0)] * d for _ in range(nk)]
    for i in range(nq):
        keys = range(min(nk, i + 1)) if causal else range(nk)
        x = {j: sum(Q[i][c] * K[j][c] for c in range(d)) for j in keys}
        w = {j: Fraction(2) ** int(x[j]) for j in keys}
        tot = sum(w.values())
        p = {j: w[j] / tot for j in keys}
        dp = {j: sum(dO[i][c] * V[j][c] for c in range(d)) for j in keys}
        Di = sum(p[j] * dp[j] for j in keys)
        for j in keys:
            dz = p[j] * (dp[j] - Di)
            for c in range(d):
                dq[i][c] += dz * K[j][c]
                dk[j][c] += dz * Q[i][c]
                dv[j][c] += p[j] * dO[i][c]
    return dq, dk, dv


def pin_bwd_exact_rationals(bwd):
    g = json.load(open(GOLDEN))
    Q, K, V = _frac_matrix(g["Q"]), _frac_matrix(g["K"]), _frac_matrix(g["V"])
    for x in (q for row in Q + K for q in row):
        assert x.denominator == 1, "the example's scores are integers"
    dO = [[Fraction(1), Fraction(-2)], [Fraction(3), Fraction(1)]]
    for causal in (False, True):
        eq, ek, ev = _exact_grads(Q, K, V, dO, causal)
        f = lambda m: np.array([[float(x) for x in row] for row in m])
        dq, dk, dv = bwd(f(Q)[None], f(K)[None], f(V)[None], f(dO)[None], LN2, causal)
        np.testing.assert_allclose(dq[0], LN2 * f(eq), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk[0], LN2 * f(ek), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[0], f(ev), rtol=0, atol=1e-13)


# --- closed form: Q = 0 ------------------------------------------------------------------------

def pin_bwd_zero_query_closed_form(bwd):
    """Q = 0: every valid key has weight 1/n_i, so dV_j = sum_i dO_i / n_i over the rows that
    see key j, dK = 0, and dQ_i = (s / n_i) sum_j (dO_i . (v_j - mean_i v)) k_j."""
    rng = np.random.default_rng(2)
    n, d, s = 9, 4, 0.6
    k = rng.standard_normal((1, n, d)); v = rng.standard_normal((1, n, d)); do = rng.standard_normal((1, n, d))
    q = np.zeros((1, n, d))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, s, causal)
        ev = np.zeros((n, d)); eq = np.zeros((n, d))
        for i in range(n):
            keys = np.arange(i + 1) if causal else np.arange(n)
            ni = len(keys)
            ev[keys] += do[0, i] / ni
            vbar = v[0, keys].mean(axis=0)
            eq[i] = (s / ni) * ((v[0, keys] - vbar) @ do[0, i]) @ k[0, keys]
        np.testing.assert_allclose(dv[0], ev, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq[0], eq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[0], 0.0, rtol=0, atol=1e-14)


# --- invariants --------------------------------------------------------------------------------

def pin_bwd_invariants(bwd):
    rng = np.random.default_rng(3)
    nq, nk, d, s = 6, 8, 5, 0.9
    q = rng.standard_normal((2, nq, d)); k = rng.standard_normal((2, nk, d))
    v = rng.standard_normal((2, nk, d)); do = rng.standard_normal((2, nq, d))
    for causal, align in ((False, "top-left"), (True, "bottom-right")):
        dq, dk, dv = bwd(q, k, v, do, s, causal, align=align)
        # each row's score gradients sum to zero, so the key gradients of a slice do too
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        # each row's weights sum to one: dV sums to the dO of the rows that see a key
        seen = np.array([(not causal) or (i + nk - nq >= 0) for i in range(nq)])
        np.testing.assert_allclose(dv.sum(axis=1), do[:, seen].sum(axis=1), atol=1e-12)
        # a common shift of every key (scores shift per row) or of every value changes nothing
        c = rng.standard_normal(d)
        for kk, vv in ((k + c, v), (k, v + c)):
            dq2, dk2, dv2 = bwd(q, kk, vv, do, s, causal, align=align)
            np.testing.assert_allclose(dq2, dq, atol=1e-12)
            np.testing.assert_allclose(dk2, dk, atol=1e-12)
            np.testing.assert_allclose(dv2, dv, atol=1e-12)


def pin_bwd_against_torch_autograd(bwd):
    rng = np.random.default_rng(4)
    for causal, nq, nk in ((False, 7, 9), (True, 8, 8), (True, 5, 9)):
        q = torch.tensor(rng.standard_normal((3, nq, 6)), dtype=torch.float64, requires_grad=True)
        k = torch.tensor(rng.standard_normal((3, nk, 6)), dtype=torch.float64, requires_grad=True)
        v = torch.tensor(rng.standard_normal((3, nk, 6)), dtype=torch.float64, requires_grad=True)
        do = torch.tensor(rng.standard_normal((3, nq, 6)), dtype=torch.float64)
        s = 0.45
        z = s * (q @ k.transpose(-1, -2))
        if causal:
            i = torch.arange(nq)[:, None]; j = torch.arange(nk)[None, :]
            z = z.masked_fill(j > i + nk - nq, float("-inf"))
        o = torch.softmax(z, dim=-1) @ v
        o.backward(do)
        dq, dk, dv = bwd(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), do.numpy(), s, causal,
                         align="bottom-right")
        np.testing.assert_allclose(dq, q.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, k.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, v.grad.numpy(), rtol=0, atol=1e-12)


def pin_bwd_slices_independent(bwd):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 5, 4)); k = rng.standard_normal((3, 6, 4))
    v = rng.standard_normal((3, 6, 4)); do = rng.standard_normal((3, 5, 4))
    full = bwd(q, k, v, do, 0.5, True, align="bottom-right")
    for b in range(3):
        one = bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], do[b:b + 1], 0.5, True, align="bottom-right")
        for a, c in zip(full, one):
            np.testing.assert_allclose(a[b], c[0], rtol=0, atol=0)


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_exact_rationals, pin_bwd_zero_query_closed_form,
                pin_bwd_invariants, pin_bwd_against_torch_autograd, pin_bwd_slices_independent]


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_bwd_pin(pin):
    pin(_bwd())


def test_bwd_degenerate_sizes():
    z = np.zeros((2, 0, 4))
    dq, dk, dv = oracle.attention_bwd(z, np.ones((2, 3, 4)), np.ones((2, 3, 4)), z, 0.5)
    assert dq.shape == (2, 0, 4) and np.all(dk == 0) and np.all(dv == 0)
    # no keys: every gradient is zero
    q = np.ones((1, 3, 4))
    dq, dk, dv = oracle.attention_bwd(q, np.zeros((1, 0, 4)), np.zeros((1, 0, 4)), q, 0.5)
    assert np.all(dq == 0) and dk.shape == (1, 0, 4)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, q, q, q, -1.0)


BWD_MUTATIONS = {
    "drop_delta": ("const double dz = pr[j] * (dp[j] - Di);", "const double dz = pr[j] * dp[j];"),
    "dk_without_scale": ("dks[j * d + c] += scale * dz * qi[c];", "dks[j * d + c] += dz * qi[c];"),
    "dv_uses_score_grad": ("dvs[j * d + c] += pr[j] * doi[c];", "dvs[j * d + c] += dz * doi[c];"),
    "dq_uses_v": ("dqi[c] += scale * dz * ks[j * d + c];", "dqi[c] += scale * dz * vs[j * d + c];"),
    "dp_drops_last_term": ("for (int64_t c = 0; c < d; ++c) x += doi[c] * vs[j * d + c];",
                           "for (int64_t c = 0; c + 1 < d; ++c) x += doi[c] * vs[j * d + c];"),
    "unnormalised_p": ("for (int64_t j = 0; j < nv; ++j) pr[j] = exp(z[j] - m) / l;",
                       "for (int64_t j = 0; j < nv; ++j) pr[j] = exp(z[j] - m);"),
    "bwd_causal_off_by_one": ("if (causal == 1) nv = (i + 1 < Nk) ? (i + 1) : Nk;",
                              "if (causal == 1) nv = (i < Nk) ? i : Nk;"),
    "bwd_bottom_right_sign": ("if (causal == 2) nv = (i + Nk - Nq + 1 < Nk) ? (i + Nk - Nq + 1) : Nk;",
                              "if (causal == 2) nv = (i - Nk + Nq + 1 < Nk) ? (i - Nk + Nq + 1) : Nk;"),
    "dk_slice_offset": ("double* dks = dk + bh * Nk * d;", "double* dks = dk + bh * Nq * d;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_planted_bwd_mistakes_are_caught(name):
    src_path = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")
    src = open(src_path).read()
    old, new = BWD_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation target for {name} not found once in the oracle source"
    tmpdir = tempfile.mkdtemp(prefix="oracle_bwd_mut_")
    try:
        mpath = os.path.join(tmpdir, "mut.c")
        with open(mpath, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.load_library(oracle.build(src=mpath, out=os.path.join(tmpdir, "libmut.so")))
        caught = []
        for pin in ALL_BWD_PINS:
            try:
                pin(_bwd(lib))
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
        assert caught, f"planted mistake {name} passed every pin"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
