"""Pins for the fp64 C oracle (CPU only).

Each check ties the oracle to something other than itself: the blog's printed
worked example, values derived by hand from the blog's causal figure, closed forms
(Q = 0 gives prefix means), a one-hot limit, scipy's softmax / logsumexp on tiny
inputs, and invariants of softmax attention. ``test_planted_mistakes_are_caught``
plants plausible mistakes into a copy of the oracle source and checks that these
pins catch every one.
"""
import math
import os
import shutil
import tempfile

import numpy as np
import pytest
import scipy.special

import oracle
from golden_io import load_worked_example

LN2 = math.log(2.0)


def _example():
    g = load_worked_example()
    return g["Q"], g["K"], g["V"], g


# --- printed worked example ------------------------------------------------------------

def pin_worked_example(fwd):
    q, k, v, g = _example()
    o, lse = fwd(q, k, v, LN2, False)
    np.testing.assert_allclose(o, g["O"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["LSE"], rtol=0, atol=1e-14)


def pin_worked_example_causal(fwd):
    q, k, v, g = _example()
    o, lse = fwd(q, k, v, LN2, True)
    np.testing.assert_allclose(o, g["causal"]["O"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["causal"]["LSE"], rtol=0, atol=1e-14)


def pin_worked_example_bottom_right(fwd):
    q, k, v, g = _example()
    o, lse = fwd(q, k, v, LN2, True, align="bottom-right")
    np.testing.assert_allclose(o, g["bottom_right"]["O"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["bottom_right"]["LSE"], rtol=0, atol=1e-14)


def pin_bottom_right_reductions(fwd):
    """Bottom-right causal reduces to known cases: with Nq = Nk it is top-left; a
    single query sees every key (non-causal); with Nq > Nk the first Nq - Nk rows
    have no valid key (O = 0, LSE = -inf) and row i >= Nq - Nk is top-left row
    i - (Nq - Nk)."""
    rng = np.random.default_rng(21)
    d, s = 6, 0.45
    K = rng.standard_normal((9, d)); V = rng.standard_normal((9, d))
    Q = rng.standard_normal((9, d))
    o_br, l_br = fwd(Q, K, V, s, True, align="bottom-right")
    o_tl, l_tl = fwd(Q, K, V, s, True)
    np.testing.assert_array_equal(o_br, o_tl)
    np.testing.assert_array_equal(l_br, l_tl)
    o1, l1 = fwd(Q[4:5], K, V, s, True, align="bottom-right")
    o2, l2 = fwd(Q[4:5], K, V, s, False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    Qb = rng.standard_normal((13, d))
    o3, l3 = fwd(Qb, K, V, s, True, align="bottom-right")
    assert np.all(o3[:4] == 0.0) and np.all(np.isneginf(l3[:4]))
    o4, l4 = fwd(Qb[4:], K, V, s, True)
    np.testing.assert_array_equal(o3[4:], o4)
    np.testing.assert_array_equal(l3[4:], l4)


def pin_embedded_example(fwd):
    """The worked example as a square N=4 problem with d padded to 64 by zeros and
    query rows 2,3 set to 0 (the form the GPU parity test uses). Rows 0,1 keep the
    printed results; rows 2,3 get uniform weights over their valid keys."""
    q, k, v, g = _example()
    d = 64
    Q = np.zeros((4, d)); Q[:2, :2] = q
    K = np.zeros((4, d)); K[:, :2] = k
    V = np.zeros((4, d)); V[:, :2] = v
    o, lse = fwd(Q, K, V, LN2, False)
    np.testing.assert_allclose(o[:2, :2], g["O"], atol=1e-14)
    np.testing.assert_allclose(o[2:, :2], [[1.0, 0.5], [1.0, 0.5]], atol=1e-14)
    np.testing.assert_allclose(lse, [g["LSE"][0], g["LSE"][1], math.log(4), math.log(4)], atol=1e-14)
    assert np.all(o[:, 2:] == 0.0)
    o, lse = fwd(Q, K, V, LN2, True)
    np.testing.assert_allclose(o[:2, :2], g["causal"]["O"], atol=1e-14)
    np.testing.assert_allclose(o[2:, :2], [[2 / 3, 2 / 3], [1.0, 0.5]], atol=1e-14)
    np.testing.assert_allclose(lse, [0.0, math.log(3), math.log(3), math.log(4)], atol=1e-14)


# --- closed forms ----------------------------------------------------------------------

def pin_zero_query_prefix_mean(fwd):
    """Q = 0: every valid key scores 0, so O[i] is the mean of the valid V rows and
    LSE[i] = ln(#valid). Causal: prefix means and ln(i+1)."""
    rng = np.random.default_rng(7)
    for n, d in [(1, 3), (5, 2), (70, 3), (129, 8)]:
        V = rng.standard_normal((n, d))
        K = rng.standard_normal((n, d))
        Q = np.zeros((n, d))
        o, lse = fwd(Q, K, V, 0.37, True)
        counts = np.arange(1, n + 1)[:, None]
        np.testing.assert_allclose(o, np.cumsum(V, axis=0) / counts, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)
        o, lse = fwd(Q, K, V, 0.37, False)
        np.testing.assert_allclose(o, np.broadcast_to(V.mean(axis=0), (n, d)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, np.full(n, math.log(n)), rtol=0, atol=1e-13)


def pin_one_hot_limit(fwd):
    """Key j = perm[i] scores 50/s above every other key for query i, so O[i] equals
    V[perm[i]] up to n*e^-50 and LSE[i] is 50 above the others' scaled score."""
    rng = np.random.default_rng(11)
    n, d, s = 12, 12, 0.25
    perm = rng.permutation(n)
    K = np.eye(n, d)                              # key j is the unit vector e_j
    Q = np.zeros((n, d))
    Q[np.arange(n), perm] = 50.0 / s              # query i points at key perm[i]
    V = rng.standard_normal((n, d))
    o, lse = fwd(Q, K, V, s, False)
    np.testing.assert_allclose(o, V[perm], rtol=0, atol=1e-15)  # n e^-50 is far below fp64 rounding
    np.testing.assert_allclose(lse, np.full(n, 50.0), rtol=0, atol=1e-12)


def pin_against_scipy(fwd):
    """Tiny random problems against scipy.special.softmax / logsumexp applied to the
    scaled score matrix built with numpy (masked entries -inf for causal)."""
    rng = np.random.default_rng(3)
    for (nq, nk, d, causal) in [(1, 1, 1, False), (3, 5, 2, False), (7, 7, 4, True),
                                (9, 9, 16, False), (6, 11, 5, True), (33, 33, 8, True),
                                (6, 11, 5, "bottom-right"), (1, 9, 3, "bottom-right"),
                                (10, 10, 4, "bottom-right")]:
        Q = rng.standard_normal((nq, d)); K = rng.standard_normal((nk, d))
        V = rng.standard_normal((nk, d)); s = 1.0 / math.sqrt(d)
        z = s * (Q @ K.T)
        off = (nk - nq) if causal == "bottom-right" else 0
        if causal:
            z = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + off, z, -np.inf)
        if causal == "bottom-right":
            o, lse = fwd(Q, K, V, s, True, align="bottom-right")
        else:
            o, lse = fwd(Q, K, V, s, causal)
        np.testing.assert_allclose(o, scipy.special.softmax(z, axis=1) @ V, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-13, atol=1e-13)


# --- invariants ------------------------------------------------------------------------

def pin_invariants(fwd):
    rng = np.random.default_rng(5)
    n, d, s = 40, 8, 0.3
    Q = 2 * rng.standard_normal((n, d)); K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    for causal in (False, True):
        o, lse = fwd(Q, K, V, s, causal)
        nvalid = np.arange(1, n + 1) if causal else np.full(n, n)
        # weights sum to one: V = ones gives O = 1
        o1, _ = fwd(Q, K, np.ones((n, d)), s, causal)
        np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-13)
        # convex hull of the valid V rows, per coordinate
        for i in range(n):
            vv = V[:nvalid[i]]
            assert np.all(o[i] >= vv.min(axis=0) - 1e-12) and np.all(o[i] <= vv.max(axis=0) + 1e-12)
        # max z <= LSE <= max z + ln(#valid)
        z = s * (Q @ K.T)
        zmax = np.array([z[i, :nvalid[i]].max() for i in range(n)])
        assert np.all(lse >= zmax - 1e-12) and np.all(lse <= zmax + np.log(nvalid) + 1e-12)
        # shifting every key by w leaves O and moves LSE_i by s * q_i . w
        w = rng.standard_normal(d)
        o2, lse2 = fwd(Q, K + w, V, s, causal)
        np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(lse2, lse + s * Q @ w, rtol=1e-11, atol=1e-11)
    # joint key/value permutation (non-causal) changes nothing
    o, lse = fwd(Q, K, V, s, False)
    p = rng.permutation(n)
    o3, lse3 = fwd(Q, K[p], V[p], s, False)
    np.testing.assert_allclose(o3, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, rtol=1e-13, atol=1e-13)


def pin_heads_independent(fwd):
    """A [B, H, N, d] call equals one call per (b, h) slice."""
    rng = np.random.default_rng(9)
    B, H, n, d = 2, 3, 17, 4
    Q = rng.standard_normal((B, H, n, d)); K = rng.standard_normal((B, H, n, d))
    V = rng.standard_normal((B, H, n, d))
    for causal in (False, True):
        o, lse = fwd(Q, K, V, 0.5, causal)
        for b in range(B):
            for h in range(H):
                o1, l1 = fwd(Q[b, h], K[b, h], V[b, h], 0.5, causal)
                np.testing.assert_array_equal(o[b, h], o1)
                np.testing.assert_array_equal(lse[b, h], l1)
        # a head's output depends on its own K and V only: perturb another head
        K2 = K.copy(); K2[1, 2] += 1.0
        V2 = V.copy(); V2[1, 2] *= 3.0
        o2, lse2 = fwd(Q, K2, V2, 0.5, causal)
        np.testing.assert_array_equal(o2[0], o[0])
        np.testing.assert_array_equal(lse2[1, :2], lse[1, :2])
        assert not np.allclose(o2[1, 2], o[1, 2])


ALL_PINS = [pin_worked_example, pin_worked_example_causal, pin_worked_example_bottom_right,
            pin_bottom_right_reductions, pin_embedded_example,
            pin_zero_query_prefix_mean, pin_one_hot_limit, pin_against_scipy, pin_invariants,
            pin_heads_independent]


def _fwd(lib=None):
    return lambda q, k, v, s, c, align="top-left": oracle.attention_fwd(q, k, v, s, c, lib=lib, align=align)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(_fwd())


def test_rows_entry_matches_full():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((2, 3, 50, 8)); K = rng.standard_normal((2, 3, 50, 8))
    V = rng.standard_normal((2, 3, 50, 8))
    o, lse = oracle.attention_fwd(Q, K, V, 0.4, True)
    rows = np.array([0, 49, 50, 149, 299, 123])
    o_r, lse_r = oracle.attention_rows(Q, K, V, 0.4, True, rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(lse_r, lse.reshape(-1)[rows])
    with pytest.raises(ValueError):
        oracle.attention_rows(Q, K, V, 0.4, True, [300])


def test_degenerate_sizes_and_errors():
    # no keys: O = 0, LSE = -inf; no queries: empty outputs
    o, lse = oracle.attention_fwd(np.ones((3, 2)), np.zeros((0, 2)), np.zeros((0, 2)), 1.0, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = oracle.attention_fwd(np.zeros((0, 2)), np.ones((3, 2)), np.ones((3, 2)), 1.0, True)
    assert o.shape == (0, 2) and lse.shape == (0,)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.attention_fwd(np.ones((2, 2)), np.ones((2, 2)), np.ones((2, 2)), bad, False)


# --- planted mistakes ------------------------------------------------------------------

MUTATIONS = {
    "drop_scale": ("z[j] = scale * x;", "z[j] = x;"),
    "causal_off_by_one": ("nvalid = (i + 1 < Nk) ? (i + 1) : Nk;", "nvalid = (i < Nk) ? i : Nk;"),
    "bottom_right_sign": ("const int64_t last = i + Nk - Nq;", "const int64_t last = i - Nk + Nq;"),
    "bottom_right_off_by_one": ("nvalid = (last + 1 < Nk) ? (last + 1) : Nk;", "nvalid = (last < Nk) ? last : Nk;"),
    "k_for_v": ("const double* k_row = k + j * d;", "const double* k_row = v + j * d;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "exp_sign": ("l += exp(z[j] - m);", "l += exp(m - z[j]);"),
    "no_normalisation": ("double p = exp(z[j] - m) / l;", "double p = exp(z[j] - m);"),
    "first_head_v": ("k + bh * Nk * d, v + bh * Nk * d, Nq, Nk, d, scale, causal, i, z,\n"
                     "                       o + r * d", "k + bh * Nk * d, v, Nq, Nk, d, scale, causal, i, z,\n"
                     "                       o + r * d"),
    "dot_drops_last_term": ("for (int64_t c = 0; c < d; ++c) x += q_row[c] * k_row[c];",
                            "for (int64_t c = 0; c + 1 < d; ++c) x += q_row[c] * k_row[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    src_path = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")
    src = open(src_path).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation target for {name} no longer in the oracle source"
    tmpdir = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        mpath = os.path.join(tmpdir, "mut.c")
        with open(mpath, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.load_library(oracle.build(src=mpath, out=os.path.join(tmpdir, "libmut.so")))
        caught = []
        for pin in ALL_PINS:
            try:
                pin(_fwd(lib))
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"planted mistake {name} passed every pin"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
