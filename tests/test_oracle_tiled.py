"""Pins for the tiled online-softmax emulator (CPU only).

The blog's worked example at two keys per round reproduces every intermediate it
prints (Fig. 5 scores, Fig. 6/7 weights, l0, alpha, l1, Fig. 8-10 numerators,
Fig. 12 output). A brute-force sweep over sizes, tile shapes and causal flags then
checks that the tiled recurrence and the three-pass C oracle agree to 1e-12: two
independent codes for the same definition.
"""
import math

import numpy as np
import pytest

import oracle
from golden_io import load_worked_example
from oracle.tiled import online_softmax_attention, round_to

LN2 = math.log(2.0)
EXACT = dict(rtol=0, atol=1e-14)


def test_worked_example_rounds():
    g = load_worked_example()
    o, lse, steps = online_softmax_attention(g["Q"], g["K"], g["V"], LN2, causal=False,
                                             block_m=2, block_n=2, trace=True)
    assert len(steps) == 2
    r0, r1 = steps
    np.testing.assert_allclose(np.hstack([r0["S"], r1["S"]]), g["S"], **EXACT)   # Fig. 5
    np.testing.assert_allclose(r0["m"], g["m0"], **EXACT)
    np.testing.assert_allclose(r0["E"], g["E0"], **EXACT)                         # Fig. 6
    np.testing.assert_allclose(r0["l"], g["l0"], **EXACT)
    np.testing.assert_allclose(r0["U"], g["U0"], **EXACT)                         # Fig. 8
    np.testing.assert_allclose(r1["alpha"], g["alpha1"], **EXACT)
    np.testing.assert_allclose(r1["m"], g["m1"], **EXACT)
    np.testing.assert_allclose(r1["E"], g["E1"], **EXACT)                         # Fig. 7
    np.testing.assert_allclose(r1["E"] @ g["V"][2:4], g["dU"], **EXACT)           # Fig. 9
    np.testing.assert_allclose(r1["U"], g["U1"], **EXACT)                         # Fig. 10
    np.testing.assert_allclose(r1["l"], g["l1"], **EXACT)
    np.testing.assert_allclose(o, g["O"], **EXACT)                                # Fig. 12
    np.testing.assert_allclose(lse, g["LSE"], **EXACT)
    # rescaled old denominator 3/2 -> 3/4 (text before Fig. 7)
    np.testing.assert_allclose(r1["alpha"] * r0["l"], [0.75, 0.75], **EXACT)


def test_worked_example_causal():
    g = load_worked_example()
    o, lse, steps = online_softmax_attention(g["Q"], g["K"], g["V"], LN2, causal=True,
                                             block_m=2, block_n=2, trace=True)
    np.testing.assert_array_equal(np.hstack([steps[0]["S"], steps[1]["S"]]), g["causal"]["S_masked"])  # Fig. 11
    # the second key block lies wholly in the future of both queries: weights all zero
    assert np.all(steps[1]["E"] == 0) and np.all(steps[1]["alpha"] == 1)
    np.testing.assert_allclose(o, g["causal"]["O"], **EXACT)
    np.testing.assert_allclose(lse, g["causal"]["LSE"], **EXACT)


def test_fully_masked_row_guard():
    """With one key per block, every block after a row's diagonal is wholly in its
    future; such blocks must leave the row's state unchanged (no NaN, alpha = 1)."""
    rng = np.random.default_rng(0)
    q = rng.standard_normal((8, 4)); k = rng.standard_normal((8, 4)); v = rng.standard_normal((8, 4))
    o, lse = online_softmax_attention(q, k, v, 0.5, causal=True, block_m=1, block_n=1)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    # no keys at all: O = 0, LSE = -inf, like the C oracle
    o, lse = online_softmax_attention(q, np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


SWEEP = [(n, d, bm, bn, causal)
         for n in (1, 2, 3, 17, 64, 70)
         for d in (1, 2, 3, 8)
         for (bm, bn) in ((1, 1), (2, 3), (5, 2), (64, 64), (3, 64))
         for causal in (False, True)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiled_matches_three_pass(seed):
    rng = np.random.default_rng(100 + seed)
    for (n, d, bm, bn, causal) in SWEEP:
        q = 2 * rng.standard_normal((n, d)); k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d)); s = 1.0 / math.sqrt(d)
        o_ref, lse_ref = oracle.attention_fwd(q, k, v, s, causal)
        o, lse = online_softmax_attention(q, k, v, s, causal=causal, block_m=bm, block_n=bn)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12, err_msg=str((n, d, bm, bn, causal)))
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12, err_msg=str((n, d, bm, bn, causal)))


def test_unequal_lengths_match():
    rng = np.random.default_rng(4)
    for (nq, nk) in [(2, 4), (5, 9), (9, 5), (1, 64)]:
        q = rng.standard_normal((nq, 3)); k = rng.standard_normal((nk, 3)); v = rng.standard_normal((nk, 3))
        for causal in (False, True):
            o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.7, causal)
            o, lse = online_softmax_attention(q, k, v, 0.7, causal=causal, block_m=2, block_n=3)
            np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_round_to_formats():
    # fp16: 1 + 2^-11 is a tie between 1 and 1 + 2^-10 -> even (1.0); 1 + 3*2^-11 -> 1 + 2^-9
    x = np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 1e-8])
    np.testing.assert_array_equal(round_to(x, "f16"), [1.0, 1.0, 1 + 2.0 ** -9, 65504.0, 0.0])
    # bf16 keeps 8 significand bits: 1 + 2^-8 is a tie -> 1.0; 1 + 3*2^-8 -> 1 + 2^-6
    # and 3 + 2^-7 is a tie between 3 (even) and 3 + 2^-6
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 3 + 2.0 ** -7, 3 + 2.0 ** -7 + 2.0 ** -12])
    np.testing.assert_array_equal(round_to(x, "bf16"), [1.0, 1.0, 1 + 2.0 ** -6, -2.5, 3.0, 3 + 2.0 ** -6])
    assert np.isnan(round_to(np.array([np.nan]), "bf16")[0])
