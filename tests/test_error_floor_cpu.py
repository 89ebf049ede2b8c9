"""Predicted GPU error floor per workload, from the tiled emulator with the kernel's
two 16-bit roundings switched on (CPU only).

The kernel keeps scores, weights, row sums and the output numerator in fp32, and
rounds twice: the weights P to the input type before the P V product (the in-register
downcast of "用 CuTe 读懂 FlashAttention" step 5) and O once at the end (its final
section). ``oracle.tiled.online_softmax_attention`` with ``p_round`` and ``o_round``
performs exactly those two roundings in otherwise exact (fp64) arithmetic, so its
distance from the fp64 oracle is the error the roundings alone cause: the floor the
GPU result sits on (fp32 accumulation adds far less). The notes of the pwwt.cn
FlashAttention-forward page advise this CPU simulation of the tiling and of the
fp16/fp32 split before trusting a kernel (§7, §6.2).

Rows: the tight ones of each workload. Under a causal mask the first rows average
only a handful of values, so |O| is largest there and the output rounding (half an
ulp of |O|) dominates; for the N = 16384 workload the spiked rows (1% of Q rows x20),
whose running maximum jumps and forces the alpha rescaling. The test prints the
prediction per workload and asserts that it stays below the parity tolerance of
the target contract (2e-3 fp16, 1e-2 bf16).
"""
import numpy as np
import pytest

import oracle
from exact_attention_forward_fwd_amd.workloads import WORKLOADS, make_inputs
from oracle.tiled import online_softmax_attention

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3


def _f64(t):
    return t.double().numpy()


def _predict(idx):
    """(max|dO|, max|dLSE|, rows compared) of the rounding emulator against the oracle."""
    w = WORKLOADS[idx]
    q, k, v, spikes = make_inputs(w)
    q, k, v = _f64(q), _f64(k), _f64(v)
    bm, bn = w.tile if w.tile else (128, 64 if (not w.causal or w.d == 64) else 32)
    err_o = err_l = 0.0
    n_rows = 0
    for b in range(w.B):
        for h in range(w.H):
            if spikes.numel():
                rows = np.concatenate([np.sort(spikes[b, h].numpy()), np.arange(64)])
            elif w.causal:
                rows = np.arange(64)                      # the shortest causal rows
            else:
                rows = np.arange(min(w.N, 128))
            # a causal row i sees keys 0..i: the emulator is given the row prefix itself
            qs = q[b, h, :rows.max() + 1] if w.causal else q[b, h, rows]
            o_e, l_e = online_softmax_attention(qs, k[b, h], v[b, h], w.scale, w.causal, block_m=bm,
                                                block_n=bn, p_round=w.dtype, o_round=w.dtype)
            if w.causal:
                o_e, l_e = o_e[rows], l_e[rows]
            flat = (b * w.H + h) * w.N + rows
            o_r, l_r = oracle.attention_rows(q, k, v, w.scale, w.causal, flat)
            err_o = max(err_o, float(np.abs(o_e - o_r).max()))
            err_l = max(err_l, float(np.abs(l_e - l_r).max()))
            n_rows += rows.size
    return err_o, err_l, n_rows


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_predicted_error_floor_below_tolerance(idx):
    w = WORKLOADS[idx]
    err_o, err_l, n = _predict(idx)
    print(f"[floor] {w.name}: predicted max|dO| = {err_o:.4e} (tol {TOL_O[w.dtype]}, "
          f"{100 * err_o / TOL_O[w.dtype]:.0f}% of it), max|dLSE| = {err_l:.2e}, over {n} rows")
    # the roundings are on: the floor is not zero, and it is below the contract
    assert err_o > 0.0
    assert err_o < TOL_O[w.dtype], f"{w.name}: the roundings alone exceed the tolerance"
    assert err_l < TOL_LSE
