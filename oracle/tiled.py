"""Tiled online-softmax attention in numpy fp64 — TEST INFRASTRUCTURE ONLY.

Follows the FA2 forward loop order of "CUDA 算子工程" ch. 14 §14.5 (outer loop
over query blocks, inner loop over key/value blocks, one normalisation at the end)
with the per-row state and recurrence of "用 CuTe 读懂 FlashAttention", step 4
(Table 2 and the equations for alpha, l' and U'):

    m  : running maximum of the RAW scores x_j (not yet multiplied by s)
    l  : sum_j exp(s (x_j - m))
    U  : sum_j exp(s (x_j - m)) v_j            (unnormalised output numerator)
    m' = max(m, max_{j in block} x_j)
    alpha = exp(s (m - m'))
    l' = alpha l + sum_{j in block} exp(s (x_j - m'))
    U' = alpha U + sum_{j in block} exp(s (x_j - m')) v_j
    finally O = U / l and LSE = s m + log l   (the blog's final section)

Masked positions (causal k > q, top-left aligned, per the blog's causal section)
score -inf. When a row's running maximum is still -inf after a block, the
exponent base is taken as 0 so that exp(-inf - (-inf)) never appears, the guard
ch. 14 §14.5 asks for in its pseudocode comment.

Optionally the roundings a 16-bit GPU kernel performs can be switched on: the
block weights E are rounded to fp16/bf16 (through fp32, round-to-nearest-even)
before the E @ V product, and O is rounded at the end. l is always summed from
the unrounded weights. This is used only to predict the GPU's error floor.

This module shares no code with the C oracle or with the HIP path.
"""
from __future__ import annotations

import numpy as np


def round_to(x: np.ndarray, fmt: str | None) -> np.ndarray:
    """Round fp64 values through fp32 to fp16 or bf16 (RNE) and back to fp64."""
    if fmt is None:
        return x
    x32 = np.asarray(x, dtype=np.float32)
    if fmt == "f16":
        return x32.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        is_nan = np.isnan(x32)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        out = u.astype(np.uint32).view(np.float32).astype(np.float64)
        out[is_nan] = np.nan
        return out
    raise ValueError(f"unknown rounding format {fmt!r}")


def online_softmax_attention(q, k, v, s: float, causal: bool = False, block_m: int = 64,
                             block_n: int = 64, p_round: str | None = None,
                             o_round: str | None = None, trace: bool = False):
    """One (batch, head) slice: q [Nq, d], k and v [Nk, d] -> (O [Nq, d], LSE [Nq]).

    With ``trace=True`` also returns a list with one dict per (query block, key block)
    step holding that step's raw scores S, weights E, alpha, l, U (after the update)
    and the running maximum m, so that the per-round figures can be compared.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, d = q.shape
    nk = k.shape[0]
    o = np.zeros((nq, d))
    lse = np.full((nq,), -np.inf)
    steps = []
    for q0 in range(0, nq, block_m):
        qb = q[q0:q0 + block_m]
        rows = np.arange(q0, q0 + qb.shape[0])
        m = np.full((qb.shape[0],), -np.inf)
        l = np.zeros((qb.shape[0],))
        u = np.zeros((qb.shape[0], d))
        for k0 in range(0, nk, block_n):
            kb = k[k0:k0 + block_n]
            vb = v[k0:k0 + block_n]
            cols = np.arange(k0, k0 + kb.shape[0])
            x = qb @ kb.T                                    # raw scores of this block
            if causal:
                x = np.where(cols[None, :] <= rows[:, None], x, -np.inf)
            m_new = np.maximum(m, x.max(axis=1))
            base = np.where(np.isneginf(m_new), 0.0, m_new)  # -inf guard
            e = np.exp(s * (x - base[:, None]))
            alpha = np.exp(s * (m - base))
            l = alpha * l + e.sum(axis=1)
            u = alpha[:, None] * u + round_to(e, p_round) @ vb
            m = m_new
            if trace:
                steps.append(dict(q0=q0, k0=k0, S=x.copy(), E=e.copy(), alpha=alpha.copy(),
                                  m=m.copy(), l=l.copy(), U=u.copy()))
        safe_l = np.where(l > 0, l, 1.0)
        ob = np.where((l > 0)[:, None], u / safe_l[:, None], 0.0)
        o[q0:q0 + qb.shape[0]] = round_to(ob, o_round)
        lse[q0:q0 + qb.shape[0]] = np.where(l > 0, s * m + np.log(safe_l), -np.inf)
    if trace:
        return o, lse, steps
    return o, lse
