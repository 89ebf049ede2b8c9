"""Seeded random shapes through the general entry points, against the fp64 oracle.

The dedicated tests cover each feature on its own grid; this sweep draws their
combinations: batch, query heads over K/V heads (grouped or not), query and key
lengths (ragged, N_q above and below N_k, the packed few-row decoding range), head
size, dtype, causal mask, split count, tile, and q/o layouts ([B, H, N, d], [B, N,
H, d], padded rows). Every case is also run backward through fa_bwd_ex when the
layout is contiguous. Tolerances as in the other parity tests: forward max |dO| <=
2e-3 (fp16) / 1e-2 (bf16) and max |dLSE| <= 1e-3; backward max|d| <= 8 u max|ref| per
gradient. Shapes stay small enough for the oracle (a few seconds in all).
"""
import math
import random
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
import oracle
from grad_tolerance import check_grad

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
TOL_O = {"f16": 2e-3, "bf16": 1e-2}
DEV = torch.device("cuda:0")
TILES = [(64, 64), (128, 64), (128, 32), (256, 32), (256, 64)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def _draw(rng):
    d = rng.choice([64, 128])
    dtype = rng.choice(["f16", "bf16"])
    hk = rng.choice([1, 2, 3])
    group = rng.choice([1, 1, 2, 4, 5])
    B = rng.choice([1, 2, 3])
    nq = rng.choice([1, 2, 3, 7, 16, 31, 33, 63, 64, 65, 100, 129, 257])
    nk = rng.choice([1, 5, 31, 64, 65, 127, 200, 333, 700])
    causal = rng.random() < 0.5
    layout = rng.choice(["bhnd", "bhnd", "bnhd", "padded"])
    splits = rng.choice([None, 1, 2, 3, 7])
    tile = rng.choice([None, None] + [t for t in TILES if fa.fa_tile_supported(d, *t)])
    return dict(B=B, hq=hk * group, hk=hk, nq=nq, nk=nk, d=d, dtype=dtype, causal=causal, layout=layout,
                splits=splits, tile=tile)


def _place(t, layout):
    """A GPU copy of t [B, H, N, d] stored in the given layout (same logical values)."""
    if layout == "bhnd":
        return t.to(DEV)
    if layout == "bnhd":
        return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    buf = torch.zeros(t.shape[:3] + (t.shape[3] + 8,), dtype=t.dtype)
    buf[..., : t.shape[3]] = t
    return buf.to(DEV)[..., : t.shape[3]]


def _empty_like_layout(shape, dtype, layout):
    B, H, N, d = shape
    if layout == "bnhd":
        return torch.empty((B, N, H, d), dtype=dtype, device=DEV).transpose(1, 2)
    if layout == "padded":
        return torch.empty((B, H, N, d + 8), dtype=dtype, device=DEV)[..., :d]
    return torch.empty(shape, dtype=dtype, device=DEV)


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(seed):
    rng = random.Random(1000 + seed)
    for case in range(8):
        c = _draw(rng)
        B, hq, hk, nq, nk, d, dtype = c["B"], c["hq"], c["hk"], c["nq"], c["nk"], c["d"], c["dtype"]
        scale = 1 / math.sqrt(d)
        _say(f"[random] seed={seed} case={case} {c}")
        g = torch.Generator("cpu").manual_seed(seed * 100 + case)
        q = torch.randn((B, hq, nq, d), generator=g).to(TORCH_DT[dtype])
        k = torch.randn((B, hk, nk, d), generator=g).to(TORCH_DT[dtype])
        v = (torch.randn((B, hk, nk, d), generator=g) * 0.5).to(TORCH_DT[dtype])
        grp = hq // hk
        kr, vr = k.repeat_interleave(grp, dim=1), v.repeat_interleave(grp, dim=1)
        o_ref, l_ref = oracle.attention_fwd(q.double().numpy(), kr.double().numpy(), vr.double().numpy(), scale,
                                            c["causal"], align="bottom-right")
        qd, kd, vd = _place(q, c["layout"]), k.to(DEV), v.to(DEV)
        out = _empty_like_layout(q.shape, q.dtype, c["layout"])
        bm, bn = c["tile"] if c["tile"] else (None, None)
        if c["splits"] is None:
            o, lse = fa.fwd_ex(qd, kd, vd, scale=scale, causal=c["causal"], block_m=bm, block_n=bn, out=out)
        else:
            o, lse = fa.fwd_split(qd, kd, vd, scale=scale, causal=c["causal"], num_splits=c["splits"], block_m=bm,
                                  block_n=bn, out=out)
        torch.cuda.synchronize()
        o_g, l_g = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(l_g), empty), "rows without a visible key differ"
        assert np.all(o_g[empty] == 0.0)
        err_o = np.abs(o_g - o_ref).max()
        err_l = np.abs(l_g[~empty] - l_ref[~empty]).max() if (~empty).any() else 0.0
        _say(f"[random]   fwd max|dO|={err_o:.2e} max|dLSE|={err_l:.2e}")
        assert err_o <= TOL_O[dtype] and err_l <= 1e-3
        if c["layout"] != "bhnd":
            continue
        # backward on the same inputs (contiguous tensors)
        do = torch.randn((B, hq, nq, d), generator=g).to(TORCH_DT[dtype])
        o2, lse2 = fa.fwd_ex(qd, kd, vd, scale=scale, causal=c["causal"])
        dq, dk, dv = fa.bwd_ex(qd, kd, vd, o2, do.to(DEV), lse2, scale=scale, causal=c["causal"])
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_bwd(q.double().numpy(), kr.double().numpy(), vr.double().numpy(),
                                          do.double().numpy(), scale, c["causal"], align="bottom-right")
        rk = rk.reshape(B, hk, grp, nk, d).sum(axis=2)
        rv = rv.reshape(B, hk, grp, nk, d).sum(axis=2)
        res = [check_grad(name, got.float().cpu().double().numpy(), ref, dtype, f"random seed {seed} case {case}")
               for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))]
        _say("[random]   bwd errors in u (normalised / big-entry relative): "
             + " ".join(f"{n} {a:.2f}/{b:.2f}" for n, (a, b) in zip(("dq", "dk", "dv"), res)))
