"""GPU parity of split-KV (fa_fwd_split, through the C ABI) and of decoding with grouped
K/V heads (fewer than 64 query rows per head, the heads of a group packed into one
slice per K/V head) against the fp64 CPU oracle.

Tolerances as in test_parity_gpu.py (max |dO| <= 2e-3 fp16, <= 1e-2 bf16, max
|dLSE| <= 1e-3). Split-KV computes the same attention: every key range's partial
output and LSE come from the same tile loop, and the merge combines them in fp32, so
the bound is the same. V ~ N(0, 0.5^2) as in test_general_gpu.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
import oracle
from exact_attention_forward_fwd_amd.workloads import SPLIT_WORKLOADS, make_general_inputs

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEV = torch.device("cuda:0")
_CACHE = {}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def _rand(shape, dtype, seed, std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(TORCH_DT[dtype])


def _qkv(B, hq, hk, nq, nk, d, dtype, seed):
    return (_rand((B, hq, nq, d), dtype, seed), _rand((B, hk, nk, d), dtype, seed + 1),
            _rand((B, hk, nk, d), dtype, seed + 2, std=0.5))


def _reference(q, k, v, scale, causal):
    g = q.shape[1] // k.shape[1]
    return oracle.attention_fwd(q.double().numpy(), k.repeat_interleave(g, dim=1).double().numpy(),
                                v.repeat_interleave(g, dim=1).double().numpy(), scale, causal, align="bottom-right")


def _compare(o, lse, ref, dtype, label):
    o_g = o.float().cpu().double().numpy()
    l_g = lse.cpu().double().numpy()
    o_ref, l_ref = ref
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_g), empty), f"{label}: rows without a visible key differ"
    assert np.all(o_g[empty] == 0.0), f"{label}: rows without a visible key must give O = 0"
    err_o = np.abs(o_g - o_ref).max() if o_g.size else 0.0
    err_l = np.abs(l_g[~empty] - l_ref[~empty]).max() if (~empty).any() else 0.0
    _say(f"[split]   max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} rows without keys={int(empty.sum())}")
    assert err_o <= TOL_O[dtype], f"{label}: max|dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{label}: max|dLSE| = {err_l}"


def check_split(q, k, v, scale, causal, dtype, splits, tile=None, label="", ref=None):
    _say(f"[split] {label} q={tuple(q.shape)} k={tuple(k.shape)} {dtype} causal={causal} splits={splits} tile={tile}")
    bm, bn = tile if tile else (None, None)
    ws_bytes = fa.fa_split_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3], splits) if splits else 0
    # the workspace's previous contents must not matter
    ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = fa.fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal, num_splits=splits,
                          block_m=bm, block_n=bn, workspace=ws if splits else None)
    torch.cuda.synchronize()
    _compare(o, lse, ref if ref is not None else _reference(q, k, v, scale, causal), dtype, label)


@pytest.mark.parametrize("nq,nk", [(1, 4096), (64, 4096), (300, 1000), (1000, 1000), (37, 515), (128, 64),
                                   (300, 100)])
@pytest.mark.parametrize("splits", [2, 3, 7, 64])
def test_split_matches_oracle(nq, nk, splits):
    for d, dtype, tiles in ((64, "f16", (None, (128, 64), (256, 64))), (128, "bf16", (None, (128, 32), (128, 64), (256, 32), (256, 64)))):
        q, k, v = _qkv(2, 2, 2, nq, nk, d, dtype, seed=nq + 7 * nk + d + splits)
        for tile in tiles:
            for causal in (False, True):
                check_split(q, k, v, 1 / math.sqrt(d), causal, dtype, splits, tile, label=f"Nq={nq} Nk={nk}")


@pytest.mark.parametrize("hq,hk", [(8, 2), (6, 3), (4, 4)])
def test_split_grouped_heads(hq, hk):
    for d, dtype in ((64, "f16"), (128, "bf16")):
        q, k, v = _qkv(2, hq, hk, 200, 2000, d, dtype, seed=hq + hk + d)
        for causal in (False, True):
            check_split(q, k, v, 1 / math.sqrt(d), causal, dtype, 5, label=f"gqa {hq}/{hk}")


def _workload(idx):
    """Inputs and full oracle result of a split-KV benchmark workload (cached)."""
    if idx not in _CACHE:
        w = SPLIT_WORKLOADS[idx]
        q, k, v = make_general_inputs(w)
        _CACHE[idx] = (w, q, k, v, _reference(q, k, v, w.scale, w.causal))
    return _CACHE[idx]


@pytest.mark.parametrize("splits", [None, 1, 16, 256])
def test_decode_long_context(splits):
    """The decoding benchmark workload: one query row per head against 128K keys, 32
    query heads on 8 K/V heads (the long-context decoding case of the chapter on
    IO-aware attention, §14.7.1). None = the suggested split count, which the
    benchmark times; every row against the oracle."""
    w, q, k, v, ref = _workload(6)
    s = splits if splits is not None else fa.fa_split_default(w.B, w.Hq, w.Hk, w.Nq, w.Nk, w.d, w.causal)
    check_split(q, k, v, w.scale, w.causal, w.dtype, s, label=f"{w.name} default={splits is None}", ref=ref)


@pytest.mark.parametrize("splits", [None, 1, 4])
def test_shard_workload(splits):
    """The one-GPU share of the N = 16384 workload (2 heads): every row against the oracle,
    in the launch configuration the benchmark times (None = suggested splits)."""
    w, q, k, v, ref = _workload(7)
    s = splits if splits is not None else fa.fa_split_default(w.B, w.Hq, w.Hk, w.Nq, w.Nk, w.d, w.causal)
    check_split(q, k, v, w.scale, w.causal, w.dtype, s, label=f"{w.name} default={splits is None}", ref=ref)


def test_split_one_is_fwd_ex_bitwise():
    q, k, v = _qkv(2, 4, 2, 515, 777, 128, "bf16", seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o1, l1 = fa.fwd_ex(qd, kd, vd, scale=0.1, causal=causal)
        o2, l2 = fa.fwd_split(qd, kd, vd, scale=0.1, causal=causal, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_is_deterministic_and_ignores_workspace_contents():
    q, k, v = _qkv(1, 4, 4, 256, 3000, 64, "f16", seed=4)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n = fa.fa_split_workspace_bytes(1, 4, 256, 64, 6) // 4
    outs = []
    for fill in (0.0, float("nan"), float("inf"), -1e30):
        ws = torch.full((n,), fill, dtype=torch.float32, device=DEV)
        outs.append(fa.fwd_split(qd, kd, vd, causal=True, num_splits=6, workspace=ws))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


@pytest.mark.parametrize("layout", ["bhnd", "bnhd", "padded"])
@pytest.mark.parametrize("hq,hk", [(8, 2), (32, 8), (4, 1), (3, 3)])
def test_decode_grouped_heads_fwd_ex(layout, hq, hk):
    """Nq = 1 with grouped heads: the query heads of a group are processed as the rows
    of one block (any q/o layout: their rows are one head stride apart)."""
    for d, dtype in ((64, "f16"), (128, "bf16")):
        q, k, v = _qkv(2, hq, hk, 1, 3000, d, dtype, seed=hq * 3 + hk + d)
        if layout == "bhnd":
            qd = q.to(DEV)
            out = torch.empty_like(qd)
        elif layout == "bnhd":
            qd = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
            out = torch.empty((2, 1, hq, d), dtype=q.dtype, device=DEV).transpose(1, 2)
        else:
            buf = torch.zeros((2, hq, 1, d + 8), dtype=q.dtype)
            buf[..., :d] = q
            qd = buf.to(DEV)[..., :d]
            out = torch.zeros((2, hq, 1, d + 8), dtype=q.dtype, device=DEV)[..., :d]
        for causal in (False, True):
            _say(f"[decode] {layout} hq={hq} hk={hk} d={d} causal={causal}")
            o, lse = fa.fwd_ex(qd, k.to(DEV), v.to(DEV), scale=1 / math.sqrt(d), causal=causal, out=out)
            torch.cuda.synchronize()
            _compare(o, lse, _reference(q, k, v, 1 / math.sqrt(d), causal), dtype, f"decode {layout}")


_TILES = [(64, 64), (128, 64), (128, 32), (256, 32), (256, 64)]


@pytest.mark.parametrize("nq,nk", [(2, 1500), (4, 1500), (7, 1500), (33, 1500), (63, 1500), (64, 1500), (33, 20)])
@pytest.mark.parametrize("hq,hk", [(8, 2), (32, 8), (4, 1)])
def test_decode_grouped_heads_several_rows(nq, nk, hq, hk):
    """A few query rows per head (draft tokens) with grouped heads. With fewer than 64
    rows and head-contiguous q and o the heads of a group are packed into one slice per
    K/V head, and the bottom-right causal mask takes row mod Nq as the query index; 64
    rows and the [B, N, H, d] layout run unpacked. Both against the oracle: unsplit
    (default and every compiled tile), split-KV at the suggested count and at 5 ranges.
    (33, 20) has causal rows that see no key."""
    for d, dtype in ((64, "f16"), (128, "bf16")):
        scale = 1 / math.sqrt(d)
        q, k, v = _qkv(2, hq, hk, nq, nk, d, dtype, seed=nq * 7 + hq + hk + d + nk)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        for causal in (False, True):
            ref = _reference(q, k, v, scale, causal)
            _say(f"[rows] nq={nq} nk={nk} hq={hq} hk={hk} d={d} causal={causal}")
            o, lse = fa.fwd_ex(qd, kd, vd, scale=scale, causal=causal)
            torch.cuda.synchronize()
            _compare(o, lse, ref, dtype, f"rows nq={nq} default tile")
            for bm, bn in _TILES:
                if fa.fa_tile_supported(d, bm, bn):
                    o, lse = fa.fwd_ex(qd, kd, vd, scale=scale, causal=causal, block_m=bm, block_n=bn)
                    torch.cuda.synchronize()
                    _compare(o, lse, ref, dtype, f"rows nq={nq} tile ({bm},{bn})")
            for splits in (None, 5):
                check_split(q, k, v, scale, causal, dtype, splits, label=f"rows nq={nq}", ref=ref)
            # [B, N, H, d] storage: head stride d, not Nq rows, so the heads are not packed
            qt = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
            out = torch.empty((2, nq, hq, d), dtype=q.dtype, device=DEV).transpose(1, 2)
            o, lse = fa.fwd_ex(qt, kd, vd, scale=scale, causal=causal, out=out)
            torch.cuda.synchronize()
            _compare(o, lse, ref, dtype, f"rows nq={nq} bnhd")
