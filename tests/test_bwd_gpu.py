"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the fp64 CPU
oracle's gradients on the very 16-bit inputs the GPU received.

The contract is fa_fwd's: o and lse come from fa_fwd on the same q, k, v (the
backward recomputes P from lse and uses o for the row sums D = dO . O).

Tolerance: grad_tolerance.check_grad (a normalised bound per gradient tensor and an
element-wise relative bound on its large entries, both in units of the dtype's unit
roundoff u, derived from the arithmetic). The tests print the measured errors in u.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
import oracle
from exact_attention_forward_fwd_amd.workloads import WORKLOADS, make_inputs
from grad_tolerance import U, check_grad

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def _rand(shape, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(TORCH_DT[dtype])


def run_bwd(q, k, v, do, scale, causal, ws_fill=None):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    ws = None
    if ws_fill is not None:
        B, H, N, _ = q.shape
        ws = torch.full((max(fa.fa_bwd_workspace_bytes(B, H, N), 16) // 4,), ws_fill, dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(q, k, v, do, scale, causal, dtype, label):
    _say(f"[bwd] {label} shape={tuple(q.shape)} {dtype} causal={causal}")
    got = run_bwd(q, k, v, do, scale, causal)
    ref = oracle.attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                               scale, causal)
    res = [check_grad(name, g.float().cpu().double().numpy(), r, dtype, label)
           for name, g, r in zip(("dq", "dk", "dv"), got, ref)]
    _say("[bwd]   errors in u (normalised / big-entry relative): "
         + " ".join(f"{n} {a:.2f}/{b:.2f}" for n, (a, b) in zip(("dq", "dk", "dv"), res)))


@pytest.mark.parametrize("n", [1, 17, 32, 64, 100, 129, 300, 513])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_sizes(n, d):
    for dtype in ("f16", "bf16"):
        for causal in (False, True):
            seed = 7 * n + d + (1 if causal else 0)
            q, k, v, do = (_rand((1, 2, n, d), dtype, seed + i) for i in range(4))
            check(q, k, v, do, 1 / math.sqrt(d), causal, dtype, f"N={n} d={d}")


@pytest.mark.parametrize("idx", [2, 3, 5])
def test_bwd_workloads(idx):
    """The forward benchmark workloads, with dO ~ N(0, 1) of the same shape: every
    gradient element against the oracle."""
    w = WORKLOADS[idx]
    q, k, v, _ = make_inputs(w)
    do = _rand(q.shape, w.dtype, 5000 + idx)
    check(q, k, v, do, w.scale, w.causal, w.dtype, w.name)


def test_bwd_deterministic_and_ignores_workspace_contents():
    q, k, v, do = (_rand((2, 3, 700, 64), "f16", 90 + i) for i in range(4))
    runs = [run_bwd(q, k, v, do, 0.125, True, ws_fill=f) for f in (0.0, float("nan"), 1e30)]
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_bwd_uniform_weights_closed_form():
    """Q = 0 makes every valid key's weight 1/n_i: dV_j = sum_i dO_i / n_i over the rows
    that see key j, and dK = 0 exactly."""
    n, d = 200, 64
    q = torch.zeros((1, 1, n, d), dtype=torch.float16)
    k, v, do = (_rand((1, 1, n, d), "f16", 300 + i) for i in range(3))
    for causal in (False, True):
        dq, dk, dv = run_bwd(q, k, v, do, 0.125, causal)
        dof = do[0, 0].double().numpy()
        ev = np.zeros((n, d))
        for i in range(n):
            keys = np.arange(i + 1) if causal else np.arange(n)
            ev[keys] += dof[i] / len(keys)
        assert torch.count_nonzero(dk) == 0
        check_grad("dv", dv[0, 0].float().cpu().double().numpy(), ev, "f16", "uniform weights")


def check_ex(B, hq, hk, nq, nk, d, dtype, causal, seed, label):
    """fa_bwd_ex against the oracle on K/V repeated per query head (the definition of
    the grouping); the gradient of a shared K/V head is the sum over its query heads."""
    _say(f"[bwd_ex] {label} hq={hq} hk={hk} nq={nq} nk={nk} d={d} {dtype} causal={causal}")
    q, do = _rand((B, hq, nq, d), dtype, seed), _rand((B, hq, nq, d), dtype, seed + 3)
    k, v = _rand((B, hk, nk, d), dtype, seed + 1), _rand((B, hk, nk, d), dtype, seed + 2)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fwd_ex(qd, kd, vd, scale=1 / math.sqrt(d), causal=causal)
    dq, dk, dv = fa.bwd_ex(qd, kd, vd, o, dod, lse, scale=1 / math.sqrt(d), causal=causal)
    torch.cuda.synchronize()
    g = hq // hk
    rq, rk, rv = oracle.attention_bwd(q.double().numpy(), k.repeat_interleave(g, dim=1).double().numpy(),
                                      v.repeat_interleave(g, dim=1).double().numpy(), do.double().numpy(),
                                      1 / math.sqrt(d), causal, align="bottom-right")
    rk = rk.reshape(B, hk, g, nk, d).sum(axis=2)
    rv = rv.reshape(B, hk, g, nk, d).sum(axis=2)
    res = [check_grad(name, gg.float().cpu().double().numpy(), r, dtype, label)
           for name, gg, r in zip(("dq", "dk", "dv"), (dq, dk, dv), (rq, rk, rv))]
    if causal and nq > nk:   # rows that see no key
        assert torch.count_nonzero(dq[:, :, : nq - nk]) == 0
    _say("[bwd_ex]   errors in u (normalised / big-entry relative): "
         + " ".join(f"{n} {a:.2f}/{b:.2f}" for n, (a, b) in zip(("dq", "dk", "dv"), res)))


@pytest.mark.parametrize("hq,hk", [(8, 2), (4, 1), (6, 3)])
def test_bwd_grouped_kv_heads(hq, hk):
    for d, dtype in ((64, "f16"), (128, "bf16")):
        for causal in (False, True):
            check_ex(2, hq, hk, 300, 300, d, dtype, causal, seed=hq * 7 + hk + d, label="gqa")


@pytest.mark.parametrize("nq,nk", [(1, 300), (37, 515), (300, 100), (100, 1), (64, 1000), (513, 129), (129, 513)])
def test_bwd_unequal_lengths(nq, nk):
    for d, dtype in ((64, "f16"), (128, "bf16")):
        for causal in (False, True):
            check_ex(1, 4, 2, nq, nk, d, dtype, causal, seed=nq + 3 * nk + d, label="lengths")


def test_bwd_no_keys_and_no_queries():
    for d in (64, 128):
        q = _rand((1, 2, 50, d), "f16", 1).to(DEV)
        kz = torch.zeros((1, 2, 0, d), dtype=torch.float16, device=DEV)
        o, lse = fa.fwd_ex(q, kz, kz, causal=False)
        dq, dk, dv = fa.bwd_ex(q, kz, kz, o, q.clone(), lse)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dq) == 0 and dk.numel() == 0
        # no queries: dk = dv = 0 for every key
        qz = torch.zeros((1, 2, 0, d), dtype=torch.float16, device=DEV)
        k = _rand((1, 2, 70, d), "f16", 2).to(DEV)
        oz, lz = fa.fwd_ex(qz, k, k, causal=True)
        dk0 = torch.full_like(k, float("nan"))
        dv0 = torch.full_like(k, float("nan"))
        fa.bwd_ex(qz, k, k, oz, qz, lz, causal=True, dk=dk0, dv=dv0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dk0) == 0 and torch.count_nonzero(dv0) == 0


def test_bwd_ex_equals_bwd_when_plain():
    q, k, v, do = (_rand((2, 3, 333, 128), "bf16", 40 + i).to(DEV) for i in range(4))
    for causal in (False, True):
        o, lse = fa.fwd(q, k, v, causal=causal)
        a = fa.bwd(q, k, v, o, do, lse, causal=causal)
        b = fa.bwd_ex(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
