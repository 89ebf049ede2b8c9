"""GPU checks at the largest key count the library accepts (the 32-bit byte range of
one K/V slice: (N + 512) * row stride < 2^30 elements), through the C ABI.

At this size the oracle's own pass over 8-17 million keys per row would dominate, so
the inputs are built so that the exact result has a closed form that holds at any
size (the definition of attention, evaluated by hand):

- Q = 0: every visible key gets the same weight, so O is the mean of V over the keys
  and LSE = ln N_k. V[j, c] = ((j + c) mod 7 - 3) / 4 is exact in both 16-bit types,
  so the mean is a sum of residue counts. Every key of the range must be read once.
- K = 0 except the last key, which aligns with q: that key's score z = 40 dominates
  every other weight (e^-40 N_k < 1e-10), so O = V[last] and
  LSE = z + ln(1 + (N_k - 1) e^-z). The last key sits at the top of the addressable
  range.

Both the unsplit general entry point (packed decoding: one query row for each of 4
query heads over one K/V head) and split-KV at the suggested count are checked; both
must accept this N_k (the binding raises on any other status). That N_k + 1 is
refused is checked without a GPU, in the boundary tests.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
from grad_tolerance import NORM_U, check_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
TOL_O = {"f16": 2e-3, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def _max_keys(d):
    return (1 << 30) // d - 512 - 1


def _pattern_v(nk, d, dtype):
    table = torch.tensor([[((r + c) % 7 - 3) / 4 for c in range(d)] for r in range(7)], dtype=torch.float32)
    idx = torch.arange(nk, device=DEV) % 7
    return table.to(DEV).to(TORCH_DT[dtype])[idx].reshape(1, 1, nk, d)


def _pattern_mean(nk, d):
    """Mean over j < nk of ((j + c) mod 7 - 3) / 4, per column c, from residue counts."""
    out = np.zeros(d)
    for c in range(d):
        tot = 0.0
        for r in range(7):
            cnt = nk // 7 + (1 if (r - c) % 7 < nk % 7 else 0)   # j = r - c (mod 7)
            tot += cnt * (r - 3) / 4
        out[c] = tot / nk
    return out


def _run(q, k, v, splits, scale):
    if splits is None:
        return fa.fwd_ex(q, k, v, scale=scale, causal=False)
    return fa.fwd_split(q, k, v, scale=scale, causal=False, num_splits=splits)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_largest_key_count(d, dtype):
    nk = _max_keys(d)
    scale = 1 / math.sqrt(d)
    hq = 4
    print(f"[limits] d={d} {dtype} Nk={nk}", flush=True)
    k = torch.zeros((1, 1, nk, d), dtype=TORCH_DT[dtype], device=DEV)
    v = _pattern_v(nk, d, dtype)
    suggested = fa.fa_split_default(1, hq, 1, 1, nk, d, False)
    assert suggested > 1

    # Q = 0: uniform weights
    q = torch.zeros((1, hq, 1, d), dtype=TORCH_DT[dtype], device=DEV)
    mean = _pattern_mean(nk, d)
    for splits in (None, suggested):
        o, lse = _run(q, k, v, splits, scale)
        torch.cuda.synchronize()
        err_o = np.abs(o.float().cpu().double().numpy()[0, :, 0] - mean[None, :]).max()
        err_l = np.abs(lse.cpu().double().numpy() - math.log(nk)).max()
        print(f"[limits]   Q=0 splits={splits}: max|dO| {err_o:.2e} max|dLSE| {err_l:.2e}", flush=True)
        assert err_o <= TOL_O[dtype] and err_l <= 1e-3

    # one dominant key at the top of the range
    t = 40.0 / scale                             # stored rounded to the dtype; z is taken from that value
    k[0, 0, nk - 1, 0] = t
    t16 = float(k[0, 0, nk - 1, 0].float())
    q[..., 0] = 1.0
    z = scale * t16
    lse_ref = z + math.log1p((nk - 1) * math.exp(-z))
    v_last = v[0, 0, nk - 1].float().cpu().double().numpy()
    for splits in (None, suggested):
        o, lse = _run(q, k, v, splits, scale)
        torch.cuda.synchronize()
        err_o = np.abs(o.float().cpu().double().numpy()[0, :, 0] - v_last[None, :]).max()
        err_l = np.abs(lse.cpu().double().numpy() - lse_ref).max()
        print(f"[limits]   last key splits={splits}: max|dO| {err_o:.2e} max|dLSE| {err_l:.2e}", flush=True)
        assert err_o <= TOL_O[dtype] and err_l <= 1e-3
    del k, v
    torch.cuda.empty_cache()



def test_backward_largest_key_count():
    """fa_bwd_ex at the largest accepted key count (d = 128, bf16; with fp16 the weights
    1/N_k ~ 1e-7 would be subnormal), 4 query heads of 64 rows over one K/V head,
    against closed forms that hold at any size. Q = 0 makes every weight 1/N_k, so
    dV_j = (1/N_k) sum of dO over the group's rows for every key, dK = 0 exactly, and
    dQ_i = (s/N_k) sum_j (dO_i . (v_j - vbar)) k_j. K and V are periodic in j mod 7
    (v_j as above, k_j[c] = ((2 j + 3 c) mod 7 - 3) / 4), so the sums over j are residue
    counts."""
    d, dtype, hq, nq = 128, "bf16", 4, 64
    nk = _max_keys(d)
    scale = 1 / math.sqrt(d)
    print(f"[limits] backward d={d} {dtype} Nk={nk}", flush=True)
    idx = torch.arange(nk, device=DEV) % 7
    v7 = np.array([[((a + c) % 7 - 3) / 4 for c in range(d)] for a in range(7)])
    k7 = np.array([[((2 * a + 3 * c) % 7 - 3) / 4 for c in range(d)] for a in range(7)])
    v = torch.tensor(v7, dtype=torch.float32, device=DEV).to(TORCH_DT[dtype])[idx].reshape(1, 1, nk, d)
    k = torch.tensor(k7, dtype=torch.float32, device=DEV).to(TORCH_DT[dtype])[idx].reshape(1, 1, nk, d)
    del idx
    q = torch.zeros((1, hq, nq, d), dtype=TORCH_DT[dtype], device=DEV)
    g = torch.Generator("cpu").manual_seed(77)
    do = torch.randn((1, hq, nq, d), generator=g).to(TORCH_DT[dtype])
    o, lse = fa.fwd_split(q, k, v, scale=scale)
    dq, dk, dv = fa.bwd_ex(q, k, v, o, do.to(DEV), lse, scale=scale)
    torch.cuda.synchronize()
    cnt = np.array([nk // 7 + (1 if a < nk % 7 else 0) for a in range(7)], dtype=np.float64)
    vbar = (cnt[:, None] * v7).sum(0) / nk
    # the forward on the way: O = mean of V, LSE = ln N_k
    assert np.abs(o.float().cpu().double().numpy() - vbar).max() <= TOL_O[dtype]
    assert np.abs(lse.cpu().double().numpy() - math.log(nk)).max() <= 1e-3
    dod = do.double().numpy()[0]                                   # [hq, nq, d]
    dv_ref = dod.sum(axis=(0, 1)) / nk                             # the same row for every key
    ksum = (cnt[:, None] * k7).sum(0)
    proj = np.einsum("hid,ad->hia", dod, v7)                       # dO_i . v7[a]
    dq_ref = scale / nk * (np.einsum("hia,a,ad->hid", proj, cnt, k7) - (dod @ vbar)[..., None] * ksum)
    assert torch.count_nonzero(dk) == 0
    u = 2.0 ** -8
    for name, got, ref in (("dq", dq[0].float().cpu().double().numpy(), dq_ref),
                           ("dv", None, dv_ref)):
        if name == "dv":
            # every key's row: check the first, the last and a sample in between
            rows = torch.tensor([0, 1, 2, 3, nk // 2, nk - 2, nk - 1], device=DEV)
            got = dv[0, 0, rows].float().cpu().double().numpy()
            ref = np.broadcast_to(ref, got.shape)
            spread = (dv[0, 0].float().amax(dim=0) - dv[0, 0].float().amin(dim=0)).abs().max().item()
            print(f"[limits]   dv spread over all keys {spread:.2e}", flush=True)
            assert spread <= NORM_U * u * np.abs(ref).max()
        norm, rel = check_grad(name, got, ref, "bf16", "largest key count")
        print(f"[limits]   {name}: errors in u (normalised / big-entry relative) {norm:.2f}/{rel:.2f}", flush=True)
    del k, v, dk, dv
    torch.cuda.empty_cache()
