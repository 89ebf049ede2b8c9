"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (written here, from the target contract): max |dO| <= 2e-3 for fp16 and
<= 1e-2 for bf16, max |dLSE| <= 1e-3, both against the oracle evaluated on the very
16-bit inputs the GPU received. The output buffers are pre-filled with NaN, so a
row the kernel fails to write fails the comparison.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
import oracle
from exact_attention_forward_fwd_amd.workloads import WORKLOADS, make_inputs, make_random
from golden_io import load_worked_example

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
ALL_TILES = [(64, 64), (128, 64), (128, 32), (256, 32), (256, 64)]
# tiles of the software-pipelined kernel at d = 128 (all of them) and of the 256-row
# workgroups at d = 64
PP_TILES = [(128, 32), (128, 64), (256, 32), (256, 64)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def run_gpu(q, k, v, scale, causal, tile=None, stream=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    bm, bn = tile if tile else (None, None)
    fa.fwd(qd, kd, vd, scale=scale, causal=causal, block_m=bm, block_n=bn, out=o, lse=lse,
           stream=stream)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def f64(t):
    return t.double().numpy()


def check_against_oracle(q, k, v, scale, causal, dtype, tile=None, rows=None, label=""):
    _say(f"[parity] {label} shape={tuple(q.shape)} {dtype} causal={causal} tile={tile}")
    o, lse = run_gpu(q, k, v, scale, causal, tile)
    B, H, N, d = q.shape
    if rows is None:
        o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), scale, causal)
        o_g, lse_g = o, lse
    else:
        o_ref, lse_ref = oracle.attention_rows(f64(q), f64(k), f64(v), scale, causal, rows)
        o_g, lse_g = o.reshape(-1, d)[rows], lse.reshape(-1)[rows]
        assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten output rows"
    err_o = np.abs(o_g - o_ref).max() if o_g.size else 0.0
    err_l = np.abs(lse_g - lse_ref).max() if lse_g.size else 0.0
    _say(f"[parity]   max|dO|={err_o:.3e} (tol {TOL_O[dtype]}) max|dLSE|={err_l:.3e} (tol {TOL_LSE})")
    assert err_o <= TOL_O[dtype], f"{label}: max|dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{label}: max|dLSE| = {err_l}"
    return o, lse


# --- the blog's worked example, embedded in the ABI's square, d = 64 form --------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [None] + ALL_TILES)
def test_worked_example(dtype, causal, tile):
    g = load_worked_example()
    # embedded in d = 64, or in d = 128 for a tile compiled at d = 128 only
    d = 64 if tile is None or fa.fa_tile_supported(64, *tile) else 128
    Q = torch.zeros(1, 1, 4, d); K = torch.zeros(1, 1, 4, d); V = torch.zeros(1, 1, 4, d)
    Q[0, 0, :2, :2] = torch.tensor(g["Q"]); K[0, 0, :, :2] = torch.tensor(g["K"])
    V[0, 0, :, :2] = torch.tensor(g["V"])
    dt = TORCH_DT[dtype]
    o, lse = run_gpu(Q.to(dt), K.to(dt), V.to(dt), math.log(2.0), causal, tile)
    if causal:
        exp_o = np.vstack([g["causal"]["O"], [[2 / 3, 2 / 3], [1.0, 0.5]]])
        exp_l = [0.0, math.log(3), math.log(3), math.log(4)]
    else:
        exp_o = np.vstack([g["O"], [[1.0, 0.5], [1.0, 0.5]]])
        exp_l = [g["LSE"][0], g["LSE"][1], math.log(4), math.log(4)]
    np.testing.assert_allclose(o[0, 0, :, :2], exp_o, rtol=0, atol=TOL_O[dtype])
    assert np.all(o[0, 0, :, 2:] == 0.0)
    np.testing.assert_allclose(lse[0, 0], exp_l, rtol=0, atol=TOL_LSE)


# --- closed form: Q = 0 gives prefix means (causal) / column means -------------------

@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_query_closed_form(N, d, dtype):
    _, k, v = make_random(1, 2, N, d, dtype, seed=50 + N + d)
    q = torch.zeros_like(k)
    vv = f64(v)
    for causal in (False, True):
        o, lse = run_gpu(q, k, v, 1 / math.sqrt(d), causal)
        if causal:
            cnt = np.arange(1, N + 1)
            exp_o = np.cumsum(vv, axis=2) / cnt[None, None, :, None]
            exp_l = np.broadcast_to(np.log(cnt), lse.shape)
        else:
            exp_o = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
            exp_l = np.full(lse.shape, math.log(N))
        assert np.abs(o - exp_o).max() <= TOL_O[dtype], (N, d, dtype, causal)
        assert np.abs(lse - exp_l).max() <= TOL_LSE, (N, d, dtype, causal)


# --- the five workloads ----------------------------------------------------------------

def _spiked_rows(w, spikes):
    """Flat row indices of the rows scaled x20 in every (b, h) slice."""
    return np.array(sorted((b * w.H + h) * w.N + int(i) for b in range(w.B) for h in range(w.H)
                           for i in spikes[b, h].tolist()), dtype=np.int64)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_full_oracle(idx):
    """Every row of every workload against the full oracle, in the launch configuration
    the benchmark times. For the N = 16384 workload (about 20 s of host time) the
    spiked rows, whose running maximum jumps and forces the alpha rescaling, are also
    reported on their own."""
    w = WORKLOADS[idx]
    q, k, v, spikes = make_inputs(w)
    _say(f"[parity] {w.name}: full oracle over {w.B * w.H * w.N} rows")
    o, lse = check_against_oracle(q, k, v, w.scale, w.causal, w.dtype, tile=w.tile, label=w.name)
    if spikes.numel():
        rows = _spiked_rows(w, spikes)
        o_ref, lse_ref = oracle.attention_rows(f64(q), f64(k), f64(v), w.scale, w.causal, rows)
        err_o = np.abs(o.reshape(-1, w.d)[rows] - o_ref).max()
        err_l = np.abs(lse.reshape(-1)[rows] - lse_ref).max()
        _say(f"[parity]   spiked rows ({rows.size}): max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
        assert err_o <= TOL_O[w.dtype] and err_l <= TOL_LSE


def test_workload_1_default_tile_matches_forced():
    w = WORKLOADS[1]
    q, k, v, _ = make_inputs(w)
    assert fa.fa_default_tile(w.B, w.H, w.N, w.d, w.causal) == (64, 64)
    o1, l1 = run_gpu(q, k, v, w.scale, w.causal, None)
    o2, l2 = run_gpu(q, k, v, w.scale, w.causal, (64, 64))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# --- sizes, ragged tails and tiles -----------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 31, 33, 64, 100, 129, 257, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_edge_sizes(N, d, dtype):
    q, k, v = make_random(2, 3, N, d, dtype, seed=N * 7 + d)
    for causal in (False, True):
        check_against_oracle(q, k, v, 1 / math.sqrt(d), causal, dtype, label=f"edge N={N}")


@pytest.mark.parametrize("tile", ALL_TILES)
@pytest.mark.parametrize("d", [64, 128])
def test_every_tile_shape(tile, d):
    if not fa.fa_tile_supported(d, *tile):
        pytest.skip(f"tile {tile} is not compiled for d={d}")
    for dtype in ("f16", "bf16"):
        q, k, v = make_random(1, 4, 333, d, dtype, seed=tile[0] + d)
        for causal in (False, True):
            check_against_oracle(q, k, v, 0.09, causal, dtype, tile=tile, label=f"tile {tile}")


@pytest.mark.parametrize("N", [1, 31, 32, 33, 64, 95, 257, 511, 513, 1000])
@pytest.mark.parametrize("tile", PP_TILES)
@pytest.mark.parametrize("d", [64, 128])
def test_pp_tiles_edge_sizes(N, tile, d):
    """The pipelined and 256-row tiles at sizes where a workgroup has one, two or three
    key tiles, waves whose rows start past N, and ragged last tiles."""
    if not fa.fa_tile_supported(d, *tile):
        pytest.skip(f"tile {tile} is not compiled for d={d}")
    for dtype in ("f16", "bf16"):
        q, k, v = make_random(1, 3, N, d, dtype, seed=N * 3 + tile[0] + tile[1] + d)
        for causal in (False, True):
            check_against_oracle(q, k, v, 1 / math.sqrt(d), causal, dtype, tile=tile,
                                 label=f"pp N={N} tile {tile}")


def test_large_scores_rescaling():
    """Scores spanning hundreds of units force many alpha rescalings per row. V keeps
    |O| < 4, where fp16's own rounding of O (half an ulp) stays under the tolerance."""
    q, k, _ = make_random(1, 2, 700, 64, "f16", seed=3, std=3.0)
    _, _, v = make_random(1, 2, 700, 64, "f16", seed=4, std=0.5)
    check_against_oracle(q, k, v, 0.5, False, "f16", label="large scores")
    check_against_oracle(q, k, v, 0.5, True, "f16", label="large scores causal")


def _one_tile_rows(dtype, N=256, d=64, seed=41):
    """Inputs whose every row has its softmax mass in one 32-key group: row i's query
    is A e_(i mod 8) and the keys of group t are B u_j e_t (u_j in [0.85, 1]), so with
    scale 1/8 and A B / 8 = 20 a row scores 17..20 on its own group and 0 elsewhere
    (weights e^-3 .. 1 against e^-20): l is, to 1e-7, the sum over one tile."""
    g = torch.Generator("cpu").manual_seed(seed)
    A = B = math.sqrt(160.0)
    q = torch.zeros(1, 4, N, d)
    k = torch.zeros(1, 4, N, d)
    rows = torch.arange(N)
    q[0, :, rows, rows % 8] = A
    u = 0.85 + 0.15 * torch.rand(4, N, generator=g)
    k[0, :, rows, (rows // 32) % 8] = B * u
    v = torch.randn(1, 4, N, d, generator=g)
    dt = TORCH_DT[dtype]
    return q.to(dt), k.to(dt), v.to(dt)


@pytest.mark.parametrize("tile", [None, (128, 64), (256, 32), (64, 64)])
def test_row_sums_of_one_tile_stay_within_their_bound(tile):
    """fp16 weights in unmasked tiles are summed as rounded fp16 values by two levels
    of packed adds; a lane's tile sum is then within 3 * 2^-12 = 7.3e-4 of the exact
    sum, relative, and where one tile holds a row's mass that is LSE's error (plus
    fp32 rounding). bf16 weights keep fp32 sums: there LSE is exact to fp32 rounding."""
    q, k, v = _one_tile_rows("f16")
    _, lse = check_against_oracle(q, k, v, 0.125, False, "f16", tile=tile, label="one-tile rows f16")
    _, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), 0.125, False)
    err = np.abs(lse - lse_ref).max()
    _say(f"[rowsum] f16 tile {tile}: max|dLSE| = {err:.3e} against the bound 7.3e-4")
    assert err <= 3 * 2.0 ** -12 + 1e-5
    q, k, v = _one_tile_rows("bf16")
    _, lse = check_against_oracle(q, k, v, 0.125, False, "bf16", tile=tile, label="one-tile rows bf16")
    _, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), 0.125, False)
    err = np.abs(lse - lse_ref).max()
    _say(f"[rowsum] bf16 tile {tile}: max|dLSE| = {err:.3e}")
    assert err <= 2e-5


def test_empty_problems_are_noops():
    dev = torch.device("cuda:0")
    for shape in [(0, 2, 16, 64), (2, 0, 16, 64), (2, 2, 0, 64)]:
        q = torch.zeros(shape, dtype=torch.float16, device=dev)
        o, lse = fa.fwd(q, q, q, causal=True)
        torch.cuda.synchronize()
        assert o.shape == shape and lse.shape == shape[:3]


def test_side_stream_and_repeat_determinism():
    q, k, v = make_random(2, 4, 515, 128, "bf16", seed=77)
    s = torch.cuda.Stream()
    o1, l1 = run_gpu(q, k, v, 0.1, True, stream=s)
    o2, l2 = run_gpu(q, k, v, 0.1, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_pending_hip_error_of_the_caller_is_neither_reported_nor_cleared():
    """A HIP error that an earlier, unrelated call of the caller's thread left pending
    (here hipSetDevice with an ordinal no machine has) must not turn a successful
    launch into FA_ERR_HIP, and must still be pending afterwards. Covers the forward,
    the split-KV forward (two launches) and the backward (two launches)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    hip.hipPeekAtLastError.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    q, k, v = make_random(1, 2, 300, 128, "bf16", seed=91)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_b, l_b = fa.fwd(qd, kd, vd, causal=True)
    dout = torch.randn(qd.shape, generator=torch.Generator("cpu").manual_seed(92)).to(qd.dtype).to(dev)
    calls = [
        ("fwd", lambda: fa.fwd(qd, kd, vd, causal=True)),
        ("fwd_split", lambda: fa.fwd_split(qd, kd, vd, causal=True, num_splits=3)),
        ("bwd", lambda: fa.bwd(qd, kd, vd, o_b, dout, l_b, causal=True)),
    ]
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), 1 / math.sqrt(128), True)
    for name, call in calls:
        hip.hipGetLastError()                     # start from a clean state
        st = hip.hipSetDevice(1 << 20)            # fails on the host, touches no device
        assert st != 0, "an out-of-range device ordinal was accepted"
        out = call()                              # raises FaError on any status but FA_OK
        torch.cuda.synchronize()
        assert hip.hipGetLastError() == st, f"{name}: the caller's pending error was cleared or replaced"
        if name != "bwd":
            o, lse = out
            assert np.abs(o.float().cpu().double().numpy() - ref_o).max() <= TOL_O["bf16"]
            assert np.abs(lse.cpu().double().numpy() - ref_l).max() <= TOL_LSE
        _say(f"[pending-error] {name}: launched, caller's error {st} still pending")


def test_library_loaded_before_torch_shares_its_runtime():
    """In a fresh process that loads libfa.so before it has imported torch, the library
    still runs on the HIP runtime torch uses (torch ships its own copy; two copies in
    one process do not share the device), and a forward matches an fp32 CPU reference."""
    import subprocess
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys\n"
        f"sys.path.insert(0, {root!r})\n"
        "import exact_attention_forward_fwd_amd as fa\n"
        "assert 'torch' not in sys.modules\n"
        "fa.load_library()\n"
        "import torch\n"
        "g = torch.Generator().manual_seed(5)\n"
        "q, k, v = (torch.randn(1, 2, 200, 64, generator=g).half() for _ in range(3))\n"
        "o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda())\n"
        "ref = torch.softmax((q.float() @ k.float().transpose(-1, -2)) * 0.125, -1) @ v.float()\n"
        "print(float((o.float().cpu() - ref).abs().max()))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    err = float(r.stdout.strip().splitlines()[-1])
    _say(f"[load-order] max |dO| = {err:.2e}")
    assert err <= TOL_O["f16"]


def test_invalid_arguments_return_status():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device=dev)
    p = (q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr())
    assert fa.fa_fwd(*p, 1, 1, 64, 96, 0.1, 0, fa.FA_F16, None) == 3
    assert fa.fa_fwd(*p, 1, 1, 64, 64, 0.0, 0, fa.FA_F16, None) == 4
    assert fa.fa_fwd(*p, 1, 1, 64, 64, 0.1, 0, 5, None) == 5
    assert fa.fa_fwd(p[0] + 2, *p[1:], 1, 1, 64, 64, 0.1, 0, fa.FA_F16, None) == 6
    assert fa.fa_fwd_tiled(*p, 1, 1, 64, 64, 0.1, 0, fa.FA_F16, None, 96, 64) == 8
    torch.cuda.synchronize()


def test_lse_does_not_drift_over_many_tiles():
    """Regression: with the maximum reached early, 256 key tiles of rescaling by
    alpha must leave l untouched (alpha exactly 1 when the maximum does not move).
    Without drift the LSE error of a spiked row (|LSE| ~ 90) is a few fp32 ulps of
    the reference plus s times the score error, ~1e-5; 2e-4 catches a compounding
    per-tile factor long before the 1e-3 contract does."""
    g = torch.Generator("cpu").manual_seed(31)
    N, d = 16384, 128
    q = torch.randn(1, 2, N, d, generator=g)
    k = torch.randn(1, 2, N, d, generator=g)
    v = torch.rand(1, 2, N, d, generator=g) * 2 - 1
    rows = torch.randperm(N, generator=g)[:64]
    q[:, :, rows] *= 20.0
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = run_gpu(q, k, v, 1 / math.sqrt(d), False)
    flat = np.concatenate([rows.numpy(), rows.numpy() + N, np.arange(0, 2 * N, 997)])
    o_ref, lse_ref = oracle.attention_rows(f64(q), f64(k), f64(v), 1 / math.sqrt(d), False, flat)
    err = np.abs(lse.reshape(-1)[flat] - lse_ref).max()
    _say(f"[drift] max|dLSE| over spiked and sampled rows = {err:.2e}")
    assert err <= 2e-4
