"""fa_fwd_split_noalloc (the split-KV entry point that uses the library's per-GPU
scratch array instead of a caller workspace) against fa_fwd_split with a workspace,
through the C ABI: the same kernels on the same inputs, so the results must agree bit
for bit. Two calls in a row, the second with a smaller input, so that the scratch is
reused with stale contents from the first call."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_fwd_amd as fa
from exact_attention_forward_fwd_amd.workloads import make_random

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield


def _inputs(B, Hq, Hk, Nq, Nk, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    q = torch.randn((B, Hq, Nq, d), generator=g).to(dt).cuda()
    k = torch.randn((B, Hk, Nk, d), generator=g).to(dt).cuda()
    v = torch.randn((B, Hk, Nk, d), generator=g).to(dt).cuda()
    return q, k, v


def _both(q, k, v, causal, splits):
    B, Hq, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    code = fa.FA_F16 if q.dtype == torch.float16 else fa.FA_BF16
    scale = 1 / math.sqrt(d)
    st = torch.cuda.current_stream().cuda_stream
    res = []
    for noalloc in (False, True):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=q.device)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hk, Nq, Nk, d,
                None, None, None, None, scale, causal, code, st, 0, 0, splits)
        if noalloc:
            rc = fa.fa_fwd_split_noalloc(*args)
        else:
            need = fa.fa_split_workspace_bytes(B, Hq, Nq, d, splits)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            rc = fa.fa_fwd_split(*args, ws.data_ptr(), need)
        assert rc == 0, fa.status_str(rc)
        torch.cuda.synchronize()
        res.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    return res


CASES = [
    # (B, Hq, Hk, Nq, Nk, d, dtype, causal, splits): a decoding-like shape first, then a
    # smaller one reusing the scratch
    (1, 32, 8, 1, 32768, 128, "bf16", True, None),
    (2, 4, 4, 100, 3000, 64, "f16", True, 5),
]


def test_noalloc_matches_workspace_form_twice_in_a_row():
    for i, (B, Hq, Hk, Nq, Nk, d, dtype, causal, splits) in enumerate(CASES):
        q, k, v = _inputs(B, Hq, Hk, Nq, Nk, d, dtype, seed=300 + i)
        if splits is None:
            splits = fa.fa_split_default(B, Hq, Hk, Nq, Nk, d, causal, 0, 0)
        _say(f"[noalloc] call {i}: B={B} Hq={Hq} Hk={Hk} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
             f"splits={splits}")
        assert splits > 1
        (o_ws, l_ws), (o_na, l_na) = _both(q, k, v, causal, splits)
        assert not np.isnan(o_na).any() and not np.isnan(l_na).any()
        np.testing.assert_array_equal(o_na, o_ws)
        np.testing.assert_array_equal(l_na, l_ws)


def test_noalloc_single_range_and_limit():
    q, k, v = _inputs(1, 2, 2, 64, 500, 64, "f16", seed=310)
    (o_ws, l_ws), (o_na, l_na) = _both(q, k, v, False, 1)
    np.testing.assert_array_equal(o_na, o_ws)
    np.testing.assert_array_equal(l_na, l_ws)
    # partials beyond the scratch: refused, outputs untouched
    B, Hq, Nq, d = 1, 8, 1024, 128
    fits = fa.SPLIT_SCRATCH_BYTES // (B * Hq * Nq * (d + 1) * 4)
    q, k, v = _inputs(B, Hq, Hq, Nq, 8192, d, "bf16", seed=311)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=q.device)
    rc = fa.fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                 Hq, Nq, 8192, d, None, None, None, None, 0.088, 0, fa.FA_BF16,
                                 torch.cuda.current_stream().cuda_stream, 0, 0, fits + 1)
    torch.cuda.synchronize()
    assert rc == 13
    assert torch.isnan(o).all()


def test_noalloc_captured_in_a_graph_replays_like_eager():
    """The callers this entry point is for: capture one call (attention launch + merge
    launch) in a HIP graph and replay it. Each replay, with eager work and a
    synchronisation in between, must equal the eager call bit for bit; after the
    inputs are overwritten in place, a replay must equal a fresh eager call on them."""
    B, Hq, Hk, Nq, Nk, d = 1, 32, 8, 1, 16384, 128
    q, k, v = _inputs(B, Hq, Hk, Nq, Nk, d, "bf16", seed=320)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    call = lambda: fa.fwd_split_noalloc(q, k, v, causal=True, num_splits=16, out=o, lse=lse)
    call()                                   # eager; also looks up the scratch address
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep} differs from the eager call"
        _say(f"[noalloc-graph] replay {rep} equals the eager call")
    q2, k2, v2 = _inputs(B, Hq, Hk, Nq, Nk, d, "bf16", seed=321)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    o_new, l_new = fa.fwd_split(q2, k2, v2, causal=True, num_splits=16)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(o, o_new) and torch.equal(lse, l_new)
