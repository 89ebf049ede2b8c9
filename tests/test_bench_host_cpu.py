"""Host-side logic of the benchmark and of the seeded input generators (no GPU).

- bench.py refuses more than one GPU before it touches any device;
- the HBM-traffic record scales each counter by what it reads for a plain copy of
  known size (checked on synthetic counter files whose answer is known);
- a stored traffic record is used only while its kernel-source hash matches;
- the algorithmic FLOP and byte counts equal their closed forms, and the visible
  (query, key) pairs of a bottom-right causal mask equal a brute-force count;
- the generators are deterministic per seed, give the stated shapes, types and
  distributions, and plant the stated number of spiked rows.
"""
import csv
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_attention_forward_fwd_amd.workloads import (GeneralWorkload, SPLIT_WORKLOADS, WORKLOADS,  # noqa: E402
                                                       make_general_inputs, make_inputs, spike_count)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2", "--steps", "1", "--warmup", "0"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write_counters(d, counter, attn_values, copy_values, kernel="void fa_fwd_kernel<64, false, false, 4, 1, 64>(Params)"):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        i = 0
        for v in attn_values:
            i += 1
            wr.writerow([i, kernel, counter, v])
        for v in copy_values:
            i += 1
            wr.writerow([i, "__amd_rocclr_copyBuffer", counter, v])


def test_traffic_record_scales_by_the_copy(tmp_path):
    """FETCH_SIZE reading half of the copy's bytes gives factor 2, WRITE_SIZE reading
    all of them factor 1; the attention kernel's counters are averaged per dispatch."""
    w = WORKLOADS[2]
    copy_kib = bench.COPY_BYTES / 1024
    _write_counters(tmp_path / "f", "FETCH_SIZE", [1000.0, 1002.0, 998.0], [copy_kib / 2])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [500.0, 500.0, 500.0], [copy_kib])
    rec = bench.traffic_record(w, str(tmp_path / "f"), str(tmp_path / "w"))
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(1000.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2 + 500.0 * 1024)
    assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(w)
    assert rec["traffic_over_algorithmic"] == pytest.approx(rec["hbm_bytes_per_launch"] / bench.algorithmic_bytes(w))
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def test_traffic_record_needs_both_kinds_of_dispatch(tmp_path):
    _write_counters(tmp_path / "f", "FETCH_SIZE", [1000.0], [])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [500.0], [1.0])
    with pytest.raises(SystemExit):
        bench.traffic_record(WORKLOADS[2], str(tmp_path / "f"), str(tmp_path / "w"))


def test_stored_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    w = WORKLOADS[2]
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic(w) is None
    rec = {"kernel_source_sha256": "0" * 64, "hbm_bytes_per_launch": 1.0}
    (tmp_path / f"traffic_{w.name}.json").write_text(json.dumps(rec))
    assert bench.stored_traffic(w) is None
    rec["kernel_source_sha256"] = bench.kernel_source_hash()
    (tmp_path / f"traffic_{w.name}.json").write_text(json.dumps(rec))
    assert bench.stored_traffic(w)["hbm_bytes_per_launch"] == 1.0


def test_algorithmic_counts_closed_forms():
    w = WORKLOADS[2]   # B=2, H=16, N=4096, d=64
    assert w.flops == 4.0 * 2 * 16 * 4096 ** 2 * 64
    assert bench.algorithmic_bytes(w) == 4 * 2 * 16 * 4096 * 64 * 2 + 2 * 16 * 4096 * 4 == 67633152
    w3 = WORKLOADS[3]  # causal: half of the square, as the counted convention states
    assert w3.flops == 2.0 * 4 * 32 * 2048 ** 2 * 128


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 7), (5, 3), (3, 5), (7, 7), (64, 1000), (1000, 64), (0, 5)])
def test_visible_pairs_brute_force(nq, nk):
    """Bottom-right causal: key j is visible to query i iff j <= i + nk - nq."""
    w = GeneralWorkload(0, "t", 1, 1, 1, nq, nk, 64, "f16", True, 0.125)
    count = sum(1 for i in range(nq) for j in range(nk) if j <= i + nk - nq)
    assert w.visible_pairs == count
    assert GeneralWorkload(0, "t", 1, 1, 1, nq, nk, 64, "f16", False, 0.125).visible_pairs == nq * nk


def test_split_workload_counts():
    dec = SPLIT_WORKLOADS[6]
    # one query row per head sees every key (its row is the last one)
    assert dec.visible_pairs == dec.Nk
    assert dec.hbm_bytes == (2 * dec.B * dec.Hq * dec.d * 2 + 2 * dec.B * dec.Hk * dec.Nk * dec.d * 2
                             + 4 * dec.B * dec.Hq)
    sh = SPLIT_WORKLOADS[7]
    assert sh.flops == 4.0 * 128 * 2 * 16384 ** 2


@pytest.mark.parametrize("idx", [1, 2, 5])
def test_make_inputs_is_seeded_and_shaped(idx):
    w = WORKLOADS[idx]
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a[:3], b[:3]):
        assert x.shape == (w.B, w.H, w.N, w.d) and x.dtype == w.torch_dtype
        assert torch.equal(x, y)
    other = make_inputs(w, seed=w.seed + 1)
    assert not torch.equal(a[0], other[0])


def test_workload_5_distributions():
    """n1000_d64_f16_causal_ragged: Q, K ~ N(0, 0.5^2), V ~ N(0, 0.5^2)."""
    w = WORKLOADS[5]
    q, k, v, spikes = make_inputs(w)
    for t in (q, k, v):
        s = t.float().std().item()
        assert abs(s - 0.5) < 0.01, s
    assert spikes.shape == (w.B, w.H, 0)


def test_spiked_rows_are_planted():
    """A small spiked workload of the same recipe: spike_frac of the Q rows per (b, h)
    scaled by spike_mult, V ~ U(-1, 1)."""
    w = WORKLOADS[4]
    small = type(w)(99, "small_spiked", 1, 2, 1000, 64, "bf16", False, 0.125, v_dist="uniform",
                    spike_frac=w.spike_frac, spike_mult=w.spike_mult)
    q, k, v, spikes = make_inputs(small)
    cnt = spike_count(small)
    assert cnt == 10 and spikes.shape == (1, 2, cnt)
    norms = q.float().norm(dim=-1)
    for h in range(2):
        idx = spikes[0, h]
        rest = torch.ones(small.N, dtype=torch.bool)
        rest[idx] = False
        assert norms[0, h, idx].min() > 5 * norms[0, h, rest].max()
        assert len(set(idx.tolist())) == cnt
    assert v.float().min() >= -1 and v.float().max() <= 1


def test_make_general_inputs_shapes():
    w = GeneralWorkload(5, "g", 2, 8, 2, 3, 70, 128, "bf16", True, 0.1, v_std=0.5)
    q, k, v = make_general_inputs(w)
    assert q.shape == (2, 8, 3, 128) and k.shape == (2, 2, 70, 128) and v.shape == k.shape
    assert q.dtype == torch.bfloat16
    q2, _, _ = make_general_inputs(w)
    assert torch.equal(q, q2)
