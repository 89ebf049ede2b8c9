"""The C-ABI library loads, exports every function include/fa.h declares, and its
argument validation answers without touching a GPU (no compute calls here: every
call below is rejected, or is an empty problem, before anything is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_forward_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings():
    for code in range(14):
        s = fa.status_str(code)
        assert s and s != "unknown status"
    assert fa.status_str(99) == "unknown status"


def test_tile_queries():
    assert fa.fa_tile_supported(64, 64, 64) and fa.fa_tile_supported(128, 128, 64)
    assert not fa.fa_tile_supported(96, 64, 64) and not fa.fa_tile_supported(64, 48, 64)
    assert fa.fa_default_tile(1, 1, 128, 64, False) == (64, 64)
    bm, bn = fa.fa_default_tile(2, 16, 4096, 64, False)
    assert fa.fa_tile_supported(64, bm, bn)
    with pytest.raises(fa.FaError):
        fa.fa_default_tile(1, 1, 128, 80, False)


@pytest.mark.parametrize("B,H,N,causal,tile", [
    (1, 16, 16384, False, (256, 64)),   # 1024 blocks of 256 rows: eight waves, 64-key tiles
    (1, 16, 4096, False, (256, 64)),    # 256 blocks: one per CU
    (1, 8, 4096, False, (128, 64)),     # 128 blocks of 256 rows would leave half the CUs idle
    (2, 16, 4096, True, (256, 64)),     # causal: 512 blocks
    (1, 16, 8192, True, (256, 64)),
    (1, 8, 8192, True, (128, 64)),      # causal: 256 blocks of uneven length are too few
    (2, 16, 2048, False, (128, 64)),
    (2, 16, 256, False, (128, 32)),
    (4, 32, 2048, True, (128, 32)),     # short rows: 128-row blocks; several rounds of them: 32-key tiles
    (2, 16, 2048, True, (128, 64)),     # one round of 512 workgroups: 64-key tiles
    (2, 16, 3072, True, (128, 32)),     # 768 workgroups
    (1, 8, 200, True, (128, 32)),
    (1, 1, 1 << 40, True, (256, 64)),   # sizes far past any real grid: no overflow
    (1 << 40, 1 << 40, 4096, False, (256, 64)),
])
def test_default_tile_d128_follows_the_grid(B, H, N, causal, tile):
    """At d = 128 the eight-wave 256-row tile is chosen only when its grid covers the CUs
    (256 workgroups; 512 under a causal mask)."""
    assert fa.fa_default_tile(B, H, N, 128, causal) == tile


@pytest.mark.parametrize("B,H,N,causal,tile", [
    (2, 16, 4096, False, (256, 32)),    # two query blocks per wave: 512 workgroups of 256 rows
    (1, 16, 4096, False, (128, 64)),    # 256 of them would leave one per CU
    (1, 8, 200, False, (128, 32)),
    (8, 16, 1000, True, (128, 32)),     # 1024 causal row blocks: 32-key tiles, three per CU
    (4, 32, 2048, True, (128, 32)),
    (2, 16, 2048, True, (128, 64)),     # one round of 512: 64-key tiles
    (4, 16, 1024, True, (128, 64)),
    (4, 24, 1024, True, (128, 32)),     # 768 short rows
    (2, 16, 3072, True, (128, 64)),     # 768 long rows: 1.5 rounds
    (4, 16, 3072, True, (128, 32)),
    (1, 8, 200, True, (128, 32)),
])
def test_default_tile_d64_follows_the_grid(B, H, N, causal, tile):
    """At d = 64 the two-block tile needs two 256-row workgroups per CU; under a causal
    mask the 64-key tile is chosen while its grid is about one round of 512."""
    assert fa.fa_default_tile(B, H, N, 64, causal) == tile


# Fake, aligned, never-dereferenced addresses: validation rejects before any launch.
A = 0x10000


def call(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=64, d=64, scale=0.125, causal=0, dtype=0):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def test_validation_codes_without_gpu():
    assert call(q=None) == 1 and call(lse=None) == 1 and call(o=None) == 1
    assert call(B=-1) == 2 and call(N=-5) == 2
    assert call(d=96) == 3 and call(d=0) == 3
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert call(scale=s) == 4
    assert call(dtype=2) == 5 and call(dtype=-1) == 5
    assert call(q=A + 8) == 6 and call(o=A + 2) == 6 and call(lse=A + 2) == 6
    assert call(N=1 << 25) == 7                       # N*d >= 2^31 with d = 64
    assert call(B=1 << 20, H=1 << 20, N=1 << 10) == 7  # grid too large
    assert fa.fa_fwd_tiled(A, A, A, A, A, 1, 1, 64, 64, 0.1, 0, 0, None, 96, 64) == 8


def call_ex(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=4, Hk=2, Nq=64, Nk=100, d=64, qs=None, ks=None, vs=None,
            os_=None, causal=0, bm=0, bn=0):
    return fa.fa_fwd_ex(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, qs, ks, vs, os_, 0.125, causal, 0, None, bm, bn)


def test_general_entry_validation_without_gpu():
    assert call_ex(Hk=3) == 2 and call_ex(Hk=0) == 2 and call_ex(Nk=-1) == 2
    assert call_ex(qs=(0, 0, 60)) == 10              # row stride < d
    assert call_ex(ks=(8, 8, 68)) == 10              # not a multiple of 8
    assert call_ex(vs=(-64, 64, 64)) == 10           # negative
    assert call_ex(os_=(0, 64, 64), q=None) == 1     # null checked first
    assert call_ex(k=None) == 1                      # Nk > 0 needs k and v
    assert call_ex(qs=(0, 0, 1 << 24), Nq=100) == 7  # rows exceed 32-bit offsets
    assert call_ex(bm=96, bn=64) == 8
    assert call_ex(q=None, k=None, v=None, o=None, lse=None, Nq=0) == 0
    assert call_ex(q=None, k=None, v=None, o=None, lse=None, Hq=0, Hk=0) == 0


def test_key_count_limit_without_gpu():
    """One key beyond the 32-bit slice range ((N + 512) * row stride < 2^30 elements) is
    refused before any launch; the GPU tests run the largest accepted count."""
    for d in (64, 128):
        nk = (1 << 30) // d - 513 + 1
        assert call_ex(Hq=4, Hk=1, Nq=1, Nk=nk, d=d) == 7
        assert call_ex(Hq=4, Hk=1, Nq=1, Nk=nk - 1, d=d, ks=(0, 0, 2 * d)) == 7   # a wider row stride counts
        assert call_split(Hq=4, Hk=1, Nq=1, Nk=nk, d=d, ws=A, ws_bytes=1 << 20) == 7


def call_split(ws=None, ws_bytes=0, splits=2, q=A, B=1, Hq=4, Hk=2, Nq=64, Nk=100, d=64, causal=0, bm=0, bn=0):
    return fa.fa_fwd_split(q, A, A, A, A, B, Hq, Hk, Nq, Nk, d, None, None, None, None, 0.125, causal, 0, None,
                           bm, bn, splits, ws, ws_bytes)


def test_split_entry_validation_without_gpu():
    assert call_split(splits=0) == 11 and call_split(splits=257) == 11 and call_split(splits=-3) == 11
    assert call_split(splits=0, Nq=0) == 11            # the split count is checked before the empty case
    assert call_split(ws=None, ws_bytes=0) == 12       # Nk = 100 has two 64-key tiles: a split is made
    need = fa.fa_split_workspace_bytes(1, 4, 64, 64, 2)
    assert need == 2 * (1 * 4 * 64) * (64 + 1) * 4
    assert call_split(ws=A, ws_bytes=need - 4) == 12   # too small
    assert call_split(ws=A + 8, ws_bytes=need) == 12   # not 16-byte aligned
    assert call_split(q=None, ws=A, ws_bytes=need) == 1
    assert call_split(Hk=3, ws=A, ws_bytes=need) == 2
    assert call_split(bm=96, bn=64, ws=A, ws_bytes=need) == 8
    assert call_split(q=None, Nq=0) == 0               # empty: nothing to do, nothing checked further


def test_split_sizes_and_default():
    assert fa.fa_split_workspace_bytes(2, 8, 100, 128, 1) == 0
    assert fa.fa_split_workspace_bytes(2, 8, 100, 96, 4) == 0
    assert fa.fa_split_workspace_bytes(2, 8, 100, 128, 257) == 0
    assert fa.fa_split_workspace_bytes(2, 8, 100, 128, 3) == 3 * 1600 * 129 * 4
    # query blocks alone fill the GPU: no split
    assert fa.fa_split_default(2, 16, 16, 4096, 4096, 64, False) == 1
    # decoding, one query row per head, 128K keys: many ranges, within the limit
    s = fa.fa_split_default(1, 32, 8, 1, 131072, 128, True)
    assert 16 <= s <= 256
    # no more ranges than key tiles
    assert fa.fa_split_default(1, 1, 1, 64, 128, 64, False, 64, 64) <= 2
    assert fa.fa_split_default(1, 1, 1, 64, 0, 64, False) == 1


def call_bwd(ptr=A, lse=A, ws=A, ws_bytes=1 << 20, B=1, H=2, N=100, d=64, scale=0.125, dtype=0):
    return fa.fa_bwd(ptr, A, A, A, A, lse, A, A, A, B, H, N, d, scale, 0, dtype, ws, ws_bytes, None)


def test_bwd_entry_validation_without_gpu():
    assert call_bwd(B=-1) == 2 and call_bwd(N=-1) == 2
    assert call_bwd(d=96) == 3
    assert call_bwd(scale=0.0) == 4 and call_bwd(scale=float("nan")) == 4
    assert call_bwd(dtype=7) == 5
    assert call_bwd(ptr=None) == 1 and call_bwd(lse=None) == 1
    assert call_bwd(ptr=A + 8) == 6 and call_bwd(lse=A + 2) == 6
    assert call_bwd(ws=None) == 12 and call_bwd(ws_bytes=2 * 100 * 4 - 4) == 12 and call_bwd(ws=A + 4) == 12
    assert call_bwd(N=1 << 24, d=128, ws_bytes=1 << 40) == 7
    assert call_bwd(ptr=None, lse=None, ws=None, N=0) == 0
    assert fa.fa_bwd_workspace_bytes(2, 3, 5) == 240 and fa.fa_bwd_workspace_bytes(0, 3, 5) == 0


def call_bwd_ex(ptr=A, ws=A, ws_bytes=1 << 20, B=1, Hq=4, Hk=2, Nq=100, Nk=70, d=64):
    return fa.fa_bwd_ex(ptr, A, A, A, A, A, A, A, A, B, Hq, Hk, Nq, Nk, d, 0.125, 1, 0, ws, ws_bytes, None)


def test_bwd_ex_validation_without_gpu():
    assert call_bwd_ex(Hk=3) == 2 and call_bwd_ex(Hk=0) == 2 and call_bwd_ex(Nk=-1) == 2
    assert call_bwd_ex(ptr=None) == 1
    assert call_bwd_ex(ws=None) == 12 and call_bwd_ex(ws_bytes=4 * 100 * 4 - 4) == 12
    assert call_bwd_ex(ptr=None, ws=None, Nq=0, Nk=0) == 0
    assert call_bwd_ex(ptr=None, ws=None, B=0) == 0


def test_empty_problems_need_no_pointers():
    assert call(q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert call(q=None, k=None, v=None, o=None, lse=None, B=0) == 0
    assert call(q=None, k=None, v=None, o=None, lse=None, H=0, causal=1) == 0


def test_product_path_does_not_reference_the_oracle():
    """The HIP library and the binding never load or import the CPU oracle."""
    pkg = os.path.dirname(fa.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f
    out = subprocess.run(["nm", "-D", fa.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in out


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError):
        fa.load_library(str(tmp_path / "libfa.so"))


def test_noalloc_split_refuses_partials_beyond_the_scratch():
    """fa_fwd_split_noalloc checks the partials' size against the built-in scratch
    before any HIP call: one range more than fits is refused, nothing is launched."""
    d, rows = 128, 8 * 1024                       # B * Hq * Nq query rows
    per_range = rows * (d + 1) * 4
    fits = fa.SPLIT_SCRATCH_BYTES // per_range
    assert fa.fa_split_workspace_bytes(1, 8, 1024, d, fits) <= fa.SPLIT_SCRATCH_BYTES
    st = fa.fa_fwd_split_noalloc(A, A, A, A, A, 1, 8, 8, 1024, 4096, d, None, None, None, None, 0.088, 0, 1,
                                 None, 0, 0, fits + 1)
    assert st == 13 and "scratch" in fa.status_str(st)
    # the other checks are those of fa_fwd_split (nothing launched either)
    assert fa.fa_fwd_split_noalloc(A, A, A, A, A, 1, 8, 8, 1024, 4096, 96, None, None, None, None, 0.088, 0, 1,
                                   None, 0, 0, 4) == 3
    assert fa.fa_fwd_split_noalloc(A, A, A, A, A, 1, 8, 8, 1024, 4096, d, None, None, None, None, 0.088, 0, 1,
                                   None, 0, 0, 257) == 11
