"""ctypes binding of libfa.so: the same entry points as include/fa.h, argument
marshalling only. Every step of the attention forward runs in the HIP kernels of
the library; there is no fallback of any kind. If the library is missing or fails
to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_F16 = 0
FA_BF16 = 1

STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_UNSUPPORTED_HEADDIM",
    4: "FA_ERR_BAD_SCALE", 5: "FA_ERR_BAD_DTYPE", 6: "FA_ERR_MISALIGNED", 7: "FA_ERR_TOO_LARGE",
    8: "FA_ERR_UNSUPPORTED_TILE", 9: "FA_ERR_HIP", 10: "FA_ERR_BAD_STRIDE", 11: "FA_ERR_BAD_SPLITS",
    12: "FA_ERR_WORKSPACE", 13: "FA_ERR_SCRATCH_LIMIT",
}
# size of the per-GPU scratch array of fa_fwd_split_noalloc (FA_SPLIT_SCRATCH_BYTES in fa.h)
SPLIT_SCRATCH_BYTES = 64 << 20
EXPORTED = ("fa_fwd", "fa_fwd_tiled", "fa_fwd_ex", "fa_fwd_split", "fa_fwd_split_noalloc", "fa_split_workspace_bytes",
            "fa_split_default",
            "fa_bwd", "fa_bwd_ex", "fa_bwd_workspace_bytes", "fa_tile_supported", "fa_default_tile", "fa_status_str")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfa.so and declare the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run "
                           "`python -m exact_attention_forward_fwd_amd.build` first")
    # libfa.so must use the HIP runtime that torch (which owns the tensors and streams
    # passed in) has loaded. torch ships its own libamdhip64 (file libamdhip64.so,
    # soname libamdhip64.so.7). Loaded first, it satisfies libfa.so's dependency on
    # libamdhip64.so.7; loaded after libfa.so, which would bring in the system runtime,
    # it becomes a second runtime in the process, and the one libfa.so calls then
    # finds no device (every launch returns FA_ERR_HIP).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    common = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, i32, i32, vp]
    lib.fa_fwd.argtypes = common
    lib.fa_fwd.restype = i32
    lib.fa_fwd_tiled.argtypes = common + [i32, i32]
    lib.fa_fwd_tiled.restype = i32
    i64p = ctypes.POINTER(i64)
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p,
                              ctypes.c_float, i32, i32, vp, i32, i32]
    lib.fa_fwd_ex.restype = i32
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p,
                                 ctypes.c_float, i32, i32, vp, i32, i32, i32, vp, ctypes.c_size_t]
    lib.fa_fwd_split.restype = i32
    lib.fa_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p,
                                         ctypes.c_float, i32, i32, vp, i32, i32, i32]
    lib.fa_fwd_split_noalloc.restype = i32
    lib.fa_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.fa_split_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_split_default.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32]
    lib.fa_split_default.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, i32, i32, vp,
                           ctypes.c_size_t, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, i32,
                              i32, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_ex.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_tile_supported.argtypes = [i64, i32, i32]
    lib.fa_tile_supported.restype = i32
    lib.fa_default_tile.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fa_default_tile.restype = i32
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw C call; pointers are integers (device addresses). Returns the fa_status."""
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, int(causal), dtype, stream)


def fa_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream, block_m, block_n) -> int:
    return load_library().fa_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, int(causal), dtype,
                                       stream, block_m, block_n)


def _strides(st):
    """{batch, head, row} element strides as a C array, or NULL for None."""
    if st is None:
        return None
    return (ctypes.c_int64 * 3)(*[int(x) for x in st])


def fa_fwd_ex(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides,
              scale, causal, dtype, stream, block_m=0, block_n=0) -> int:
    """Raw C call of the general entry point; strides are 3-sequences or None."""
    return load_library().fa_fwd_ex(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, _strides(q_strides),
                                    _strides(k_strides), _strides(v_strides), _strides(o_strides),
                                    scale, int(causal), dtype, stream, int(block_m), int(block_n))


def fa_fwd_split(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides,
                 scale, causal, dtype, stream, block_m, block_n, num_splits, workspace, workspace_bytes) -> int:
    """Raw C call of the split-KV entry point; workspace is a device address (or 0)."""
    return load_library().fa_fwd_split(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, _strides(q_strides),
                                       _strides(k_strides), _strides(v_strides), _strides(o_strides),
                                       scale, int(causal), dtype, stream, int(block_m), int(block_n),
                                       int(num_splits), workspace, int(workspace_bytes))


def fa_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides,
                         scale, causal, dtype, stream, block_m, block_n, num_splits) -> int:
    """Raw C call of the split-KV entry point that uses the library's built-in scratch."""
    return load_library().fa_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, _strides(q_strides),
                                               _strides(k_strides), _strides(v_strides), _strides(o_strides),
                                               scale, int(causal), dtype, stream, int(block_m), int(block_n),
                                               int(num_splits))


def fa_split_workspace_bytes(B: int, Hq: int, Nq: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_split_workspace_bytes(B, Hq, Nq, d, int(num_splits)))


def fa_split_default(B: int, Hq: int, Hk: int, Nq: int, Nk: int, d: int, causal: bool, block_m: int = 0,
                     block_n: int = 0) -> int:
    return int(load_library().fa_split_default(B, Hq, Hk, Nq, Nk, d, int(causal), int(block_m), int(block_n)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace, workspace_bytes,
           stream) -> int:
    """Raw C call of the backward entry point; pointers are device addresses."""
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, int(causal), dtype,
                                 workspace, int(workspace_bytes), stream)


def fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hk, Nq, Nk, d, scale, causal, dtype, workspace,
              workspace_bytes, stream) -> int:
    """Raw C call of the general backward entry point."""
    return load_library().fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hk, Nq, Nk, d, scale, int(causal),
                                    dtype, workspace, int(workspace_bytes), stream)


def fa_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N))


def fa_tile_supported(d: int, block_m: int, block_n: int) -> bool:
    return bool(load_library().fa_tile_supported(d, block_m, block_n))


def fa_default_tile(B: int, H: int, N: int, d: int, causal: bool):
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    st = load_library().fa_default_tile(B, H, N, d, int(causal), ctypes.byref(bm), ctypes.byref(bn))
    if st != 0:
        raise FaError(st, "fa_default_tile")
    return bm.value, bn.value


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"dtype must be float16 or bfloat16, got {t.dtype}")


def _check_tensor(name, t, device, shape=None, dtype=None, contiguous=False, last_contiguous=False):
    """Raise ValueError unless ``t`` is a GPU tensor on ``device`` with the given shape,
    dtype and layout. Every pointer handed to the library passes through here: a host
    pointer or an undersized buffer would reach a kernel as a bad address."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if last_contiguous and t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}'s last dimension must be contiguous")


def _workspace_args(workspace, device):
    """(pointer, bytes) of a caller's workspace tensor (contiguous, on the GPU), or (0, 0)."""
    if workspace is None:
        return 0, 0
    _check_tensor("workspace", workspace, device, contiguous=True)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fwd(q, k, v, scale: float | None = None, causal: bool = False, block_m: int | None = None,
        block_n: int | None = None, out=None, lse=None, stream=None):
    """Attention forward on torch tensors [B, H, N, d] (contiguous, same device/dtype).

    Returns (o, lse): o like q, lse float32 [B, H, N]. ``scale`` defaults to 1/sqrt(d).
    Runs asynchronously on ``stream`` (default: torch's current stream).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape [B, H, N, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, q.device, shape=q.shape, dtype=q.dtype, contiguous=True)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor("lse", lse, q.device, shape=(B, H, N), dtype=torch.float32, contiguous=True)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
            float(scale), causal, dt, sp)
    if block_m is None and block_n is None:
        st = fa_fwd(*args)
    else:
        st = fa_fwd_tiled(*args, int(block_m), int(block_n))
    if st != 0:
        raise FaError(st, "fa_fwd")
    return out, lse


def _general_args(q, k, v, scale, out, lse, stream):
    """Checks and defaults shared by fwd_ex and fwd_split."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, heads, N, d]")
        if t.stride(-1) != 1:
            raise ValueError(f"{name}'s last dimension must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, Hq, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hk, Nk, d] with q's B and d")
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, q.device, shape=q.shape, dtype=q.dtype, last_contiguous=True)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_tensor("lse", lse, q.device, shape=(B, Hq, Nq), dtype=torch.float32, contiguous=True)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return scale, out, lse, sp


def fwd_ex(q, k, v, scale: float | None = None, causal: bool = False, block_m: int | None = None,
           block_n: int | None = None, out=None, lse=None, stream=None):
    """General attention forward on torch tensors: q [B, Hq, Nq, d], k and v [B, Hk, Nk, d]
    with any strides whose last dimension is contiguous; Hq a multiple of Hk (query
    head h reads K/V head h // (Hq // Hk)). ``causal`` masks key j > i + Nk - Nq
    (bottom-right alignment). Returns (o, lse): o [B, Hq, Nq, d] laid out like q
    unless ``out`` is given, lse float32 [B, Hq, Nq] contiguous.
    """
    scale, out, lse, sp = _general_args(q, k, v, scale, out, lse, stream)
    B, Hq, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hk,
                   Nq, Nk, d, q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3],
                   float(scale), causal, _dtype_code(q), sp, block_m or 0, block_n or 0)
    if st != 0:
        raise FaError(st, "fa_fwd_ex")
    return out, lse


def fwd_split(q, k, v, scale: float | None = None, causal: bool = False, num_splits: int | None = None,
              block_m: int | None = None, block_n: int | None = None, out=None, lse=None, workspace=None,
              stream=None):
    """fwd_ex with the keys of every query block divided among ``num_splits`` workgroups
    (split-KV) and merged by a second kernel. ``num_splits`` defaults to the library's
    suggestion (fa_split_default). ``workspace``: a device tensor of at least
    fa_split_workspace_bytes(...) bytes; allocated here if None.
    """
    import torch
    scale, out, lse, sp = _general_args(q, k, v, scale, out, lse, stream)
    B, Hq, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    bm, bn = block_m or 0, block_n or 0
    if num_splits is None:
        num_splits = fa_split_default(B, Hq, Hk, Nq, Nk, d, causal, bm, bn)
    need = fa_split_workspace_bytes(B, Hq, Nq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = _workspace_args(workspace, q.device)
    st = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hk,
                      Nq, Nk, d, q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3],
                      float(scale), causal, _dtype_code(q), sp, bm, bn, num_splits, ws_ptr, ws_bytes)
    if st != 0:
        raise FaError(st, "fa_fwd_split")
    return out, lse


def fwd_split_noalloc(q, k, v, scale: float | None = None, causal: bool = False, num_splits: int | None = None,
                      block_m: int | None = None, block_n: int | None = None, out=None, lse=None, stream=None):
    """fwd_split through fa_fwd_split_noalloc: the partials go to the library's per-GPU
    scratch array instead of a workspace. With ``out`` and ``lse`` given, nothing is
    allocated on the device by this call (the C entry point never allocates)."""
    scale, out, lse, sp = _general_args(q, k, v, scale, out, lse, stream)
    B, Hq, Nq, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    bm, bn = block_m or 0, block_n or 0
    if num_splits is None:
        num_splits = fa_split_default(B, Hq, Hk, Nq, Nk, d, causal, bm, bn)
    st = fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                              Hk, Nq, Nk, d, q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3],
                              float(scale), causal, _dtype_code(q), sp, bm, bn, num_splits)
    if st != 0:
        raise FaError(st, "fa_fwd_split_noalloc")
    return out, lse


def bwd(q, k, v, o, dout, lse, scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the attention forward on torch tensors [B, H, N, d]
    (contiguous, same device and 16-bit dtype): o and lse as returned by ``fwd`` for
    the same q, k, v, scale and causal; dout = dL/dO. ``workspace``: a device tensor of
    at least fa_bwd_workspace_bytes(B, H, N) bytes, allocated here if None.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor [B, H, N, d]")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape and dtype")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q.device)
    _check_tensor("lse", lse, q.device, shape=(B, H, N), dtype=torch.float32, contiguous=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.device, shape=q.shape, dtype=q.dtype, contiguous=True)
    need = fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = _workspace_args(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), causal, _dtype_code(q),
                ws_ptr, ws_bytes, sp)
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def bwd_ex(q, k, v, o, dout, lse, scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """Gradients for ``fwd_ex`` with contiguous tensors: q, o, dout [B, Hq, Nq, d]; k, v
    [B, Hk, Nk, d]; lse [B, Hq, Nq] (o and lse from fwd_ex on the same inputs). Returns
    (dq, dk, dv); dk and dv of a K/V head sum over the query heads that share it."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor of q's dtype")
    B, Hq, Nq, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hk, Nk, d] with q's B and d")
    Hk, Nk = k.shape[1], k.shape[2]
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q.device)
    _check_tensor("lse", lse, q.device, shape=(B, Hq, Nq), dtype=torch.float32, contiguous=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, q.device, shape=q.shape, dtype=q.dtype, contiguous=True)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.device, shape=k.shape, dtype=q.dtype, contiguous=True)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(B, Hq, Nq), 16), dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = _workspace_args(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hk, Nq, Nk, d, float(scale), causal,
                   _dtype_code(q), ws_ptr, ws_bytes, sp)
    if st != 0:
        raise FaError(st, "fa_bwd_ex")
    return dq, dk, dv
