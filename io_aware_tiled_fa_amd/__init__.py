"""Python binding of libfa_fwd.so, the gfx950 FlashAttention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fa.h``.  PyTorch is used for
device memory and the current HIP stream, nothing else.  There is no fallback:
if the library is missing or fails to load, every call raises.

Functions with the C names take raw integers (device addresses, sizes) exactly
as the C ABI does; :func:`fwd` is the tensor-level convenience wrapper.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FaError", "lib_path", "load", "fa_fwd", "fa_fwd_general", "fa_check_args",
           "fa_fwd_splitkv", "fa_splitkv_workspace_bytes", "fa_splitkv_check_args",
           "fa_fwd_splitkv_noalloc", "NOALLOC_MAX_BYTES", "fa_bwd",
           "fa_bwd_check_args", "fa_status_string", "fa_abi_version", "fwd", "bwd", "DTYPE_F32",
           "DTYPE_F16", "DTYPE_BF16", "STATUS", "MAX_SPLITS"]

DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_BAD_DTYPE",
    4: "FA_ERR_UNSUPPORTED_D", 5: "FA_ERR_BAD_SCALE", 6: "FA_ERR_MISALIGNED",
    7: "FA_ERR_TOO_LARGE", 8: "FA_ERR_HIP", 9: "FA_ERR_WORKSPACE", 10: "FA_ERR_SCRATCH_LIMIT",
}
MAX_SPLITS = 64
NOALLOC_MAX_BYTES = 64 << 20  # FA_NOALLOC_MAX_BYTES in include/fa.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str = "fa_fwd"):
        self.status = status
        super().__init__(f"{where} failed: {fa_status_string(status)} ({status})")


def lib_path() -> str:
    return os.path.join(_HERE, "libfa_fwd.so")


def load():
    """Load libfa_fwd.so (once) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m io_aware_tiled_fa_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    i64, vp, fp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, fp, ctypes.c_int,
                           ctypes.c_int, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_general.argtypes = lib.fa_fwd.argtypes
    lib.fa_fwd_general.restype = ctypes.c_int
    lib.fa_check_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, fp,
                                  ctypes.c_int, ctypes.c_int]
    lib.fa_check_args.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, fp, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, fp,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.fa_splitkv_workspace_bytes.restype = i64
    lib.fa_splitkv_check_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, fp,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64]
    lib.fa_splitkv_check_args.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp] * 10 + [i64, i64, i64, i64, i64, fp, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_check_args.argtypes = [vp] * 10 + [i64, i64, i64, i64, i64, fp, ctypes.c_int,
                                                  ctypes.c_int]
    lib.fa_bwd_check_args.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream=None) -> int:
    """Direct call of the C entry point; pointers are integer device addresses."""
    return load().fa_fwd(q, k, v, o, lse, B, H, M, N, D, float(scale), int(causal), int(dtype),
                         stream)


def fa_fwd_general(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream=None) -> int:
    """Direct call of the C entry point that always runs the general kernel."""
    return load().fa_fwd_general(q, k, v, o, lse, B, H, M, N, D, float(scale), int(causal),
                                 int(dtype), stream)


def fa_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype) -> int:
    return load().fa_check_args(q, k, v, o, lse, B, H, M, N, D, float(scale), int(causal),
                                int(dtype))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, splits, workspace,
                   workspace_bytes, stream=None) -> int:
    """Direct call of the C entry point; pointers are integer device addresses."""
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, H, M, N, D, float(scale), int(causal),
                                 int(dtype), int(splits), workspace, int(workspace_bytes), stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, splits,
                           stream=None) -> int:
    """Direct call of the allocation-free split-KV entry point (static scratch)."""
    return load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, M, N, D, float(scale),
                                         int(causal), int(dtype), int(splits), stream)


def fa_splitkv_workspace_bytes(B, H, M, D, splits) -> int:
    return load().fa_splitkv_workspace_bytes(B, H, M, D, int(splits))


def fa_splitkv_check_args(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, splits, workspace,
                          workspace_bytes) -> int:
    return load().fa_splitkv_check_args(q, k, v, o, lse, B, H, M, N, D, float(scale), int(causal),
                                        int(dtype), int(splits), workspace, int(workspace_bytes))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale, causal, dtype,
           stream=None) -> int:
    """Direct call of the C entry point; pointers are integer device addresses."""
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, float(scale),
                         int(causal), int(dtype), stream)


def fa_bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale, causal,
                      dtype) -> int:
    return load().fa_bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D,
                                    float(scale), int(causal), int(dtype))


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_abi_version() -> int:
    return load().fa_abi_version()


def _dtype_code(t):
    import torch

    codes = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return codes[t.dtype]


def _check_given(t, name, shape, dtype, device):
    """A caller-supplied output or workspace tensor must match what the kernels
    write through its pointer: shape, dtype, device and a contiguous layout."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
        stream=None, general: bool = False, splits: int | None = None, workspace=None):
    """O, LSE = attention forward of q [B,H,M,D], k/v [B,H,N,D] (device tensors).

    Allocates ``o`` (like q) and ``lse`` ([B,H,M] fp32) unless given, enqueues
    fa_fwd on ``stream`` (default: torch's current stream) and returns them.
    ``general=True`` calls fa_fwd_general instead; ``splits=S`` calls
    fa_fwd_splitkv with S key chunks (allocating the workspace unless a device
    tensor of enough bytes is given).
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, seq, D]")
    B, H, M, D = q.shape
    N = k.shape[2]
    if tuple(k.shape) != (B, H, N, D) or tuple(v.shape) != (B, H, N, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda:
            raise ValueError("q, k, v must be device tensors")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for t in (k, v):
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_given(out, "out", (B, H, M, D), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    else:
        _check_given(lse, "lse", (B, H, M), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if splits is not None:
        need = max(fa_splitkv_workspace_bytes(B, H, M, D, splits), 0)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        elif workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, H, M, N, D, scale, 1 if causal else 0, code,
                            splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            stream)
        if st != 0:
            raise FaError(st, "fa_fwd_splitkv")
        return out, lse
    entry = fa_fwd_general if general else fa_fwd
    st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, M, N, D, scale, 1 if causal else 0, code, stream)
    if st != 0:
        raise FaError(st)
    return out, lse


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None, dq=None,
        dk=None, dv=None, delta=None, stream=None):
    """dq, dk, dv = gradients of fwd's o (with its lse) for the incoming gradient dout.

    q [B,H,M,D], k/v [B,H,N,D], o and dout [B,H,M,D] (device tensors of one
    dtype: float32, float16 or bfloat16), lse [B,H,M] fp32.  Allocates dq, dk, dv and the
    fp32 workspace ``delta`` [2,B,H,M] unless given, enqueues fa_bwd on
    ``stream`` (default: torch's current stream) and returns (dq, dk, dv).
    """
    import torch

    for t in (q, k, v, o, dout):
        if t.dim() != 4:
            raise ValueError("q, k, v, o, dout must be [B, H, seq, D]")
    B, H, M, D = q.shape
    N = k.shape[2]
    if tuple(k.shape) != (B, H, N, D) or tuple(v.shape) != (B, H, N, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if tuple(o.shape) != (B, H, M, D) or tuple(dout.shape) != (B, H, M, D):
        raise ValueError("o and dout must have the shape of q")
    if tuple(lse.shape) != (B, H, M) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, H, M]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o, dout must share one dtype")
    for t in (q, k, v, o, dout, lse):
        if not t.is_cuda:
            raise ValueError("all tensors must be device tensors")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for t in (k, v, o, dout, lse):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_given(t, name, like.shape, like.dtype, like.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((2, B, H, M), dtype=torch.float32, device=q.device)
    elif (delta.dtype != torch.float32 or delta.numel() < 2 * B * H * M
          or not delta.is_contiguous() or delta.device != q.device):
        raise ValueError("delta must be a contiguous fp32 workspace on q's device "
                         "of at least 2*B*H*M elements")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                B, H, M, N, D, scale, 1 if causal else 0, code, stream)
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv
