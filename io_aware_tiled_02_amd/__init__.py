"""Exact attention forward pass for AMD Instinct MI355X (gfx950).

A thin ctypes binding of the C ABI declared in include/fa.h and implemented
by the in-tree HIP library libfa_fwd.so.  Every step of the computation runs
in that library's kernels; this module only marshals arguments.  PyTorch is
used for device memory and streams.  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
# size of the device array behind fa_fwd_splitkv_noalloc (include/fa.h)
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")
_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fa_fwd failed: {code} ({msg})")
        self.code = code


def load():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        # PyTorch ships its own HIP runtime, which its libraries ask for by a
        # file name other than the soname this library asks for.  Loaded
        # first, this library would bring in the system runtime and torch
        # then a second one, and torch's streams and memory would be foreign
        # to this library's launches (FA_ERR_HIP).  With torch loaded first,
        # both ask for the one runtime already in the process.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_strerror.argtypes = [i]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_last_hip_error.argtypes = []
        lib.fa_last_hip_error.restype = i
        lib.fa_fwd_tiling.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                      ctypes.POINTER(ctypes.c_longlong)]
        lib.fa_fwd_tiling.restype = i
        lib.fa_splitkv_splits.argtypes = [i, i, i]
        lib.fa_splitkv_splits.restype = i
        lib.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        lib.fa_fwd_splitkv.restype = i
        lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        lib.fa_fwd_splitkv_noalloc.restype = i
        lib.fa_combine.argtypes = [vp, vp, i, i, i, i, i, vp, vp, i, vp]
        lib.fa_combine.restype = i
        lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        lib.fa_bwd.restype = i
        lib.fa_quantize_fp8.argtypes = [vp, i, i, i, i, i, i, vp, vp, vp]
        lib.fa_quantize_fp8.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, vp]
        lib.fa_fwd_fp8.restype = i
        _lib = lib
    return _lib


def fa_fwd(q, k, v, o, lse, B, H, L, d, scale, causal, dtype, stream) -> int:
    """The C entry point as is: raw device addresses (ints) and a raw stream handle."""
    return load().fa_fwd(q, k, v, o, lse, B, H, L, d, scale, causal, dtype, stream)


def fa_splitkv_splits(B, H, Lk) -> int:
    return load().fa_splitkv_splits(B, H, Lk)


def fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit) -> int:
    return load().fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, workspace, workspace_size,
                   stream) -> int:
    """The C entry point as is (raw device addresses and stream handle)."""
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, workspace,
                                 workspace_size, stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, stream) -> int:
    """The C entry point as is (raw device addresses and stream handle); the
    partial results go to the library's own per-GPU scratch array."""
    return load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, stream)


def fa_combine(o_part, lse_part, nsplit, B, H, Lq, d, o, lse, dtype, stream) -> int:
    """The C entry point as is (raw device addresses and stream handle)."""
    return load().fa_combine(o_part, lse_part, nsplit, B, H, Lq, d, o, lse, dtype, stream)


def fa_bwd_workspace_bytes(B, H, L) -> int:
    return load().fa_bwd_workspace_bytes(B, H, L)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, L, d, scale, causal, dtype, workspace, workspace_size,
           stream) -> int:
    """The C entry point as is (raw device addresses and stream handle)."""
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, L, d, scale, causal, dtype, workspace,
                         workspace_size, stream)


def fa_quantize_fp8(x, dtype, B, H, L, d, block, x8, scales, stream) -> int:
    """The C entry point as is (raw device addresses and stream handle)."""
    return load().fa_quantize_fp8(x, dtype, B, H, L, d, block, x8, scales, stream)


def fa_fwd_fp8(q8, k8, q_scale, k_scale, v, o, lse, B, H, L, d, scale, causal, dtype, block_q, block_k,
               stream) -> int:
    """The C entry point as is (raw device addresses and stream handle)."""
    return load().fa_fwd_fp8(q8, k8, q_scale, k_scale, v, o, lse, B, H, L, d, scale, causal, dtype, block_q,
                             block_k, stream)


def fa_strerror(code: int) -> str:
    return load().fa_strerror(code).decode()


def fa_last_hip_error() -> int:
    return load().fa_last_hip_error()


def fa_fwd_tiling(B, H, L, d, causal, dtype):
    """(block_rows, block_cols, workgroups) that fa_fwd uses for this shape."""
    br, bc, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_longlong()
    rc = load().fa_fwd_tiling(B, H, L, d, causal, dtype, ctypes.byref(br), ctypes.byref(bc), ctypes.byref(wg))
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return br.value, bc.value, wg.value


def _check(t, name, shape, dtype, device):
    """A caller-given tensor must be a contiguous device tensor of exactly this
    shape and dtype on `device`: the kernels index it as such, so anything
    else would be read or written out of bounds."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         + ("" if t.is_contiguous() else " (not contiguous)"))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def forward(q, k, v, scale: float, causal: bool = False, out=None, lse=None, stream=None):
    """O and lse for torch device tensors q, k, v of shape (B, H, L, d).

    Outputs are allocated with torch unless given.  The work is enqueued on
    `stream` (default: torch's current stream) and not waited for.
    """
    import torch
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 4:
        raise ValueError("q, k, v must share one (B, H, L, d) shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors on one device")
    B, H, L, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    _check(out, "out", q.shape, q.dtype, q.device)
    _check(lse, "lse", (B, H, L), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, L, d, float(scale), int(bool(causal)), _dtype_code(q), stream.cuda_stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return out, lse


def forward_splitkv(q, k, v, scale: float, nsplit: int = 0, out=None, lse=None, workspace=None, stream=None):
    """Split-K/V attention of q (B, H, Lq, d) against k, v (B, H, Lk, d), Lq <= 8.

    The workspace (a uint8 device tensor) is allocated with torch unless given.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q is (B, H, Lq, d); k and v share one (B, H, Lk, d) shape")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("q and k/v disagree on B, H or d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors on one device")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    _check(out, "out", q.shape, q.dtype, q.device)
    _check(lse, "lse", (B, H, Lq), torch.float32, q.device)
    need = fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, Lq, Lk, d, float(scale), _dtype_code(q), int(nsplit), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return out, lse


def backward(q, k, v, o, lse, dout, scale: float, causal: bool = False, workspace=None, stream=None):
    """dq, dk, dv for torch device tensors (B, H, L, d); o, lse from forward()."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be (B, H, L, d)")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(t, name, q.shape, q.dtype, q.device)
    B, H, L, d = q.shape
    _check(lse, "lse", (B, H, L), torch.float32, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa_bwd_workspace_bytes(B, H, L)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, float(scale), int(bool(causal)),
                _dtype_code(q), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                stream.cuda_stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return dq, dk, dv


def quantize_fp8(x, block: int, x8=None, scales=None, stream=None):
    """E4M3 codes (uint8, x's shape) and float32 block scales (B*H, ceil(L/block))
    of a 16-bit device tensor x (B, H, L, d)."""
    import torch
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous (B, H, L, d) device tensor")
    B, H, L, d = x.shape
    if block < 1:
        raise ValueError("block must be >= 1")
    if x8 is None:
        x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B * H, (L + block - 1) // block), dtype=torch.float32, device=x.device)
    _check(x8, "x8", x.shape, torch.uint8, x.device)
    _check(scales, "scales", (B * H, (L + block - 1) // block), torch.float32, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    rc = fa_quantize_fp8(x.data_ptr(), _dtype_code(x), B, H, L, d, int(block), x8.data_ptr(), scales.data_ptr(),
                         stream.cuda_stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return x8, scales


def forward_fp8(q8, k8, q_scale, k_scale, v, scale: float, causal: bool, block_q: int, block_k: int, out=None,
                lse=None, stream=None):
    """O (v's dtype) and lse of attention on block-quantised q8, k8 (uint8
    E4M3 codes (B, H, L, d)) with their scales, and 16-bit v (B, H, L, d)."""
    import torch
    if q8.shape != k8.shape or q8.shape != v.shape or q8.dim() != 4:
        raise ValueError("q8, k8, v must share one (B, H, L, d) shape")
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise TypeError("q8 and k8 hold E4M3 codes as uint8")
    for t in (q8, k8, q_scale, k_scale, v):
        if not t.is_cuda or not t.is_contiguous() or t.device != v.device:
            raise ValueError("inputs must be contiguous tensors on one device")
    B, H, L, d = q8.shape
    if block_q < 1 or block_k < 1:
        raise ValueError("block_q and block_k must be >= 1")
    if q_scale.dtype != torch.float32 or k_scale.dtype != torch.float32 or \
            q_scale.numel() != B * H * ((L + block_q - 1) // block_q) or \
            k_scale.numel() != B * H * ((L + block_k - 1) // block_k):
        raise ValueError("scale tensors must hold B*H*ceil(L/block) float32 values")
    if out is None:
        out = torch.empty_like(v)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=v.device)
    _check(out, "out", v.shape, v.dtype, v.device)
    _check(lse, "lse", (B, H, L), torch.float32, v.device)
    if stream is None:
        stream = torch.cuda.current_stream(v.device)
    rc = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(), v.data_ptr(),
                    out.data_ptr(), lse.data_ptr(), B, H, L, d, float(scale), int(bool(causal)), _dtype_code(v),
                    int(block_q), int(block_k), stream.cuda_stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return out, lse
