"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``io_aware_tiled_02_amd``) never imports it, and this package never imports
the product library: the two share no code.

Contents
  * ``fwd``   -- the plain definition (materialised score row, safe softmax,
                 weighted sum, logsumexp) in C, float64, OpenMP over rows.
  * ``brute`` -- a separate C brute-force twin for tiny shapes.
  * ``bwd``   -- gradients dQ, dK, dV for an upstream dO (definition, fp64).
  * ``attn_range`` / ``merge`` -- one K/V block's attention for a few query
                 rows (rectangular, no mask) and the merge of such partial
                 results: the Flash-Decoding task and its combine step.
  * ``e4m3_value`` / ``e4m3_code`` / ``quantize_fp8`` / ``fwd_fp8`` -- the
                 E4M3 format, FP8 block quantisation of Q and K, and attention
                 on the quantised Q and K (exact dequantisation, then ``fwd``'s
                 definition).
  * ``tiled`` -- float64 NumPy models of the tiled online-softmax algorithm
                 itself, used only to pin that the tiled method is exact.

Every function here is pinned by the CPU tests against closed forms,
invariants, library routines and values printed on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (float64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.fa_oracle_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, d, i, vp, i, vp, vp, i]
        lib.fa_oracle_fwd.restype = i
        lib.fa_oracle_brute.argtypes = [vp, vp, vp, i, i, i, i, d, i, vp, vp]
        lib.fa_oracle_brute.restype = i
        lib.fa_oracle_range.argtypes = [vp, vp, vp, i, i, i, i, i, i, d, i, i, vp, vp, i]
        lib.fa_oracle_range.restype = i
        lib.fa_oracle_merge.argtypes = [vp, vp, i, i, i, vp, vp]
        lib.fa_oracle_merge.restype = i
        lib.fa_oracle_bwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, d, i, vp, vp, vp, i]
        lib.fa_oracle_bwd.restype = i
        lib.fa_oracle_e4m3_value.argtypes = [i]
        lib.fa_oracle_e4m3_value.restype = d
        lib.fa_oracle_e4m3_code.argtypes = [ctypes.c_float]
        lib.fa_oracle_e4m3_code.restype = i
        lib.fa_oracle_quantize_fp8.argtypes = [vp, i, i, i, i, i, i, vp, vp]
        lib.fa_oracle_quantize_fp8.restype = i
        lib.fa_oracle_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, d, i, i, i, vp, i, vp, vp, i]
        lib.fa_oracle_fwd_fp8.restype = i
        lib.fa_oracle_max_threads.argtypes = []
        lib.fa_oracle_max_threads.restype = i
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().fa_oracle_max_threads()


def _storage_check(a: np.ndarray, dtype: int) -> np.ndarray:
    want = {0: np.float32, 1: np.float16, 2: np.uint16, 3: np.float64}[dtype]
    if a.dtype != want:
        raise TypeError(f"dtype code {dtype} expects storage {want}, got {a.dtype}")
    return np.ascontiguousarray(a)


def fwd(q, k, v, dtype: int, scale: float, causal: int, rows=None, nthreads: int = 0):
    """O (B,H,nrows,d) and lse (B,H,nrows), float64, for the given query rows.

    q, k, v: storage arrays (B, H, L, d) -- float32, float16, or uint16 holding
    bfloat16 bits -- exactly as handed to the GPU library; dtype code 3 takes
    float64 arrays (for the oracle's own pins).
    """
    q = _storage_check(q, dtype)
    k = _storage_check(k, dtype)
    v = _storage_check(v, dtype)
    B, H, L, d = q.shape
    if rows is None:
        nrows, rows_arr, rows_ptr = L, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        nrows = int(rows_arr.size)
        rows_ptr = rows_arr.ctypes.data
    o = np.empty((B, H, nrows, d), dtype=np.float64)
    lse = np.empty((B, H, nrows), dtype=np.float64)
    rc = _load().fa_oracle_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dtype,
                               B, H, L, d, float(scale), int(causal), rows_ptr, nrows,
                               o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"fa_oracle_fwd rejected its arguments (rc={rc})")
    return o, lse


def brute(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: int):
    """Brute-force O and lse from float64 (B,H,L,d) inputs; tiny shapes only."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    o = np.empty((B, H, L, d), dtype=np.float64)
    lse = np.empty((B, H, L), dtype=np.float64)
    rc = _load().fa_oracle_brute(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                 B, H, L, d, float(scale), int(causal),
                                 o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"fa_oracle_brute rejected its arguments (rc={rc})")
    return o, lse


def attn_range(q, k, v, dtype: int, scale: float, kv_begin: int, kv_end: int, nthreads: int = 0):
    """O (B,H,Lq,d) and lse (B,H,Lq), float64, of q (B,H,Lq,d) against keys
    [kv_begin, kv_end) of k, v (B,H,Lk,d).  Empty range: O = 0, lse = -inf."""
    q = _storage_check(q, dtype)
    k = _storage_check(k, dtype)
    v = _storage_check(v, dtype)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != k.shape:
        raise ValueError("k and v must be (B, H, Lk, d) matching q")
    o = np.empty((B, H, Lq, d), dtype=np.float64)
    lse = np.empty((B, H, Lq), dtype=np.float64)
    rc = _load().fa_oracle_range(q.ctypes.data, k.ctypes.data, v.ctypes.data, dtype,
                                 B, H, Lq, Lk, d, float(scale), int(kv_begin), int(kv_end),
                                 o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"fa_oracle_range rejected its arguments (rc={rc})")
    return o, lse


def merge(o_parts, lse_parts):
    """Merge partial results: o_parts (S, ..., d), lse_parts (S, ...) float64
    -> o (..., d), lse (...)."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S = o_parts.shape[0]
    d = o_parts.shape[-1]
    rows_shape = o_parts.shape[1:-1]
    if lse_parts.shape != (S,) + rows_shape:
        raise ValueError("lse_parts must be o_parts' shape without its last axis")
    n = int(np.prod(rows_shape)) if rows_shape else 1
    o = np.empty(rows_shape + (d,), dtype=np.float64)
    lse = np.empty(rows_shape, dtype=np.float64)
    rc = _load().fa_oracle_merge(o_parts.ctypes.data, lse_parts.ctypes.data, S, n, d,
                                 o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"fa_oracle_merge rejected its arguments (rc={rc})")
    return o, lse


def bwd(q, k, v, dout, dtype: int, scale: float, causal: int, nthreads: int = 0):
    """dQ, dK, dV (each float64 (B,H,L,d)) of attention for upstream gradient dout."""
    q = _storage_check(q, dtype)
    k = _storage_check(k, dtype)
    v = _storage_check(v, dtype)
    dout = _storage_check(dout, dtype)
    B, H, L, d = q.shape
    for a in (k, v, dout):
        if a.shape != q.shape:
            raise ValueError("q, k, v, dout must share one (B, H, L, d) shape")
    dq = np.empty((B, H, L, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = _load().fa_oracle_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, dtype,
                               B, H, L, d, float(scale), int(causal), dq.ctypes.data, dk.ctypes.data,
                               dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"fa_oracle_bwd rejected its arguments (rc={rc})")
    return dq, dk, dv


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code (NaN for the NaN codes)."""
    return _load().fa_oracle_e4m3_value(int(code))


def e4m3_code(x: float) -> int:
    """E4M3 code of a float32 value |x| <= 448, round to nearest even (-1 if out of range)."""
    return _load().fa_oracle_e4m3_code(float(np.float32(x)))


def quantize_fp8(x, dtype: int, block: int):
    """Block quantisation of x (B, H, L, d) in storage type `dtype` to E4M3.

    Returns codes uint8 (B, H, L, d) and float32 scales (B*H, ceil(L/block))."""
    x = _storage_check(x, dtype)
    B, H, L, d = x.shape
    nblk = (L + block - 1) // block
    x8 = np.empty((B, H, L, d), dtype=np.uint8)
    sc = np.empty((B * H, nblk), dtype=np.float32)
    rc = _load().fa_oracle_quantize_fp8(x.ctypes.data, dtype, B, H, L, d, int(block), x8.ctypes.data, sc.ctypes.data)
    if rc != 0:
        raise ValueError(f"fa_oracle_quantize_fp8 rejected its arguments (rc={rc})")
    return x8, sc


def fwd_fp8(q8, k8, q_scale, k_scale, v, dtype: int, scale: float, causal: int, block_q: int, block_k: int,
            rows=None, nthreads: int = 0):
    """O (B,H,nrows,d) and lse (B,H,nrows), float64, of attention on the
    dequantised q8 * q_scale and k8 * k_scale, with v in storage type `dtype`."""
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v = _storage_check(v, dtype)
    B, H, L, d = q8.shape
    if k8.shape != q8.shape or v.shape != q8.shape:
        raise ValueError("q8, k8, v must share one (B, H, L, d) shape")
    sq = np.ascontiguousarray(q_scale, dtype=np.float32)
    sk = np.ascontiguousarray(k_scale, dtype=np.float32)
    if sq.size != B * H * ((L + block_q - 1) // block_q) or sk.size != B * H * ((L + block_k - 1) // block_k):
        raise ValueError("scale arrays must hold B*H*ceil(L/block) values")
    if rows is None:
        nrows, rows_arr, rows_ptr = L, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        nrows = int(rows_arr.size)
        rows_ptr = rows_arr.ctypes.data
    o = np.empty((B, H, nrows, d), dtype=np.float64)
    lse = np.empty((B, H, nrows), dtype=np.float64)
    rc = _load().fa_oracle_fwd_fp8(q8.ctypes.data, k8.ctypes.data, sq.ctypes.data, sk.ctypes.data, v.ctypes.data,
                                   dtype, B, H, L, d, float(scale), int(causal), int(block_q), int(block_k),
                                   rows_ptr, nrows, o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"fa_oracle_fwd_fp8 rejected its arguments (rc={rc})")
    return o, lse
