"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, the bench and the smoke check.  It holds
no attention arithmetic: it only turns (seed, stream, index) into numbers and
rounds them to the storage type that both the CPU oracle and the GPU library
read.  Everything is counter-based, so element n of a stream never depends on
how many elements were drawn before it or on chunking.

Generator (its published definitions, restated):
  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the 64-bit finaliser
        z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
        z ^= z >> 27; z *= 0x94D049BB133111EB
        z ^= z >> 31
    applied to key + (n + 1) * 0x9E3779B97F4A7C15 (mod 2**64), where the key
    mixes the seed and the stream id.
  * A uniform in (0, 1): ((x >> 11) + 0.5) * 2**-53.
  * A standard normal by Box-Muller (cosine branch only): element n uses the
    uniforms with counters 2n and 2n+1:  z = sqrt(-2 ln u1) * cos(2 pi u2).
  * value = sigma * z in float64, rounded to float32 (round-to-nearest-even),
    then, for the 16-bit types, rounded again to fp16 / bf16 (RNE).

The floating-point steps (Box-Muller and the roundings) have one definition,
the C library fa_inputs/libfa_gen.so (source fa_gen.c, declared in
include/fa_gen.h, built with gcc by ``build()``): ``normal`` and ``fill`` call
it.  It uses the C library's log, cos and sqrt; numpy's own log differs from
it in the last bit for a fraction of arguments, so the normals are not
recomputed in numpy.  The integer steps (SplitMix64 and the uniforms) are
exact in both languages; they are also written out here in numpy (used to
draw sampled rows) and checked against the C library by the tests.

This is not torch.randn; values are i.i.d. N(0, sigma^2) up to the rounding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import BWD, CONFIGS, DECODE, FP8, BwdConfig, Config, DecodeConfig, Fp8Config, config  # noqa: F401

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_KEY_STREAM = np.uint64(0xD1B54A32D192ED03)

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_SRC = os.path.join(_HERE, "fa_gen.c")
LIB_PATH = os.path.join(_HERE, "libfa_gen.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the generator with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-I" + os.path.join(_ROOT, "include"), "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    """The loaded generator library (built on first use if missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        l = ctypes.CDLL(LIB_PATH)
        vp, i, sz, u64, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_double
        l.fa_gen_key.argtypes = [u64, u64]
        l.fa_gen_key.restype = u64
        l.fa_gen_splitmix64.argtypes = [u64, u64]
        l.fa_gen_splitmix64.restype = u64
        l.fa_gen_fill.argtypes = [vp, i, sz, u64, u64, d]
        l.fa_gen_fill.restype = i
        l.fa_gen_fill_range.argtypes = [vp, i, sz, sz, u64, u64, d]
        l.fa_gen_fill_range.restype = i
        l.fa_gen_normal.argtypes = [vp, sz, sz, u64, u64, d]
        l.fa_gen_normal.restype = i
        l.fa_gen_f32_to_f16.argtypes = [vp, vp, sz]
        l.fa_gen_f32_to_f16.restype = None
        l.fa_gen_f32_to_bf16.argtypes = [vp, vp, sz]
        l.fa_gen_f32_to_bf16.restype = None
        _lib = l
    return _lib


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return np.uint64(seed) * _GOLDEN ^ (np.uint64(stream) + np.uint64(1)) * _KEY_STREAM


def splitmix64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit outputs with counters start .. start+count-1."""
    return splitmix64_from_state(_key(seed, stream), start, count)


def splitmix64_from_state(key, start: int, count: int) -> np.ndarray:
    """SplitMix64 outputs start .. start+count-1 from the initial state `key`.

    Output n is the finaliser applied to key + (n + 1) * 0x9E3779B97F4A7C15,
    i.e. the (n+1)-th value of the sequential generator seeded with `key`.
    """
    key = np.uint64(key)
    n = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (n + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Uniforms in the open interval (0, 1), float64."""
    x = splitmix64(seed, stream, start, count)
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, stream: int, count: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    """sigma * N(0,1) in float64 for element counters start .. start+count-1."""
    out = np.empty(count, dtype=np.float64)
    rc = lib().fa_gen_normal(out.ctypes.data, start, count, seed, stream, float(sigma))
    if rc != 0:
        raise RuntimeError(f"fa_gen_normal failed: {rc}")
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def fill(dtype: int, shape, seed: int, stream: int, sigma: float = 1.0) -> np.ndarray:
    """A contiguous array in the storage type of `dtype`.

    F32 -> float32, F16 -> float16, BF16 -> uint16 holding bfloat16 bits.
    """
    n = int(np.prod(shape, dtype=np.int64))
    if dtype == F32:
        out = np.empty(n, dtype=np.float32)
    elif dtype == F16:
        out = np.empty(n, dtype=np.float16)
    elif dtype == BF16:
        out = np.empty(n, dtype=np.uint16)
    else:
        raise ValueError(f"unknown dtype code {dtype}")
    rc = lib().fa_gen_fill(out.ctypes.data, dtype, n, seed, stream, float(sigma))
    if rc != 0:
        raise RuntimeError(f"fa_gen_fill failed: {rc}")
    return out.reshape(shape)


def to_float64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of a storage array to float64 (for building test inputs)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def from_float64(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to the storage type (via float32, RNE at each step)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == F16:
        return x32.astype(np.float16)
    return f32_to_bf16_bits(x32)


ROWS_STREAM = 7


def sample_rows(L: int, count: int, seed: int) -> np.ndarray:
    """`count` distinct query indices in [0, L), sorted.

    Always contains {0, 1, 127, 128, L//2, L-1} (those inside [0, L)); the rest
    are drawn uniformly without replacement from stream ROWS_STREAM of `seed`.
    """
    fixed = [r for r in (0, 1, 127, 128, L // 2, L - 1) if 0 <= r < L]
    chosen = list(dict.fromkeys(fixed))
    count = min(count, L)
    ctr = 0
    while len(chosen) < count:
        u = uniform01(seed, ROWS_STREAM, ctr, 1)[0]
        ctr += 1
        r = min(int(u * L), L - 1)
        if r not in chosen:
            chosen.append(r)
    return np.array(sorted(chosen[:count]), dtype=np.int32)


def make_qkv(cfg: "Config"):
    """Q, K, V storage arrays of shape (B, H, L, d) for a workload definition."""
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    q = fill(cfg.dtype, shape, cfg.seed, 0, cfg.sigma_q)
    k = fill(cfg.dtype, shape, cfg.seed, 1, cfg.sigma_k)
    v = fill(cfg.dtype, shape, cfg.seed, 2, cfg.sigma_v)
    return q, k, v


def make_decode_qkv(cfg):
    """Q (B, H, Lq, d) and K, V (B, H, Lk, d) storage arrays for a decoding shape."""
    q = fill(cfg.dtype, (cfg.B, cfg.H, cfg.Lq, cfg.d), cfg.seed, 0, cfg.sigma_q)
    k = fill(cfg.dtype, (cfg.B, cfg.H, cfg.Lk, cfg.d), cfg.seed, 1, cfg.sigma_k)
    v = fill(cfg.dtype, (cfg.B, cfg.H, cfg.Lk, cfg.d), cfg.seed, 2, cfg.sigma_v)
    return q, k, v


def make_bwd_inputs(cfg):
    """Q, K, V and dO storage arrays (B, H, L, d) for a backward shape."""
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    return tuple(fill(cfg.dtype, shape, cfg.seed, s) for s in range(4))


def make_fp8_inputs(cfg):
    """Q, K, V storage arrays (B, H, L, d) in cfg.dtype for an FP8 shape (before quantisation)."""
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    return (fill(cfg.dtype, shape, cfg.seed, 0, cfg.sigma_q), fill(cfg.dtype, shape, cfg.seed, 1, cfg.sigma_k),
            fill(cfg.dtype, shape, cfg.seed, 2, cfg.sigma_v))
