"""The seeded input generator: published test vectors, determinism, rounding."""
import numpy as np
import pytest
import torch

import fa_inputs as gen


def test_splitmix64_published_vector():
    # the sequential SplitMix64 seeded with 1234567: its first five outputs
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = gen.splitmix64_from_state(1234567, 0, 5)
    assert [int(x) for x in got] == want


def test_counter_based_and_chunk_independent():
    a = gen.normal(3, 1, 1000)
    b = gen.normal(3, 1, 400, start=600)
    np.testing.assert_array_equal(a[600:], b)
    big = gen.fill(gen.BF16, (5_000_000,), 9, 2)     # split over the fill's threads
    tail = gen.from_float64(gen.normal(9, 2, 100, start=4_999_900), gen.BF16)
    np.testing.assert_array_equal(big[-100:], tail)


def test_streams_and_seeds_differ():
    a = gen.normal(1, 0, 64)
    assert not np.array_equal(a, gen.normal(1, 1, 64))
    assert not np.array_equal(a, gen.normal(2, 0, 64))


def test_normal_moments():
    z = gen.normal(0, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3
    assert abs(z.var() - 1.0) < 5e-3
    u = gen.uniform01(0, 0, 0, 1 << 16)
    assert u.min() > 0.0 and u.max() < 1.0


def test_bf16_rounding_matches_torch():
    x = gen.normal(4, 4, 1 << 16, 3.0).astype(np.float32)
    # include exact ties
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], np.float32)
    x = np.concatenate([x, ties])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_fill_storage_types():
    for dt, want in ((gen.F32, np.float32), (gen.F16, np.float16), (gen.BF16, np.uint16)):
        a = gen.fill(dt, (2, 3, 4), 1, 0)
        assert a.dtype == want and a.shape == (2, 3, 4)
    f16 = gen.fill(gen.F16, (1000,), 1, 0)
    np.testing.assert_array_equal(f16, gen.normal(1, 0, 1000).astype(np.float32).astype(np.float16))


def test_sample_rows():
    r = gen.sample_rows(16384, 64, 4)
    assert r.size == 64 and np.all(np.diff(r) > 0)
    for must in (0, 1, 127, 128, 8192, 16383):
        assert must in r
    np.testing.assert_array_equal(r, gen.sample_rows(16384, 64, 4))
    assert gen.sample_rows(3, 64, 4).tolist() == [0, 1, 2]


@pytest.mark.parametrize("idx", range(5))
def test_config_metric_flops(idx):
    c = gen.config(idx)
    full = 4 * c.B * c.H * c.L * c.L * c.d
    assert c.flops == (full // 2 if c.causal else full)


# ---- the C library behind fill / normal (include/fa_gen.h) ----

def _u16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def test_c_splitmix64_matches_numpy_and_published_vector():
    lib = gen.lib()
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [lib.fa_gen_splitmix64(1234567, c) for c in range(5)] == want
    for seed, stream in ((0, 0), (3, 1), (2**40 + 7, 5)):
        key = lib.fa_gen_key(seed, stream)
        assert key == int(gen._key(seed, stream))
        ctrs = [0, 1, 2, 1000, 2**33 + 5]
        ref = [int(gen.splitmix64(seed, stream, c, 1)[0]) for c in ctrs]
        assert [lib.fa_gen_splitmix64(key, c) for c in ctrs] == ref


def test_c_normal_is_box_muller_of_the_uniforms():
    # the definition evaluated element by element with Python floats (the
    # math module calls the same C library log, cos and sqrt)
    import math
    for seed, stream, start, sigma in ((0, 0, 0, 1.0), (7, 2, 123456789, 3.0), (4, 1, 5, 0.25)):
        n = 3000
        u = gen.uniform01(seed, stream, 2 * start, 2 * n)
        ref = [sigma * (math.sqrt(-2.0 * math.log(float(u[2 * i]))) * math.cos(2.0 * math.pi * float(u[2 * i + 1])))
               for i in range(n)]
        np.testing.assert_array_equal(gen.normal(seed, stream, n, sigma, start=start), np.array(ref))


def test_c_fill_roundings():
    n = 50_000
    z = gen.normal(11, 3, n, 2.5)
    z32 = z.astype(np.float32)
    np.testing.assert_array_equal(gen.fill(gen.F32, (n,), 11, 3, 2.5), z32)
    np.testing.assert_array_equal(_u16(gen.fill(gen.F16, (n,), 11, 3, 2.5)), _u16(z32.astype(np.float16)))
    ref_bf16 = torch.from_numpy(z32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.fill(gen.BF16, (n,), 11, 3, 2.5), ref_bf16)


def test_c_half_rounding_against_numpy_over_the_exponent_range():
    # every binade from below the smallest binary16 subnormal to past its
    # overflow, 2**16 mantissa patterns each (low 7 bits cycling, so the
    # rounding bit, the sticky bits and exact ties all occur), both signs
    lib = gen.lib()
    e = np.arange(98, 146, dtype=np.uint32)
    m = np.arange(1 << 16, dtype=np.uint32)
    mant = ((m << np.uint32(7)) | (m & np.uint32(0x7F))) & np.uint32(0x7FFFFF)
    bits = ((e[:, None] << np.uint32(23)) | mant[None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000),
                           np.array([0, 0x80000000, 0x33000000, 0x33000001, 0x477FE000, 0x477FEFFF,
                                     0x477FF000, 0x7F7FFFFF, 0x7F800000, 0xFF800000], np.uint32)])
    x = bits.view(np.float32)
    out = np.empty(x.size, np.uint16)
    lib.fa_gen_f32_to_f16(x.ctypes.data, out.ctypes.data, x.size)
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(out, _u16(x.astype(np.float16)))
    out_bf = np.empty(x.size, np.uint16)
    lib.fa_gen_f32_to_bf16(x.ctypes.data, out_bf.ctypes.data, x.size)
    finite = np.isfinite(x)
    ref = torch.from_numpy(x[finite]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out_bf[finite], ref)


def test_c_fill_range_and_error_codes():
    lib = gen.lib()
    whole = gen.fill(gen.BF16, (10_000,), 5, 1, 1.5)
    part = np.empty(3_000, np.uint16)
    assert lib.fa_gen_fill_range(part.ctypes.data, gen.BF16, 7_000, 3_000, 5, 1, 1.5) == 0
    np.testing.assert_array_equal(part, whole[7_000:])
    buf = np.zeros(4, np.float32)
    assert lib.fa_gen_fill(buf.ctypes.data, 3, 4, 0, 0, 1.0) == -2
    assert lib.fa_gen_fill(None, gen.F32, 4, 0, 0, 1.0) == -1
    assert lib.fa_gen_fill(None, gen.F32, 0, 0, 0, 1.0) == 0
    assert lib.fa_gen_normal(None, 0, 1, 0, 0, 1.0) == -1
    np.testing.assert_array_equal(buf, 0)


def test_fp8_algorithmic_bytes():
    # B1 H32 L8192 d128, 128-row blocks: codes 2 x 32 MiB, V and O 2 x 64 MiB,
    # lse 1 MiB, 2 x 32 x 64 float32 scales
    c = gen.FP8[0]
    assert c.algorithmic_bytes == 2 * 2**25 + 2 * 2**26 + 2**20 + 2 * 32 * 64 * 4 == 202391552
