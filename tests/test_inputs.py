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
    big = gen.fill(gen.BF16, (5_000_000,), 9, 2)     # spans two internal chunks
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
