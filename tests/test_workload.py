"""The seeded input generator: Philox4x32-10 known answers, random access,
Gaussian statistics, storage rounding and the workload recipe."""
import numpy as np
import pytest
import torch
from scipy import stats

from routing_permute_grouped_router_amd import workload as wl


def test_philox_known_answers():
    # Known-answer vectors of the Random123 distribution for philox4x32-10.
    assert wl.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert wl.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert wl.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_random_access_and_determinism():
    a = wl.normal(5, 3, 0, 1001, 1.0, "f64")
    for start in (0, 1, 2, 7, 500):
        b = wl.normal(5, 3, start, 1001 - start, 1.0, "f64")
        assert np.array_equal(a[start:], b)
    assert not np.array_equal(a, wl.normal(6, 3, 0, 1001, 1.0, "f64"))
    assert not np.array_equal(a, wl.normal(5, 4, 0, 1001, 1.0, "f64"))


def test_gaussian_statistics():
    z = wl.normal(123, 0, 0, 400000, 1.0, "f64")
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3
    z2 = wl.normal(123, 0, 0, 100000, 0.02, "f64")
    assert abs(z2.std() - 0.02) < 0.001


def test_storage_rounding():
    d = wl.normal(9, 1, 0, 50000, 3.0, "f64")
    f = wl.normal(9, 1, 0, 50000, 3.0, "f32")
    b = wl.normal(9, 1, 0, 50000, 3.0, "bf16")
    assert np.array_equal(f, d.astype(np.float32))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_workload_recipe_shapes_and_stds():
    s = wl.small_shapes()[2]
    w = wl.Workload(s)
    x = w.x()
    assert x.shape == (s.T, s.H) and x.dtype == np.uint16
    w1 = wl.bf16_bits_to_f32(w.w1())
    w2 = wl.bf16_bits_to_f32(w.w2())
    assert w1.shape == (s.E, 2 * s.F, s.H) and w2.shape == (s.E, s.H, s.F)
    assert abs(w1.std() * np.sqrt(s.H) - 1) < 0.02
    assert abs(w2.std() * np.sqrt(s.F) - 1) < 0.02
    # per-expert slices equal the whole
    assert np.array_equal(w.w1(3, 5), w.w1()[3:5])
    assert np.array_equal(w.w2(2, 3), w.w2()[2:3])
    lg = w.logits()
    assert lg.dtype == np.float32 and lg.shape == (s.T, s.E)
    ref = (wl.bf16_bits_to_f32(x).astype(np.float64) @ w.router_weight()).astype(np.float32)
    assert np.array_equal(lg, ref)


def test_zipf_bias_formula():
    b = wl.zipf_bias(128, 1.2)
    r = np.arange(1, 129)
    p = r ** -1.2 / np.sum(r ** -1.2)
    np.testing.assert_allclose(np.exp(b / 2), p, rtol=1e-12)
    assert np.all(np.diff(b) < 0)


def test_tiny_workload_stds():
    s = wl.WORKLOADS[0]
    w = wl.Workload(s)
    assert w.x().dtype == np.float32
    w2 = w.w2()
    assert abs(w2.std() * np.sqrt(s.H) - 1) < 0.03  # down weights use H^-1/2 here
