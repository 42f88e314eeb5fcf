"""Pins for the router-GEMM reference in the CPU oracle (no GPU).

The source article's Router GEMM splits each fp32 weight into two bf16 parts,
the high part and a residual scaled by 1/256, and runs two bf16 tensor-core
products whose results are combined [Tencent HPC lands in SGLang, challenging
default inference kernels, sec. "Dynamic Attention and Fused MoE target
different bottlenecks"]. The reading: hi = bf16(w), lo = bf16(256 (w - hi)),
w ~ hi + lo / 256. These tests pin the oracle's rounding, split and fp64
products against torch's own bf16 conversion, NumPy, closed forms and the
error bound that follows from two 8-bit roundings.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _torch_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def _special_values():
    rng = np.random.default_rng(0)
    v = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-40, -1e-40, 1.1754944e-38]
    # exact ties: low 16 bits 0x8000, kept lsb even and odd
    for hi in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x0001, 0x7F7E, 0x7F7F):
        v.append(np.array([(hi << 16) | 0x8000], np.uint32).view(np.float32)[0])
        v.append(np.array([(hi << 16) | 0x7FFF], np.uint32).view(np.float32)[0])
        v.append(np.array([(hi << 16) | 0x8001], np.uint32).view(np.float32)[0])
    v += list(rng.normal(0, 1, 2000).astype(np.float32))
    v += list((rng.normal(0, 1, 2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32))
    return np.array(v, np.float32)


def test_bf16_rounding_matches_torch():
    v = _special_values()
    mine = np.array([oracle.bf16_rne(float(x)) for x in v], np.uint16)
    assert np.array_equal(mine, _torch_bits(v))


def test_bf16_rounding_keeps_nan():
    nan = np.array([0x7FC00001, 0xFF800001, 0x7F800001], np.uint32).view(np.float32)
    for x in nan:
        b = oracle.bf16_rne(float(x))
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_split_matches_an_independent_construction():
    rng = np.random.default_rng(1)
    w = np.concatenate([rng.normal(0, 0.02, 5000), rng.normal(0, 3, 5000), rng.uniform(-1e-3, 1e-3, 5000)])
    w = w.astype(np.float32)
    hi, lo = oracle.router_split(w)
    hi_t = torch.from_numpy(w).to(torch.bfloat16)
    r = (torch.from_numpy(w) - hi_t.float()) * 256.0
    assert np.array_equal(hi, hi_t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(lo, r.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_split_of_bf16_values_is_exact():
    rng = np.random.default_rng(2)
    b = _torch_bits(rng.normal(0, 1, 4000).astype(np.float32))
    w = _bits_to_f32(b)
    hi, lo = oracle.router_split(w)
    assert np.array_equal(hi, b)
    assert np.all((lo & 0x7FFF) == 0)        # +-0


def test_split_error_bound():
    """hi is w to 8 significant bits (|w - hi| <= 2^-8 |w|), lo is 256 (w - hi)
    to 8 bits, so |w - (hi + lo/256)| <= 2^-8 * 2^-8 |w| = 2^-16 |w| for normal
    values (tiny weights, whose residual falls below the normal range, excepted)."""
    rng = np.random.default_rng(3)
    w = (rng.normal(0, 1, 20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    hi, lo = oracle.router_split(w)
    approx = _bits_to_f32(hi).astype(np.float64) + _bits_to_f32(lo).astype(np.float64) / 256.0
    err = np.abs(w.astype(np.float64) - approx)
    assert np.all(err <= 2.0 ** -16 * np.abs(w.astype(np.float64)))
    # and the split is much closer than bf16 alone (what a single bf16 product would use)
    assert np.median(err / np.abs(w)) < 2.0 ** -6 * np.median(np.abs(w - _bits_to_f32(hi)) / np.abs(w))


def _x_bits(rng, M, K, scale=1.0):
    return _torch_bits((rng.normal(0, scale, (M, K))).astype(np.float32))


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 7, 5), (4, 128, 16), (17, 300, 9)])
def test_gemm_matches_numpy(shape):
    M, K, E = shape
    rng = np.random.default_rng(sum(shape))
    x = _x_bits(rng, M, K)
    w = rng.normal(0, 0.05, (E, K)).astype(np.float32)
    ye, ys = oracle.router_gemm(x, w)
    xf = _bits_to_f32(x).astype(np.float64)
    np.testing.assert_allclose(ye, xf @ w.astype(np.float64).T, rtol=1e-12, atol=1e-14)
    hi, lo = oracle.router_split(w)
    ws = _bits_to_f32(hi).astype(np.float64) + _bits_to_f32(lo).astype(np.float64) / 256.0
    np.testing.assert_allclose(ys, xf @ ws.T, rtol=1e-12, atol=1e-14)


def test_gemm_one_hot_rows_select_weights():
    rng = np.random.default_rng(4)
    K, E = 64, 12
    w = rng.normal(0, 1, (E, K)).astype(np.float32)
    x = np.zeros((K, K), np.float32)
    np.fill_diagonal(x, 1.0)
    ye, ys = oracle.router_gemm(_torch_bits(x), w)
    assert np.array_equal(ye, w.T.astype(np.float64))
    hi, lo = oracle.router_split(w)
    assert np.array_equal(ys, (_bits_to_f32(hi).astype(np.float64) + _bits_to_f32(lo).astype(np.float64) / 256.0).T)


def test_split_product_within_the_bound_of_the_exact_product():
    rng = np.random.default_rng(5)
    M, K, E = 8, 4096, 32
    x = _x_bits(rng, M, K)
    w = rng.normal(0, 0.02, (E, K)).astype(np.float32)
    ye, ys = oracle.router_gemm(x, w)
    bound = 2.0 ** -16 * (np.abs(_bits_to_f32(x).astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(ys - ye) <= bound)
    assert math.isfinite(float(np.abs(ye).max()))
