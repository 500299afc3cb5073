"""Pins of the oracle's MXFP4 dequantisation and of the MXFP4 input generator.

The format (OCP Microscaling Formats v1.0): FP4 E2M1 elements, whose sixteen
values are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, and one E8M0 scale
2^(s - 127) per block of 32 elements. The pages name the format only (page
"FreeToken-benchmark", model table, DeepSeek-V4-Flash row).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import gen

FP4_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the format's value table


def test_e2m1_table_is_the_format_table():
    assert list(oracle.E2M1[:8]) == FP4_MAGNITUDES
    assert list(oracle.E2M1[8:]) == [-v for v in FP4_MAGNITUDES]
    assert math.copysign(1.0, oracle.E2M1[8]) == -1.0  # code 8 is -0


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(120) == 2.0 ** -7
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def test_dequant_block_and_column_boundaries():
    # 64 rows of K, 3 columns; every block/column gets its own scale, so a
    # transposed index or an off-by-one block boundary changes the result
    K, N = 64, 3
    codes = np.zeros((K, N), np.uint8)
    codes[31, 0] = 7     # +6, last row of block 0
    codes[32, 0] = 15    # -6, first row of block 1
    codes[0, 1] = 3      # +1.5
    codes[63, 2] = 9     # -0.5
    scales = np.array([[127, 120, 130], [125, 131, 100]], np.uint8)  # [K/32, N]
    w = oracle.dequant_mxfp4(codes, scales)
    assert w.shape == (K, N)
    assert w[31, 0] == 6.0 * 2.0 ** 0
    assert w[32, 0] == -6.0 * 2.0 ** -2
    assert w[0, 1] == 1.5 * 2.0 ** -7
    assert w[63, 2] == -0.5 * 2.0 ** -27
    assert np.count_nonzero(w) == 4


def test_dequant_matmul_brute_force():
    # x . W with W from codes and scales, against a term-by-term sum of the table values
    r = np.random.default_rng(1)
    K, N = 64, 4
    codes = r.integers(0, 16, size=(K, N)).astype(np.uint8)
    scales = r.integers(115, 135, size=(K // 32, N)).astype(np.uint8)
    x = r.standard_normal(K)
    got = x @ oracle.dequant_mxfp4(codes, scales)
    for n in range(N):
        ref = math.fsum(x[k] * FP4_MAGNITUDES[codes[k, n] & 7] * (-1.0 if codes[k, n] & 8 else 1.0)
                        * 2.0 ** (int(scales[k // 32, n]) - 127) for k in range(K))
        assert abs(got[n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_quantizer_grid_values_round_trip_exactly():
    # values already on the FP4 grid times a power of two come back unchanged
    grid = torch.tensor(FP4_MAGNITUDES + [-v for v in FP4_MAGNITUDES[1:]], dtype=torch.float32)
    w = torch.zeros(32, 3)
    w[:15, 0] = grid * 2.0 ** -5
    w[:15, 1] = grid * 2.0 ** 3
    w[:15, 2] = grid
    c, s = gen.quantize_mxfp4(w)
    assert np.array_equal(oracle.dequant_mxfp4(c, s), w.double().numpy())
    # max |w| = 6 * 2^X gives shared exponent X (floor(log2 6) - 2 = 0)
    assert [int(v) for v in s[0]] == [127 - 5, 127 + 3, 127]


def test_quantizer_ties_to_even_and_saturation():
    # block max 4 -> X = 0: the values are quantised as they are
    vals = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.3, 2.6, -0.25, -5.0]
    want = [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 0.5, 3.0, -0.0, -4.0]
    w = torch.zeros(32, 1)
    w[:len(vals), 0] = torch.tensor(vals)
    c, s = gen.quantize_mxfp4(w)
    assert int(s[0, 0]) == 127
    assert list(oracle.dequant_mxfp4(c, s)[:len(vals), 0]) == want
    # block max 7.9 -> X = floor(log2 7.9) - 2 = 0 as well; 7.9 saturates to 6
    w = torch.zeros(32, 1)
    w[0, 0] = 7.9
    c, s = gen.quantize_mxfp4(w)
    assert int(s[0, 0]) == 127 and oracle.dequant_mxfp4(c, s)[0, 0] == 6.0


@pytest.mark.parametrize("std", [1e-3, 0.02, 1.0])
def test_quantizer_error_bound(std):
    # in units of 2^X: |w - deq| <= half the FP4 spacing at |w| (0.25 up to 2, 0.5 up to 4, 1 up
    # to 6), and values in (6, 8) saturate to 6; the block maximum lies in [4, 8) units
    torch.manual_seed(3)
    w = torch.randn(256, 8) * std
    c, s = gen.quantize_mxfp4(w)
    d = oracle.dequant_mxfp4(c, s)
    X = np.repeat(s.numpy().astype(np.int64) - 127, 32, axis=0)
    err = np.abs(d - w.double().numpy()) / np.ldexp(1.0, X)
    a = np.abs(w.double().numpy()) / np.ldexp(1.0, X)
    half = np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))
    bound = np.maximum(half, a - 6.0)
    assert np.all(err <= bound + 1e-12)
    blockmax = a.reshape(8, 32, 8).max(axis=1)
    assert np.all((blockmax >= 4.0) & (blockmax < 8.0))
