"""Pins of the oracle's dequantizing matmul and group ordering.

The oracle forms Y = A W_hat^T from the packed outputs (unpack, dequantize,
one matrix product).  These tests tie it to values fixed independently of that
path: a hand-worked example, the zero-point identity, the round-to-nearest
reconstruction of the sweep code (a different code path), the rounding bound
against the original weights, and invariance under the act-order column
permutation.
"""
import numpy as np
import pytest

import oracle


def _packed(codes, bits):
    return oracle.pack(np.asarray(codes, dtype=np.int64), bits)


def test_worked_example_one_hot_rows():
    # 3 output rows, 256 input columns = 2 groups of 128, 4-bit.
    bits, rows, n = 4, 3, 256
    codes = np.full((rows, n), 5, dtype=np.int64)
    codes[0, 3] = 15
    codes[0, 130] = 13
    codes[1, 200] = 0
    codes[2, 255] = 9
    scales = oracle.to_fp16([[0.5, 0.25, 2.0], [0.25, 0.125, 0.0625]])   # [G, rows]
    zeros = oracle.to_fp16([[3, 8, 0], [8, 1, 15]])
    g_idx = np.arange(n) // 128
    A = np.zeros((4, n))
    A[0, 3] = 1.0
    A[1, 130] = 1.0
    A[2, 200] = -2.0
    A[3, 255] = 0.5
    Y = oracle.dequant_matmul(A, _packed(codes, bits), scales, zeros, g_idx, bits, rows, n)
    # by hand: y = a * s[g, r] * (code - z[g, r])
    expect = np.array([
        [0.5 * (15 - 3), 0.25 * (5 - 8), 2.0 * (5 - 0)],            # column 3, group 0
        [0.25 * (13 - 8), 0.125 * (5 - 1), 0.0625 * (5 - 15)],       # column 130, group 1
        [-2 * 0.25 * (5 - 8), -2 * 0.125 * (0 - 1), -2 * 0.0625 * (5 - 15)],   # column 200
        [0.5 * 0.25 * (5 - 8), 0.5 * 0.125 * (5 - 1), 0.5 * 0.0625 * (9 - 15)],  # column 255
    ])
    assert np.array_equal(Y, expect)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codes_at_zero_point_give_zero(bits):
    rng = np.random.default_rng(bits)
    rows, n, gs = 8, 256, 64
    zeros = rng.integers(0, 1 << bits, size=(n // gs, rows))
    g_idx = np.arange(n) // gs
    codes = zeros[g_idx].T                      # code == zero point everywhere
    scales = oracle.to_fp16(rng.uniform(0.01, 1.0, size=(n // gs, rows)))
    A = rng.standard_normal((5, n))
    Y = oracle.dequant_matmul(A, _packed(codes, bits), scales, oracle.to_fp16(zeros), g_idx, bits, rows, n)
    assert np.array_equal(Y, np.zeros((5, rows)))


@pytest.mark.parametrize("bits,gs,sym", [(4, 128, 0), (3, 64, 0), (2, 32, 1), (8, -1, 2)])
def test_matches_round_to_nearest_reconstruction(bits, gs, sym):
    """The sweep's own reconstruction of each weight (quantize_column, used by
    round-to-nearest) against unpack + dequantize + product.  They differ only
    by the fp16 rounding of the scale: |ds| <= 2^-11 s per group."""
    rng = np.random.default_rng(100 + bits)
    rows, n = 24, 256
    W = rng.standard_normal((rows, n)) * 0.02
    cfg = oracle.QuantConfig(bits=bits, group_size=gs, sym=sym)
    r = oracle.rtn(W, cfg)
    G = r["S"].shape[0]
    gsz = n // G
    g_idx = np.arange(n) // gsz
    A = rng.standard_normal((7, n))
    Y = oracle.dequant_matmul(A, _packed(r["codes"], bits), oracle.to_fp16(r["S"]), oracle.to_fp16(r["Z"]),
                              g_idx, bits, rows, n)
    ref = A @ r["What"].T
    s_col = r["S"][g_idx].T                     # [rows, n] scale of each weight
    z_col = r["Z"][g_idx].T
    bound = np.abs(A) @ (2.0 ** -11 * s_col * np.abs(r["codes"] - z_col)).T
    assert np.all(np.abs(Y - ref) <= bound + 1e-15)
    # and the product is within rounding of the original weights: each weight
    # lies within one grid step of its reconstruction
    err = np.abs(Y - A @ W.T)
    assert np.all(err <= np.abs(A) @ (1.001 * s_col).T)


def test_act_order_storage_is_a_joint_permutation():
    """Storing columns in another order (with g_idx and the activations permuted
    the same way) does not change the product."""
    rng = np.random.default_rng(7)
    bits, rows, n, gs = 4, 16, 384, 128
    codes = rng.integers(0, 16, size=(rows, n))
    scales = oracle.to_fp16(rng.uniform(0.01, 0.1, size=(n // gs, rows)))
    zeros = oracle.to_fp16(rng.integers(0, 16, size=(n // gs, rows)))
    g_idx = np.arange(n) // gs
    A = oracle.to_fp16(rng.standard_normal((3, n))).astype(np.float64)
    p = rng.permutation(n)
    Y0 = oracle.dequant_matmul(A, _packed(codes, bits), scales, zeros, g_idx, bits, rows, n)
    Y1 = oracle.dequant_matmul(A[:, p], _packed(codes[:, p], bits), scales, zeros, g_idx[p], bits, rows, n)
    assert np.allclose(Y0, Y1, rtol=1e-12, atol=1e-12)


def test_grouped_order():
    assert oracle.grouped_order([1, 0, 1, 0, 2, 2]).tolist() == [1, 3, 0, 2, 4, 5]
    assert oracle.grouped_order(np.arange(512) // 128).tolist() == list(range(512))
    g = np.array([2, 0, 1, 0, 2, 1, 1, 0, 2])
    o = oracle.grouped_order(g)
    assert sorted(o.tolist()) == list(range(9))
    assert g[o].tolist() == sorted(g.tolist())
