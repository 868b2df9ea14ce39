"""Pins of the oracle's quantization grid and packing."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages():
    with open(os.path.join(GOLDEN, "pages_numbers.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("sym", [0, 1, 2])
@pytest.mark.parametrize("qdtype", [np.float64, np.float32])
def test_code_is_nearest_grid_point_bruteforce(bits, sym, qdtype):
    rng = np.random.default_rng(bits * 10 + sym)
    w = rng.standard_normal((16, 64)) * 0.02
    w[3] = np.abs(w[3])           # all-positive group
    w[4] = -np.abs(w[4])          # all-negative group
    w[5] = 0.0                    # degenerate group
    s, z = oracle.grid_params(w, bits, sym, qdtype)
    lo = 1 if sym == 1 else 0
    hi = (1 << bits) - 1
    for r in range(w.shape[0]):
        c, q = oracle.quantize_column(w[r], np.full(64, s[r]), np.full(64, z[r]), bits, sym, qdtype)
        grid = float(s[r]) * (np.arange(lo, hi + 1) - float(z[r]))
        dist = np.abs(w[r][:, None] - grid[None, :])
        best = dist.min(axis=1)
        mine = np.abs(w[r] - float(s[r]) * (c - float(z[r])))
        # chosen point is a nearest one (ties: either neighbour), up to rounding of w/s
        # and, when the decision is taken in binary32, of w itself (|w/s| reaches
        # 2^(b-1), so that rounding matters at 8 bits)
        eps = 1e-6 * float(s[r]) + (2.0 ** -22 * np.abs(w[r]) if qdtype == np.float32 else 0.0)
        assert np.all(mine <= best + eps), r
        assert np.all((c >= lo) & (c <= hi))
        np.testing.assert_allclose(q, float(s[r]) * (c - float(z[r])), rtol=1e-6)


@pytest.mark.parametrize("bits", [3, 4])
def test_symmetric_grid_matches_page_range(bits):
    page = _pages()["sym_range"]
    k = page["bits"].index(bits)
    rng = np.random.default_rng(5)
    w = rng.standard_normal((8, 128))
    s, z = oracle.grid_params(w, bits, True)
    a = np.maximum(-np.minimum(w.min(1), 0), np.maximum(w.max(1), 0))
    np.testing.assert_allclose(s, a / page["levels_max"][k])
    c, q = oracle.quantize_column(w[:, 0] * 0, s, z, bits, True)
    assert np.all(q == 0.0)                               # zero is exactly representable
    c, _ = oracle.quantize_column(w.T, s, z, bits, True)
    lev = c - z[None, :]
    assert lev.min() >= page["levels_min"][k] and lev.max() <= page["levels_max"][k]
    assert lev.min() == page["levels_min"][k] or lev.max() == page["levels_max"][k]


@pytest.mark.parametrize("bits", [3, 4])
def test_asymmetric_grid_covers_range(bits):
    rng = np.random.default_rng(6)
    w = rng.standard_normal((32, 128)) * 0.01 + 0.004
    s, z = oracle.grid_params(w, bits, False)
    assert np.all(z == np.rint(z)) and np.all((z >= 0) & (z <= (1 << bits) - 1))
    c, q = oracle.quantize_column(w.T, s, z, bits, False)
    assert np.all(np.abs(w.T - q) <= s / 2 * (1 + 1e-9))   # every weight within half a step


def test_degenerate_group_uses_unit_range():
    s, z = oracle.grid_params(np.zeros((2, 8)), 4, False)
    np.testing.assert_allclose(s, 2.0 / 15)
    assert np.all(z == 8)          # rint(7.5) = 8, ties to even
    s, z = oracle.grid_params(np.zeros((2, 8)), 4, True)
    np.testing.assert_allclose(s, 1.0 / 7)


def test_worked_example_group_count():
    ex = _pages()["group_worked_example"]
    assert ex["rows"] * ex["n"] == ex["elements"]
    rng = np.random.default_rng(7)
    W = rng.standard_normal((ex["rows"], ex["n"])).astype(np.float32) * 0.02
    r = oracle.rtn(W, oracle.QuantConfig(bits=4, group_size=ex["group_size"]))
    assert r["S"].shape == (ex["n"] // ex["group_size"], ex["rows"])
    assert r["S"].size == ex["groups"] and r["Z"].size == ex["groups"]


def test_quantize_layer_output_shapes():
    rng = np.random.default_rng(8)
    rows, n = 24, 256
    W = rng.standard_normal((rows, n)) * 0.02
    U = np.eye(n)
    for bits in (3, 4):
        out = oracle.quantize_layer(W, U, np.arange(n), np.zeros(n, bool),
                                    oracle.QuantConfig(bits=bits))
        assert out["qweight"].shape == (n * bits // 32, rows) and out["qweight"].dtype == np.int32
        assert out["scales"].shape == (n // 128, rows) and out["scales"].dtype == np.float16
        assert out["zeros"].shape == (n // 128, rows)
        assert out["g_idx"].tolist() == [i // 128 for i in range(n)]


def test_pack_golden_vectors():
    with open(os.path.join(GOLDEN, "pack_vectors.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        codes = np.array(case["codes"])[None, :]
        q = oracle.pack(codes, case["bits"])
        assert q[:, 0].tolist() == case["words"], (case["bits"], case["name"])
        assert oracle.unpack(q, case["bits"], codes.shape[1]).tolist() == codes.tolist()


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(7, 96))
    q = oracle.pack(codes, bits)
    assert q.shape == (96 * bits // 32, 7)
    assert np.array_equal(oracle.unpack(q, bits, 96), codes)


def test_pack_3bit_straddling_columns():
    # In each 32-column chunk, columns 10 and 21 are split across two words.
    codes = np.zeros((1, 64), dtype=np.int64)
    codes[0, 10] = 0b111
    codes[0, 32 + 21] = 0b101
    q = oracle.pack(codes, 3).view(np.uint32)[:, 0]
    assert q[0] == (0b11 << 30) and q[1] == 0b1
    assert q[4] == (0b1 << 31) and q[5] == 0b10


def test_pack_density_matches_pages():
    p = _pages()
    m = p["memory_175b_4bit"]
    rows, n = 64, 512
    q = oracle.pack(np.zeros((rows, n), dtype=np.int64), 4)
    bytes_per_weight = q.nbytes / (rows * n)
    assert bytes_per_weight == 0.5
    assert m["params"] * bytes_per_weight / 1e9 == pytest.approx(m["gb_4bit"])
    assert m["params"] * 2 / 1e9 == pytest.approx(m["gb_16bit"])
    m70 = p["memory_70b_4bit"]
    assert m70["params"] * bytes_per_weight / 1e9 == pytest.approx(m70["gb_4bit"])
    assert m70["gb_fp16"] / m70["gb_4bit"] == m70["reduction"] == 2 / bytes_per_weight


def test_fp16_cast_round_to_nearest_even():
    # 1 + 2^-11 is exactly halfway between 1 and 1 + 2^-10: ties to the even mantissa (1.0)
    assert oracle.to_fp16(np.float32(1 + 2 ** -11)) == np.float16(1.0)
    assert oracle.to_fp16(np.float32(1 + 3 * 2 ** -11)) == np.float16(1 + 2 ** -9)


def test_dequantize_roundtrip():
    rng = np.random.default_rng(9)
    rows, n, gs, bits = 5, 256, 128, 4
    codes = rng.integers(0, 16, size=(rows, n))
    S = rng.random((n // gs, rows)).astype(np.float16)
    Z = rng.integers(0, 16, size=(n // gs, rows)).astype(np.float16)
    g_idx = np.arange(n) // gs
    What = oracle.dequantize(oracle.pack(codes, bits), S, Z, g_idx, bits, rows, n)
    for r in range(rows):
        for i in (0, 127, 128, 255):
            g = g_idx[i]
            assert What[r, i] == float(S[g, r]) * (codes[r, i] - float(Z[g, r]))


@pytest.mark.parametrize("bits", [3, 4])
def test_full_range_symmetric_grid(bits):
    """sym = 2 keeps the symmetric range [-a, a] but spends all 2^b codes on it:
    a dense ramp over the range lands on every code, zero is exact, and no
    weight of the range is more than half a step from its grid point.  The
    pages' grid (sym = 1) uses 2^b - 1 codes on the same ramp."""
    a = 0.037
    ramp = np.linspace(-a, a, 4001)[None, :]
    s2, z2 = oracle.grid_params(ramp, bits, 2)
    c2, q2 = oracle.quantize_column(ramp[0], s2[0], z2[0], bits, 2)
    assert s2[0] == pytest.approx(2 * a / ((1 << bits) - 1), rel=1e-15)
    assert z2[0] == 1 << (bits - 1)
    assert set(np.unique(c2)) == set(range(1 << bits))
    assert np.max(np.abs(ramp[0] - q2)) <= s2[0] / 2 * (1 + 1e-12)
    c0, q0 = oracle.quantize_column(np.zeros(3), s2[0], z2[0], bits, 2)
    assert np.all(q0 == 0.0)
    s1, z1 = oracle.grid_params(ramp, bits, 1)
    c1, _ = oracle.quantize_column(ramp[0], s1[0], z1[0], bits, 1)
    assert len(np.unique(c1)) == (1 << bits) - 1
