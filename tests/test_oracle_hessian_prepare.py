"""Pins of the oracle's Hessian and prepare steps against things other than itself."""
import numpy as np
import pytest
import scipy.linalg as sla

import oracle
import synth


def test_hessian_bruteforce_tiny():
    # (2/N) sum_t x_t x_t^T with plain Python loops on a 5-feature, 7-token input.
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 5))
    H, N = oracle.hessian(x)
    assert N == 7
    for i in range(5):
        for j in range(5):
            acc = 0.0
            for t in range(7):
                acc += x[t, i] * x[t, j]
            assert H[i, j] == pytest.approx(2.0 * acc / 7, rel=1e-14, abs=1e-15)


def test_hessian_chunked_equals_oneshot_and_is_psd():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1000, 24))
    H1, _ = oracle.hessian(x)
    H2, n2 = oracle.hessian([x[:300], x[300:301], x[301:]])
    assert n2 == 1000
    np.testing.assert_allclose(H1, H2, rtol=1e-12, atol=1e-13)
    assert np.array_equal(H1, H1.T) or np.abs(H1 - H1.T).max() < 1e-14
    assert np.linalg.eigvalsh(H1).min() > -1e-12


def test_hessian_entries_match_full():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((500, 40)).astype(np.float32)
    H, _ = oracle.hessian(x)
    pairs = np.array([[0, 0], [3, 17], [17, 3], [39, 39], [5, 38]])
    np.testing.assert_allclose(oracle.hessian_entries(x, pairs), H[pairs[:, 0], pairs[:, 1]],
                               rtol=1e-12)


def test_hessian_expectation_factor_model():
    # The factor-model generator draws x = s * (B g + 0.5 eps); its covariance is
    # S (B B^T + 0.25 I) S, so E[H] = 2 S (B B^T + 0.25 I) S.  Checked to sampling error.
    wl = synth.get("attn4096").resized(rows=8, n=48, tokens=65536)
    x = synth.activations(wl)                   # bf16-gridded; the rounding bias is ~1e-3
    H, _ = oracle.hessian(x)
    kind, scale, loadings = synth._static(wl, 0)
    cov = (loadings.astype(np.float64) @ loadings.T.astype(np.float64) + 0.25 * np.eye(48))
    expect = 2.0 * (scale[:, None] * cov * scale[None, :])
    rel = np.linalg.norm(H - expect) / np.linalg.norm(expect)
    assert rel < 0.03, rel
    # and a dropped factor 2 or a missing 1/N would be far outside that
    assert np.linalg.norm(H / 2 - expect) / np.linalg.norm(expect) > 0.3


def _spd(n, seed, cond=1e3):
    rng = np.random.default_rng(seed)
    q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.geomspace(1.0, 1.0 / cond, n)
    return (q * ev) @ q.T


def test_prepare_inverse_factor_invariant():
    H = _spd(40, 1, cond=1e4)
    p = oracle.prepare(H, damp=0.01, desc_act=False)
    U = p["U"]
    assert np.allclose(U, np.triu(U))
    assert np.all(np.diag(U) > 0)
    err = np.abs(U.T @ U @ p["Hd"] - np.eye(40)).max()
    assert err < 1e-9, err


def test_prepare_matches_reversed_cholesky_route():
    # A second route to the same factor: with J the index reversal, L = chol(J Hd J)
    # (lower) gives Hd = (J L J)(J L J)^T with J L J upper, so U = J L^{-1} J.
    H = _spd(33, 2, cond=1e3)
    p = oracle.prepare(H, damp=0.05, desc_act=False)
    P = p["Hd"][::-1, ::-1]
    L = sla.cholesky(P, lower=True)
    U2 = sla.solve_triangular(L, np.eye(33), lower=True)[::-1, ::-1]
    np.testing.assert_allclose(p["U"], U2, rtol=1e-9, atol=1e-12)


def test_prepare_rows_closed_form():
    # Row j of U is the first row of (Hd[F,F])^{-1} over its first entry's square root,
    # F = {j..n-1}: the OBS inverse restricted to the not-yet-quantized weights.
    H = _spd(12, 3, cond=50)
    p = oracle.prepare(H, damp=0.01)
    Hd = p["Hd"]
    for j in range(12):
        M = np.linalg.inv(Hd[j:, j:])
        np.testing.assert_allclose(p["U"][j, j:], M[0] / np.sqrt(M[0, 0]), rtol=1e-10)


def test_damping_hand_example():
    H = np.diag([1.0, 2.0, 3.0, 6.0])
    p = oracle.prepare(H, damp=0.01)
    assert p["lam"] == pytest.approx(0.03)
    np.testing.assert_allclose(np.diag(p["Hd"]), [1.03, 2.03, 3.03, 6.03])
    np.testing.assert_allclose(np.diag(p["U"]), 1.0 / np.sqrt([1.03, 2.03, 3.03, 6.03]))


def test_dead_columns():
    H = _spd(6, 4)
    H[2, :] = 0.0
    H[:, 2] = 0.0
    p = oracle.prepare(H, damp=0.0)
    assert p["dead"].tolist() == [False, False, True, False, False, False]
    assert p["Hd"][2, 2] == 1.0


def test_act_order_stable_descending():
    H = np.diag([1.0, 3.0, 3.0, 2.0, 0.0])
    p = oracle.prepare(H, damp=0.01, desc_act=True)
    # dead column 4 gets diagonal 1 and ties with column 0 (lower index first)
    assert p["perm"].tolist() == [1, 2, 3, 0, 4]
    np.testing.assert_allclose(np.diag(p["Hd"]) - p["lam"], [3.0, 3.0, 2.0, 1.0, 1.0])


@pytest.mark.parametrize("H", [-np.eye(3), np.array([[1.0, 2.0], [2.0, 1.0]]),
                               np.array([[1.0, np.nan], [np.nan, 1.0]])])
def test_not_positive_definite_raises(H):
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.prepare(H, damp=0.0)
