"""Pins of the oracle's column sweep: special cases, closed forms, brute force, invariants."""
import numpy as np
import pytest

import oracle
import synth


def _layer(rows=16, n=64, tokens=512, seed=0, outliers=2):
    """Small correlated layer: X with a decaying spectrum and a few outlier channels."""
    rng = np.random.default_rng(seed)
    q1, _ = np.linalg.qr(rng.standard_normal((n, n)))
    A = q1 * (1.0 / (np.arange(n) + 1.0))[None, :]
    X = (A @ rng.standard_normal((n, tokens)) + 0.05 * rng.standard_normal((n, tokens))).T
    X[:, rng.choice(n, outliers, replace=False)] *= 20
    W = rng.standard_normal((rows, n)) * 0.02
    H, _ = oracle.hessian(X)
    return W, H


@pytest.mark.parametrize("bits,sym,gs", [(4, 0, 128), (3, 0, 128), (4, 1, 128), (3, 1, 128), (4, 2, 128),
                                         (4, 0, 32), (3, 1, 64), (4, 0, -1), (4, 2, -1)])
@pytest.mark.parametrize("qdtype", [np.float64, np.float32])
def test_identity_hessian_equals_rtn_exactly(bits, sym, gs, qdtype):
    rng = np.random.default_rng(bits + 2 * sym)
    W = (rng.standard_normal((20, 256)) * 0.02).astype(np.float32).astype(np.float64)
    cfg = oracle.QuantConfig(bits=bits, group_size=gs, sym=sym, desc_act=True, damp=0.01)
    g = oracle.gptq_layer(W, np.eye(256), cfg, qdtype=qdtype)
    r = oracle.rtn(W, cfg, qdtype=qdtype)
    assert np.array_equal(g["perm"], np.arange(256))
    assert np.array_equal(g["codes"], r["codes"])
    assert np.array_equal(g["What"], r["What"])
    assert np.array_equal(g["S"], r["S"]) and np.array_equal(g["Z"], r["Z"])


def test_single_column_matches_closed_forms():
    W, H = _layer(rows=6, n=24, seed=1)
    cfg = oracle.QuantConfig(bits=4, group_size=8)
    p = oracle.prepare(H, cfg.damp)
    Hd = p["Hd"]
    st = oracle.sweep(W, p["U"], cfg, stop=1)
    s, z = oracle.grid_params(W[:, 0:8], 4, False)
    _, q0 = oracle.quantize_column(W[:, 0], s, z, 4, False)
    err = W[:, 0] - q0
    delta = st["W"][:, 1:] - W[:, 1:]
    Hinv = np.linalg.inv(Hd)
    obs = -np.outer(err / Hinv[0, 0], Hinv[0, 1:])                 # OBS form
    lsq = np.outer(err, Hd[0, 1:] @ np.linalg.inv(Hd[1:, 1:]))      # least-squares minimiser
    np.testing.assert_allclose(delta, obs, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(delta, lsq, rtol=1e-9, atol=1e-15)
    assert np.allclose(st["W"][:, 0], W[:, 0])   # quantized column itself untouched until output


@pytest.mark.parametrize("gs", [8, 32, -1])
def test_bruteforce_obs_tiny(gs):
    W, H = _layer(rows=8, n=32, seed=2)
    cfg = oracle.QuantConfig(bits=3, group_size=gs)
    p = oracle.prepare(H, cfg.damp)
    g = oracle.sweep(W, p["U"], cfg)
    b = oracle.obs_bruteforce(W, p["Hd"], cfg)
    assert np.array_equal(g["codes"], b["codes"])
    np.testing.assert_allclose(g["What"], b["What"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [1, 8, 32, 128])
def test_lazy_blocks_do_not_change_result(block):
    W, H = _layer(rows=12, n=256, seed=3)
    cfg = oracle.QuantConfig(bits=4, group_size=32)
    p = oracle.prepare(H, cfg.damp)
    a = oracle.sweep(W, p["U"], cfg)
    b = oracle.sweep(W, p["U"], cfg, block=block)
    assert np.array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["What"], b["What"], atol=1e-13)
    assert a["L"] == pytest.approx(b["L"], rel=1e-10)


def test_loss_identities():
    W, H = _layer(rows=10, n=128, seed=4)
    cfg = oracle.QuantConfig(bits=4, group_size=32)
    p = oracle.prepare(H, cfg.damp)
    r = oracle.sweep(W, p["U"], cfg)
    D = W - r["What"]
    L = r["L"]
    assert L == pytest.approx(0.5 * np.sum((D @ p["Hd"]) * D), rel=1e-9)
    Hp = H   # desc_act off: sweep order is the original order
    assert np.sum((D @ Hp) * D) == pytest.approx(2 * L - p["lam"] * np.sum(D * D), rel=1e-8)


@pytest.mark.parametrize("name,bits,sym,factor", [("toy256", 4, False, 0.5), ("toy256", 3, True, 0.5),
                                                  ("attn4096", 4, False, 0.5),
                                                  ("mlpdown11008", 3, False, 1.0)])
def test_gptq_beats_rtn(name, bits, sym, factor):
    # GPTQ's loss is below RTN's on every workload; on the correlated ones (decaying
    # spectrum, factor model) by at least 2x.  The SiLU x Student-t activations are
    # nearly uncorrelated, so there the margin is small but still strict.
    wl = synth.get(name)
    if name != "toy256":
        wl = wl.resized(rows=32, n=256, tokens=4096)
    W = synth.weights(wl)
    H, _ = oracle.hessian(synth.activations(wl))
    cfg = oracle.QuantConfig(bits=bits, group_size=128, sym=sym, desc_act=wl.desc_act)
    g = oracle.gptq_layer(W, H, cfg)
    r = oracle.rtn(W, cfg)
    rtn_loss = oracle.rel_loss(W, r["What"], H)
    assert g["rel_loss"] < factor * rtn_loss, (g["rel_loss"], rtn_loss)


def test_hessian_scale_invariance():
    W, H = _layer(rows=16, n=128, seed=5)
    cfg = oracle.QuantConfig(bits=4, group_size=64, desc_act=True)
    a = oracle.gptq_layer(W, H, cfg)
    b = oracle.gptq_layer(W, 4.0 * H, cfg)          # power of two: exact in every step
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert b["L"] == pytest.approx(4.0 * a["L"], rel=1e-12)
    c = oracle.gptq_layer(W, 3.7 * H, cfg)
    assert np.array_equal(a["codes"], c["codes"])
    assert c["rel_loss"] == pytest.approx(a["rel_loss"], rel=1e-9)


def test_rows_are_independent():
    W, H = _layer(rows=20, n=128, seed=6)
    cfg = oracle.QuantConfig(bits=4, group_size=128)
    p = oracle.prepare(H, cfg.damp)
    full = oracle.sweep(W, p["U"], cfg)
    sub = [3, 7, 19]
    part = oracle.sweep(W[sub], p["U"], cfg)
    assert np.array_equal(full["codes"][sub], part["codes"])
    assert np.array_equal(full["What"][sub], part["What"])


def test_act_order_equivariance():
    W, H = _layer(rows=8, n=128, seed=7)
    cfg_on = oracle.QuantConfig(bits=4, group_size=32, desc_act=True)
    cfg_off = oracle.QuantConfig(bits=4, group_size=32, desc_act=False)
    a = oracle.gptq_layer(W, H, cfg_on)
    perm = np.argsort(-np.diag(H), kind="stable")
    assert np.array_equal(a["perm"], perm) and not np.array_equal(perm, np.arange(128))
    b = oracle.gptq_layer(W[:, perm], H[np.ix_(perm, perm)], cfg_off)
    codes = np.empty_like(b["codes"])
    codes[:, perm] = b["codes"]
    assert np.array_equal(a["codes"], codes)
    assert np.array_equal(a["scales"], b["scales"])
    assert np.array_equal(a["g_idx"][perm], np.arange(128) // 32)


def test_dead_column_is_zeroed():
    W, H = _layer(rows=6, n=64, seed=8)
    H[5, :] = 0.0
    H[:, 5] = 0.0
    cfg = oracle.QuantConfig(bits=4, group_size=32)
    out = oracle.gptq_layer(W, H, cfg)
    assert out["dead"][5]
    assert np.all(out["What"][:, 5] == 0.0)
    assert np.all(out["E"][:, 5] == 0.0)
