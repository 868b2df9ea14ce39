"""Pins of the block-sequential oracle (oracle/block.py): closed forms of each
forward piece, a brute-force per-token forward, and the stage wiring."""
import math

import numpy as np
import pytest

import oracle
from oracle import block as B


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0]])
    assert B.rmsnorm(x, eps=0.0) == pytest.approx(np.array([[3.0, 4.0]]) / math.sqrt(12.5), rel=1e-15)
    rng = np.random.default_rng(0)
    y = rng.standard_normal((5, 64)) * 7
    r = B.rmsnorm(y, eps=0.0)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-14)            # unit mean square
    np.testing.assert_allclose(B.rmsnorm(3.5 * y, eps=0.0), r, rtol=1e-14)          # scale invariant
    assert B.rmsnorm(np.zeros((1, 4)))[0, 0] == 0.0                                 # eps keeps zero rows finite


def test_rope_hand_example_and_invariants():
    # head_dim 2: one frequency, base^0 = 1 rad per position
    x = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 2.0]])
    r = B.rope(x, head_dim=2)
    np.testing.assert_allclose(r[0], [1.0, 0.0], atol=1e-15)                       # position 0: identity
    np.testing.assert_allclose(r[1], [math.cos(1), math.sin(1)], rtol=1e-15)
    np.testing.assert_allclose(r[2], [-2 * math.sin(2), 2 * math.cos(2)], rtol=1e-14)
    rng = np.random.default_rng(1)
    L, hd = 9, 8
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    Rq = B.rope(np.tile(q, (L, 1)), head_dim=hd)
    Rk = B.rope(np.tile(k, (L, 1)), head_dim=hd)
    # norms kept; scores depend on the position difference only
    np.testing.assert_allclose(np.linalg.norm(Rq, axis=1), np.linalg.norm(q), rtol=1e-14)
    for m, n in ((3, 1), (7, 2), (4, 4)):
        assert Rq[m] @ Rk[n] == pytest.approx(Rq[m - n] @ Rk[0], rel=1e-12, abs=1e-12)


def _attention_bruteforce(q, k, v, hd):
    L, d = q.shape
    out = np.zeros((L, d))
    for h in range(d // hd):
        for t in range(L):
            sc = [sum(q[t, h * hd + i] * k[u, h * hd + i] for i in range(hd)) / math.sqrt(hd) for u in range(t + 1)]
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            z = sum(w)
            for i in range(hd):
                out[t, h * hd + i] = sum(w[u] * v[u, h * hd + i] for u in range(t + 1)) / z
    return out


def test_causal_attention_bruteforce_and_special_cases():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((5, 8)) for _ in range(3))
    np.testing.assert_allclose(B.causal_attention(q, k, v, head_dim=4), _attention_bruteforce(q, k, v, 4),
                               rtol=1e-13, atol=1e-15)
    o = B.causal_attention(np.zeros((6, 8)), k[:1].repeat(6, 0), np.arange(48.0).reshape(6, 8), head_dim=4)
    np.testing.assert_allclose(o, np.cumsum(np.arange(48.0).reshape(6, 8), 0) / np.arange(1, 7)[:, None],
                               rtol=1e-14)   # zero queries: the mean of the values so far
    np.testing.assert_allclose(B.causal_attention(q, k, v, head_dim=4)[0], v[0], rtol=1e-14)


def test_silu_closed_form():
    assert B.silu(0.0) == 0.0
    assert B.silu(2.0) == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert B.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert B.silu(-40.0) == pytest.approx(0.0, abs=1e-15)


def test_to_half_rounding():
    assert B.to_half(1.0 + 2.0 ** -11) == 1.0                     # half way: to even
    assert B.to_half(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert B.to_half(65504.0) == 65504.0


def _tiny_block(seed=3, d=8, f=12, hd=4, seqs=2, L=3):
    rng = np.random.default_rng(seed)
    X0 = rng.standard_normal((seqs * L, d))
    rows = (d, d, d, d, f, f, d)
    cols = (d, d, d, d, d, d, f)
    Ws = [rng.standard_normal((r, c)) * 0.3 for r, c in zip(rows, cols)]
    return X0, Ws, hd, L


def test_block_forward_against_a_per_token_bruteforce():
    """The stage wiring, recomputed token by token with plain loops from the
    quantized weights the oracle returns (a separate implementation of the
    Llama block's forward)."""
    X0, Ws, hd, L = _tiny_block()
    cfg = oracle.QuantConfig(bits=4, group_size=-1, desc_act=False)
    # widths 8 and 12 are not multiples of 32: use 8-bit codes so packing is defined
    cfg = oracle.QuantConfig(bits=8, group_size=-1, desc_act=False)
    r = B.block_sequential(X0, Ws, cfg, seq_len=L, head_dim=hd)
    Wq, Wk, Wv, Wo, Wg, Wu, Wd = (r["layers"][i]["What"] for i in range(7))
    T, d = X0.shape
    half = lambda x: float(np.float16(x))

    def rms(v):
        m = sum(t * t for t in v) / len(v)
        return [t / math.sqrt(m + 1e-5) for t in v]

    def mv(W, v):
        return [sum(W[o][i] * v[i] for i in range(len(v))) for o in range(len(W))]

    def rot(v, p):
        out = list(v)
        for h in range(len(v) // hd):
            for i in range(hd // 2):
                a, b = v[h * hd + i], v[h * hd + hd // 2 + i]
                ang = p * 10000.0 ** (-2.0 * i / hd)
                out[h * hd + i] = a * math.cos(ang) - b * math.sin(ang)
                out[h * hd + hd // 2 + i] = b * math.cos(ang) + a * math.sin(ang)
        return out

    xa = [[half(t) for t in rms(X0[i])] for i in range(T)]
    np.testing.assert_array_equal(r["acts"]["attn_in"], xa)
    Q = [rot(mv(Wq, xa[t]), t % L) for t in range(T)]
    K = [rot(mv(Wk, xa[t]), t % L) for t in range(T)]
    V = [mv(Wv, xa[t]) for t in range(T)]
    xo = []
    for t in range(T):
        s0 = t - t % L
        row = []
        for h in range(d // hd):
            sc = [sum(Q[t][h * hd + i] * K[u][h * hd + i] for i in range(hd)) / math.sqrt(hd) for u in range(s0, t + 1)]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            row += [sum(w[u - s0] * V[u][h * hd + i] for u in range(s0, t + 1)) / sum(w) for i in range(hd)]
        xo.append([half(x) for x in row])
    np.testing.assert_allclose(r["acts"]["o_in"], xo, rtol=2 ** -10, atol=0)
    h1 = [[X0[t][i] + mv(Wo, xo[t])[i] for i in range(d)] for t in range(T)]
    xm = [[half(x) for x in rms(h1[t])] for t in range(T)]
    np.testing.assert_allclose(r["acts"]["mlp_in"], xm, rtol=2 ** -10, atol=0)
    xd = [[half(g / (1 + math.exp(-g)) * u) for g, u in zip(mv(Wg, xm[t]), mv(Wu, xm[t]))] for t in range(T)]
    np.testing.assert_allclose(r["acts"]["down_in"], xd, rtol=2 ** -10, atol=0)
    out = [[h1[t][i] + mv(Wd, xd[t])[i] for i in range(d)] for t in range(T)]
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_block_stages_use_the_quantized_weights_and_their_own_hessians():
    X0, Ws, hd, L = _tiny_block(seed=4)
    cfg = oracle.QuantConfig(bits=8, group_size=-1)
    r = B.block_sequential(X0, Ws, cfg, seq_len=L, head_dim=hd)
    for stage, idx in B.STAGES:
        H, _ = oracle.hessian(r["acts"][stage])
        np.testing.assert_array_equal(r["H"][stage], H)
        for li in idx:
            assert np.array_equal(r["layers"][li]["plain"]["codes"],
                                  oracle.gptq_layer(Ws[li], H, cfg)["codes"])
    # the o input comes from the quantized q/k/v, not from the original weights
    Xo_orig = B.attention_output(r["acts"]["attn_in"], Ws[0], Ws[1], Ws[2], L, hd)
    assert not np.array_equal(Xo_orig, r["acts"]["o_in"])
    # following its own results changes nothing
    fol = [dict(codes=r["layers"][i]["plain"]["codes"], zeros=r["layers"][i]["plain"]["Z"]) for i in range(7)]
    r2 = B.block_sequential(X0, Ws, cfg, seq_len=L, head_dim=hd, follow=fol, tie_tol=2.0 ** -15)
    for stage in r["acts"]:
        np.testing.assert_array_equal(r["acts"][stage], r2["acts"][stage])
    for i in range(7):
        assert r2["layers"][i]["followed"]["follow"]["unexplained"] == 0
