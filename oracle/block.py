"""Float64 oracle of block-sequential calibration (test infrastructure only).

wikiprompt.org "GPTQ", "Approche technique": the layers are treated one after
another.  polydesk.ai "GPTQ", "Comment fonctionne l'algorithme GPTQ": each
linear layer is solved on its own input activations X, obtained by running
the calibration data through the model.  Read together: inside a decoder
block the linears are quantized in the order their inputs become available,
and each one's Hessian is taken from the activations that reach it through
the already-quantized linears before it:

    Xa = rmsnorm(X0)                              -> q, k, v   (one Hessian)
    Xo = attention(rope(Xa Wq^T), rope(Xa Wk^T), Xa Wv^T)  with quantized Wq, Wk, Wv
                                                  -> o
    h1 = X0 + Xo Wo^T                             with quantized Wo
    Xm = rmsnorm(h1)                              -> gate, up  (one Hessian)
    Xd = silu(Xm Wg^T) * (Xm Wu^T)                with quantized Wg, Wu
                                                  -> down
    out = h1 + Xd Wd^T                            (the next block's input)

The pages do not describe the block itself; it is the Llama-2-7B-shaped
decoder block of the workload (the architecture's published form): RMSNorm
with unit weight (a random-init block) and eps 1e-5, rotary embeddings in the
rotate-half form with base 10000, causal softmax attention over heads of 128,
SiLU-gated MLP.

Rounding points (a reading): every linear's input is held in fp16 (round to
nearest even), the precision a 16-bit model feeds its matmul kernel; the
Hessian of a linear is taken from those fp16 values.  Everything else is
float64 here.  The quantized weights used in the forward are the stored form,
fp16 scale times (code - zero).
"""
from __future__ import annotations

import numpy as np

from .gptq import QuantConfig, dequantize, gptq_layer, hessian, prepare, quantize_layer, rel_loss

EPS = 1e-5
ROPE_BASE = 10000.0


def to_half(x):
    """The value an fp16 activation holds: round to nearest even, back to float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def rmsnorm(x, eps=EPS):
    """x / sqrt(mean(x^2) + eps) along the feature axis (unit weight)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, head_dim=128, base=ROPE_BASE):
    """Rotary position embedding of one sequence x [L, heads * head_dim] at
    positions 0..L-1, rotate-half form: inside each head, features i and
    i + head_dim/2 (i < head_dim/2) are rotated by the angle p * base^(-2i/head_dim)."""
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape
    half = head_dim // 2
    inv = base ** (-2.0 * np.arange(half) / head_dim)
    ang = np.arange(L)[:, None] * inv[None, :]                     # [L, half]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    for h in range(d // head_dim):
        a = x[:, h * head_dim:h * head_dim + half]
        b = x[:, h * head_dim + half:(h + 1) * head_dim]
        out[:, h * head_dim:h * head_dim + half] = a * c - b * s
        out[:, h * head_dim + half:(h + 1) * head_dim] = b * c + a * s
    return out


def causal_attention(q, k, v, head_dim=128):
    """softmax(q k^T / sqrt(head_dim)) v per head over one sequence, each
    position attending to itself and the positions before it."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, d = q.shape
    out = np.empty_like(q)
    mask = np.tril(np.ones((L, L), dtype=bool))
    for h in range(d // head_dim):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        s = q[:, sl] @ k[:, sl].T / np.sqrt(head_dim)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ v[:, sl]
    return out


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def attention_input(X0):
    """Input of q, k and v: fp16 of rmsnorm(X0)."""
    return to_half(rmsnorm(X0))


def attention_output(Xa, Wq, Wk, Wv, seq_len, head_dim=128):
    """Input of o: fp16 of causal attention over each sequence of ``seq_len``
    tokens, with rotary q and k, from the (quantized) q, k, v weights."""
    Q, K, V = Xa @ Wq.T, Xa @ Wk.T, Xa @ Wv.T
    out = np.empty_like(Q)
    for t0 in range(0, Xa.shape[0], seq_len):
        sl = slice(t0, t0 + seq_len)
        out[sl] = causal_attention(rope(Q[sl], head_dim), rope(K[sl], head_dim), V[sl], head_dim)
    return to_half(out)


def mlp_input(X0, Xo, Wo):
    """(h1, input of gate and up): h1 = X0 + Xo Wo^T, then fp16 of rmsnorm(h1)."""
    h1 = np.asarray(X0, dtype=np.float64) + Xo @ Wo.T
    return h1, to_half(rmsnorm(h1))


def down_input(Xm, Wg, Wu):
    """Input of down: fp16 of silu(Xm Wg^T) * (Xm Wu^T)."""
    return to_half(silu(Xm @ Wg.T) * (Xm @ Wu.T))


# linear order of the block and the input each one reads
LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
STAGES = (("attn_in", (0, 1, 2)), ("o_in", (3,)), ("mlp_in", (4, 5)), ("down_in", (6,)))


def solve_stage(X, weights, cfg: QuantConfig, follow=None, tie_tol=None):
    """The Hessian of one stage's input X and the plain solve of each linear
    that reads it (with ``follow``, also the re-run that takes another
    solver's choices at verified ties; see ``sweep``).  Returns (H, [dict(
    plain, followed, What, rel_loss)]) where What, the stored form
    scale * (code - zero) of the followed result (the plain one without
    follow), is what the forward of the later stages uses."""
    H, _ = hessian(X)
    p = prepare(H, cfg.damp, cfg.desc_act)
    out = []
    for k, Wk in enumerate(weights):
        W = np.asarray(Wk, dtype=np.float64)
        plain = gptq_layer(W, H, cfg)
        fol = None
        use = plain
        if follow is not None and follow[k] is not None:
            fol = quantize_layer(W, p["U"], p["perm"], p["dead"], cfg, follow=follow[k], tie_tol=tie_tol)
            use = fol
        rows, n = W.shape
        What = dequantize(use["qweight"], use["scales"], use["zeros"], use["g_idx"], cfg.bits, rows, n)
        out.append(dict(plain=plain, followed=fol, What=What, rel_loss=rel_loss(W, What, H)))
    return H, out


def block_sequential(X0, weights, cfg: QuantConfig, seq_len, head_dim=128, follow=None, tie_tol=None):
    """Calibrates the seven linears of one block in order (see the module
    docstring).  X0 [T, d] holds whole sequences of ``seq_len`` tokens;
    ``weights`` are the seven float arrays [rows, n] in LINEARS order.

    Each linear is solved by the plain per-column sweep (``gptq_layer``) on
    its stage's Hessian.  ``follow`` (optional list of seven dicts, see
    ``sweep``) makes each linear take another solver's code or zero point
    where it differs from this one's at a verified rounding tie, so that the
    forward of the later stages runs with that solver's quantized weights
    whenever its only differences are such ties.

    Returns dict(acts: stage name -> fp16-valued input, H: stage -> Hessian,
    layers: list of seven dicts with the plain result ("plain"), the followed
    one ("followed", None without follow) and the dequantized weights used
    downstream ("What"), h1, out)."""
    X0 = np.asarray(X0, dtype=np.float64)
    acts, Hs, layers = {}, {}, [None] * 7

    def solve(stage_x, idx):
        H, res = solve_stage(stage_x, [weights[li] for li in idx], cfg,
                             None if follow is None else [follow[li] for li in idx], tie_tol)
        for li, r in zip(idx, res):
            layers[li] = r
        return H

    acts["attn_in"] = attention_input(X0)
    Hs["attn_in"] = solve(acts["attn_in"], (0, 1, 2))
    acts["o_in"] = attention_output(acts["attn_in"], layers[0]["What"], layers[1]["What"], layers[2]["What"],
                                    seq_len, head_dim)
    Hs["o_in"] = solve(acts["o_in"], (3,))
    h1, acts["mlp_in"] = mlp_input(X0, acts["o_in"], layers[3]["What"])
    Hs["mlp_in"] = solve(acts["mlp_in"], (4, 5))
    acts["down_in"] = down_input(acts["mlp_in"], layers[4]["What"], layers[5]["What"])
    Hs["down_in"] = solve(acts["down_in"], (6,))
    out = h1 + acts["down_in"] @ layers[6]["What"].T
    return dict(acts=acts, H=Hs, layers=layers, h1=h1, out=out)
