"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Sizes here are small enough for the oracle to finish in seconds but span
several tiles with ragged tails: Hessian tiles are 128 features and stages of
32 tokens, the factorization uses 64-blocks, the sweep 64-row strips and
128-column blocks.  The full-size workloads are in test_gpu_fullsize.py.

Acceptance: Hessian within 1e-5 relative Frobenius; against the plain
float64 oracle (per-column sweep, float64 decisions) >= 99.9 % identical
codes, scales within 1e-3 relative and zero points equal on >= 99.9 % of
groups, relative loss within 1 %, g_idx exact, packing bit-exact; then every
remaining difference verified as a rounding tie, after which the oracle's
path reproduces every code, zero point and scale (gpu_helpers: follow_check).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_stated_bar, compare_layer, follow_check, layer_inputs, rel_frobenius, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    import post_weight_quantization_13_amd as g
    g.lib()
    torch.cuda.init()
    return g


def _cfg(g, wl):
    return g.Config(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                    damp_percent=wl.damp, block_size=wl.block_size)


def _ocfg(wl):
    return oracle.QuantConfig(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                              damp=wl.damp)


# --------------------------------------------------------------------------- Hessian
@pytest.mark.parametrize("name,n,tokens", [("toy256", None, None), ("attn4096", 300, 1000),
                                           ("attn4096", 640, 5000), ("mlpdown11008", 257, 333),
                                           ("attn4096", 4104, 3001)])
def test_hessian_matches_oracle(g, name, n, tokens):
    import torch
    wl = synth.get(name)
    if n is not None:
        wl = wl.resized(rows=8, n=n, tokens=tokens)
    _, _, xv, xd = layer_inputs(wl)
    H = torch.empty((wl.n, wl.n), dtype=torch.float64, device="cuda")
    cnt = g.gptq_hessian_accumulate(H, 0, xd)
    torch.cuda.synchronize()
    assert cnt == wl.tokens
    Hg = H.cpu().numpy()
    Href, _ = oracle.hessian(xv)
    err = rel_frobenius(Hg, Href)
    print(f"{name} n={wl.n} tokens={wl.tokens}: H rel Frobenius {err:.3e}")
    assert err <= 1e-5
    assert np.array_equal(Hg, Hg.T)


def test_hessian_token_chunks_pieces_and_tails(g):
    """n = 8200 (65 tile rows: rounds of whole tiles plus leftover tiles cut
    into token pieces, a ragged last feature tile) over 40001 tokens, which
    the direct-to-LDS kernel splits into token chunks with a ragged last one.
    Compared with the oracle on a sampled set of 96 features (all pairs among
    them, including features of the ragged tile and at tile boundaries);
    H must also be exactly symmetric."""
    import torch
    wl = synth.get("attn4096").resized(rows=8, n=8200, tokens=40001)
    raw = synth.activations_raw(wl)
    rng = np.random.default_rng(8200)
    cols = np.unique(np.concatenate([[0, 127, 128, 8191, 8192, 8199],
                                     rng.choice(8200, size=90, replace=False)]))
    Href, _ = oracle.hessian(synth.bf16_value(raw[:, cols]))
    H = torch.empty((8200, 8200), dtype=torch.float64, device="cuda")
    assert g.gptq_hessian_accumulate(H, 0, to_device(raw, "bf16")) == 40001
    del raw
    torch.cuda.synchronize()
    assert torch.equal(H, H.T)
    idx = torch.from_numpy(cols).cuda()
    sub = H[idx][:, idx].cpu().numpy()
    err = rel_frobenius(sub, Href)
    print(f"n=8200 tokens=40001: sampled H rel Frobenius {err:.3e}")
    assert err <= 1e-5


@pytest.mark.parametrize("n", [640, 300, 4104])
def test_hessian_graph_replay(g, n):
    """The Hessian call captured in a graph and replayed several times with
    eager work in between: every replay equals the eager result bitwise.
    n = 640 and 4104 take the direct-to-LDS kernel (4104 also its leftover-tile
    pieces and their reduction), n = 300 the register-staged one."""
    import torch
    wl = synth.get("attn4096").resized(rows=8, n=n, tokens=5000)
    xd = to_device(synth.activations_raw(wl), "bf16")
    ws = g.hessian_workspace(n, xd)
    eager = torch.empty((n, n), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(eager, 0, xd, workspace=ws)
    H = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.gptq_hessian_accumulate(H, 0, xd, workspace=ws)      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.gptq_hessian_accumulate(H, 0, xd, workspace=ws)
    for i in range(4):
        H.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(H, eager), i
        _ = (xd.float() * 2).sum().item()                      # eager work between replays


def test_hessian_chunked_and_fp16(g):
    import torch
    wl = synth.get("attn4096").resized(rows=8, n=384, tokens=3000)
    xv = synth.activations(wl)
    Href, _ = oracle.hessian(xv)
    xd = to_device(synth.activations_raw(wl), "bf16")
    H = torch.full((384, 384), float("nan"), dtype=torch.float64, device="cuda")  # ignored when count is 0
    cnt = g.gptq_hessian_accumulate(H, 0, xd[:1234])
    cnt = g.gptq_hessian_accumulate(H, cnt, xd[1234:1234])    # empty chunk: no-op
    cnt = g.gptq_hessian_accumulate(H, cnt, xd[1234:])
    torch.cuda.synchronize()
    assert cnt == 3000
    assert rel_frobenius(H.cpu().numpy(), Href) <= 1e-5
    # fp16 activations (the values rounded to fp16)
    x16 = torch.from_numpy(xv.astype(np.float16)).cuda()
    H16 = torch.empty((384, 384), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H16, 0, x16)
    Href16, _ = oracle.hessian(xv.astype(np.float16).astype(np.float64))
    assert rel_frobenius(H16.cpu().numpy(), Href16) <= 1e-5
    # strided X (ldx > n): a column slice of a wider matrix
    wide = torch.zeros((3000, 400), dtype=torch.bfloat16, device="cuda")
    wide[:, :384] = xd
    Hs = torch.empty((384, 384), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(Hs, 0, wide[:, :384])
    assert rel_frobenius(Hs.cpu().numpy(), Href) <= 1e-5


# --------------------------------------------------------------------------- prepare
def _spd_with_dead(n, seed, dead=()):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3 * n, n)) @ np.diag(np.geomspace(1, 30, n)) + rng.standard_normal((3 * n, n))
    x[:, list(dead)] = 0.0
    H, _ = oracle.hessian(x)
    return H


# n = 4608 is the smallest size here whose trailing passes and last inverse
# level have enough 128x128 tiles to run on the 128-tile fp64 kernels; at
# n = 4096 the factorization's trailing passes switch to them from 128 tiles.
@pytest.mark.parametrize("n,desc_act,dead", [(64, False, ()), (300, True, (7, 299)), (640, False, ()),
                                             (1000, True, (0,)), (4096, False, (5,)), (4608, True, (3, 4000))])
def test_prepare_matches_oracle(g, n, desc_act, dead):
    import torch
    H = _spd_with_dead(n, n, dead)
    cfg = g.Config(desc_act=desc_act, damp_percent=0.01)
    U, perm, deadg = g.prepare(torch.from_numpy(H).cuda(), cfg)
    ref = oracle.prepare(H, 0.01, desc_act)
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(deadg.cpu().numpy().astype(bool), ref["dead"])
    Ug = U.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(Ug, -1) == 0.0)
    err = rel_frobenius(Ug, ref["U"])
    inv_err = np.abs(Ug.T @ Ug @ ref["Hd"] - np.eye(n)).max()
    print(f"prepare n={n}: U rel Frobenius {err:.3e}, |U^T U Hd - I|max {inv_err:.3e}")
    assert err < 1e-6
    assert inv_err < 1e-3


def test_prepare_not_positive_definite(g):
    import torch
    for H in (-np.eye(70), np.diag(np.r_[np.ones(69), np.nan])):
        with pytest.raises(g.GptqError) as ei:
            g.prepare(torch.from_numpy(np.ascontiguousarray(H)).cuda(), g.Config(damp_percent=0.0))
        assert ei.value.status == g.GPTQ_ERR_NOT_PD


# --------------------------------------------------------------------------- quantize
@pytest.mark.parametrize("bits,sym,gs", [(4, 0, 128), (3, 0, 128), (4, 1, 128), (3, 1, 128), (4, 2, 128),
                                         (3, 2, 128), (4, 0, 32), (3, 1, 64), (4, 2, 32), (4, 0, -1), (3, 2, -1),
                                         (2, 0, 128), (2, 1, 64), (8, 0, 128), (8, 1, 32), (8, 2, -1)])
def test_identity_hessian_is_rtn_bit_exact(g, bits, sym, gs):
    import torch
    rows, n = 200, 384
    rng = np.random.default_rng(bits + 10 * sym + gs)
    W = synth.bf16_round((rng.standard_normal((rows, n)) * 0.02).astype(np.float32))
    W[5, :128] = 0.0                                   # a degenerate group (for gs <= 128)
    W[6, :] = 0.0                                      # a degenerate row
    wd = to_device(synth.bf16_bits(W), "bf16")
    cfg = g.Config(bits=bits, sym=sym, group_size=gs, desc_act=True)
    U, perm, dead = g.prepare(torch.eye(n, dtype=torch.float64, device="cuda"), cfg)
    out = g.quantize_layer(U, perm, dead, cfg, wd)
    ocfg = oracle.QuantConfig(bits=bits, group_size=gs, sym=sym)
    r = oracle.rtn(W.astype(np.float64), ocfg, qdtype=np.float32)
    codes = oracle.unpack(out["qweight"].cpu().numpy(), bits, n)
    assert np.array_equal(codes, r["codes"])
    assert np.array_equal(out["scales"].cpu().numpy(), oracle.to_fp16(r["S"]))
    assert np.array_equal(out["zeros"].cpu().numpy(), oracle.to_fp16(r["Z"]))
    assert np.array_equal(out["g_idx"].cpu().numpy(), np.arange(n) // gs if gs > 0 else np.zeros(n, np.int32))


CASES = [
    ("toy256", None),
    ("attn4096", dict(rows=200, n=512, tokens=4096)),
    # three super-blocks of 512 columns: the first one's errors reach the
    # third through the wide update (the second stream); 200 rows leave a
    # ragged row tile
    ("attn4096", dict(rows=200, n=1536, tokens=4096)),
    ("mlpdown11008", dict(rows=136, n=640, tokens=4096)),
    ("down28672", dict(rows=72, n=768, tokens=8192)),
]


def _check_against_plain_oracle(out, rel, wv, Href, ocfg, label):
    """The stated bar against the plain float64 oracle, then the tie check."""
    ref = oracle.gptq_layer(wv.astype(np.float64), Href, ocfg)
    n = wv.shape[1]
    m = compare_layer(out, ref, ocfg.bits, n, wv, Href, rel)
    print(f"{label}: {m}", flush=True)
    assert_stated_bar(m)
    # internal loss: sum e^2 / 2 agrees with the oracle's to the same tolerance
    assert abs(out["loss"] - ref["L"]) <= 0.01 * ref["L"]
    follow_check(out, wv, ref["U"], ref["perm"], ref["dead"], ocfg, ocfg.bits, label=label)
    return ref


@pytest.mark.parametrize("name,size", CASES)
def test_layer_end_to_end(g, name, size):
    import torch
    wl = synth.get(name)
    if size:
        wl = wl.resized(**size)
    wv, wd, xv, xd = layer_inputs(wl)
    cfg = _cfg(g, wl)
    H = torch.empty((wl.n, wl.n), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H, 0, xd)
    U, perm, dead = g.prepare(H, cfg)
    out = g.quantize_layer(U, perm, dead, cfg, wd)
    rel = g.layer_loss(H, wd, out, cfg)
    Href, _ = oracle.hessian(xv)
    _check_against_plain_oracle(out, rel, wv, Href, _ocfg(wl), wl.name)
    rtn = oracle.rtn(wv.astype(np.float64), _ocfg(wl))
    assert rel < oracle.rel_loss(wv, rtn["What"], Href)


@pytest.mark.parametrize("desc_act", [False, True])
def test_layer_with_dead_features(g, desc_act):
    """Calibration features that never fire (zeroed columns of X: H_ii = 0)
    through hessian -> prepare -> quantize: their weight columns are zeroed
    and their diagonal taken as 1 (the dead-column reading of the oracle);
    with act-order the dead features sort last.  Columns 0 (first of the
    first block), 130 (inside the second block), 511 (last column) and a run
    of 40 inside the third block."""
    import torch
    wl = synth.get("attn4096").resized(rows=136, n=512, tokens=4096)
    w_raw = synth.weights_raw(wl)
    x_raw = synth.activations_raw(wl).copy()
    dead_cols = np.r_[0, 130, 300:340, 511]
    x_raw[:, dead_cols] = 0                      # bf16 zero bits
    wv, xv = synth.bf16_value(w_raw), synth.bf16_value(x_raw)
    cfg = g.Config(bits=4, group_size=128, sym=0, desc_act=desc_act, damp_percent=0.01)
    H = torch.empty((512, 512), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H, 0, to_device(x_raw, "bf16"))
    U, perm, dead = g.prepare(H, cfg)
    wd = to_device(w_raw, "bf16")
    out = g.quantize_layer(U, perm, dead, cfg, wd)
    rel = g.layer_loss(H, wd, out, cfg)
    Href, _ = oracle.hessian(xv)
    ocfg = oracle.QuantConfig(bits=4, group_size=128, sym=0, desc_act=desc_act, damp=0.01)
    ref = _check_against_plain_oracle(out, rel, wv, Href, ocfg, f"dead features, desc_act={desc_act}")
    assert np.array_equal(np.nonzero(dead.cpu().numpy())[0], dead_cols)
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    # every dead column dequantizes to exactly 0 in the GPU's packed output
    What = oracle.dequantize(out["qweight"].cpu().numpy(), out["scales"].cpu().numpy(), out["zeros"].cpu().numpy(),
                             out["g_idx"].cpu().numpy(), 4, wl.rows, 512)
    assert np.all(What[:, dead_cols] == 0.0)


@pytest.mark.parametrize("bits,sym,desc_act", [(4, 0, False), (3, 1, True)])
def test_layer_fp16_weights(g, bits, sym, desc_act):
    """W given in fp16 (the values of the bf16 workload re-rounded to fp16)."""
    import torch
    wl = synth.get("attn4096").resized(rows=200, n=640, tokens=4096)
    _, _, xv, xd = layer_inputs(wl)
    w16 = synth.weights(wl).astype(np.float16)
    wv = w16.astype(np.float32)
    wd = torch.from_numpy(w16).cuda()
    cfg = g.Config(bits=bits, group_size=128, sym=sym, desc_act=desc_act, damp_percent=0.01)
    H = torch.empty((wl.n, wl.n), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H, 0, xd)
    U, perm, dead = g.prepare(H, cfg)
    out = g.quantize_layer(U, perm, dead, cfg, wd)
    rel = g.layer_loss(H, wd, out, cfg)
    Href, _ = oracle.hessian(xv)
    ocfg = oracle.QuantConfig(bits=bits, group_size=128, sym=sym, desc_act=desc_act, damp=0.01)
    _check_against_plain_oracle(out, rel, wv, Href, ocfg, f"fp16 W {bits}-bit sym={sym}")


# Group sizes and grids beyond 128 / the pages' sym grid, on the same layers:
# skillmd "Configurações de quantização" ("Máxima precisão": 4-bit, groups of
# 32, act-order, damp 0.005) and polydesk "Paramètres clés" (group_size 64, 32
# and -1 for one group per row).  Groups of 32 and 64 start inside a 128-column
# block, where the kernel takes their grid after the errors of the previous
# sub-block have reached all of the group's columns.
VARIANTS = [
    ("attn4096", dict(rows=200, n=512, tokens=4096), dict(bits=4, group_size=32, sym=0, desc_act=True, damp=0.005)),
    ("attn4096", dict(rows=200, n=1536, tokens=4096), dict(bits=4, group_size=64, sym=0, desc_act=False, damp=0.01)),
    ("mlpdown11008", dict(rows=136, n=640, tokens=4096), dict(bits=3, group_size=32, sym=1, desc_act=True, damp=0.01)),
    ("attn4096", dict(rows=200, n=512, tokens=4096), dict(bits=4, group_size=-1, sym=0, desc_act=True, damp=0.01)),
    ("down28672", dict(rows=72, n=768, tokens=8192), dict(bits=4, group_size=128, sym=2, desc_act=True, damp=0.01)),
    ("attn4096", dict(rows=200, n=512, tokens=4096), dict(bits=3, group_size=64, sym=2, desc_act=False, damp=0.005)),
    # the other widths "Paramètres clés" lists (bits 3, 4 or 8) and 2 bits
    ("attn4096", dict(rows=200, n=512, tokens=4096), dict(bits=8, group_size=128, sym=0, desc_act=True, damp=0.01)),
    ("mlpdown11008", dict(rows=136, n=640, tokens=4096), dict(bits=8, group_size=64, sym=1, desc_act=False, damp=0.01)),
    ("attn4096", dict(rows=200, n=512, tokens=4096), dict(bits=2, group_size=128, sym=0, desc_act=True, damp=0.01)),
    ("down28672", dict(rows=72, n=768, tokens=8192), dict(bits=2, group_size=32, sym=2, desc_act=True, damp=0.01)),
]


@pytest.mark.parametrize("name,size,qc", VARIANTS)
def test_layer_group_and_grid_variants(g, name, size, qc):
    import torch
    wl = synth.get(name).resized(**size)
    wv, wd, xv, xd = layer_inputs(wl)
    cfg = g.Config(bits=qc["bits"], group_size=qc["group_size"], sym=qc["sym"], desc_act=qc["desc_act"],
                   damp_percent=qc["damp"])
    H = torch.empty((wl.n, wl.n), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H, 0, xd)
    U, perm, dead = g.prepare(H, cfg)
    out = g.quantize_layer(U, perm, dead, cfg, wd)
    rel = g.layer_loss(H, wd, out, cfg)
    Href, _ = oracle.hessian(xv)
    ocfg = oracle.QuantConfig(bits=qc["bits"], group_size=qc["group_size"], sym=qc["sym"],
                              desc_act=qc["desc_act"], damp=qc["damp"])
    ngroups = wl.n // qc["group_size"] if qc["group_size"] > 0 else 1
    assert tuple(out["scales"].shape) == (ngroups, wl.rows)
    _check_against_plain_oracle(out, rel, wv, Href, ocfg, f"{wl.name} {qc}")


def test_shared_hessian_several_layers(g):
    """One Hessian and one prepare serve several linears with the same inputs
    (q, k, v of a decoder block); each quantize call matches the oracle."""
    import dataclasses
    import torch
    base = synth.get("llama2block")
    n = 384
    wl = dataclasses.replace(
        base, name="llama2block@qkv", tokens=4096, xsets=((n, "factor", 0, 1.0),),
        linears=tuple(dataclasses.replace(lin, rows=r, n=n) for lin, r in zip(base.linears[:3], (96, 128, 160))))
    x_raw = synth.activations_raw(wl, 0)
    xv = synth.bf16_value(x_raw)
    cfg = _cfg(g, wl)
    H = torch.empty((n, n), dtype=torch.float64, device="cuda")
    g.gptq_hessian_accumulate(H, 0, to_device(x_raw, "bf16"))
    U, perm, dead = g.prepare(H, cfg)
    Href, _ = oracle.hessian(xv)
    p = oracle.prepare(Href, wl.damp, wl.desc_act)
    for li, lin in enumerate(wl.linears):
        w_raw = synth.weights_raw(wl, li)
        wv = synth.bf16_value(w_raw)
        wd = to_device(w_raw, "bf16")
        out = g.quantize_layer(U, perm, dead, cfg, wd)
        rel = g.layer_loss(H, wd, out, cfg)
        ref = oracle.quantize_layer(wv.astype(np.float64), p["U"], p["perm"], p["dead"], _ocfg(wl))
        What16 = oracle.dequantize(ref["qweight"], ref["scales"], ref["zeros"], ref["g_idx"], wl.bits, lin.rows, n)
        ref["rel_loss"] = oracle.rel_loss(wv, What16, Href)
        m = compare_layer(out, ref, wl.bits, n, wv, Href, rel)
        print(f"{lin.name}: {m}")
        assert_stated_bar(m)
        follow_check(out, wv, p["U"], p["perm"], p["dead"], _ocfg(wl), wl.bits, label=lin.name)


def test_quantize_deterministic_and_rows_independent(g):
    import torch
    wl = synth.get("attn4096").resized(rows=130, n=384, tokens=2048)
    _, wd, _, xd = layer_inputs(wl)
    cfg = _cfg(g, wl)
    H, _ = g.hessian(xd)
    H2, _ = g.hessian(xd)
    assert torch.equal(H, H2)
    U, perm, dead = g.prepare(H, cfg)
    U2, _, _ = g.prepare(H, cfg)
    assert torch.equal(U, U2)
    a = g.quantize_layer(U, perm, dead, cfg, wd)
    b = g.quantize_layer(U, perm, dead, cfg, wd)
    for k in ("qweight", "scales", "zeros", "g_idx"):
        assert torch.equal(a[k], b[k])
    assert a["loss"] == b["loss"]
    sub = g.quantize_layer(U, perm, dead, cfg, wd[65:130].contiguous())
    assert torch.equal(sub["qweight"], a["qweight"][:, 65:130])
    assert torch.equal(sub["scales"], a["scales"][:, 65:130])


# --------------------------------------------------------------------------- ABI edge cases
def test_abi_edge_cases(g):
    import torch
    cfg = g.Config()
    n = 256
    U, perm, dead = g.prepare(torch.eye(n, dtype=torch.float64, device="cuda"), cfg)
    W = torch.zeros((0, n), dtype=torch.bfloat16, device="cuda")
    out = g.quantize_layer(U, perm, dead, cfg, W)          # rows == 0: no work, loss 0
    assert out["loss"] == 0.0
    U200, perm200, dead200 = g.prepare(torch.eye(200, dtype=torch.float64, device="cuda"), cfg)
    W = torch.randn((8, 200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GptqError) as ei:
        g.quantize_layer(U200, perm200, dead200, cfg, W)    # n % 128 != 0
    assert ei.value.status == g.GPTQ_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        g.quantize_layer(U, perm, dead, cfg, W)             # U for another n: rejected by the binding
    W = torch.randn((8, n), dtype=torch.bfloat16, device="cuda")
    q, s, z, gi = g.alloc_outputs(8, n, cfg, "cuda")
    with pytest.raises(g.GptqError) as ei:
        g.gptq_quantize_layer(U, perm, dead, cfg, W, q, s, z, gi, g.workspace(16, "cuda"))
    assert ei.value.status == g.GPTQ_ERR_WORKSPACE
    with pytest.raises(g.GptqError) as ei:
        g.quantize_layer(U, perm, dead, g.Config(bits=5), W)
    assert ei.value.status == g.GPTQ_ERR_UNSUPPORTED


def _midpoint_cases(count, seed=0):
    """(xmax, w) pairs, 0 <= w <= xmax, for which rint(w * (1/s)) != rint(w / s)
    in fp32 with s = xmax / 15: the reciprocal form would pick the other code."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    out = []
    while len(out) < count:
        xmax = f32(rng.uniform(0.01, 0.05))
        s = f32(xmax) / f32(15)
        k = rng.integers(0, 15, size=4000)
        w = ((k + 0.5) * np.float64(s)).astype(np.float32)
        bad = np.nonzero(np.rint(w / s) != np.rint(w * (f32(1) / s)))[0]
        out += [(xmax, w[b]) for b in bad[:1] if w[b] <= xmax]
    return out


def test_quantizer_exact_division_near_midpoints(g):
    import torch
    rows, n = 24, 256
    rng = np.random.default_rng(5)
    W = (rng.random((rows, n)) * 0.01).astype(np.float32)       # all >= 0: xmin = 0, z = 0
    for r, (xmax, w) in enumerate(_midpoint_cases(rows)):
        W[r, :128] = np.minimum(W[r, :128], xmax)
        W[r, 0] = xmax                                          # group max -> s = xmax / 15
        W[r, 77] = w                                            # a quotient the reciprocal rounds wrong
    cfg = g.Config(bits=4, sym=False)
    U, perm, dead = g.prepare(torch.eye(n, dtype=torch.float64, device="cuda"), cfg)
    out = g.quantize_layer(U, perm, dead, cfg, torch.from_numpy(W).cuda())
    r = oracle.rtn(W.astype(np.float64), oracle.QuantConfig(bits=4), qdtype=np.float32)
    codes = oracle.unpack(out["qweight"].cpu().numpy(), 4, n)
    s = r["S"][0]
    fast = np.rint(W[:, 77] * (np.float32(1) / s))
    assert np.all(fast != np.rint(W[:, 77] / s))                # the planted cases are real
    assert np.array_equal(codes, r["codes"])
