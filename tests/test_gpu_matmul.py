"""GPU parity of the dequantizing matmul (pack + matmul through the C ABI)
against the oracle's Y = A W_hat^T on the same seeded inputs.

Tolerance (written out per element): the kernel multiplies fp16 activations by
the exact integers code - zero (products exact in fp32), sums them in fp32
along a chain of at most n/32 + 44 additions (MFMA steps of 32 products, the
group folds, the sum of the 8 waves), scales each group's partial sum by its
fp16 scale in fp32 and rounds once to the output type.  So
    |Y_gpu - Y| <= (n/32 + 64) u sum_i |A_i W_hat_i| + out_ulp(Y),
u = 2^-24, out_ulp the half-ulp of the output type (2^-11 |Y| + 2^-25 for
fp16, 2^-24 |Y| for fp32).  A Frobenius check at the typical fp32 level keeps
the test sensitive below that worst case.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_13_amd as g
    g.lib()
    return g


def _device_layer(codes, scales, zeros, g_idx, bits):
    import torch
    qweight = oracle.pack(codes, bits)
    return (torch.from_numpy(qweight.view(np.int32)).cuda(),
            torch.from_numpy(np.asarray(scales, np.float16)).cuda(),
            torch.from_numpy(np.asarray(zeros, np.float16)).cuda(),
            torch.from_numpy(np.asarray(g_idx, np.int32)).cuda(), qweight)


def _reference(a16, qweight, scales, zeros, g_idx, bits, rows, n):
    A = a16.astype(np.float64)
    What = oracle.dequantize(qweight, scales, zeros, g_idx, bits, rows, n)
    Y = oracle.dequant_matmul(A, qweight, scales, zeros, g_idx, bits, rows, n)
    mag = np.abs(A) @ np.abs(What).T
    return Y, mag


def _check(Y_gpu, Y, mag, n, out):
    acc = (n / 32 + 64) * U32 * mag
    if out == "fp16":
        tol = 1.001 * acc + 2.0 ** -11 * np.abs(Y) + 2.0 ** -25
        frob = 4e-4
    else:
        tol = 1.001 * acc + U32 * np.abs(Y)
        frob = 2e-6
    err = np.abs(Y_gpu - Y)
    bad = err > tol
    assert not bad.any(), (int(bad.sum()), float(err[bad].max()), float(tol[bad].min()))
    rel = float(np.linalg.norm(Y_gpu - Y) / np.linalg.norm(Y))
    assert rel <= frob, rel
    return rel


CASES = [
    # bits, group_size, act_order, rows, n, tokens, output
    (4, 128, False, 64, 128, 1, "fp32"),     # one chunk: fewer chunks than waves
    (4, 128, False, 50, 384, 3, "fp16"),     # ragged output tile, 3 chunks
    (4, 64, True, 200, 1152, 16, "fp32"),    # act-order; 9 chunks = 2 rounds, ragged; full token tile
    (4, 32, False, 96, 2048, 17, "fp16"),    # two token slices
    (4, -1, False, 32, 1024, 2, "fp32"),     # one group per row
    (3, 128, True, 80, 1152, 5, "fp32"),
    (3, 32, False, 48, 640, 1, "fp16"),
    (2, 64, False, 64, 896, 4, "fp32"),
    (2, 128, True, 16, 256, 1, "fp32"),
    (8, 128, False, 112, 1024, 7, "fp32"),
    (8, 32, True, 40, 512, 16, "fp16"),
    (8, -1, False, 16, 384, 1, "fp32"),
    (4, 128, False, 32, 4096, 16, "fp32"),   # activations beyond the LDS budget: windowed staging
    (2, 32, False, 16, 5120, 9, "fp32"),     # windowed, odd number of rounds
    (3, 64, True, 48, 3072, 12, "fp32"),
    # one slice too large to stage per tile: the persistent kernel, several
    # tiles per work-group (one per compute unit), ragged last tile
    (4, 128, False, 8200, 4096, 16, "fp16"),
    (3, 32, True, 4500, 3584, 12, "fp32"),    # four groups per chunk, act-order
    (8, -1, False, 4200, 4096, 10, "fp32"),   # one group per row
    # windowed staging: one slice too wide for the persistent kernel, and several slices
    (4, 128, False, 40, 11008, 16, "fp32"),
    (3, 64, False, 48, 4096, 40, "fp16"),
    (4, 64, False, 48, 512, 255, "fp32"),       # the decode kernel's largest size: 16 slices
    # prefill sizes (256 tokens and up): 128-token x 64-output tiles
    (4, 128, False, 96, 640, 256, "fp16"),      # the smallest prefill size: two token tiles
    (3, 32, True, 70, 768, 700, "fp32"),        # ragged token and output tiles, act-order
    (4, 128, False, 200, 1152, 1100, "fp32"),   # ragged token and output tiles, 9 chunks
    (4, 32, True, 300, 1024, 1024, "fp16"),     # act-order, four groups per chunk
    (3, 64, True, 96, 512, 1030, "fp16"),
    (2, -1, False, 64, 640, 1500, "fp32"),      # one group per row
    (8, 128, False, 130, 384, 2048, "fp32"),
    (8, 32, False, 16, 256, 1024, "fp32"),
]


@pytest.mark.parametrize("bits,gs,act,rows,n,M,out", CASES)
def test_random_layers(g, bits, gs, act, rows, n, M, out):
    import torch
    seed = 1000 + bits * 100 + len(str(gs)) + rows
    codes, scales, zeros, g_idx = synth.quantized_layer(seed, rows, n, bits, gs, act_order=act)
    qw, sc, ze, gi, qweight = _device_layer(codes, scales, zeros, g_idx, bits)
    layer = g.PackedLayer(qw, sc, ze, gi, bits, gs)
    assert (layer.col_order is None) == (not act)
    if act:
        assert np.array_equal(layer.col_order.cpu().numpy(), oracle.grouped_order(g_idx))
    a16 = synth.decode_activations_raw(seed, M, n).view(np.float16)
    A = torch.from_numpy(a16).cuda()
    Y = layer.matmul(A, out_dtype=torch.float16 if out == "fp16" else torch.float32)
    torch.cuda.synchronize()
    Yref, mag = _reference(a16, qweight, scales, zeros, g_idx, bits, rows, n)
    rel = _check(Y.cpu().numpy().astype(np.float64), Yref, mag, n, out)
    print(f"matmul bits={bits} gs={gs} act={act} {rows}x{n} M={M} {out}: rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("n,M,offset,pad", [
    (1152, 1030, 1, 3),    # unaligned activations, odd row stride: the 2-byte staging of the row gather
    (32896, 3, 0, 0),      # rows longer than the LDS row buffer: the plain gather
])
def test_act_order_gather_paths(g, n, M, offset, pad):
    """The act-order column gather for activations that are not 16-byte
    aligned (a view one element into a buffer with an odd row stride) and for
    rows too long to stage in LDS, against the oracle."""
    import torch
    bits, gs, rows = 4, 128, 48
    seed = 77 + n
    codes, scales, zeros, g_idx = synth.quantized_layer(seed, rows, n, bits, gs, act_order=True)
    qw, sc, ze, gi, qweight = _device_layer(codes, scales, zeros, g_idx, bits)
    layer = g.PackedLayer(qw, sc, ze, gi, bits, gs)
    assert layer.col_order is not None
    a16 = synth.decode_activations_raw(seed, M, n).view(np.float16)
    big = torch.zeros((M, n + pad), dtype=torch.float16, device="cuda")
    A = big[:, offset:offset + n]
    A.copy_(torch.from_numpy(a16).cuda())
    assert (A.data_ptr() % 16 != 0) == (offset != 0) and A.stride(0) == n + pad
    Y = layer.matmul(A, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Yref, mag = _reference(a16, qweight, scales, zeros, g_idx, bits, rows, n)
    rel = _check(Y.cpu().numpy().astype(np.float64), Yref, mag, n, "fp32")
    print(f"act-order gather n={n} M={M} offset={offset} lda={n + pad}: rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("desc_act", [False, True])
def test_layer_from_the_oracle_quantizer(g, desc_act):
    """Codes, scales, zeros and g_idx as the GPTQ sweep itself produces them
    (the oracle's, with act-order), then the GPU matmul on them."""
    import torch
    wl = synth.get("attn4096").resized(rows=96, n=512, tokens=4096)
    W = synth.weights(wl).astype(np.float64)
    X = synth.activations(wl)
    H, _ = oracle.hessian(X)
    cfg = oracle.QuantConfig(bits=4, group_size=128, desc_act=desc_act)
    ref = oracle.gptq_layer(W, H, cfg, qdtype=np.float32)
    qw = torch.from_numpy(ref["qweight"].view(np.int32)).cuda()
    sc = torch.from_numpy(ref["scales"]).cuda()
    ze = torch.from_numpy(ref["zeros"]).cuda()
    gi = torch.from_numpy(ref["g_idx"].astype(np.int32)).cuda()
    layer = g.PackedLayer(qw, sc, ze, gi, 4, 128)
    assert (layer.col_order is None) == (not desc_act)
    a16 = synth.decode_activations_raw(7, 4, 512).view(np.float16)
    Y = layer.matmul(torch.from_numpy(a16).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    Yref, mag = _reference(a16, ref["qweight"], ref["scales"], ref["zeros"], ref["g_idx"], 4, 96, 512)
    _check(Y.cpu().numpy().astype(np.float64), Yref, mag, 512, "fp32")


@pytest.mark.parametrize("rows,n", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_full_size_decode(g, rows, n):
    """The decode shapes of a Llama-2-7B block at 4-bit g128, one token and a
    batch of 8, every output compared."""
    import torch
    codes, scales, zeros, g_idx = synth.quantized_layer(11, rows, n, 4, 128)
    qw, sc, ze, gi, qweight = _device_layer(codes, scales, zeros, g_idx, 4)
    layer = g.PackedLayer(qw, sc, ze, gi, 4, 128)
    What = oracle.dequantize(qweight, scales, zeros, g_idx, 4, rows, n)
    for M in (1, 8):
        a16 = synth.decode_activations_raw(12 + M, M, n).view(np.float16)
        Y = layer.matmul(torch.from_numpy(a16).cuda())
        torch.cuda.synchronize()
        A = a16.astype(np.float64)
        Yref = A @ What.T
        _check(Y.cpu().numpy().astype(np.float64), Yref, np.abs(A) @ np.abs(What).T, n, "fp16")
        print(f"full size {rows}x{n} M={M}: ok", flush=True)


def test_edges_and_errors(g):
    import torch
    codes, scales, zeros, g_idx = synth.quantized_layer(5, 32, 256, 4, 128)
    qw, sc, ze, gi, _ = _device_layer(codes, scales, zeros, g_idx, 4)
    layer = g.PackedLayer(qw, sc, ze, gi, 4, 128)
    # no tokens: nothing written
    Y = torch.full((1, 32), 7.0, dtype=torch.float32, device="cuda")
    g.gptq_matmul(torch.empty((0, 256), dtype=torch.float16, device="cuda"), layer.packed, None, 32, 256, 4, 128,
                  Y[:0])
    assert torch.all(Y == 7.0)
    # deterministic: the same bits twice
    A = torch.from_numpy(synth.decode_activations_raw(3, 5, 256).view(np.float16)).cuda()
    y1 = layer.matmul(A, out_dtype=torch.float32)
    y2 = layer.matmul(A, out_dtype=torch.float32)
    assert torch.equal(y1, y2)
    # g_idx that is not a grouping into groups of 128 columns
    bad = gi.clone()
    bad[0] = 1
    with pytest.raises(g.GptqError, match="INVALID_ARG"):
        g.PackedLayer(qw, sc, ze, bad, 4, 128)
    bad[0] = 5                                   # out of range
    with pytest.raises(g.GptqError, match="INVALID_ARG"):
        g.PackedLayer(qw, sc, ze, bad, 4, 128)
    with pytest.raises(g.GptqError, match="UNSUPPORTED"):
        layer.matmul(A.to(torch.bfloat16))


def test_graph_replay(g):
    """The matmul (and the act-order gather before it) captured in a graph and
    replayed several times, with eager work between replays, equals the
    eager result on every replay."""
    import torch
    codes, scales, zeros, g_idx = synth.quantized_layer(9, 128, 1024, 4, 64, act_order=True)
    qw, sc, ze, gi, _ = _device_layer(codes, scales, zeros, g_idx, 4)
    layer = g.PackedLayer(qw, sc, ze, gi, 4, 64)
    A = torch.from_numpy(synth.decode_activations_raw(9, 2, 1024).view(np.float16)).cuda()
    ws = layer.workspace(2)
    eager = layer.matmul(A, out_dtype=torch.float32, ws=ws)
    Y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.matmul(A, Y=Y, ws=ws)               # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.matmul(A, Y=Y, ws=ws)
    for i in range(4):
        Y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), i
        _ = (A.float() * 2).sum().item()          # eager work between replays
