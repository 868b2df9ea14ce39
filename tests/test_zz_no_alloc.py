"""The allocation-free matmul entry point (gptq_matmul_static) through the C
ABI against gptq_matmul with a caller-supplied workspace: the same kernels
and the same gathered activations, so the outputs must be bitwise equal.
Two calls in a row, the second with a smaller input (fewer tokens, a
narrower layer), on act-order layers (which gather into the library's own
device array) and a layer without act-order (no scratch); a graph capture
of the static call replayed with eager work in between; and the size limit
of the library's array (rejected before anything is launched)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    import post_weight_quantization_13_amd as g
    g.lib()
    torch.cuda.init()
    return g


def _layer(g, seed, rows, n, bits, gs, act_order):
    import torch
    codes, scales, zeros, g_idx = synth.quantized_layer(seed, rows, n, bits, gs, act_order)
    qw = torch.from_numpy(oracle.pack(codes, bits).view(np.int32)).cuda()
    layer = g.PackedLayer(qw, torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(),
                          torch.from_numpy(g_idx).cuda(), bits, gs)
    assert (layer.col_order is None) == (not act_order)
    return layer


def _acts(seed, M, n):
    import torch
    return torch.from_numpy(synth.decode_activations_raw(seed, M, n).view(np.float16)).cuda()


def _both(g, layer, A):
    """(Y from gptq_matmul with its own workspace, Y from gptq_matmul_static)."""
    import torch
    M = A.shape[0]
    y_ws = torch.full((M, layer.rows), float("nan"), dtype=torch.float32, device="cuda")
    y_st = torch.full_like(y_ws, float("nan"))
    g.gptq_matmul(A, layer.packed, layer.col_order, layer.rows, layer.n, layer.bits, layer.group_size, y_ws,
                  layer.workspace(M))
    g.gptq_matmul_static(A, layer.packed, layer.col_order, layer.rows, layer.n, layer.bits, layer.group_size, y_st)
    torch.cuda.synchronize()
    return y_ws, y_st


@pytest.mark.parametrize("bits,gs,act_order", [(4, 128, True), (3, 32, True), (4, 64, False)])
def test_static_matches_workspace_twice_second_smaller(g, bits, gs, act_order):
    import torch
    big = _layer(g, 71, 200, 2048, bits, gs, act_order)
    small = _layer(g, 72, 48, 384, bits, gs, act_order)
    for layer, M, seed in ((big, 16, 81), (small, 3, 82)):
        print(f"[no-alloc] {bits}-bit g{gs} act_order={act_order}: rows {layer.rows} n {layer.n} tokens {M}",
              flush=True)
        A = _acts(seed, M, layer.n)
        y_ws, y_st = _both(g, layer, A)
        assert not torch.isnan(y_ws).any()
        assert torch.equal(y_ws, y_st)


def test_static_in_a_graph(g):
    import torch
    layer = _layer(g, 73, 96, 1152, 4, 128, True)
    A = _acts(83, 5, 1152)
    y_ws, y_eager = _both(g, layer, A)
    Y = torch.empty_like(y_ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.gptq_matmul_static(A, layer.packed, layer.col_order, layer.rows, layer.n, 4, 128, Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.gptq_matmul_static(A, layer.packed, layer.col_order, layer.rows, layer.n, 4, 128, Y)
    other = _layer(g, 74, 32, 640, 3, 32, True)
    for i in range(3):
        Y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, y_eager), i
        _both(g, other, _acts(84 + i, 7, 640))          # eager static calls reuse the array in between


def test_static_scratch_limit(g):
    import torch
    cap = g.gptq_matmul_static_scratch_bytes()
    assert cap == 4 << 20
    n = 32768
    order = torch.arange(n, dtype=torch.int32, device="cuda")
    packed = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    A = torch.zeros((cap // (2 * n) + 1, n), dtype=torch.float16, device="cuda")
    Y = torch.zeros((A.shape[0], 16), dtype=torch.float32, device="cuda")
    with pytest.raises(g.GptqError) as ei:
        g.gptq_matmul_static(A, packed, order, 16, n, 4, 128, Y)
    assert ei.value.status == g.GPTQ_ERR_WORKSPACE
    assert torch.count_nonzero(Y) == 0                   # nothing was launched
