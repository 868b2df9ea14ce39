"""The stream-ordered forms of prepare and quantize (no host round trip):
bit-identical to the synchronizing forms, with the positive-definiteness flag
and the loss delivered to device memory in stream order.  Several layers are
queued back to back on one stream, as a caller quantizing a model would, and
only then read."""
import numpy as np
import pytest

import synth
from gpu_helpers import layer_inputs

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


@pytest.mark.parametrize("name,rows,n,tokens", [("toy256", None, None, None), ("attn4096", 200, 1536, 4096),
                                                ("mlpdown11008", 136, 640, 3000)])
def test_async_forms_match_sync(g, name, rows, n, tokens):
    import torch
    wl = synth.get(name)
    if n is not None:
        wl = wl.resized(rows=rows, n=n, tokens=tokens)
    _, wd, _, xd = layer_inputs(wl)
    cfg = _cfg(g, wl)
    dev = wd.device
    n = wl.n
    H, _ = g.hessian(xd)
    U, perm, dead = g.prepare(H, cfg)
    ref = g.quantize_layer(U, perm, dead, cfg, wd)

    reps = 3
    info = torch.full((reps,), 7, dtype=torch.int32, device=dev)
    loss = torch.full((reps,), -1.0, dtype=torch.float64, device=dev)
    ws_p = g.workspace(g.gptq_prepare_workspace_bytes(n, cfg), dev)
    ws_q = g.workspace(g.gptq_quantize_workspace_bytes(wl.rows, n, cfg), dev)
    outs = []
    torch.cuda.synchronize()
    for r in range(reps):   # queued without any synchronization in between
        Ua = torch.empty((n, n), dtype=torch.float32, device=dev)
        pa = torch.empty(n, dtype=torch.int32, device=dev)
        da = torch.empty(n, dtype=torch.uint8, device=dev)
        g.gptq_prepare_hinv_async(H, cfg, Ua, pa, da, info[r:r + 1], ws_p)
        q, s, z, gi = g.alloc_outputs(wl.rows, n, cfg, dev)
        g.gptq_quantize_layer_async(Ua, pa, da, cfg, wd, q, s, z, gi, loss[r:r + 1], ws_q)
        outs.append((Ua, pa, da, q, s, z, gi))
    torch.cuda.synchronize()
    assert info.tolist() == [0] * reps
    for r, (Ua, pa, da, q, s, z, gi) in enumerate(outs):
        assert torch.equal(Ua, U) and torch.equal(pa, perm) and torch.equal(da, dead)
        for k, t in (("qweight", q), ("scales", s), ("zeros", z), ("g_idx", gi)):
            assert torch.equal(t, ref[k]), (r, k)
        assert float(loss[r]) == ref["loss"]
    print(f"{name} {wl.rows}x{n}: {reps} queued layers bit-identical, loss {ref['loss']:.6e}")


def test_async_not_pd_flag_and_empty_layer(g):
    import torch
    cfg = g.Config(damp_percent=0.0)
    dev = torch.device("cuda")
    info = torch.full((3,), 7, dtype=torch.int32, device=dev)
    ws = g.workspace(g.gptq_prepare_workspace_bytes(70, cfg), dev)
    for i, H in enumerate((-np.eye(70), np.diag(np.r_[np.ones(69), np.nan]), np.eye(70))):
        Hd = torch.from_numpy(np.ascontiguousarray(H)).to(dev)
        U = torch.empty((70, 70), dtype=torch.float32, device=dev)
        perm = torch.empty(70, dtype=torch.int32, device=dev)
        dead = torch.empty(70, dtype=torch.uint8, device=dev)
        g.gptq_prepare_hinv_async(Hd, cfg, U, perm, dead, info[i:i + 1], ws)
    torch.cuda.synchronize()
    assert info.tolist() == [1, 1, 0]
    # rows == 0: the loss is written as 0 in stream order
    cfg = g.Config()
    U, perm, dead = g.prepare(torch.eye(256, dtype=torch.float64, device=dev), cfg)
    W = torch.zeros((0, 256), dtype=torch.bfloat16, device=dev)
    q, s, z, gi = g.alloc_outputs(0, 256, cfg, dev)
    loss = torch.full((1,), 5.0, dtype=torch.float64, device=dev)
    g.gptq_quantize_layer_async(U, perm, dead, cfg, W, q, s, z, gi, loss, None)
    torch.cuda.synchronize()
    assert float(loss[0]) == 0.0
    with pytest.raises(ValueError):
        g.gptq_prepare_hinv_async(torch.eye(256, dtype=torch.float64, device=dev), cfg, U, perm, dead,
                                  torch.zeros(1, dtype=torch.int64, device=dev), None)
