"""Shared helpers for the GPU parity tests (device transfer and comparisons)."""
import numpy as np

import oracle
import synth


def to_device(raw: np.ndarray, dtype: str):
    """Stored synth array (uint16 bf16 bits or float32) -> torch tensor on cuda:0."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).cuda()


def layer_inputs(wl, li=0):
    """(W float32 values, W on device, X float32 values, X on device) for linear li."""
    lin = wl.linears[li]
    w_raw = synth.weights_raw(wl, li)
    x_raw = synth.activations_raw(wl, lin.xset)
    wv = synth.bf16_value(w_raw) if wl.dtype == "bf16" else w_raw
    xv = synth.bf16_value(x_raw) if wl.dtype == "bf16" else x_raw
    return wv, to_device(w_raw, wl.dtype), xv, to_device(x_raw, wl.dtype)


def rel_frobenius(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def gpu_codes(out, bits, n):
    return oracle.unpack(out["qweight"].cpu().numpy(), bits, n)


def compare_layer(out, ref, bits, n, W, H, gpu_rel_loss):
    """Acceptance numbers of a GPU layer against the oracle's outputs."""
    codes = gpu_codes(out, bits, n)
    agree = float(np.mean(codes == ref["codes"]))
    s_gpu = out["scales"].cpu().numpy().astype(np.float64)
    s_ref = ref["scales"].astype(np.float64)
    z_gpu = out["zeros"].cpu().numpy().astype(np.float64)
    z_ref = ref["zeros"].astype(np.float64)
    s_rel = float(np.max(np.abs(s_gpu - s_ref) / np.abs(s_ref)))
    s_frac = float(np.mean(np.abs(s_gpu - s_ref) <= 1e-3 * np.abs(s_ref)))
    z_frac = float(np.mean(z_gpu == z_ref))
    gidx_ok = bool(np.array_equal(out["g_idx"].cpu().numpy(), ref["g_idx"]))
    repack = oracle.pack(codes, bits)
    pack_ok = bool(np.array_equal(repack, out["qweight"].cpu().numpy()))
    loss_rel = abs(gpu_rel_loss - ref["rel_loss"]) / ref["rel_loss"]
    return dict(agree=agree, s_rel=s_rel, s_frac=s_frac, z_frac=z_frac, gidx_ok=gidx_ok, pack_ok=pack_ok,
                loss_rel=loss_rel, gpu_rel_loss=gpu_rel_loss, ref_rel_loss=ref["rel_loss"])


def groups_before_first_flip(codes_gpu, codes_ref, g_idx, G):
    """Mask [G, rows] of the groups whose parameters were taken before the
    first differing code of their row (in sweep order, groups are numbered by
    sweep position; a group's grid is taken at its first column, so a group
    is upstream of a flip when its index is at most the flipped column's
    group).  Rows with no differing code: every group."""
    rows = codes_gpu.shape[0]
    mask = np.ones((G, rows), dtype=bool)
    g_idx = np.asarray(g_idx)
    for r in np.nonzero((codes_gpu != codes_ref).any(axis=1))[0]:
        first = int(g_idx[codes_gpu[r] != codes_ref[r]].min())
        mask[first + 1:, r] = False
    return mask
