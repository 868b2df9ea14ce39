"""Python binding of libgptq, the gfx950 GPTQ layer-wise solver.

The C ABI (include/gptq.h) is the product; this module only marshals
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t, status codes become exceptions.  Every step of the
computation runs in the HIP kernels of libgptq.so.  There is no fallback: if
the library is missing, importing the functions raises.

Functions keep the C names:
    gptq_hessian_accumulate(H, n_tokens, X)             -> new n_tokens
    gptq_prepare_hinv(H, cfg, U, perm, dead, ws)
    gptq_quantize_layer(U, perm, dead, cfg, W, qweight, scales, zeros, g_idx, ws) -> loss
    gptq_layer_loss(H, W, qweight, scales, zeros, g_idx, cfg, ws) -> relative loss
    gptq_matmul_pack(qweight, scales, zeros, g_idx, bits, group_size, packed, col_order) -> identity
    gptq_matmul(A, packed, col_order, rows, n, bits, group_size, Y, ws)
plus the workspace queries and small allocating helpers (``quantize_layer``,
``hessian``, ``prepare``, ``PackedLayer``) that create the output tensors with
torch, and ``quantize_block``, which sequences those calls for the linears of a
decoder block that share activation sets.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = -1
GPTQ_ERR_UNSUPPORTED = -2
GPTQ_ERR_NOT_PD = -3
GPTQ_ERR_HIP = -4
GPTQ_ERR_WORKSPACE = -5
_STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "NOT_PD", -4: "HIP", -5: "WORKSPACE"}

GPTQ_BF16, GPTQ_FP16, GPTQ_FP32 = 0, 1, 2

# Every symbol include/gptq.h declares.
EXPORTS = (
    "gptq_hessian_workspace_bytes", "gptq_hessian_chain_tokens", "gptq_hessian_accumulate",
    "gptq_prepare_workspace_bytes", "gptq_prepare_hinv",
    "gptq_quantize_workspace_bytes", "gptq_quantize_layer",
    "gptq_layer_loss_workspace_bytes", "gptq_layer_loss",
    "gptq_matmul_packed_bytes", "gptq_matmul_pack", "gptq_matmul_workspace_bytes", "gptq_matmul",
    "gptq_last_error", "gptq_version",
)


class GptqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class gptq_config(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("desc_act", ctypes.c_int32), ("damp_percent", ctypes.c_float),
                ("block_size", ctypes.c_int32)]


@dataclass(frozen=True)
class Config:
    """The pages' quantize config: bits, group_size, sym, desc_act, damp_percent, block_size."""
    bits: int = 4
    group_size: int = 128       # 128, 64, 32, or -1 (one group per row)
    sym: int = 0                # 0 asymmetric, 1 the pages' symmetric grid, 2 full-range symmetric
    desc_act: bool = False
    damp_percent: float = 0.01
    block_size: int = 128

    def c(self) -> gptq_config:
        return gptq_config(int(self.bits), int(self.group_size), int(self.sym), int(bool(self.desc_act)),
                           float(self.damp_percent), int(self.block_size))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgptq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m post_weight_quantization_13_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    cfgp = ctypes.POINTER(gptq_config)
    L.gptq_hessian_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
    L.gptq_hessian_workspace_bytes.restype = sz
    L.gptq_hessian_chain_tokens.argtypes = []
    L.gptq_hessian_chain_tokens.restype = i64
    L.gptq_hessian_accumulate.argtypes = [vp, i64, ctypes.POINTER(i64), vp, ctypes.c_int, i64, i64, vp, sz, vp]
    L.gptq_hessian_accumulate.restype = ctypes.c_int
    L.gptq_prepare_workspace_bytes.argtypes = [i64, cfgp]
    L.gptq_prepare_workspace_bytes.restype = sz
    L.gptq_prepare_hinv.argtypes = [vp, i64, cfgp, vp, vp, vp, vp, sz, vp]
    L.gptq_prepare_hinv.restype = ctypes.c_int
    L.gptq_quantize_workspace_bytes.argtypes = [i64, i64, cfgp]
    L.gptq_quantize_workspace_bytes.restype = sz
    L.gptq_quantize_layer.argtypes = [vp, vp, vp, i64, cfgp, vp, ctypes.c_int, i64, i64, vp, vp, vp, vp,
                                      ctypes.POINTER(ctypes.c_double), vp, sz, vp]
    L.gptq_quantize_layer.restype = ctypes.c_int
    L.gptq_layer_loss_workspace_bytes.argtypes = [i64, i64]
    L.gptq_layer_loss_workspace_bytes.restype = sz
    L.gptq_layer_loss.argtypes = [vp, i64, vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, cfgp,
                                  ctypes.POINTER(ctypes.c_double), vp, sz, vp]
    L.gptq_layer_loss.restype = ctypes.c_int
    i32 = ctypes.c_int32
    L.gptq_matmul_packed_bytes.argtypes = [i64, i64, i32, i32]
    L.gptq_matmul_packed_bytes.restype = sz
    L.gptq_matmul_pack.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, vp, sz, vp, ctypes.POINTER(i32), vp]
    L.gptq_matmul_pack.restype = ctypes.c_int
    L.gptq_matmul_workspace_bytes.argtypes = [i64, i64, i32]
    L.gptq_matmul_workspace_bytes.restype = sz
    L.gptq_matmul.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, i64, vp,
                              sz, vp]
    L.gptq_matmul.restype = ctypes.c_int
    L.gptq_last_error.argtypes = []
    L.gptq_last_error.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != GPTQ_OK:
        raise GptqError(status, lib().gptq_last_error().decode())


# ---------------------------------------------------------------- marshalling
def _dtype_code(t) -> int:
    import torch
    m = {torch.bfloat16: GPTQ_BF16, torch.float16: GPTQ_FP16, torch.float32: GPTQ_FP32}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _row_major_2d(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _cfg(cfg):
    return ctypes.byref((cfg if isinstance(cfg, Config) else Config(**cfg)).c())


# ---------------------------------------------------------------- C entry points
def gptq_hessian_workspace_bytes(n: int, tokens: int, dtype_code: int) -> int:
    return lib().gptq_hessian_workspace_bytes(n, tokens, dtype_code)


def gptq_hessian_chain_tokens() -> int:
    return lib().gptq_hessian_chain_tokens()


def gptq_hessian_accumulate(H, n_tokens: int, X, workspace="auto", stream=None) -> int:
    """H (float64 [n, n], device) <- running mean of 2 x x^T; returns the new token count.

    workspace="auto" allocates the scratch the call needs (a torch tensor)."""
    n = H.shape[0]
    if isinstance(workspace, str):
        workspace = hessian_workspace(n, X) if X.shape[0] > 0 else None
    ldx = _row_major_2d(X, "X")
    cnt = ctypes.c_int64(int(n_tokens))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gptq_hessian_accumulate(_ptr(H), n, ctypes.byref(cnt), _ptr(X), _dtype_code(X), X.shape[0], ldx,
                                         _ptr(workspace), ws_bytes, _stream(stream, H.device)))
    return cnt.value


def gptq_prepare_workspace_bytes(n: int, cfg) -> int:
    return lib().gptq_prepare_workspace_bytes(n, _cfg(cfg))


def gptq_prepare_hinv(H, cfg, U, perm, dead, workspace, stream=None) -> None:
    n = H.shape[0]
    _check(lib().gptq_prepare_hinv(_ptr(H), n, _cfg(cfg), _ptr(U), _ptr(perm), _ptr(dead), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream, H.device)))


def gptq_quantize_workspace_bytes(rows: int, n: int, cfg) -> int:
    return lib().gptq_quantize_workspace_bytes(rows, n, _cfg(cfg))


def gptq_quantize_layer(U, perm, dead, cfg, W, qweight, scales, zeros, g_idx, workspace, stream=None,
                        want_loss: bool = True):
    """Quantize W; writes qweight/scales/zeros/g_idx; returns the internal loss (or None)."""
    rows, n = W.shape
    ldw = _row_major_2d(W, "W")
    loss = ctypes.c_double(0.0)
    _check(lib().gptq_quantize_layer(_ptr(U), _ptr(perm), _ptr(dead), n, _cfg(cfg), _ptr(W), _dtype_code(W), rows,
                                     ldw, _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                     ctypes.byref(loss) if want_loss else None, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream, W.device)))
    return loss.value if want_loss else None


def gptq_layer_loss_workspace_bytes(rows: int, n: int) -> int:
    return lib().gptq_layer_loss_workspace_bytes(rows, n)


def gptq_layer_loss(H, W, qweight, scales, zeros, g_idx, cfg, workspace, stream=None) -> float:
    rows, n = W.shape
    ldw = _row_major_2d(W, "W")
    out = ctypes.c_double(0.0)
    _check(lib().gptq_layer_loss(_ptr(H), n, _ptr(W), _dtype_code(W), rows, ldw, _ptr(qweight), _ptr(scales),
                                 _ptr(zeros), _ptr(g_idx), _cfg(cfg), ctypes.byref(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream, W.device)))
    return out.value


def gptq_matmul_packed_bytes(rows: int, n: int, bits: int, group_size: int) -> int:
    return lib().gptq_matmul_packed_bytes(rows, n, bits, group_size)


def gptq_matmul_pack(qweight, scales, zeros, g_idx, bits: int, group_size: int, packed, col_order,
                     stream=None) -> bool:
    """Tiled copy of a quantized layer for gptq_matmul; returns True if col_order is the identity."""
    rows = qweight.shape[1]
    n = g_idx.shape[0]
    ident = ctypes.c_int32(0)
    _check(lib().gptq_matmul_pack(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(g_idx), rows, n, bits, group_size,
                                  _ptr(packed), packed.numel() * packed.element_size(), _ptr(col_order),
                                  ctypes.byref(ident), _stream(stream, qweight.device)))
    return bool(ident.value)


def gptq_matmul_workspace_bytes(M: int, n: int, has_col_order: bool) -> int:
    return lib().gptq_matmul_workspace_bytes(M, n, int(bool(has_col_order)))


def gptq_matmul(A, packed, col_order, rows: int, n: int, bits: int, group_size: int, Y, workspace=None,
                stream=None) -> None:
    """Y[:M, :rows] = A W_hat^T for fp16 activations A [M, >= n]."""
    lda = _row_major_2d(A, "A")
    ldy = _row_major_2d(Y, "Y")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gptq_matmul(_ptr(A), _dtype_code(A), A.shape[0], lda, _ptr(packed), _ptr(col_order), rows, n, bits,
                             group_size, _ptr(Y), _dtype_code(Y), ldy, _ptr(workspace), ws_bytes,
                             _stream(stream, A.device)))


def gptq_version() -> str:
    return lib().gptq_version().decode()


# ---------------------------------------------------------------- allocating helpers
def workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def hessian(X, H=None, n_tokens: int = 0):
    """Allocate (if needed) and accumulate H from X; returns (H, n_tokens)."""
    import torch
    n = X.shape[1]
    if H is None:
        H = torch.empty((n, n), dtype=torch.float64, device=X.device)
    ws = hessian_workspace(n, X)
    return H, gptq_hessian_accumulate(H, n_tokens, X, ws)


def hessian_workspace(n: int, X):
    """Workspace tensor (or None) for accumulating X into an n x n Hessian."""
    nb = gptq_hessian_workspace_bytes(n, X.shape[0], _dtype_code(X))
    return workspace(nb, X.device) if nb else None


def prepare(H, cfg):
    """Returns (U, perm, dead) for H."""
    import torch
    n = H.shape[0]
    U = torch.empty((n, n), dtype=torch.float32, device=H.device)
    perm = torch.empty(n, dtype=torch.int32, device=H.device)
    dead = torch.empty(n, dtype=torch.uint8, device=H.device)
    ws = workspace(gptq_prepare_workspace_bytes(n, cfg), H.device)
    gptq_prepare_hinv(H, cfg, U, perm, dead, ws)
    return U, perm, dead


def alloc_outputs(rows: int, n: int, cfg, device):
    import torch
    c = cfg if isinstance(cfg, Config) else Config(**cfg)
    qweight = torch.empty((n * c.bits // 32, rows), dtype=torch.int32, device=device)
    groups = n // c.group_size if c.group_size > 0 else 1
    scales = torch.empty((groups, rows), dtype=torch.float16, device=device)
    zeros = torch.empty((groups, rows), dtype=torch.float16, device=device)
    g_idx = torch.empty(n, dtype=torch.int32, device=device)
    return qweight, scales, zeros, g_idx


def quantize_layer(U, perm, dead, cfg, W):
    """Returns dict(qweight, scales, zeros, g_idx, loss)."""
    rows, n = W.shape
    qweight, scales, zeros, g_idx = alloc_outputs(rows, n, cfg, W.device)
    ws = workspace(gptq_quantize_workspace_bytes(rows, n, cfg), W.device)
    loss = gptq_quantize_layer(U, perm, dead, cfg, W, qweight, scales, zeros, g_idx, ws)
    return dict(qweight=qweight, scales=scales, zeros=zeros, g_idx=g_idx, loss=loss)


def layer_loss(H, W, out, cfg) -> float:
    rows, n = W.shape
    ws = workspace(gptq_layer_loss_workspace_bytes(rows, n), W.device)
    return gptq_layer_loss(H, W, out["qweight"], out["scales"], out["zeros"], out["g_idx"], cfg, ws)


class PackedLayer:
    """A quantized layer in the matmul's tiled layout (see gptq_matmul_pack)."""

    def __init__(self, qweight, scales, zeros, g_idx, bits: int, group_size: int):
        import torch
        self.rows = qweight.shape[1]
        self.n = g_idx.shape[0]
        self.bits, self.group_size = int(bits), int(group_size)
        dev = qweight.device
        self.packed = torch.empty(gptq_matmul_packed_bytes(self.rows, self.n, self.bits, self.group_size),
                                  dtype=torch.uint8, device=dev)
        order = torch.empty(self.n, dtype=torch.int32, device=dev)
        ident = gptq_matmul_pack(qweight, scales, zeros, g_idx, self.bits, self.group_size, self.packed, order)
        self.col_order = None if ident else order

    def workspace(self, M: int):
        nb = gptq_matmul_workspace_bytes(M, self.n, self.col_order is not None)
        return workspace(nb, self.packed.device) if nb else None

    def matmul(self, A, out_dtype=None, Y=None, ws=None):
        """Y = A W_hat^T (fp16 A [M, n]); out_dtype float16 (default) or float32."""
        import torch
        M = A.shape[0]
        if Y is None:
            Y = torch.empty((M, self.rows), dtype=out_dtype or torch.float16, device=A.device)
        if ws is None and self.col_order is not None:
            ws = self.workspace(M)
        gptq_matmul(A, self.packed, self.col_order, self.rows, self.n, self.bits, self.group_size, Y, ws)
        return Y


def quantize_block(X_sets, weights, xset_of, cfg, want_loss: bool = True):
    """Quantize the linears of a decoder block whose inputs come in a few
    shared activation sets (q/k/v read one, gate/up another): one Hessian and
    one prepare per set, then one quantize per linear with its set's factor.

    X_sets: list of [tokens, n_s] device tensors; weights: list of [rows, n]
    device tensors; xset_of[i]: the set linear i reads.  Returns a list of
    dicts (qweight, scales, zeros, g_idx, loss, rel_loss) in the order of
    ``weights``, plus the Hessians (for the caller's checks).
    """
    Hs, factors = [], []
    for X in X_sets:
        H, _ = hessian(X)
        Hs.append(H)
        factors.append(prepare(H, cfg))
    outs = []
    for W, s in zip(weights, xset_of):
        U, perm, dead = factors[s]
        out = quantize_layer(U, perm, dead, cfg, W)
        out["rel_loss"] = layer_loss(Hs[s], W, out, cfg) if want_loss else None
        outs.append(out)
    return outs, Hs
