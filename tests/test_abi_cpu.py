"""The C-ABI library on a machine without a GPU: it loads, exports every symbol
include/gptq.h declares, and rejects bad arguments with status codes before
any device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def g():
    import post_weight_quantization_13_amd as g
    if not os.path.exists(g.LIB_PATH):
        pytest.skip("libgptq.so not built")
    g.lib()
    return g


def _declared():
    text = open(os.path.join(ROOT, "include", "gptq.h")).read()
    return sorted(set(re.findall(r"^[a-z_ ]*?\b(?:size_t|int64_t|gptq_status|const char\*)\s+(gptq_\w+)\(",
                                 text, flags=re.M)))


def test_exports_every_declared_symbol(g):
    names = _declared()
    assert len(names) == 23, names
    assert set(names) == set(g.EXPORTS)
    L = g.lib()
    for n in names:
        assert getattr(L, n) is not None
    assert g.gptq_version().startswith("gptq-gfx950")
    assert L.gptq_last_error() is not None


def test_workspace_queries(g):
    cfg = g.Config()
    # 528 tiles of 128x128 on 256 compute units: 16 tiles left over after the
    # rounds, cut into token pieces with fp64 partials; the larger of the two
    # kernels' needs (16 pieces each at one work-group per compute unit, 32 at two)
    assert g.gptq_hessian_workspace_bytes(4096, 65536, g.GPTQ_BF16) == 16 * 32 * 128 * 128 * 8
    assert g.gptq_hessian_workspace_bytes(4096, 65536, g.GPTQ_FP32) == 0
    assert g.gptq_hessian_workspace_bytes(256, 65536, g.GPTQ_BF16) == 0   # 3 tiles: one round
    assert g.gptq_hessian_chain_tokens() == 256
    assert g.gptq_prepare_workspace_bytes(4096, cfg) >= 2 * 4096 * 4096 * 8
    assert g.gptq_quantize_workspace_bytes(4096, 4096, cfg) >= 4096 * 4096 * 5
    assert g.gptq_quantize_workspace_bytes(0, 4096, cfg) == 0
    assert g.gptq_layer_loss_workspace_bytes(16, 256) > 0


def _cfg(**kw):
    import post_weight_quantization_13_amd as g
    return ctypes.byref(g.Config(**kw).c())


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_argument_validation(g):
    L = g.lib()
    cnt = ctypes.c_int64(0)
    assert L.gptq_hessian_accumulate(None, 16, ctypes.byref(cnt), FAKE, 0, 10, 16, None, 0, None) == g.GPTQ_ERR_INVALID_ARG
    assert b"H" in L.gptq_last_error()
    assert L.gptq_hessian_accumulate(FAKE, 16, None, FAKE, 0, 10, 16, None, 0, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_hessian_accumulate(FAKE, 16, ctypes.byref(cnt), FAKE, 0, 10, 8, None, 0, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_hessian_accumulate(FAKE, 16, ctypes.byref(cnt), FAKE, 7, 10, 16, None, 0, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_hessian_accumulate(FAKE, 0, ctypes.byref(cnt), FAKE, 0, 10, 16, None, 0, None) == g.GPTQ_ERR_INVALID_ARG
    # tokens == 0 is a no-op that succeeds and leaves the count alone
    assert L.gptq_hessian_accumulate(FAKE, 16, ctypes.byref(cnt), None, 0, 0, 16, None, 0, None) == g.GPTQ_OK
    assert cnt.value == 0

    assert L.gptq_prepare_hinv(None, 16, _cfg(), FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_prepare_hinv(FAKE, 16, _cfg(damp_percent=-1.0), FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_prepare_hinv(FAKE, 16, _cfg(), FAKE, FAKE, FAKE, FAKE, 10, None) == g.GPTQ_ERR_WORKSPACE
    assert L.gptq_prepare_hinv(FAKE, 70000, _cfg(), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == g.GPTQ_ERR_INVALID_ARG

    args = lambda n=256, rows=8, ldw=256, ws=1 << 30, cfg=None, wdt=0: (
        FAKE, FAKE, FAKE, n, cfg or _cfg(), FAKE, wdt, rows, ldw, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert L.gptq_quantize_layer(*args(cfg=_cfg(bits=5))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(bits=1))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(bits=6))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(group_size=16))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(group_size=256))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(group_size=0))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(sym=3))) == g.GPTQ_ERR_INVALID_ARG
    # group_size 32 or 64 still needs n to be a multiple of the 128-column block
    assert L.gptq_quantize_layer(*args(n=192, ldw=192, cfg=_cfg(group_size=64))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(cfg=_cfg(block_size=64))) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(n=200, ldw=200)) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_quantize_layer(*args(ldw=128)) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_quantize_layer(*args(rows=-1)) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_quantize_layer(*args(wdt=9)) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_quantize_layer(*args(ws=16)) == g.GPTQ_ERR_WORKSPACE
    assert L.gptq_quantize_layer(None, FAKE, FAKE, 256, _cfg(), FAKE, 0, 8, 256, FAKE, FAKE, FAKE, FAKE, None,
                                 FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    loss = ctypes.c_double(7.0)
    assert L.gptq_quantize_layer(FAKE, FAKE, FAKE, 256, _cfg(), FAKE, 0, 0, 256, FAKE, FAKE, FAKE, FAKE,
                                 ctypes.byref(loss), None, 0, None) == g.GPTQ_OK
    assert loss.value == 0.0

    # the stream-ordered forms: the same checks, plus the device flag
    assert L.gptq_prepare_hinv_async(None, 16, _cfg(), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_prepare_hinv_async(FAKE, 16, _cfg(), FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    assert b"info" in L.gptq_last_error()
    assert L.gptq_prepare_hinv_async(FAKE, 16, _cfg(), FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == g.GPTQ_ERR_WORKSPACE
    assert L.gptq_prepare_hinv_async(FAKE, 16, _cfg(damp_percent=-1.0), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                     None) == g.GPTQ_ERR_INVALID_ARG
    qa = lambda n=256, rows=8, ldw=256, ws=1 << 30, cfg=None: L.gptq_quantize_layer_async(
        FAKE, FAKE, FAKE, n, cfg or _cfg(), FAKE, 0, rows, ldw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert qa(cfg=_cfg(bits=5)) == g.GPTQ_ERR_UNSUPPORTED
    assert qa(n=200, ldw=200) == g.GPTQ_ERR_UNSUPPORTED
    assert qa(ldw=128) == g.GPTQ_ERR_INVALID_ARG
    assert qa(ws=16) == g.GPTQ_ERR_WORKSPACE
    assert b"gptq_quantize_layer_async" not in L.gptq_last_error()   # argument errors name the argument

    rel = ctypes.c_double(0)
    assert L.gptq_layer_loss(None, 256, FAKE, 0, 8, 256, FAKE, FAKE, FAKE, FAKE, _cfg(), ctypes.byref(rel),
                             FAKE, 1 << 30, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_layer_loss(FAKE, 256, FAKE, 0, 8, 256, FAKE, FAKE, FAKE, FAKE, _cfg(), ctypes.byref(rel),
                             FAKE, 8, None) == g.GPTQ_ERR_WORKSPACE


def test_matmul_queries_and_validation(g):
    L = g.lib()
    # header + codes ([tiles][chunks][64 lanes][bits words]) + scale/zero words
    assert g.gptq_matmul_packed_bytes(4096, 4096, 4, 128) == 256 + 256 * 32 * 64 * 4 * 4 + 256 * 32 * 16 * 4
    assert g.gptq_matmul_packed_bytes(50, 384, 3, 32) == 256 + 4 * 3 * 64 * 3 * 4 + 4 * 12 * 16 * 4
    assert g.gptq_matmul_packed_bytes(16, 128, 8, -1) == 256 + 1 * 1 * 64 * 8 * 4 + 16 * 4
    assert g.gptq_matmul_packed_bytes(16, 200, 4, 128) == 0      # n not a multiple of 128
    assert g.gptq_matmul_packed_bytes(16, 256, 5, 128) == 0
    assert g.gptq_matmul_workspace_bytes(1, 4096, False) == 0
    assert g.gptq_matmul_workspace_bytes(3, 4096, True) == 3 * 4096 * 2
    i32 = ctypes.c_int32(0)
    pk = lambda rows=16, n=256, bits=4, gs=128, nbytes=1 << 30, order=FAKE: L.gptq_matmul_pack(
        FAKE, FAKE, FAKE, FAKE, rows, n, bits, gs, FAKE, nbytes, order, ctypes.byref(i32), None)
    assert pk(bits=5) == g.GPTQ_ERR_UNSUPPORTED
    assert pk(gs=16) == g.GPTQ_ERR_UNSUPPORTED
    assert pk(n=192, gs=64) == g.GPTQ_ERR_UNSUPPORTED
    assert pk(rows=0) == g.GPTQ_ERR_INVALID_ARG
    assert pk(order=None) == g.GPTQ_ERR_INVALID_ARG
    assert pk(nbytes=100) == g.GPTQ_ERR_WORKSPACE
    mm = lambda adt=g.GPTQ_FP16, M=1, lda=256, ydt=g.GPTQ_FP16, ldy=16, order=None, ws=None, wsb=0, A=FAKE: \
        L.gptq_matmul(A, adt, M, lda, FAKE, order, 16, 256, 4, 128, FAKE, ydt, ldy, ws, wsb, None)
    assert mm(adt=g.GPTQ_BF16) == g.GPTQ_ERR_UNSUPPORTED
    assert mm(ydt=g.GPTQ_BF16) == g.GPTQ_ERR_UNSUPPORTED
    assert mm(M=-1) == g.GPTQ_ERR_INVALID_ARG
    assert mm(lda=128) == g.GPTQ_ERR_INVALID_ARG
    assert mm(ldy=8) == g.GPTQ_ERR_INVALID_ARG
    assert mm(lda=260) == g.GPTQ_ERR_INVALID_ARG                  # rows of A must stay 16-byte aligned
    assert mm(A=ctypes.c_void_p(0x1002)) == g.GPTQ_ERR_INVALID_ARG
    assert mm(order=FAKE) == g.GPTQ_ERR_WORKSPACE                  # act-order needs the gather workspace
    assert mm(M=0, A=None) == g.GPTQ_OK                            # no tokens: nothing to do
    # the allocation-free variant: the same checks, and the size of the library's gather array
    st = lambda M=1, n=256, order=None, adt=g.GPTQ_FP16, lda=None: L.gptq_matmul_static(
        FAKE, adt, M, lda or n, FAKE, order, 16, n, 4, 128, FAKE, g.GPTQ_FP32, 16, None)
    assert g.gptq_matmul_static_scratch_bytes() == 4 << 20
    assert st(adt=g.GPTQ_BF16) == g.GPTQ_ERR_UNSUPPORTED
    assert st(lda=128) == g.GPTQ_ERR_INVALID_ARG
    assert st(M=0) == g.GPTQ_OK
    assert st(M=65, n=32768, order=FAKE) == g.GPTQ_ERR_WORKSPACE   # 65 x 32768 fp16 > 4 MiB
    assert b"4194304" in L.gptq_last_error()


def test_block_forward_validation(g):
    L = g.lib()
    # rmsnorm: X, xdt, ldx, R, T, d, eps, H_out, Y, stream
    assert L.gptq_rmsnorm(FAKE, 0, 64, None, 4, 0, 1e-5, None, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_rmsnorm(FAKE, 0, 32, None, 4, 64, 1e-5, None, FAKE, None) == g.GPTQ_ERR_INVALID_ARG   # ldx < d
    assert L.gptq_rmsnorm(FAKE, 9, 64, None, 4, 64, 1e-5, None, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_rmsnorm(FAKE, 0, 64, None, 4, 64, -1.0, None, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_rmsnorm(None, 0, 64, None, 4, 64, 1e-5, None, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_rmsnorm(None, 0, 64, None, 0, 64, 1e-5, None, None, None) == g.GPTQ_OK             # T == 0
    # rope: Q, K, T, d, head_dim, seq_len, base, stream
    assert L.gptq_rope(FAKE, FAKE, 512, 256, 127, 256, 1e4, None) == g.GPTQ_ERR_INVALID_ARG       # odd head_dim
    assert L.gptq_rope(FAKE, FAKE, 512, 200, 128, 256, 1e4, None) == g.GPTQ_ERR_INVALID_ARG       # d % head_dim
    assert L.gptq_rope(FAKE, FAKE, 500, 256, 128, 256, 1e4, None) == g.GPTQ_ERR_INVALID_ARG       # T % seq_len
    assert L.gptq_rope(FAKE, FAKE, 512, 256, 128, 256, 0.0, None) == g.GPTQ_ERR_INVALID_ARG
    # attention: Q, K, V, T, d, head_dim, seq_len, O, stream
    assert L.gptq_causal_attention(FAKE, FAKE, FAKE, 512, 256, 64, 256, FAKE, None) == g.GPTQ_ERR_UNSUPPORTED
    assert L.gptq_causal_attention(FAKE, FAKE, FAKE, 500, 256, 128, 256, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_causal_attention(FAKE, FAKE, None, 512, 256, 128, 256, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_causal_attention(ctypes.c_void_p(0x1004), FAKE, FAKE, 512, 256, 128, 256, FAKE,
                                   None) == g.GPTQ_ERR_INVALID_ARG                               # unaligned Q
    assert L.gptq_causal_attention(None, None, None, 0, 256, 128, 256, None, None) == g.GPTQ_OK
    assert L.gptq_silu_mul(FAKE, FAKE, -1, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_silu_mul(None, FAKE, 10, FAKE, None) == g.GPTQ_ERR_INVALID_ARG
    assert L.gptq_silu_mul(None, None, 0, None, None) == g.GPTQ_OK


def test_binding_fails_loudly_without_library(monkeypatch, g):
    import post_weight_quantization_13_amd as mod
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "LIB_PATH", "/nonexistent/libgptq.so")
    with pytest.raises(RuntimeError, match="missing"):
        mod.lib()


def test_binding_rejects_mismatched_tensors(g):
    """The binding checks dtype, shape, contiguity and device of every tensor
    against (n, rows, bits, group_size) before the C call: a float32 or
    non-square H, U or outputs sized for another group size, or an X with the
    wrong feature count would otherwise be read or written out of bounds.
    Every case below raises ValueError before reaching the library (CPU
    tensors; nothing is launched)."""
    import torch
    n, rows = 256, 8
    cfg = g.Config(bits=4, group_size=128)
    f64 = lambda *s: torch.zeros(s, dtype=torch.float64)
    H, U = f64(n, n), torch.zeros((n, n), dtype=torch.float32)
    perm, dead = torch.zeros(n, dtype=torch.int32), torch.zeros(n, dtype=torch.uint8)
    W = torch.zeros((rows, n), dtype=torch.bfloat16)
    qw = torch.zeros((n * 4 // 32, rows), dtype=torch.int32)
    sc = torch.zeros((2, rows), dtype=torch.float16)
    ze = torch.zeros((2, rows), dtype=torch.float16)
    gi = torch.zeros(n, dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    X = torch.zeros((10, n), dtype=torch.bfloat16)
    bad = [
        lambda: g.gptq_hessian_accumulate(H.float(), 0, X, ws),                 # H not fp64
        lambda: g.gptq_hessian_accumulate(f64(n, n + 1), 0, X, ws),             # H not square
        lambda: g.gptq_hessian_accumulate(H, 0, X[:, :200], ws),                # X narrower than n
        lambda: g.gptq_hessian_accumulate(f64(2 * n, n)[::2], 0, X, ws),       # H strided
        lambda: g.gptq_prepare_hinv(H, cfg, U.double(), perm, dead, ws),        # U not fp32
        lambda: g.gptq_prepare_hinv(H, cfg, U, perm.long(), dead, ws),          # perm not int32
        lambda: g.gptq_prepare_hinv(H, cfg, U, perm, dead[:10], ws),            # dead too short
        lambda: g.gptq_quantize_layer(U, perm, dead, cfg, W, qw, sc[:1], ze, gi, ws),        # scales for gs 256
        lambda: g.gptq_quantize_layer(U, perm, dead, g.Config(group_size=64), W, qw, sc, ze, gi, ws),
        lambda: g.gptq_quantize_layer(U, perm, dead, g.Config(bits=3), W, qw, sc, ze, gi, ws),  # qweight for 4 bits
        lambda: g.gptq_quantize_layer(U[:128, :128].contiguous(), perm, dead, cfg, W, qw, sc, ze, gi, ws),
        lambda: g.gptq_quantize_layer(U, perm, dead, cfg, W, qw.t(), sc, ze, gi, ws),        # transposed view
        lambda: g.gptq_quantize_layer(U, perm, dead, cfg, W, qw, sc.float(), ze, gi, ws),    # scales not fp16
        lambda: g.gptq_layer_loss(H.float(), W, qw, sc, ze, gi, cfg, ws),
        lambda: g.gptq_layer_loss(H, W, qw, sc, ze, gi[:100], cfg, ws),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
        print(f"case {i}: rejected")
