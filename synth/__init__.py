"""Seeded synthetic layers and calibration activations.

This module is the only code shared by the float64 oracle (``oracle/``) and the
HIP path's tests and benchmark.  It draws random numbers and shapes them into
weights W [rows, n] and calibration activations X [tokens, n]; it holds none of
the quantization method's arithmetic (no Hessian, no rounding grid, no
compensation).

Why synthetic: the pages calibrate on C4 / WikiText-2 text samples (128-256
sequences of 512 tokens, skillmd.com "Gptq" page, section "Quantizar seu
próprio modelo"; ayinedjimi-consultants "Quantization : GPTQ, GGUF, AWQ",
section "Calibration et dataset") through trained Llama/OPT weights.  Neither
the datasets nor the weights are available here, so each workload below stands
in for one of those layers with the pages' token counts and a seeded generator.

Every stream comes from numpy's PCG64 seeded by ``SeedSequence([seed, stream,
...])`` so that any token chunk can be regenerated on its own: X chunk ``c``
covers tokens ``[CHUNK*c, CHUNK*c + CHUNK)`` and uses ``SeedSequence([seed,
100, xset, c])``.  bf16 workloads are drawn in float32 and rounded to bf16 with
round-to-nearest-even; both sides read the same bf16 values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096          # tokens per independently seeded activation chunk
FACTORS = 64          # rank of the correlated part of the factor model


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only: IEEE binary32 with the low 16 bits dropped
# after round-to-nearest-even)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> the exact float32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 values on the bf16 grid (round to nearest even)."""
    return bf16_value(bf16_bits(x))


# ----------------------------------------------------------------------------
# Workload recipes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Linear:
    """One linear layer of a workload: W is [rows, n]; its inputs come from X set ``xset``."""
    name: str
    rows: int
    n: int
    xset: int
    w_std: float


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                 # "bf16" or "fp32" storage of W and X
    tokens: int
    linears: tuple             # tuple[Linear]
    xsets: tuple               # tuple of (n, kind, outlier_count, outlier_scale)
    bits: int = 4
    group_size: int = 128
    sym: bool = False
    desc_act: bool = False
    damp: float = 0.01
    block_size: int = 128
    description: str = ""

    @property
    def rows(self) -> int:
        return self.linears[0].rows

    @property
    def n(self) -> int:
        return self.linears[0].n

    def resized(self, rows=None, n=None, tokens=None, name=None) -> "Workload":
        """Same recipe at other sizes (first linear / first X set only).

        Outlier channel counts scale with n so the outlier fraction is kept.
        """
        lin = self.linears[0]
        nn = lin.n if n is None else n
        xs = self.xsets[lin.xset]
        frac = xs[2] / xs[0] if xs[0] else 0.0
        oc = xs[2] if n is None else (int(round(frac * nn)) if xs[2] else 0)
        newx = (nn, xs[1], oc, xs[3])
        newl = Linear(lin.name, lin.rows if rows is None else rows, nn, 0, lin.w_std)
        return dataclasses.replace(
            self, name=name or f"{self.name}@{newl.rows}x{nn}x{tokens or self.tokens}",
            tokens=self.tokens if tokens is None else tokens,
            linears=(newl,), xsets=(newx,))


def _ss(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


WORKLOADS = {
    # Single 256x256 fp32 layer; X = A Z with A of decaying spectrum, 4 outlier channels x20.
    "toy256": Workload(
        name="toy256", seed=1, dtype="fp32", tokens=2048,
        linears=(Linear("linear", 256, 256, 0, 0.02),),
        xsets=((256, "haar", 4, 20.0),),
        bits=4, group_size=128, sym=False, desc_act=False, damp=0.01,
        description="W 256x256 fp32 N(0,0.02^2); X 256 x 2048 tokens, A Z with decaying "
                    "spectrum, 4 outlier channels x20; 4-bit asym g128 damp 0.01"),
    # Llama-7B-shaped attention projection; 128 x 512 calibration tokens; 1% outliers x20.
    "attn4096": Workload(
        name="attn4096", seed=2, dtype="bf16", tokens=65536,
        linears=(Linear("q_proj", 4096, 4096, 0, 0.02),),
        xsets=((4096, "factor", 41, 20.0),),
        bits=4, group_size=128, sym=False, desc_act=False, damp=0.01,
        description="W 4096x4096 bf16 N(0,0.02^2); X 4096 x 65536 tokens correlated "
                    "Gaussian, 1% outlier channels x20; 4-bit asym g128 damp 0.01"),
    # MLP down projection, heavy-tailed post-SiLU-gating activations, 3-bit, act-order.
    "mlpdown11008": Workload(
        name="mlpdown11008", seed=3, dtype="bf16", tokens=65536,
        linears=(Linear("down_proj", 4096, 11008, 0, 0.015),),
        xsets=((11008, "silu_t", 0, 1.0),),
        bits=3, group_size=128, sym=False, desc_act=True, damp=0.01,
        description="W 4096x11008 bf16 N(0,0.015^2); X 11008 x 65536 tokens silu(G)*t4; "
                    "3-bit asym g128 desc_act"),
    # 70B-shaped down projection, symmetric 4-bit, act-order.
    "down28672": Workload(
        name="down28672", seed=4, dtype="bf16", tokens=131072,
        linears=(Linear("down_proj", 8192, 28672, 0, 0.01),),
        xsets=((28672, "factor", 143, 30.0),),
        bits=4, group_size=128, sym=True, desc_act=True, damp=0.01,
        description="W 8192x28672 bf16 N(0,0.01^2); X 28672 x 131072 tokens correlated "
                    "Gaussian, 0.5% outlier channels x30; 4-bit sym g128 desc_act"),
    # Llama-2-7B-shaped decoder block: 7 linears over 4 activation sets.
    "llama2block": Workload(
        name="llama2block", seed=5, dtype="bf16", tokens=262144,
        linears=(Linear("q_proj", 4096, 4096, 0, 0.02), Linear("k_proj", 4096, 4096, 0, 0.02),
                 Linear("v_proj", 4096, 4096, 0, 0.02), Linear("o_proj", 4096, 4096, 1, 0.02),
                 Linear("gate_proj", 11008, 4096, 2, 0.02), Linear("up_proj", 11008, 4096, 2, 0.02),
                 Linear("down_proj", 4096, 11008, 3, 0.02)),
        xsets=((4096, "factor", 0, 1.0), (4096, "factor", 0, 1.0),
               (4096, "factor", 0, 1.0), (11008, "factor", 0, 1.0)),
        bits=4, group_size=128, sym=False, desc_act=True, damp=0.01,
        description="Llama-2-7B-shaped block, random-init bf16; q/k/v share one Hessian, "
                    "gate/up share one; X 128 x 2048 tokens; 4-bit asym g128 desc_act"),
}


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------
def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def weights_raw(wl: Workload, li: int = 0) -> np.ndarray:
    """W of linear ``li`` as stored: uint16 bf16 bits or float32, row-major [rows, n]."""
    lin = wl.linears[li]
    g = _ss(wl.seed, 0, li)
    w = (g.standard_normal((lin.rows, lin.n), dtype=np.float32) * np.float32(lin.w_std))
    return _store(w, wl.dtype)


def weights(wl: Workload, li: int = 0) -> np.ndarray:
    """W of linear ``li`` as exact float32 values."""
    r = weights_raw(wl, li)
    return bf16_value(r) if wl.dtype == "bf16" else r


def _haar(g: np.random.Generator, n: int) -> np.ndarray:
    q, r = np.linalg.qr(g.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


def _xset_static(wl: Workload, xset: int):
    """Per-X-set quantities that do not depend on the token chunk."""
    n, kind, oc, oscale = wl.xsets[xset]
    scale = np.ones(n, dtype=np.float32)
    if oc:
        idx = _ss(wl.seed, 3, xset).choice(n, size=oc, replace=False)
        scale[idx] = np.float32(oscale)
    if kind == "haar":
        g = _ss(wl.seed, 1, xset)
        sigma = 1.0 / (np.arange(n) + 1.0)
        a = (_haar(g, n) * sigma[None, :]) @ _haar(g, n).T
        return kind, scale, a.astype(np.float32)
    loadings = (_ss(wl.seed, 2, xset).standard_normal((n, FACTORS), dtype=np.float32)
                * (1.0 / np.sqrt(np.arange(FACTORS, dtype=np.float32) + 1.0))[None, :])
    return kind, scale, np.ascontiguousarray(loadings, dtype=np.float32)


_STATIC_CACHE: dict = {}


def _static(wl: Workload, xset: int):
    # keyed by the set's index too: sets with equal descriptions (q/k/v-in,
    # o-in, gate/up-in of a block) still have their own seeded loadings
    key = (wl.name, wl.seed, xset, wl.xsets[xset])
    if key not in _STATIC_CACHE:
        _STATIC_CACHE[key] = _xset_static(wl, xset)
    return _STATIC_CACHE[key]


def n_chunks(wl: Workload) -> int:
    return (wl.tokens + CHUNK - 1) // CHUNK


def activations_chunk_raw(wl: Workload, c: int, xset: int = 0) -> np.ndarray:
    """Token chunk ``c`` of X set ``xset`` as stored, row-major [chunk_tokens, n]."""
    n = wl.xsets[xset][0]
    t0 = c * CHUNK
    t = min(CHUNK, wl.tokens - t0)
    if t <= 0:
        raise IndexError("chunk out of range")
    kind, scale, mat = _static(wl, xset)
    g = _ss(wl.seed, 100, xset, c)
    if kind == "haar":
        z = g.standard_normal((n, t), dtype=np.float32)
        x = (mat @ z).T                                   # [t, n]
    else:
        f = g.standard_normal((t, FACTORS), dtype=np.float32)
        eps = g.standard_normal((t, n), dtype=np.float32)
        x = f @ mat.T + np.float32(0.5) * eps             # [t, n]
        if kind == "silu_t":
            tails = g.standard_t(4.0, size=(t, n)).astype(np.float32) * np.float32(1.0 / np.sqrt(2.0))
            x = (x / (np.float32(1.0) + np.exp(-x))) * tails
    x = x * scale[None, :]
    return _store(np.ascontiguousarray(x, dtype=np.float32), wl.dtype)


def activations_chunk(wl: Workload, c: int, xset: int = 0) -> np.ndarray:
    r = activations_chunk_raw(wl, c, xset)
    return bf16_value(r) if wl.dtype == "bf16" else r


def activations_raw(wl: Workload, xset: int = 0) -> np.ndarray:
    """The whole X set as stored, [tokens, n]."""
    return np.concatenate([activations_chunk_raw(wl, c, xset) for c in range(n_chunks(wl))], axis=0)


def activations(wl: Workload, xset: int = 0) -> np.ndarray:
    r = activations_raw(wl, xset)
    return bf16_value(r) if wl.dtype == "bf16" else r


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------------------
# Inputs of the dequantizing matmul: a quantized layer in the quantizer's
# output shapes and fp16 decode-time activations
# ----------------------------------------------------------------------------
def group_params(seed: int, rows: int, n: int, bits: int, group_size: int, act_order: bool = False):
    """fp16 scales and integer-valued fp16 zero points [G, rows] (G = n /
    group_size, 1 for group_size -1) and the group index int32 [n] of each
    column, in the shapes the quantizer writes.

    Scales are drawn around what a 4-bit grid over N(0, 0.02^2) weights in
    groups of 128 gives (range about 6 sigma over 2^bits - 1 steps).  Without
    act_order the groups are runs of consecutive columns; with it they are
    spread over the columns by a random permutation, as a column order that
    visits columns by decreasing activation leaves them."""
    g = _ss(seed, 310, rows, n, bits, max(group_size, 0))
    gs = n if group_size <= 0 else group_size
    G = n // gs
    maxq = (1 << bits) - 1
    scales = (g.uniform(0.5, 1.5, size=(G, rows)) * 0.02 * 6.0 / maxq).astype(np.float16)
    zeros = g.integers(0, maxq + 1, size=(G, rows)).astype(np.float16)
    pos = np.arange(n)
    if act_order:
        order = g.permutation(n)                     # column visited at position j
        g_idx = np.empty(n, dtype=np.int32)
        g_idx[order] = (pos // gs).astype(np.int32)
    else:
        g_idx = (pos // gs).astype(np.int32)
    return scales, zeros, g_idx


def quantized_layer(seed: int, rows: int, n: int, bits: int, group_size: int, act_order: bool = False):
    """Random codes int64 [rows, n] in [0, 2^bits) with ``group_params``:
    (codes, scales, zeros, g_idx)."""
    codes = _ss(seed, 300, rows, n, bits).integers(0, 1 << bits, size=(rows, n), dtype=np.int64)
    return (codes, *group_params(seed, rows, n, bits, group_size, act_order))


def decode_activations_raw(seed: int, tokens: int, n: int, outlier_frac: float = 0.01,
                           outlier_scale: float = 20.0) -> np.ndarray:
    """fp16 bits uint16 [tokens, n]: N(0, 1) entries with a fixed set of outlier
    channels (outlier_frac of them) scaled by outlier_scale, the input of a
    linear layer at decode time."""
    g = _ss(seed, 400, tokens, n)
    x = g.standard_normal((tokens, n))
    k = int(round(outlier_frac * n))
    if k:
        x[:, g.choice(n, size=k, replace=False)] *= outlier_scale
    return x.astype(np.float16).view(np.uint16)


def random_qweight(seed: int, rows: int, n: int, bits: int) -> np.ndarray:
    """uint32 [n * bits / 32, rows] of uniform random bits: a packed code matrix
    in the quantizer's output shape (every bit pattern is a valid code stream)."""
    g = _ss(seed, 500, rows, n, bits)
    return g.integers(0, 1 << 32, size=(n * bits // 32, rows), dtype=np.uint64).astype(np.uint32)


def _chunk_job(args):
    wl, xset, c = args
    return c, activations_chunk_raw(wl, c, xset)


def activations_raw_parallel(wl: Workload, xset: int = 0, workers: int = 16, out=None):
    """``activations_raw`` with the chunks generated by spawned worker
    processes (each chunk is seeded on its own, so the result is identical).
    ``out``, if given, is called as out(t0, chunk) for each chunk instead of
    assembling the whole array (which is then not returned)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    n = wl.xsets[xset][0]
    full = None if out is not None else np.empty((wl.tokens, n), dtype=np.uint16 if wl.dtype == "bf16"
                                                 else np.float32)
    jobs = [(wl, xset, c) for c in range(n_chunks(wl))]
    with ProcessPoolExecutor(max_workers=max(1, workers), mp_context=mp.get_context("spawn")) as ex:
        for c, raw in ex.map(_chunk_job, jobs):
            if out is not None:
                out(c * CHUNK, raw)
            else:
                full[c * CHUNK:c * CHUNK + raw.shape[0]] = raw
    return full
