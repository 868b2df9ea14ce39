"""Float64 GPTQ oracle (test infrastructure only; see the package docstring).

Every function states which passage it follows.  Where the pages leave a step
open, the reading taken is stated in the docstring (and listed with the others
in the repository's design notes).

Conventions
-----------
* W is [rows, n] (output features x input features).  Columns are the input
  features, i.e. the Hessian dimension.
* X is [tokens, n] (one calibration token per row).
* U is upper triangular with U^T U = H_d^{-1}, in the sweep (possibly
  act-order permuted) column order.
* The "decision precision" ``qdtype`` is the floating type in which the
  quantization grid (scale, zero) and each code are decided.  The default is
  float64.  Passing ``np.float32`` decides grid and codes in IEEE binary32
  (correctly rounded division, round-half-even), which is the precision the
  GPU kernels decide them in; the error propagation stays float64 either way.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


class NotPositiveDefinite(ValueError):
    """The damped Hessian is not positive definite (no Cholesky factor)."""


@dataclass(frozen=True)
class QuantConfig:
    """The knobs of the pages' quantize config (skillmd "Configurações de quantização";
    polydesk "Paramètres clés de GPTQ"): bits, group_size, desc_act, damp_percent, sym."""
    bits: int = 4
    group_size: int = 128   # -1 (or 0): one group per row
    sym: int = 0            # 0 asymmetric, 1 the pages' symmetric grid, 2 full-range symmetric
    desc_act: bool = False
    damp: float = 0.01

    @property
    def maxq(self) -> int:
        return (1 << self.bits) - 1


# ---------------------------------------------------------------------------
# Hessian
# ---------------------------------------------------------------------------
def hessian(chunks):
    """H = (2/N) * sum_t x_t x_t^T over all calibration tokens.

    [polydesk] "Étape 2 : Compensation d'erreur via la Hessienne" gives the
    Hessian as twice X X^T (X = features x tokens).  Reading: it is taken as a
    mean over the N tokens, (2/N) X X^T, so that the scale does not grow with
    the calibration set; codes, scales and the relative loss do not depend on
    that scale (pinned by the scale-invariance test).

    ``chunks`` is an iterable of [tokens_c, n] arrays (or a single array).
    Returns (H float64 [n, n], N).
    """
    if isinstance(chunks, np.ndarray):
        chunks = [chunks]
    acc = None
    count = 0
    for x in chunks:
        x = np.asarray(x, dtype=np.float64)
        g = x.T @ x
        acc = g if acc is None else acc + g
        count += x.shape[0]
    if acc is None or count == 0:
        raise ValueError("no calibration tokens")
    return 2.0 * acc / count, count


def hessian_entries(x, pairs):
    """Selected entries H[i, j] = (2/N) sum_t x[t, i] x[t, j], one dot product each.

    Same definition as ``hessian`` for the entries named in ``pairs`` (an array
    [k, 2] of (i, j)); used where the full n x n product is too large.
    """
    x = np.asarray(x)
    pairs = np.asarray(pairs)
    out = np.empty(len(pairs), dtype=np.float64)
    for k, (i, j) in enumerate(pairs):
        out[k] = np.dot(x[:, i].astype(np.float64), x[:, j].astype(np.float64))
    return 2.0 * out / x.shape[0]


# ---------------------------------------------------------------------------
# Prepare: dead columns, act-order, damping, Cholesky factor of H^-1
# ---------------------------------------------------------------------------
def prepare(H, damp=0.01, desc_act=False):
    """Dead columns, act-order permutation, damping and U = chol(H_d^{-1}).

    * Dead columns (reading; the pages are silent): an input feature whose
      diagonal H_ii is 0 never fires; its diagonal is set to 1 so H stays
      invertible, and ``quantize_layer`` zeroes that weight column.
    * Act-order ([polydesk] "Paramètres clés", desc_act): columns are visited in
      decreasing activation magnitude.  Reading: the magnitude of feature i is
      H_ii (= 2/N sum_t x_ti^2); the order is a stable sort of -diag(H), so ties
      keep the lower original index first.
    * Damping: lambda = damp * mean(diag H_p), added to every diagonal entry
      (the damp_percent field of the config, [skillmd] "Configurações de
      quantização").
    * [polydesk] "Étape 2" propagates each error through the inverse Hessian via
      a Cholesky decomposition for numerical stability.  Reading: U is the upper
      triangular factor with positive diagonal such that U^T U = H_d^{-1},
      computed here the plain way: invert, Cholesky, transpose.

    Returns dict(U, perm, dead, Hd, lam).  Raises NotPositiveDefinite.
    """
    H = np.array(H, dtype=np.float64, copy=True)
    n = H.shape[0]
    d = np.diag(H).copy()
    dead = d == 0.0
    idx = np.nonzero(dead)[0]
    H[idx, idx] = 1.0
    if desc_act:
        perm = np.argsort(-np.diag(H), kind="stable")
    else:
        perm = np.arange(n)
    Hp = H[np.ix_(perm, perm)]
    lam = damp * float(np.mean(np.diag(Hp)))
    Hd = Hp + lam * np.eye(n)
    if not np.all(np.isfinite(Hd)):
        raise NotPositiveDefinite("damped Hessian has non-finite entries")
    try:
        np.linalg.cholesky(Hd)                  # positive-definiteness check
        Hinv = np.linalg.inv(Hd)
        Hinv = 0.5 * (Hinv + Hinv.T)
        U = np.linalg.cholesky(Hinv).T          # upper, U^T U = Hd^{-1}
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    return dict(U=U, perm=perm.astype(np.int64), dead=dead, Hd=Hd, lam=lam)


# ---------------------------------------------------------------------------
# Quantization grid
# ---------------------------------------------------------------------------
def grid_params(wg, bits, sym, qdtype=np.float64):
    """Per-row scale and zero point of one group of weights.

    [skillmd] "Quantização group-wise": every group of (typically 128) weights
    owns a scale and a zero point.  [polydesk] "Paramètres clés", sym: the
    symmetric grid spans [-2^(b-1)+1, 2^(b-1)-1] and represents zero exactly;
    the asymmetric grid uses a non-zero zero point.

    Readings (the pages give no formulas): the range is [min(0, min w),
    max(0, max w)]; a group whose range is {0} uses [-1, 1].
      sym = 0, asym: s = (xmax - xmin) / maxq,  z = rint(-xmin / s)   (z in [0, maxq])
      sym = 1:  s = max(-xmin, xmax) / (2^(b-1) - 1),  z = 2^(b-1)    (codes 1..maxq)
      sym = 2:  the symmetric range [-a, a], a = max(-xmin, xmax), spread
                over all 2^b codes: s = (a - (-a)) / maxq,  z = 2^(b-1)  (codes 0..maxq)
    sym = 1 is the grid the pages describe; sym = 2 is a reading outside
    their text (a symmetric grid that keeps every code; zero is still exact
    because z is an integer).  All arithmetic in ``qdtype``; rint is
    round-half-to-even.  Returns (s, z) arrays of length rows, dtype ``qdtype``.
    """
    dt = np.dtype(qdtype).type
    wg = np.asarray(wg).astype(dt)
    zero = dt(0)
    xmin = np.minimum(wg.min(axis=1), zero)
    xmax = np.maximum(wg.max(axis=1), zero)
    degenerate = (xmin == 0) & (xmax == 0)
    xmin = np.where(degenerate, dt(-1), xmin).astype(dt)
    xmax = np.where(degenerate, dt(1), xmax).astype(dt)
    if int(sym) == 2:
        a = np.maximum(-xmin, xmax)
        s = ((a - (-a)) / dt((1 << bits) - 1)).astype(dt)
        z = np.full_like(s, dt(1 << (bits - 1)))
    elif sym:
        a = np.maximum(-xmin, xmax)
        s = (a / dt((1 << (bits - 1)) - 1)).astype(dt)
        z = np.full_like(s, dt(1 << (bits - 1)))
    else:
        s = ((xmax - xmin) / dt((1 << bits) - 1)).astype(dt)
        z = np.rint(-xmin / s).astype(dt)
    return s, z


def quantize_column(w, s, z, bits, sym, qdtype=np.float64):
    """Nearest grid point of each weight: c = clamp(rint(w / s) + z, lo, maxq),
    w_hat = s * (c - z), with lo = 1 for the pages' symmetric grid (sym = 1)
    and 0 otherwise.

    [polydesk] "Étape 2": a column is quantized by rounding with a scale factor.
    Returns (codes int64, w_hat float64); the decision is taken in ``qdtype``.
    """
    dt = np.dtype(qdtype).type
    w = np.asarray(w).astype(dt)
    lo = dt(1 if int(sym) == 1 else 0)
    hi = dt((1 << bits) - 1)
    c = np.clip(np.rint(w / s) + z, lo, hi).astype(dt)
    q = (s * (c - z)).astype(dt)
    return c.astype(np.int64), q.astype(np.float64)


# ---------------------------------------------------------------------------
# The column sweep
# ---------------------------------------------------------------------------
def _tie_between(t, c, alt, tol):
    """True where ``alt`` is the other neighbour of the rounding of ``t`` to
    ``c`` and ``t`` lies within ``tol`` of the midpoint between them: both are
    then nearest points within an arithmetic error of ``tol`` (the pages fix no
    rounding precision, so either is a correct result)."""
    t = np.asarray(t, dtype=np.float64)
    mid = np.minimum(c, alt) + 0.5
    return (np.abs(alt - c) == 1) & (np.abs(t - mid) <= tol)


def sweep(Wp, U, cfg: QuantConfig, qdtype=np.float64, block=None, stop=None, follow=None, tie_tol=None,
          record=False):
    """GPTQ column sweep over W already in sweep order.

    [polydesk] "Étape 1 : Ordre arbitraire": all rows visit the columns in the
    same fixed order.  "Étape 2": each column is quantized, its error is
    computed and pushed onto the columns not yet quantized through the inverse
    Hessian's Cholesky factor:  e = (w_j - w_hat_j) / U[j, j] and
    W[:, k] -= e * U[j, k] for k > j.  Group parameters are taken at each
    group's first column from the current, already compensated weights of its
    ``group_size`` columns (reading; the pages do not say when).

    ``block=None`` applies every update immediately (the plain form).  With
    ``block=B`` the updates to columns beyond the current block of B columns are
    delayed and applied once per block as W[:, i2:] -= E U[i1:i2, i2:]
    ([polydesk] "Étape 3 : Mises à jour par blocs"), which the pages state does
    not change the result.

    Returns dict(codes [rows, n] in sweep order, S, Z [n/gs, rows] in
    ``qdtype``, What [rows, n] float64 in sweep order, E [rows, n], L) where
    L = sum of e^2 / 2.  With ``stop=k`` (unblocked only) the sweep ends after
    k columns and the working matrix is returned as ``W``.

    Several correct results.  A quotient w/s that lies on a rounding midpoint
    has two nearest codes, and the same holds for a zero point -xmin/s; a
    solver whose arithmetic differs from this float64 path by a small amount
    may therefore take the other code where the quotient is within that
    amount of a midpoint, and its later columns then follow from that choice.
    ``follow`` (dict with "codes" [rows, n] in sweep order and optionally
    "zeros" [n/gs, rows]) names such another result; at each decision where
    it differs, the sweep takes the followed choice only if it is the other
    neighbour and the position lies within the tolerance of the midpoint:
      codes:  tol_j = tie_tol * (|w0_j| + sum_{k<j} |e_k| |U_kj|) / s,
              w0 the column's weight before any compensation, e the errors
              of the columns already quantized on this path;
      zeros:  tol = 2 * tie_tol * (tol scale at the group's argmin column +
              at its argmax column), from the first-order error of -xmin/s.
      stored scales ("scales" [n/gs, rows], fp16 values): the scale is kept
              in working precision for the sweep and stored rounded to fp16;
              where the other solver stored the other fp16 neighbour, it is
              taken if s lies within tol_s * s of the fp16 midpoint between
              the two, tol_s = tie_tol * (tol scale at the argmin column +
              at the argmax column) / (range of the grid in steps) + 2^-22
              (the first-order error of s from its extremes, plus the
              binary32 rounding of s).
    ``tie_tol`` is the relative arithmetic error allowed on the magnitudes
    that make up the compensated weight.  Otherwise it keeps its own choice.
    The result then carries "follow" = dict(ties, zero_ties, scale_ties,
    unexplained, ratio_max): how many choices were taken from ``follow`` as
    verified ties, how many differing choices were not ties (kept), and the
    largest |distance to the midpoint| / tol among the ties taken; and "S16",
    the stored fp16 scales with the followed ones in place.
    ``record=True`` (unblocked only) also returns, in sweep order, the
    position of every decision on its own path: "t" [rows, n] = w/s + z before
    rounding, "tol_scale" [rows, n] = (|w0_j| + sum_k |e_k||U_kj|) / s, and for
    the asymmetric grid "zq" [G, rows] = -xmin/s and "zq_scale" [G, rows] =
    2 * (tol_scale at the group's argmin column + at its argmax column).
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    rows, n = W.shape
    gs = n if cfg.group_size in (-1, 0) else cfg.group_size
    if n % gs:
        raise ValueError("n must be a multiple of group_size")
    ngroups = n // gs
    codes = np.zeros((rows, n), dtype=np.int64)
    What = np.zeros((rows, n), dtype=np.float64)
    E = np.zeros((rows, n), dtype=np.float64)
    S = np.zeros((ngroups, rows), dtype=qdtype)
    Z = np.zeros((ngroups, rows), dtype=qdtype)
    B = n if block is None else block
    loss = 0.0
    s = z = None
    if stop is not None and block is not None:
        raise ValueError("stop is only defined for the unblocked sweep")
    tracking = follow is not None or record
    if tracking:
        if block is not None:
            raise ValueError("follow and record are only defined for the unblocked sweep")
        w0 = np.abs(W)
        A = np.zeros_like(W)            # sum_k |e_k| |U_kj| over the quantized columns k < j
    if follow is not None:
        f_codes = np.asarray(follow["codes"], dtype=np.int64)
        f_zeros = follow.get("zeros")
        f_scales = follow.get("scales")
        tau = float(tie_tol)
        fst = dict(ties=0, zero_ties=0, scale_ties=0, unexplained=0, ratio_max=0.0)
        S16 = np.zeros((ngroups, rows), dtype=np.float16)
    else:
        f_codes = f_zeros = f_scales = None
    if record:
        rec_t = np.zeros((rows, n))
        rec_scale = np.zeros((rows, n))
        rec_zq = np.zeros((ngroups, rows))
        rec_zs = np.zeros((ngroups, rows))
    dt = np.dtype(qdtype).type
    for i1 in range(0, n, B):
        i2 = min(i1 + B, n)
        for j in range(i1, i2):
            if stop is not None and j == stop:
                return dict(W=W, codes=codes, E=E, L=loss)
            if j % gs == 0:
                s, z = grid_params(W[:, j:j + gs], cfg.bits, cfg.sym, qdtype)
                if tracking:
                    wg = W[:, j:j + gs]
                    scale = (w0[:, j:j + gs] + A[:, j:j + gs]) / np.abs(s)[:, None]
                    r = np.arange(rows)
                    ext = scale[r, wg.argmin(axis=1)] + scale[r, wg.argmax(axis=1)]
                    zscale = 2 * ext
                    xmin = np.minimum(wg.astype(dt).min(axis=1), dt(0))
                    if record and not cfg.sym:
                        rec_zq[j // gs] = -xmin / s
                        rec_zs[j // gs] = zscale
                if f_codes is not None:
                    s16 = to_fp16(s)
                    if f_scales is not None:
                        xmax = np.maximum(wg.astype(dt).max(axis=1), dt(0))
                        span = np.maximum(xmax - xmin, np.maximum(-xmin, xmax)) / s   # the grid's range in steps
                        tol_s = tau * ext / np.maximum(span, 1.0) + 2.0 ** -22
                        alt = np.asarray(f_scales[j // gs], dtype=np.float16)
                        adjacent = np.nextafter(s16, alt) == alt
                        mid = (s16.astype(np.float64) + alt.astype(np.float64)) / 2
                        m_s = np.abs(np.asarray(s, dtype=np.float64) - mid) / (tol_s * np.abs(s))
                        differ = alt != s16
                        ok = differ & adjacent & (m_s <= 1.0)
                        fst["scale_ties"] += int(np.sum(ok))
                        fst["unexplained"] += int(np.sum(differ & ~ok))
                        if np.any(ok):
                            fst["ratio_max"] = max(fst["ratio_max"], float(m_s[ok].max()))
                        s16 = np.where(ok, alt, s16)
                    S16[j // gs] = s16
                if f_zeros is not None and not cfg.sym:
                    tol = tau * zscale
                    alt = np.asarray(f_zeros[j // gs], dtype=np.float64)
                    ok = _tie_between(-xmin / s, z, alt, tol)
                    differ = alt != z
                    fst["zero_ties"] += int(np.sum(differ & ok))
                    fst["unexplained"] += int(np.sum(differ & ~ok))
                    if np.any(differ & ok):
                        m = np.abs(-xmin / s - (np.minimum(z, alt) + 0.5)) / tol
                        fst["ratio_max"] = max(fst["ratio_max"], float(m[differ & ok].max()))
                    z = np.where(differ & ok, alt, z).astype(z.dtype)
                S[j // gs] = s
                Z[j // gs] = z
            c, q = quantize_column(W[:, j], s, z, cfg.bits, cfg.sym, qdtype)
            if record:
                rec_t[:, j] = W[:, j].astype(dt) / s + z
                rec_scale[:, j] = (w0[:, j] + A[:, j]) / np.abs(s)
            if f_codes is not None:
                alt = f_codes[:, j]
                t = W[:, j].astype(dt) / s + z
                tol = tau * (w0[:, j] + A[:, j]) / np.abs(s)
                ok = _tie_between(t, c, alt, tol)
                differ = alt != c
                fst["ties"] += int(np.sum(differ & ok))
                fst["unexplained"] += int(np.sum(differ & ~ok))
                if np.any(differ & ok):
                    m = np.abs(t - (np.minimum(c, alt) + 0.5)) / tol
                    fst["ratio_max"] = max(fst["ratio_max"], float(m[differ & ok].max()))
                    c = np.where(differ & ok, alt, c)
                    q = (s * (c.astype(dt) - z)).astype(dt).astype(np.float64)
            e = (W[:, j] - q) / U[j, j]
            W[:, j + 1:i2] -= np.outer(e, U[j, j + 1:i2])
            if tracking:
                A[:, j + 1:] += np.outer(np.abs(e), np.abs(U[j, j + 1:]))
            codes[:, j] = c
            What[:, j] = q
            E[:, j] = e
            loss += 0.5 * float(e @ e)
        if i2 < n:
            W[:, i2:] -= E[:, i1:i2] @ U[i1:i2, i2:]
    out = dict(codes=codes, S=S, Z=Z, What=What, E=E, L=loss)
    if follow is not None:
        out["follow"] = fst
        out["S16"] = S16
    if record:
        out.update(t=rec_t, tol_scale=rec_scale, zq=rec_zq, zq_scale=rec_zs)
    return out


def quantize_layer(W, U, perm, dead, cfg: QuantConfig, qdtype=np.float64, block=None, follow=None,
                   tie_tol=None, record=False):
    """One layer: zero dead columns, permute, sweep, and return the outputs in
    the original column order.

    [ayinedjimi] "Calibration et dataset": scales and zero points are stored
    as FP16 and the low-bit weights packed for on-the-fly unpacking.  Outputs:
      qweight int32 [n*bits/32, rows]  (``pack``),
      scales, zeros float16 [n/gs, rows] in sweep group order,
      g_idx int32 [n], g_idx[perm[j]] = j // gs (reading: the group of each
        original column is the sweep group that quantized it),
      codes int64 [rows, n] in original order, L (internal damped loss),
      What float64 [rows, n] (working-precision grid values, original order).
    ``follow`` (dict with "codes" [rows, n] in ORIGINAL column order and
    optionally "zeros" [n/gs, rows]) and ``tie_tol``: see ``sweep``.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    rows, n = W.shape
    perm = np.asarray(perm)
    W[:, np.asarray(dead, dtype=bool)] = 0.0
    Wp = W[:, perm]
    if follow is not None:
        follow = dict(follow, codes=np.asarray(follow["codes"])[:, perm])
    r = sweep(Wp, U, cfg, qdtype=qdtype, block=block, follow=follow, tie_tol=tie_tol, record=record)
    gs = n if cfg.group_size in (-1, 0) else cfg.group_size
    codes = np.empty_like(r["codes"])
    codes[:, perm] = r["codes"]
    What = np.empty_like(r["What"])
    What[:, perm] = r["What"]
    g_idx = np.empty(n, dtype=np.int32)
    g_idx[perm] = np.arange(n) // gs
    out = dict(qweight=pack(codes, cfg.bits), scales=r["S16"] if "S16" in r else to_fp16(r["S"]),
               zeros=to_fp16(r["Z"]),
               g_idx=g_idx, codes=codes, What=What, L=r["L"], S=r["S"], Z=r["Z"],
               codes_sweep=r["codes"], E=r["E"])
    for k in ("follow", "t", "tol_scale", "zq", "zq_scale"):
        if k in r:
            out[k] = r[k]
    return out


def gptq_layer(W, H, cfg: QuantConfig, qdtype=np.float64, block=None):
    """Whole per-layer solve from the Hessian: prepare then quantize_layer.

    Adds ``rel_loss`` = ||(W - What) X||^2 / ||W X||^2 evaluated through H on
    the stored fp16 form ([polydesk] "Comment fonctionne l'algorithme GPTQ":
    the objective is the squared output error of the layer).
    """
    p = prepare(H, cfg.damp, cfg.desc_act)
    out = quantize_layer(W, p["U"], p["perm"], p["dead"], cfg, qdtype=qdtype, block=block)
    out.update(U=p["U"], perm=p["perm"], dead=p["dead"], lam=p["lam"], Hd=p["Hd"])
    What16 = dequantize(out["qweight"], out["scales"], out["zeros"], out["g_idx"], cfg.bits,
                        W.shape[0], W.shape[1])
    out["rel_loss"] = rel_loss(W, What16, H)
    return out


# ---------------------------------------------------------------------------
# Baselines used by the pins
# ---------------------------------------------------------------------------
def rtn(W, cfg: QuantConfig, qdtype=np.float64):
    """Round-to-nearest: the same grid applied to the original weights, group by
    group in natural column order, with no compensation ([polydesk] "Le
    problème que GPTQ résout" describes RTN as rounding each weight alone)."""
    W = np.asarray(W, dtype=np.float64)
    rows, n = W.shape
    gs = n if cfg.group_size in (-1, 0) else cfg.group_size
    codes = np.zeros((rows, n), dtype=np.int64)
    What = np.zeros((rows, n), dtype=np.float64)
    S = np.zeros((n // gs, rows), dtype=qdtype)
    Z = np.zeros((n // gs, rows), dtype=qdtype)
    for g in range(n // gs):
        cols = slice(g * gs, (g + 1) * gs)
        s, z = grid_params(W[:, cols], cfg.bits, cfg.sym, qdtype)
        S[g], Z[g] = s, z
        for j in range(g * gs, (g + 1) * gs):
            codes[:, j], What[:, j] = quantize_column(W[:, j], s, z, cfg.bits, cfg.sym, qdtype)
    return dict(codes=codes, What=What, S=S, Z=Z)


def obs_bruteforce(Wp, Hd, cfg: QuantConfig, qdtype=np.float64):
    """Sequential optimal-brain style compensation with explicit inverses.

    [polydesk] "Le problème que GPTQ résout" and [ayinedjimi] "L'algorithme OBQ
    revisité": after quantizing a weight, the remaining weights are adjusted to
    compensate.  For column j with free set F = {j..n-1} and M = (Hd[F, F])^{-1}
    the least-squares compensation is W[:, F] -= ((w_j - w_hat_j) / M[0,0]) M[0, :].
    Cubic per step; tiny layers only.  Order fixed (left to right), same
    grouping rule as ``sweep``.
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    rows, n = W.shape
    gs = n if cfg.group_size in (-1, 0) else cfg.group_size
    codes = np.zeros((rows, n), dtype=np.int64)
    What = np.zeros((rows, n), dtype=np.float64)
    s = z = None
    for j in range(n):
        if j % gs == 0:
            s, z = grid_params(W[:, j:j + gs], cfg.bits, cfg.sym, qdtype)
        c, q = quantize_column(W[:, j], s, z, cfg.bits, cfg.sym, qdtype)
        M = np.linalg.inv(Hd[j:, j:])
        err = W[:, j] - q
        W[:, j:] -= np.outer(err / M[0, 0], M[0, :])
        codes[:, j] = c
        What[:, j] = q
    return dict(codes=codes, What=What)


# ---------------------------------------------------------------------------
# Storage format
# ---------------------------------------------------------------------------
def to_fp16(x):
    """IEEE binary16, round to nearest even ([ayinedjimi] "Calibration et
    dataset": scale and zero point are kept in FP16)."""
    return np.asarray(x).astype(np.float16)


def pack(codes, bits):
    """Pack integer codes into int32 words.

    Reading (the pages only say the kernels unpack the low-bit weights on the
    fly): each row's codes, in original column order, form one little-endian
    bit stream in which column i occupies bits [bits*i, bits*i + bits); word k
    of that stream is qweight[k, row].  For 4-bit this puts columns 8k..8k+7 in
    word k at bits 4i..4i+3; for 3-bit every 32 columns fill exactly 3 words and
    columns 10 and 21 of each such chunk straddle a word boundary.
    Requires n * bits to be a multiple of 32.
    """
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    if (n * bits) % 32:
        raise ValueError("n * bits must be a multiple of 32")
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError("code out of range")
    words = np.zeros((n * bits // 32, rows), dtype=np.uint64)
    for i in range(n):
        bit = bits * i
        k, off = divmod(bit, 32)
        v = codes[:, i].astype(np.uint64)
        words[k] |= (v << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + bits > 32:
            words[k + 1] |= v >> np.uint64(32 - off)
    return words.astype(np.uint32).view(np.int32)


def unpack(qweight, bits, n):
    """Inverse of ``pack``: int32 [n*bits/32, rows] -> codes int64 [rows, n]."""
    words = np.asarray(qweight).view(np.uint32).astype(np.uint64)
    rows = words.shape[1]
    mask = np.uint64((1 << bits) - 1)
    codes = np.zeros((rows, n), dtype=np.int64)
    for i in range(n):
        bit = bits * i
        k, off = divmod(bit, 32)
        v = words[k] >> np.uint64(off)
        if off + bits > 32:
            v |= words[k + 1] << np.uint64(32 - off)
        codes[:, i] = (v & mask).astype(np.int64)
    return codes


def dequantize(qweight, scales, zeros, g_idx, bits, rows, n):
    """W_hat[:, i] = fp16 scale * (code - zero) of the group g_idx[i], float64."""
    codes = unpack(qweight, bits, n)
    s = np.asarray(scales, dtype=np.float64)[np.asarray(g_idx)].T   # [rows, n]
    z = np.asarray(zeros, dtype=np.float64)[np.asarray(g_idx)].T
    return s * (codes - z)


def dequant_matmul(A, qweight, scales, zeros, g_idx, bits, rows, n):
    """Y = A W_hat^T in float64: the product an inference kernel forms with the
    packed layer.

    [ayinedjimi] "Calibration et dataset" and "Kernels d'inférence": the GPU
    kernels that serve a GPTQ model unpack and dequantize the low-bit weights on
    the fly and multiply them with the (fp16) activations, so their result is
    the product of the activations with the dequantized matrix.  A is
    [tokens, n] (fp16 values; any real array is accepted), Y is [tokens, rows].
    """
    What = dequantize(qweight, scales, zeros, g_idx, bits, rows, n)
    return np.asarray(A, dtype=np.float64) @ What.T


def grouped_order(g_idx):
    """Columns listed group by group, ascending column index inside a group.

    The order in which a kernel that keeps one scale/zero pair per run of
    consecutive columns has to visit the input features when act-order has
    scattered the groups ([polydesk] "Paramètres clés de GPTQ", desc_act).
    """
    return np.argsort(np.asarray(g_idx), kind="stable").astype(np.int32)


def rel_loss(W, What, H):
    """||W X - What X||^2 / ||W X||^2 = tr(D H D^T) / tr(W H W^T), D = W - What.

    [polydesk] "Comment fonctionne l'algorithme GPTQ": the layer objective is
    the squared output error; written through H = (2/N) X X^T both traces carry
    the same factor, so the ratio equals the ratio of output errors.
    """
    W = np.asarray(W, dtype=np.float64)
    D = W - np.asarray(What, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    num = float(np.sum((D @ H) * D))
    den = float(np.sum((W @ H) * W))
    return num / den
