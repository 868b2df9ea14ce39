"""Shared helpers for the GPU parity tests (device transfer and comparisons).

Acceptance against the oracle, in two parts:

1. The solver's stated bar, against the plain float64 oracle (per-column
   sweep, no blocking, float64 decisions): >= 99.9 % identical codes, scales
   within 1e-3 relative and zero points equal on >= 99.9 % of groups,
   relative loss within 1 %, g_idx exact, packing bit-exact.

2. Validity of every remaining difference.  A code whose quotient w/s lies
   on a rounding midpoint has two nearest values, and the rest of its row
   then follows from whichever was taken (polydesk "Paramètres clés de GPTQ":
   the result depends on the order and on each rounding).  The oracle re-runs
   its plain sweep taking the GPU's code (or zero point) wherever the two
   differ AND the oracle's own quotient is within the tie tolerance of the
   midpoint between them (likewise a stored fp16 scale that is the other
   rounding of a scale lying next to an fp16 midpoint); everything else must
   then be identical: every code, every zero point, every stored scale.

Tie tolerance.  The kernels keep W in fp32, U in fp32 (rounded from an fp64
factorization), apply the near updates on the fp32 MFMA and the far ones in
split-bf16 (x = hi + lo, three bf16 products: each product within 3 * 2^-18
of exact).  The compensated weight of column j is w0_j - sum_k e_k U_kj, so
its arithmetic error is a relative error on the magnitudes
|w0_j| + sum_k |e_k| |U_kj|.  Emulating that arithmetic against the plain
float64 sweep (256x256 to 64x2048 layers of the three workload shapes, U
additionally perturbed by 1e-6 relative) the quotient error never exceeded
7.4e-6 of (|w0_j| + sum_k |e_k||U_kj|) / s.  The tolerance is 2^-15 = 3.05e-5
of that scale: four times the emulated maximum, a per-code tie window of a
few 1e-4 quotient units at these layers' magnitudes.
"""
import numpy as np

import oracle
import synth

TIE_TOL = 2.0 ** -15


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
    # packing against the oracle's words, on every row whose codes all agree
    # (there the oracle's packed words are the expected ones)
    qw = out["qweight"].cpu().numpy()
    same = np.all(codes == ref["codes"], axis=1)
    pack_ok = bool(same.any() and np.array_equal(qw[:, same], ref["qweight"][:, same]))
    loss_rel = abs(gpu_rel_loss - ref["rel_loss"]) / ref["rel_loss"]
    return dict(agree=agree, s_rel=s_rel, s_frac=s_frac, z_frac=z_frac, gidx_ok=gidx_ok, pack_ok=pack_ok,
                rows_all_same=float(np.mean(same)), loss_rel=loss_rel, gpu_rel_loss=gpu_rel_loss,
                ref_rel_loss=ref["rel_loss"])


def assert_stated_bar(m):
    assert m["agree"] >= 0.999, m
    assert m["s_frac"] >= 0.999 and m["z_frac"] >= 0.999, m
    assert m["gidx_ok"] and m["pack_ok"], m
    assert m["loss_rel"] <= 0.01, m


def follow_check(out, W, U, perm, dead, ocfg, bits, rows_idx=None, label=""):
    """Part 2: the plain float64 oracle takes the GPU's choice at verified ties
    and must then reproduce every GPU output exactly (codes, zero points,
    stored fp16 scales).  ``U, perm, dead`` are the oracle's own (from its own
    Hessian); ``rows_idx`` restricts the check to those rows (rows are
    independent given U).  Returns the oracle's followed result."""
    n = W.shape[1]
    codes = gpu_codes(out, bits, n)
    z_gpu = out["zeros"].cpu().numpy().astype(np.float64)
    s_gpu = out["scales"].cpu().numpy()
    if rows_idx is not None:
        codes, z_gpu, s_gpu, W = codes[rows_idx], z_gpu[:, rows_idx], s_gpu[:, rows_idx], W[rows_idx]
    f = oracle.quantize_layer(np.asarray(W, dtype=np.float64), U, perm, dead, ocfg,
                              follow=dict(codes=codes, zeros=z_gpu, scales=s_gpu), tie_tol=TIE_TOL)
    st = f["follow"]
    s_bad = int(np.sum(s_gpu != f["scales"]))
    z_bad = int(np.sum(z_gpu != f["zeros"].astype(np.float64)))
    c_bad = int(np.sum(codes != f["codes"]))
    print(f"[follow] {label}: {codes.shape[0]} rows, ties taken {st['ties']} codes + {st['zero_ties']} zero points "
          f"+ {st['scale_ties']} stored scales (largest |margin|/tol {st['ratio_max']:.3f}); unexplained "
          f"{st['unexplained']}; after following: codes differing {c_bad}, zero points {z_bad}, stored scales "
          f"{s_bad}", flush=True)
    assert st["unexplained"] == 0
    assert c_bad == 0 and z_bad == 0 and s_bad == 0
    return f


# ----------------------------------------------------------------------------- rows in parallel
def _plain_and_follow(args):
    """Worker: the plain sweep of a row shard and its tie-following re-run."""
    upath, W, perm, dead, ocfg, codes, zeros, scales = args
    U = np.load(upath, mmap_mode="r")
    plain = oracle.quantize_layer(W, U, perm, dead, ocfg)
    f = oracle.quantize_layer(W, U, perm, dead, ocfg, follow=dict(codes=codes, zeros=zeros, scales=scales),
                              tie_tol=TIE_TOL)
    keep = ("codes", "scales", "zeros", "qweight")
    return {k: plain[k] for k in keep}, {k: f[k] for k in keep}, f["follow"]


def plain_and_follow_rows(out, W, U, perm, dead, ocfg, bits, rows_idx, workers=16):
    """The plain float64 sweep of the sampled rows and its tie-following re-run,
    split over worker processes by rows (rows are independent given U; each
    worker runs the unchanged oracle on its shard).  Returns (plain, followed,
    follow statistics) with the rows stacked back in ``rows_idx`` order."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import os
    import tempfile
    n = W.shape[1]
    codes = gpu_codes(out, bits, n)[rows_idx]
    zeros = out["zeros"].cpu().numpy().astype(np.float64)[:, rows_idx]
    scales = out["scales"].cpu().numpy()[:, rows_idx]
    Wr = np.asarray(W, dtype=np.float64)[rows_idx]
    shards = np.array_split(np.arange(len(rows_idx)), workers)
    with tempfile.TemporaryDirectory() as tmp:
        upath = os.path.join(tmp, "U.npy")
        np.save(upath, np.ascontiguousarray(U))
        jobs = [(upath, Wr[sh], perm, dead, ocfg, codes[sh], zeros[:, sh], scales[:, sh]) for sh in shards if len(sh)]
        with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as ex:
            res = list(ex.map(_plain_and_follow, jobs))
    cat = lambda part, k, axis: np.concatenate([r[part][k] for r in res], axis=axis)
    plain = {k: cat(0, k, 0 if k == "codes" else 1) for k in ("codes", "scales", "zeros", "qweight")}
    fol = {k: cat(1, k, 0 if k == "codes" else 1) for k in ("codes", "scales", "zeros", "qweight")}
    st = {k: sum(r[2][k] for r in res) for k in ("ties", "zero_ties", "scale_ties", "unexplained")}
    st["ratio_max"] = max(r[2]["ratio_max"] for r in res)
    return plain, fol, st


# ----------------------------------------------------------------------------- stored references
def first_divergence_check(codes_gpu, s_gpu, z_gpu, perm_gpu, ref, lp, perm_ref, gs, sym, label):
    """Sampled rows of a layer too large for the oracle to re-run in a test,
    against the plain float64 oracle's stored path (prefix ``lp``).

    For each row, the first sweep position where the two paths part is found:
    the first differing code, the start of the first group with a differing
    zero point, or the first position where the act-order permutations differ
    (checked separately as a near-tie of diag(H)).  A differing code or zero
    point there must be a verified tie: the oracle's unrounded position
    (stored for every near-tie of its path) lies within TIE_TOL of its scale
    of the midpoint to the GPU's choice.  Every group whose grid was taken at
    or before that position (the compensated weights are identical up to it)
    must have its scale within 1e-3 and, unless the tie was that zero point,
    the same zero point.  Returns (rows that part, largest |margin|/tol)."""
    rows, n = codes_gpu.shape
    G = s_gpu.shape[0]
    cs_gpu = codes_gpu[:, perm_gpu]
    cs_ref = ref[lp + "codes"].astype(np.int64)[:, perm_ref]
    s_ref = ref[lp + "scales"].astype(np.float64)
    z_ref = ref[lp + "zeros"].astype(np.float64)
    diff_perm = np.nonzero(perm_gpu != perm_ref)[0]
    p0 = int(diff_perm[0]) if len(diff_perm) else n
    if p0 < n:
        print(f"[first divergence] {label}: the act-order permutations first differ at sweep position {p0} of {n} "
              f"(a verified near-tie of diag(H)); rows are compared up to there", flush=True)
    nt = {(int(r), int(j)): (float(f), float(sc)) for r, j, f, sc in
          zip(ref[lp + "nt_row"], ref[lp + "nt_col"], ref[lp + "nt_frac"], ref[lp + "nt_scale"])}
    zt = {(int(r), int(g)): (float(f), float(sc)) for r, g, f, sc in
          zip(ref[lp + "zt_row"], ref[lp + "zt_group"], ref[lp + "zt_frac"], ref[lp + "zt_scale"])}
    parted, worst = [], 0.0
    for r in range(rows):
        dc = np.nonzero(cs_gpu[r, :p0] != cs_ref[r, :p0])[0]
        jc = int(dc[0]) if len(dc) else n
        dz = np.nonzero(z_gpu[:, r] != z_ref[:, r])[0]
        dz = dz[dz * gs < p0]
        jz = int(dz[0]) * gs if len(dz) else n
        j = min(p0, jc, jz)
        zero_tie_group = -1
        if j < n:
            parted.append(r)
        if j == jz and jz < n:                                  # a zero point parts first
            g = jz // gs
            a, c = int(z_gpu[g, r]), int(z_ref[g, r])
            frac, sc = zt.get((r, g), (None, None))
            ok = frac is not None and abs(a - c) == 1 and abs((0.5 if a > c else -0.5) - frac) <= TIE_TOL * sc
            print(f"[first divergence] {label}: row {r}: zero point of group {g}: oracle {c}, GPU {a}, "
                  f"{'verified tie' if ok else 'NOT a verified tie'}"
                  + (f" (|margin| {abs((0.5 if a > c else -0.5) - frac):.3e}, tol {TIE_TOL * sc:.3e})"
                     if frac is not None else ""), flush=True)
            assert ok, (label, r, g)
            worst = max(worst, abs((0.5 if a > c else -0.5) - frac) / (TIE_TOL * sc))
            zero_tie_group = g
        elif j == jc and jc < n:                                # a code parts first
            a, c = int(cs_gpu[r, jc]), int(cs_ref[r, jc])
            frac, sc = nt.get((r, jc), (None, None))
            ok = frac is not None and abs(a - c) == 1 and abs((0.5 if a > c else -0.5) - frac) <= TIE_TOL * sc
            print(f"[first divergence] {label}: row {r}: sweep column {jc}: oracle {c}, GPU {a}, "
                  f"{'verified tie' if ok else 'NOT a verified tie'}"
                  + (f" (|margin| {abs((0.5 if a > c else -0.5) - frac):.3e}, tol {TIE_TOL * sc:.3e})"
                     if frac is not None else ""), flush=True)
            assert ok, (label, r, jc)
            worst = max(worst, abs((0.5 if a > c else -0.5) - frac) / (TIE_TOL * sc))
        up = min(G, j // gs + 1) if j < n else G                 # groups whose grid was taken at or before j
        for g in range(up):
            assert abs(s_gpu[g, r] - s_ref[g, r]) <= 1e-3 * abs(s_ref[g, r]), (label, r, g)
            assert g == zero_tie_group or z_gpu[g, r] == z_ref[g, r], (label, r, g)
    return parted, worst
