"""Writes <workload>_sampled.npz: the oracle's results at a workload's full size,
kept for sampled rows and Hessian entries, so that the GPU test at full size
can compare without re-running the float64 oracle (minutes of CPU).

Calls only ``oracle`` and ``synth``.  For each workload named on the command
line (default mlpdown11008) and each of its activation sets it computes, in
float64:
  * the full Hessian over all calibration tokens, chunk by chunk;
  * prepare (damping, act-order permutation, U);
  * for every linear reading that set, the plain per-column sweep (float64
    decisions, no blocking) of a seeded sample of weight rows (rows are
    independent given U): codes, scales, zero points, g_idx, the relative
    loss of those rows, and the near-ties of their path: every decision
    whose unrounded position lies within NEAR_TIE * tol_scale of the
    midpoint to a neighbouring code (or zero point), with that position and
    scale (see oracle.sweep, record=True), where a solver with slightly
    different arithmetic may validly take the other neighbour;
  * a seeded sample of Hessian entries and the diagonal.
Keys carry a set{s}_ / lin{i}_ prefix for workloads with several linears.

Usage: python tests/golden/make_fullsize_refs.py [workload ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

SAMPLE_ROWS = 48
SAMPLE_PAIRS = 4096
# Near-ties kept: distance to the midpoint <= NEAR_TIE * tol_scale, a window
# well beyond any tie tolerance a test applies (2^-15 of the same scale).
NEAR_TIE = 2.0 ** -11


def sample_rows(rows: int) -> np.ndarray:
    g = np.random.default_rng(20261203)
    pick = g.choice(np.arange(1, rows - 1), size=SAMPLE_ROWS - 2, replace=False)
    return np.sort(np.concatenate([[0, rows - 1], pick])).astype(np.int64)


def sample_pairs(n: int) -> np.ndarray:
    g = np.random.default_rng(20261204)
    p = g.integers(0, n, size=(SAMPLE_PAIRS, 2))
    p[:256, 1] = p[:256, 0]                      # some diagonal entries
    return p.astype(np.int64)


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def near_ties(ref, n, gs):
    """Sparse list of the path's near-ties (sweep order): codes (row, column,
    position - code, scale) and zero points (row, group, position - zero, scale)."""
    codes = ref["codes_sweep"]
    frac = ref["t"] - codes                                # in [-0.5, 0.5] unless clamped
    dist = np.minimum(np.abs(0.5 - frac), np.abs(frac + 0.5))
    r, j = np.nonzero(dist <= NEAR_TIE * ref["tol_scale"])
    out = {"nt_row": r.astype(np.int32), "nt_col": j.astype(np.int32),
           "nt_frac": frac[r, j].astype(np.float32), "nt_scale": ref["tol_scale"][r, j].astype(np.float32)}
    zfrac = ref["zq"] - ref["Z"]                           # [G, rows]
    zdist = np.minimum(np.abs(0.5 - zfrac), np.abs(zfrac + 0.5))
    g, zr = np.nonzero((zdist <= NEAR_TIE * ref["zq_scale"]) & (ref["zq_scale"] > 0))
    out.update({"zt_row": zr.astype(np.int32), "zt_group": g.astype(np.int32),
                "zt_frac": zfrac[g, zr].astype(np.float32), "zt_scale": ref["zq_scale"][g, zr].astype(np.float32)})
    return out


def main(name: str) -> None:
    wl = synth.get(name)
    cfg = oracle.QuantConfig(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                             damp=wl.damp)
    arrays = {"tokens": np.int64(wl.tokens), "near_tie": np.float64(NEAR_TIE)}
    single = len(wl.linears) == 1
    sets = sorted({lin.xset for lin in wl.linears})
    for s in sets:
        n = wl.xsets[s][0]
        log(f"{name}: set {s}: Hessian over {wl.tokens} tokens x {n} features")

        def chunks():
            for c in range(synth.n_chunks(wl)):
                raw = synth.activations_chunk_raw(wl, c, s)
                yield synth.bf16_value(raw) if wl.dtype == "bf16" else raw

        H, cnt = oracle.hessian(chunks())
        assert cnt == wl.tokens
        pairs = sample_pairs(n)
        log("prepare")
        p = oracle.prepare(H, cfg.damp, cfg.desc_act)
        pre = "" if single else f"set{s}_"
        arrays.update({pre + "pairs": pairs, pre + "h_values": H[pairs[:, 0], pairs[:, 1]],
                       pre + "h_diag": np.diag(H).copy(), pre + "perm": p["perm"].astype(np.int32)})
        for li, lin in enumerate(wl.linears):
            if lin.xset != s:
                continue
            ridx = sample_rows(lin.rows)
            log(f"{lin.name}: plain sweep on {len(ridx)} sampled rows")
            w = synth.weights(wl, li)[ridx].astype(np.float64)
            ref = oracle.quantize_layer(w, p["U"], p["perm"], p["dead"], cfg, record=True)
            What = oracle.dequantize(ref["qweight"], ref["scales"], ref["zeros"], ref["g_idx"], wl.bits, len(ridx),
                                     lin.n)
            rel = oracle.rel_loss(w, What, H)
            lp = "" if single else f"lin{li}_"
            gs = lin.n if wl.group_size in (-1, 0) else wl.group_size
            nt = near_ties(ref, lin.n, gs)
            arrays.update({lp + "rows": ridx, lp + "codes": ref["codes"].astype(np.uint8),
                           lp + "scales": ref["scales"], lp + "zeros": ref["zeros"],
                           lp + "g_idx": ref["g_idx"].astype(np.int32), lp + "rel_loss": np.float64(rel)})
            arrays.update({lp + k: v for k, v in nt.items()})
            log(f"{lin.name}: rel loss of the sampled rows {rel:.6e}; near-ties kept: {len(nt['nt_row'])} codes, "
                f"{len(nt['zt_row'])} zero points")
        del H, p
    out = os.path.join(HERE, f"{name}_sampled.npz")
    np.savez_compressed(out, **arrays)
    log(f"wrote {out}")


if __name__ == "__main__":
    for nm in (sys.argv[1:] or ["mlpdown11008"]):
        main(nm)
