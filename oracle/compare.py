"""Parity gate between the HIP path's outputs and the oracle (TEST INFRASTRUCTURE).

For each output tensor g (GPU) against r (oracle), with (rtol, atol) =
(1e-4, 1e-4) for fp32 storage and (2e-2, 1e-2) for bf16 storage (the stated
"max relative error <= 1e-4 for fp32, <= 2e-2 with atol 1e-2 for bf16"), and
u the storage format's unit roundoff (2^-24 fp32, 2^-8 bf16):

 1. max relative error, normwise:  max|g - r| <= rtol * max|r| + a
 2. relative Frobenius error:      ||g - r||_2 <= rtol * ||r||_2
 3. elementwise band, EVERY element (no out-of-band allowance):
        |g - r| <= a + rtol * |r| + u * M
    where M >= |r| is the magnitude of the terms that form the element,
    computed by the oracle (oracle.magnitude): ||a_i|| ||b_j|| for a product
    (what a relative change u of its operand vectors can move it by), the
    sum of the summands' magnitudes for the all-reduce sums, column sums and
    the LayerNorm backward. The pages' mixed precision (overview page,
    section 2) stores the layer's intermediates in 16 bits, so an element
    whose terms cancel carries their rounding, not its own. Without M
    (mags=None) the third term is 0.

The absolute floor is a = atol * min(1, rms(r)): the stated atol for a
tensor of unit scale or larger, and proportionally less for a tensor whose
entries are small (a loss gradient is ~1/N per entry, an attention partial
~0.03), where a fixed 1e-2 would admit any error. It is never looser than
the stated atol.

The vocabulary shard's row statistics (m, se, tl) are compared as
(m, m + ln se, tl): the pair (m, se) only fixes the shard's log-sum-exp
m + ln se, and se moves by the factor exp(m' - m) when the row maximum is
taken over rounded logits; m itself, the log-sum-exp and the target logit
are each compared (each column with its own RMS).
"""
from __future__ import annotations

import numpy as np

TOLERANCES = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8}


def abs_floor(ref, dtype: str) -> float:
    """Absolute floor a = atol * min(1, rms(r)) of gates 1 and 3."""
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return TOLERANCES[dtype][1] * min(1.0, rms)


def tolerance(ref, dtype: str, mag=None):
    """Elementwise tolerance a + rtol * |r| + u * M of gate 3."""
    r = np.asarray(ref, np.float64)
    rtol = TOLERANCES[dtype][0]
    tol = abs_floor(r, dtype) + rtol * np.abs(r)
    if mag is not None:
        tol = tol + UNIT_ROUNDOFF[dtype] * np.asarray(mag, np.float64)
    return tol


def compare_tensor(got, ref, dtype: str, mag=None) -> dict:
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if g.shape != r.shape:
        return {"ok": False, "why": f"shape {g.shape} != {r.shape}"}
    rtol = TOLERANCES[dtype][0]
    if r.size == 0:
        return {"ok": True, "n": 0}
    m = np.zeros_like(r) if mag is None else np.asarray(mag, np.float64)
    if m.shape != r.shape:
        return {"ok": False, "why": f"magnitude shape {m.shape} != {r.shape}"}
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    tol = tolerance(r, dtype, m)
    bad = ~(err <= tol)                       # NaN counts as bad
    worst = int(np.argmax(np.where(np.isfinite(err), err / np.maximum(tol, 1e-300), np.inf)))
    max_ref = float(np.abs(r).max())
    max_err = float(np.max(err)) if np.isfinite(err).all() else float("inf")
    fro_err = float(np.linalg.norm(np.nan_to_num(g - r, nan=np.inf)))
    fro_ref = float(np.linalg.norm(r))
    ok_norm = max_err <= rtol * max_ref + abs_floor(r, dtype)
    ok_fro = fro_err <= rtol * fro_ref
    ok_band = not bad.any()
    return {
        "ok": bool(ok_norm and ok_fro and ok_band),
        "ok_norm": bool(ok_norm), "ok_fro": bool(ok_fro), "ok_band": bool(ok_band),
        "n_bad": int(bad.sum()),
        "n": int(r.size),
        "worst_ratio": float(err.flat[worst] / max(tol.flat[worst], 1e-300)),
        "worst_index": np.unravel_index(worst, r.shape),
        "max_abs_err": max_err,
        "max_rel_to_max": max_err / max(max_ref, 1e-300),
        "rel_fro": fro_err / max(fro_ref, 1e-300),
        "rms_ref": rms,
    }


def product_bound(ref, mag, k: int, out_dtype: str):
    """Rounding-error bound of one dense product C = A B (+ bias) over k terms
    from storage-exact operands: fp32 accumulation (every product of bf16
    operands is exact in fp32; fp32 operands add one rounding per product)
    moves C by at most gamma * M with M = |A| |B| (+ |bias|) and
    gamma = (k + 1) * 2^-23 (twice the round-to-nearest constant of Higham,
    Accuracy and Stability of Numerical Algorithms, eq. 3.5, so any fp32
    summation order and rounding of the accumulator is covered), and storing
    C in out_dtype adds u_out * |C|."""
    u_out = UNIT_ROUNDOFF[out_dtype]
    gamma = (k + 1) * 2.0 ** -23
    return u_out * np.abs(np.asarray(ref, np.float64)) + (1 + u_out) * gamma * np.asarray(mag, np.float64)


def stats_columns(stats) -> dict:
    """(m, se, tl) rows -> the compared columns (m, m + ln se, tl)."""
    s = np.asarray(stats, np.float64)
    return {"max": s[:, 0], "lse": s[:, 0] + np.log(s[:, 1]), "tl": s[:, 2]}


def compare_all(got: dict, ref: dict, dtype: str, mags: dict | None = None, keys=None) -> dict:
    keys = sorted(ref) if keys is None else keys
    rep = {}
    for k in keys:
        mag = None if mags is None else mags.get(k)
        if k.startswith("stats@"):
            gc, rc = stats_columns(got[k]), stats_columns(ref[k])
            for j, c in enumerate(("max", "lse", "tl")):
                rep[f"{k}.{c}"] = compare_tensor(gc[c], rc[c], dtype, None if mag is None else mag[:, j])
        else:
            rep[k] = compare_tensor(got[k], ref[k], dtype, mag)
    return rep


def format_report(rep: dict) -> str:
    lines = []
    for k, v in rep.items():
        if "why" in v:
            lines.append(f"{k:16s} FAIL {v['why']}")
            continue
        if v.get("n", 0) == 0:
            lines.append(f"{k:16s} ok   (empty)")
            continue
        flags = "".join(c for c, f in zip("NFB", (v["ok_norm"], v["ok_fro"], v["ok_band"])) if not f)
        lines.append(f"{k:16s} {'ok  ' if v['ok'] else 'FAIL'}{flags:3s} band_out={v['n_bad']}/{v['n']} "
                     f"worst_err/tol={v['worst_ratio']:.3g} max_abs={v['max_abs_err']:.3g} "
                     f"max_err/max_ref={v['max_rel_to_max']:.3g} rel_fro={v['rel_fro']:.3g} rms={v['rms_ref']:.3g}")
    return "\n".join(lines)
