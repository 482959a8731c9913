"""Parity gate between the HIP path's outputs and the oracle (TEST INFRASTRUCTURE).

For each output tensor g (GPU) against r (oracle), with (rtol, atol_rel) =
(1e-4, 1e-4) for fp32 storage and (2e-2, 1e-2) for bf16 storage:

 1. max relative error, normwise:  max|g - r| <= rtol * max|r| + atol_rel * rms(r)
 2. relative Frobenius error:      ||g - r||_2 <= rtol * ||r||_2
 3. elementwise band |g - r| <= atol_rel * rms(r) + rtol * |r| holds for every
    element (fp32) or for at least 97% of the elements (bf16).

The absolute floor is relative to the tensor's RMS so the gate does not depend
on each tensor's unit (a weight gradient summed over thousands of tokens is
~50 per entry, a loss gradient ~1/N per entry); for a unit-RMS tensor it is the
stated 1e-2. The bf16 allowance in (3) exists because outputs formed by
cancellation (the attention backward's dS = P*(dP - delta), weight gradients)
carry the bf16 rounding of their much larger terms: with fp32 storage the
same kernels meet (3) everywhere at 1e-4, and with bf16 the residual error is
0.3-0.6% in Frobenius norm (a few chained bf16 roundings of 2^-9 each).
"""
from __future__ import annotations

import numpy as np

TOLERANCES = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}
BAND_FRACTION = {"f32": 0.0, "bf16": 0.03}


def compare_tensor(got, ref, dtype: str) -> dict:
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if g.shape != r.shape:
        return {"ok": False, "why": f"shape {g.shape} != {r.shape}"}
    rtol, atol_rel = TOLERANCES[dtype]
    if r.size == 0:
        return {"ok": True, "n": 0}
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    tol = atol_rel * rms + rtol * np.abs(r)
    bad = ~(err <= tol)                       # NaN counts as bad
    worst = int(np.argmax(np.where(np.isfinite(err), err / np.maximum(tol, 1e-300), np.inf)))
    max_ref = float(np.abs(r).max())
    max_err = float(np.max(err)) if np.isfinite(err).all() else float("inf")
    fro_err = float(np.linalg.norm(np.nan_to_num(g - r, nan=np.inf)))
    fro_ref = float(np.linalg.norm(r))
    ok_norm = max_err <= rtol * max_ref + atol_rel * rms
    ok_fro = fro_err <= rtol * fro_ref
    ok_band = bad.sum() <= BAND_FRACTION[dtype] * r.size
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


def compare_all(got: dict, ref: dict, dtype: str, keys=None) -> dict:
    keys = sorted(ref) if keys is None else keys
    return {k: compare_tensor(got[k], ref[k], dtype) for k in keys}


def format_report(rep: dict) -> str:
    lines = []
    for k, v in rep.items():
        if "why" in v:
            lines.append(f"{k:16s} FAIL {v['why']}")
            continue
        flags = "".join(c for c, f in zip("NFB", (v["ok_norm"], v["ok_fro"], v["ok_band"])) if not f)
        lines.append(f"{k:16s} {'ok  ' if v['ok'] else 'FAIL'}{flags:3s} band_out={v['n_bad']}/{v['n']} "
                     f"worst_err/tol={v['worst_ratio']:.3g} max_abs={v['max_abs_err']:.3g} "
                     f"max_err/max_ref={v['max_rel_to_max']:.3g} rel_fro={v['rel_fro']:.3g} rms={v['rms_ref']:.3g}")
    return "\n".join(lines)
