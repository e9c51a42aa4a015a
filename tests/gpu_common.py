"""Shared helpers for the GPU tests: run the HIP path through the C ABI and
compare with the float64 oracle on the same input bytes."""

from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

from chunked_gated_delta_bwd_amd import binding as B

# Tolerances (normalised error |X - ref|_F / |ref|_F, float64): per-token
# gradients in bf16 storage, and the fp32 state-gradient / parameter outputs.
TOL_BF16 = 2e-2
TOL_FP32 = 1e-3
TOKEN_GRADS = ("dq", "dk", "dv", "dg", "db")
FP32_GRADS = ("dh0", "dA_log", "ddt_bias")


def nerr(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


# A per-row check beside the per-tensor one: a fault confined to a few rows (one
# tail chunk of one sequence in a 32k-token pack) is diluted below the per-tensor
# bar, but not below this one.  A row is one (token, head) vector of a token
# tensor, one per-token scalar, one state row (sequence, head, v) of dh0 / ht, or
# one head of the parameter gradients; its error is |row - ref_row| divided by
# the larger of |ref_row| and the root-mean-square row norm of ref (so that rows
# with a near-zero reference are held in absolute terms).
ROW_FACTOR = 5.0


def _rows(a: np.ndarray, key: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    if a.ndim <= 1 or (a.ndim == 3 and key in ("dg", "db")):
        return a.reshape(-1, 1)
    return a.reshape(-1, a.shape[-1])


def row_err(x: np.ndarray, ref: np.ndarray, key: str) -> float:
    xr, rr = _rows(x, key), _rows(ref, key)
    if rr.size == 0:
        return 0.0
    dn = np.linalg.norm(xr - rr, axis=1)
    rn = np.linalg.norm(rr, axis=1)
    rms = float(np.sqrt(np.mean(rn * rn)))
    if rms == 0.0:
        return float(dn.max())
    return float((dn / np.maximum(rn, rms)).max())


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(inp: Dict, mode: str = "fused", exports: bool = False, seq_split: int = 0) -> Dict[str, np.ndarray]:
    """Runs the backward on cuda:0 through the C ABI; float64 host copies.
    seq_split: segments per sequence for the recursions (0: the library's choice,
    1: never split)."""
    dev = B.to_device(inp)
    prob = B.Problem.from_inputs(inp, seq_split=seq_split)
    ws = B.alloc_workspace(prob)
    out = B.alloc_outputs(inp, dev)
    N, H, K, V = inp["N"], inp["H"], inp["K"], inp["V"]
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
    if mode == "fused":
        B.gdr_fwd_bwd(prob, dev, dev["dO"], dev["dht"], ws, out, ht=ht)
    elif mode == "split":
        B.gdr_fwd_recompute(prob, dev, ws, ht=ht)
        B.gdr_bwd(prob, dev, dev["dO"], dev["dht"], ws, out)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize()
    res = {k: v.double().cpu().numpy() for k, v in out.items() if v is not None}
    res["ht"] = ht.double().cpu().numpy()
    if exports:
        NC = sum((L + 63) // 64 for L in inp["lengths"])
        for name, which, shape in (("S_chunk", B.GDR_WS_STATE, (H, NC, V, K)),
                                   ("dS_chunk", B.GDR_WS_DSTATE, (H, NC, V, K))):
            off, n = B.gdr_workspace_region(prob, which)
            res[name] = ws[off:off + n].view(torch.bfloat16).view(shape).double().cpu().numpy()
    return res


def compare(got: Dict, ref: Dict, keys, tol: float, label: str, row_tol: Optional[float] = None) -> Dict:
    """Normalised error per output (|X - ref|_F / |ref|_F <= tol) and the worst
    row error (<= row_tol, default ROW_FACTOR * tol), over every head."""
    row_tol = ROW_FACTOR * tol if row_tol is None else row_tol
    errs, rows = {}, {}
    for key in keys:
        if key not in ref:
            continue
        x = got[key]
        assert np.shape(x) == np.shape(ref[key]), (label, key, np.shape(x), np.shape(ref[key]))
        errs[key] = nerr(x, ref[key])
        rows[key] = row_err(x, ref[key], key)
    log(f"[{label}] " + " ".join(f"{k}={v:.2e}/row {rows[k]:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad} above {tol}"
    bad_rows = {k: v for k, v in rows.items() if not v <= row_tol}
    assert not bad_rows, f"{label}: worst row errors {bad_rows} above {row_tol}"
    return errs
