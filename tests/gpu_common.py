"""Shared helpers for the GPU tests: run the HIP path through the C ABI and
compare with the float64 oracle on the same input bytes."""

from __future__ import annotations

import sys
from typing import Dict, Iterable, Optional

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


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(inp: Dict, mode: str = "fused", exports: bool = False) -> Dict[str, np.ndarray]:
    """Runs the backward on cuda:0 through the C ABI; float64 host copies."""
    dev = B.to_device(inp)
    prob = B.Problem.from_inputs(inp)
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


def key_heads(inp: Dict, heads: Iterable[int]) -> list:
    """The q, k heads that value heads `heads` read (grouped heads: h // (H / Hk))."""
    G = inp["H"] // (inp.get("Hk") or inp["H"])
    return sorted({h // G for h in heads})


def subset_heads(inp: Dict, heads: Iterable[int]) -> Dict:
    """The same problem restricted to some heads (heads never interact; with
    grouped heads the value heads must form whole groups, since dq and dk sum
    over a group)."""
    heads = list(heads)
    G = inp["H"] // (inp.get("Hk") or inp["H"])
    kh = key_heads(inp, heads)
    assert sorted(heads) == heads and heads == [j * G + i for j in kh for i in range(G)], "whole groups"
    idx = torch.tensor(heads, dtype=torch.long)
    kidx = torch.tensor(kh, dtype=torch.long)
    out = dict(inp)
    for key in ("q", "k"):
        out[key] = inp[key].index_select(2, kidx).contiguous()
    for key in ("v", "dO", "g", "b"):
        out[key] = inp[key].index_select(2, idx).contiguous()
    for key in ("h0", "dht"):
        if inp.get(key) is not None:
            out[key] = inp[key].index_select(1, idx).contiguous()
    for key in ("A_log", "dt_bias"):
        if inp.get(key) is not None:
            out[key] = inp[key].index_select(0, idx).contiguous()
    out["H"] = len(heads)
    out["Hk"] = len(kh)
    return out


def compare(got: Dict, ref: Dict, keys, tol: float, label: str, head_index: Optional[list] = None,
            key_index: Optional[list] = None) -> Dict:
    """Normalised error per output; `head_index` picks the value heads the oracle
    ran, `key_index` the q, k heads (dq, dk) where they differ."""
    errs = {}
    for key in keys:
        if key not in ref:
            continue
        x = got[key]
        if head_index is not None:
            axis = 0 if key in ("dA_log", "ddt_bias") else (1 if key in ("dh0", "ht") else 2)
            idx = key_index if key in ("dq", "dk") and key_index is not None else head_index
            x = np.take(x, idx, axis=axis)
        errs[key] = nerr(x, ref[key])
    log(f"[{label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad} above {tol}"
    return errs
