"""Seeded synthetic inputs for the gated delta-rule backward.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: the L2 normalisation, the sigmoid
of the beta logit and the KDA gate function are all applied by the code under
test (and, independently, by the float64 oracle), never here.  Both the HIP
path and the oracle consume the exact tensors returned by :func:`generate`.

Recipe (one ``numpy.random.PCG64`` stream per tensor, spawned from one seed in
the fixed order q, k, v, dO, b, g / g_raw, A_log, dt_bias, h0, dht, lengths):

* q, k, v, dO ~ N(0, 1), shape [B, T, H, D] (raw, not normalised); with grouped
  heads q and k have ``Hk`` heads, each shared by H / Hk value heads;
* b (beta logit) ~ N(0, 1), shape [B, T, H];
* scalar gate (GDN): the per-token log decay g = -0.1 * softplus(N(0, 1)),
  shape [B, T, H] -- this is the input distribution itself, the op takes g as
  given;
* per-channel gate (KDA, either gate function): g_raw ~ N(0, 1) [B, T, H, Dk],
  dt_bias ~ N(0, 0.5) [H, Dk], A_log ~ U(0, 1.5) [H]; the bounded sigmoid form
  also takes the fixed ``gate_scale`` of the spec (default -2);
* h0, dht ~ N(0, sigma) fp32, shape [N, H, Dv, Dk] when requested;
* varlen lengths: ``n_seqs`` draws from U[1, max_len], rescaled so that they
  sum to exactly ``total`` (floor, at least 1, remainder to the longest).

Values are generated in float64, rounded to float32, and then to bfloat16
with round-to-nearest-even when the storage dtype is bf16.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

GATE_SCALAR = 0   # GDN: one log decay per token and head
GATE_CHANNEL = 1  # KDA: one log decay per token, head and key channel
GATE_CHANNEL_SIGMOID = 2  # KDA with the bounded sigmoid gate function

_ORDER = ("q", "k", "v", "dO", "b", "g", "A_log", "dt_bias", "h0", "dht", "lengths")


@dataclasses.dataclass
class Spec:
    """Shape and distribution of one synthetic problem."""

    name: str
    gate: int
    dtype: str            # "bf16" or "f32": storage dtype of q, k, v, g, b, dO
    H: int
    K: int
    V: int
    B: int = 1
    T: int = 0            # per-sequence length when dense
    lengths: Optional[List[int]] = None  # varlen: explicit sequence lengths
    varlen_total: int = 0  # varlen: draw lengths summing to this
    varlen_n: int = 0
    varlen_max: int = 0
    h0_std: Optional[float] = None
    dht_std: Optional[float] = None
    seed: int = 0
    scale: Optional[float] = None
    gate_scale: float = -2.0   # bounded sigmoid gate only: the lower bound of the log decay
    Hk: Optional[int] = None   # key heads of q, k (grouped heads); None = H

    @property
    def eff_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.K)


def _softplus64(x: np.ndarray) -> np.ndarray:
    # input distribution of the scalar log decay (not the op's gate function)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def draw_lengths(rng: np.random.Generator, n: int, max_len: int, total: int) -> List[int]:
    """n lengths from U[1, max_len], rescaled to sum exactly to ``total``."""
    raw = rng.integers(1, max_len + 1, size=n).astype(np.float64)
    scaled = np.maximum(1, np.floor(raw * total / raw.sum())).astype(np.int64)
    scaled[int(np.argmax(scaled))] += total - int(scaled.sum())
    out = [int(x) for x in scaled]
    assert sum(out) == total and min(out) >= 1
    return out


def generate(spec: Spec) -> Dict[str, object]:
    """Draw every tensor of ``spec`` on the host.

    Returns a dict with torch CPU tensors ``q k v dO b g`` (storage dtype),
    ``A_log dt_bias h0 dht`` (fp32 or None), ``cu_seqlens`` (int64 [N+1]) and
    the scalars ``B T H K V N gate scale dtype``.  Dense problems are laid out
    [B, T, H, D]; varlen problems are packed as [1, T_total, H, D].
    """
    seeds = np.random.SeedSequence(spec.seed).spawn(len(_ORDER))
    rng = {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(_ORDER, seeds)}

    if spec.lengths is not None or spec.varlen_n:
        if spec.lengths is not None:
            lengths = list(spec.lengths)
        else:
            lengths = draw_lengths(rng["lengths"], spec.varlen_n, spec.varlen_max, spec.varlen_total)
        B, T = 1, int(sum(lengths))
    else:
        B, T = spec.B, spec.T
        lengths = [T] * B
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    H, K, V = spec.H, spec.K, spec.V

    def normal(name, shape, std=1.0):
        return rng[name].standard_normal(size=shape) * std

    out: Dict[str, object] = {}
    Hk = H if spec.Hk is None else spec.Hk
    assert H % Hk == 0, "value heads come in whole groups per key head"
    out["q"] = _round(normal("q", (B, T, Hk, K)), spec.dtype)
    out["k"] = _round(normal("k", (B, T, Hk, K)), spec.dtype)
    out["v"] = _round(normal("v", (B, T, H, V)), spec.dtype)
    out["dO"] = _round(normal("dO", (B, T, H, V)), spec.dtype)
    out["b"] = _round(normal("b", (B, T, H)), spec.dtype)
    if spec.gate == GATE_SCALAR:
        out["g"] = _round(-0.1 * _softplus64(normal("g", (B, T, H))), spec.dtype)
        out["A_log"] = None
        out["dt_bias"] = None
    else:
        out["g"] = _round(normal("g", (B, T, H, K)), spec.dtype)
        out["A_log"] = _round(rng["A_log"].uniform(0.0, 1.5, size=(H,)), "f32")
        out["dt_bias"] = _round(normal("dt_bias", (H, K), 0.5), "f32")
    out["h0"] = None if spec.h0_std is None else _round(normal("h0", (N, H, V, K), spec.h0_std), "f32")
    out["dht"] = None if spec.dht_std is None else _round(normal("dht", (N, H, V, K), spec.dht_std), "f32")
    out["cu_seqlens"] = torch.from_numpy(cu)
    out["gate_scale"] = spec.gate_scale if spec.gate == GATE_CHANNEL_SIGMOID else 0.0
    out.update(B=B, T=T, H=H, Hk=Hk, K=K, V=V, N=N, gate=spec.gate, scale=spec.eff_scale,
               dtype=spec.dtype, lengths=lengths, name=spec.name)
    return out


# ---------------------------------------------------------------------------
# Named workloads.  The seed of a named workload is 1000 + its index.
# ---------------------------------------------------------------------------

def workload(name: str) -> Spec:
    """The five evaluation workloads (and the headline variants of the last)."""
    if name == "gdn_f32_t128_h2_d64":
        return Spec(name, GATE_SCALAR, "f32", H=2, K=64, V=64, B=1, T=128, seed=1000, scale=1.0 / 8)
    if name == "gdn_bf16_b2_t4096_h16_d128":
        return Spec(name, GATE_SCALAR, "bf16", H=16, K=128, V=128, B=2, T=4096, h0_std=0.1, seed=1001)
    if name == "kda_bf16_t8192_h16_d128":
        return Spec(name, GATE_CHANNEL, "bf16", H=16, K=128, V=128, B=1, T=8192, seed=1002)
    if name == "gdn_gqa4_bf16_t32768_h32_d128":   # grouped heads: 8 key heads, 4 value heads each
        return Spec(name, GATE_SCALAR, "bf16", H=32, Hk=8, K=128, V=128, B=1, T=32768, h0_std=0.1,
                    dht_std=0.1, seed=1005)
    if name == "kdas_bf16_t8192_h16_d128":   # the bounded sigmoid gate on the same inputs
        return Spec(name, GATE_CHANNEL_SIGMOID, "bf16", H=16, K=128, V=128, B=1, T=8192, seed=1002)
    if name == "gdn_varlen12_bf16_t32768_h32_d128":
        return Spec(name, GATE_SCALAR, "bf16", H=32, K=128, V=128, varlen_n=12, varlen_max=8192,
                    varlen_total=32768, h0_std=0.1, dht_std=0.1, seed=1003)
    # H = 2 and 4: one GPU's share of the H = 16 and H = 32 problems under 8-way head sharding
    for gate_name, gate in (("gdn", GATE_SCALAR), ("kda", GATE_CHANNEL), ("kdas", GATE_CHANNEL_SIGMOID)):
        for H in (2, 4, 16, 32):
            if name == f"{gate_name}_bf16_t32768_h{H}_d128":
                return Spec(name, gate, "bf16", H=H, K=128, V=128, B=1, T=32768,
                            h0_std=0.1, dht_std=0.1, seed=1004)
    raise KeyError(name)


WORKLOADS = (
    "gdn_f32_t128_h2_d64",
    "gdn_bf16_b2_t4096_h16_d128",
    "kda_bf16_t8192_h16_d128",
    "gdn_varlen12_bf16_t32768_h32_d128",
    "gdn_bf16_t32768_h16_d128",
    "gdn_bf16_t32768_h32_d128",
    "kda_bf16_t32768_h16_d128",
    "kda_bf16_t32768_h32_d128",
    "kdas_bf16_t8192_h16_d128",
    "kdas_bf16_t32768_h16_d128",
    "gdn_gqa4_bf16_t32768_h32_d128",
    "gdn_bf16_t32768_h2_d128",
    "gdn_bf16_t32768_h4_d128",
    "kda_bf16_t32768_h2_d128",
)

HEADLINE = "gdn_bf16_t32768_h16_d128"
