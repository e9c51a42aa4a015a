"""Float64 CPU oracle for the gated delta-rule forward and backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path; both only consume the tensors drawn by the seeded generator.

* :func:`run` wraps ``gdr_oracle.c`` (token-by-token recurrence plus the
  hand-derived reverse-time adjoint, see the header of that file).
* ``oracle.chunked`` is an independent float64 rendering of the chunked
  (UT/WY) re-association in numpy; the tests use each of the two to pin the
  other.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


class _Args(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("gate", ctypes.c_int32), ("chunk", ctypes.c_int32), ("nthreads", ctypes.c_int32),
        ("do_backward", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("cu", ctypes.POINTER(ctypes.c_int64)),
        ("q", _D), ("k", _D), ("v", _D), ("dO", _D), ("b", _D), ("g", _D),
        ("A_log", _D), ("dt_bias", _D), ("h0", _D), ("dht", _D),
        ("o", _D), ("ht", _D), ("dq", _D), ("dk", _D), ("dv", _D), ("dg", _D), ("db", _D),
        ("dh0", _D), ("dA_log", _D), ("ddt_bias", _D),
        ("S_chunk", _D), ("dS_chunk", _D), ("u_out", _D), ("dqn", _D), ("dkn", _D),
        ("dbeta", _D), ("dlam", _D),
        ("gate_scale", ctypes.c_double),
        ("Hk", ctypes.c_int32),
    ]


def build() -> str:
    """Compile the oracle with gcc (plain C99, -O2, no fast-math)."""
    cmd = ["gcc", "-std=c99", "-O2", "-shared", "-fPIC", "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_run.argtypes = [ctypes.POINTER(_Args)]
        lib.oracle_run.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (any dtype) -> exact float64 values
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data_as(_D)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def run(inp: Dict, backward: bool = True, exports: bool = False, chunk: int = 64,
        nthreads: Optional[int] = None, dO=None, dht="input", b=None) -> Dict[str, np.ndarray]:
    """Run the oracle on the tensors of ``inp`` (as drawn by the generator).

    ``dO``/``dht``/``b`` override the corresponding entries of ``inp`` (use
    ``dht=None`` for a zero terminal gradient).  Returns float64 arrays shaped
    like the GPU tensors: token tensors [B, T, H, ...], states [N, H, V, K].
    """
    lib = _load()
    B, T, H, K, V, N = (int(inp[s]) for s in ("B", "T", "H", "K", "V", "N"))
    gate = int(inp["gate"])
    TT = B * T
    cu = np.ascontiguousarray(np.asarray(inp["cu_seqlens"], dtype=np.int64))
    assert cu.shape == (N + 1,) and int(cu[-1]) == TT
    q, k, v = _f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"])
    bb = _f64(inp["b"] if b is None else b)
    g = _f64(inp["g"])
    dOa = _f64(inp["dO"] if dO is None else dO)
    A_log, dt_bias = _f64(inp.get("A_log")), _f64(inp.get("dt_bias"))
    h0 = _f64(inp.get("h0"))
    dhta = _f64(inp.get("dht")) if isinstance(dht, str) and dht == "input" else _f64(dht)
    NC = int(sum((int(cu[n + 1] - cu[n]) + chunk - 1) // chunk for n in range(N)))
    gK = (K,) if gate >= 1 else ()

    out: Dict[str, np.ndarray] = {}

    def alloc(name, shape):
        arr = np.zeros(shape, dtype=np.float64)
        out[name] = arr
        return arr

    a = _Args()
    a.N, a.H, a.K, a.V, a.gate, a.chunk = N, H, K, V, gate, chunk
    a.nthreads = nthreads if nthreads is not None else default_threads()
    a.gate_scale = float(inp.get("gate_scale", 0.0))
    Hk = int(inp.get("Hk", H))
    a.Hk = Hk
    a.do_backward = 1 if backward else 0
    a.scale = float(inp["scale"])
    a.cu = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    keep = [q, k, v, bb, g, dOa, A_log, dt_bias, h0, dhta, cu]
    a.q, a.k, a.v, a.b, a.g = _ptr(q), _ptr(k), _ptr(v), _ptr(bb), _ptr(g)
    a.dO = _ptr(dOa)
    a.A_log, a.dt_bias, a.h0, a.dht = _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(dhta)
    a.o = _ptr(alloc("o", (B, T, H, V)))
    a.ht = _ptr(alloc("ht", (N, H, V, K)))
    if backward:
        a.dq = _ptr(alloc("dq", (B, T, Hk, K)))
        a.dk = _ptr(alloc("dk", (B, T, Hk, K)))
        a.dv = _ptr(alloc("dv", (B, T, H, V)))
        a.dg = _ptr(alloc("dg", (B, T, H) + gK))
        a.db = _ptr(alloc("db", (B, T, H)))
        a.dh0 = _ptr(alloc("dh0", (N, H, V, K)))
        if gate >= 1:
            a.dA_log = _ptr(alloc("dA_log", (H,)))
            a.ddt_bias = _ptr(alloc("ddt_bias", (H, K)))
    if exports:
        a.S_chunk = _ptr(alloc("S_chunk", (H, NC, V, K)))
        a.u_out = _ptr(alloc("u", (B, T, H, V)))
        if backward:
            a.dS_chunk = _ptr(alloc("dS_chunk", (H, NC, V, K)))
            a.dqn = _ptr(alloc("dqn", (B, T, H, K)))
            a.dkn = _ptr(alloc("dkn", (B, T, H, K)))
            a.dbeta = _ptr(alloc("dbeta", (B, T, H)))
            a.dlam = _ptr(alloc("dlam", (B, T, H) + gK))
    rc = lib.oracle_run(ctypes.byref(a))
    del keep
    if rc != 0:
        raise RuntimeError(f"oracle_run failed with code {rc}")
    return out
