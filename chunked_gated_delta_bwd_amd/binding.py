"""Python binding of the C ABI in include/gdr.h (argument marshalling only).

Every computation runs in the HIP library ``libgdr.so``; this module only
turns torch tensors into pointers and the current torch stream into a
``hipStream_t``.  If the library is missing the import of the entry points
fails loudly: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")
_lib = None

GDR_OK, GDR_EINVAL, GDR_EUNSUPPORTED, GDR_EWORKSPACE, GDR_EHIP = 0, 1, 2, 3, 4
GDR_GATE_SCALAR, GDR_GATE_CHANNEL, GDR_GATE_CHANNEL_SIGMOID = 0, 1, 2
GDR_BF16, GDR_F32 = 0, 1
GDR_WS_STATE, GDR_WS_DSTATE, GDR_WS_U, GDR_WS_A, GDR_WS_GAMMA = 0, 1, 2, 3, 4

GDR_STAGE_PREP, GDR_STAGE_CHAIN_FWD, GDR_STAGE_CHAIN_BWD, GDR_STAGE_CHAIN_BOTH = 0, 1, 2, 3
GDR_STAGE_GRADS, GDR_STAGE_FINISH = 4, 5
STAGE_NAMES = {GDR_STAGE_PREP: "prep", GDR_STAGE_CHAIN_FWD: "chain_fwd", GDR_STAGE_CHAIN_BWD: "chain_bwd",
               GDR_STAGE_CHAIN_BOTH: "chain_both", GDR_STAGE_GRADS: "grads", GDR_STAGE_FINISH: "finish"}

SYMBOLS = ("gdr_workspace_bytes", "gdr_fwd_recompute", "gdr_fwd", "gdr_bwd", "gdr_fwd_bwd",
           "gdr_workspace_region", "gdr_run_stage", "gdr_fwd_bwd_noalloc", "gdr_last_error")
# the device array gdr_fwd_bwd_noalloc uses as its workspace (128 MiB per GPU)
NOALLOC_WORKSPACE_BYTES = 128 << 20


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gdr status {status}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("N", ctypes.c_int32),
                ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int64)),
                ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("gate_scale", ctypes.c_float), ("Hk", ctypes.c_int32), ("seq_split", ctypes.c_int32)]


class Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta_logit", ctypes.c_void_p),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("h0", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("dh0", ctypes.c_void_p),
                ("dA_log", ctypes.c_void_p), ("ddt_bias", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdr.so (built by ``build.build()``); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with chunked_gated_delta_bwd_amd.build.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    lib.gdr_workspace_bytes.argtypes = [P(Shape), P(ctypes.c_size_t)]
    lib.gdr_fwd_recompute.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.gdr_fwd.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p]
    lib.gdr_bwd.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_size_t, P(Grads), ctypes.c_void_p]
    lib.gdr_fwd_bwd.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_size_t, P(Grads), ctypes.c_void_p, ctypes.c_void_p]
    lib.gdr_workspace_region.argtypes = [P(Shape), ctypes.c_int32, P(ctypes.c_size_t), P(ctypes.c_size_t)]
    lib.gdr_run_stage.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_size_t, P(Grads), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.gdr_fwd_bwd_noalloc.argtypes = [P(Shape), P(Inputs), ctypes.c_void_p, ctypes.c_void_p, P(Grads),
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    for name in SYMBOLS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != GDR_OK:
        raise GdrError(status, load_library().gdr_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Problem:
    """Host-side description of one problem: the C shape plus the tensors.

    ``tensors`` holds device tensors q k v g b (and optionally A_log dt_bias h0);
    ``cu_seqlens`` (host int64, or None for dense) is kept alive here because the
    C shape points into it.
    """

    def __init__(self, B: int, T: int, H: int, D: int, N: int, gate: int, dtype: int, scale: float,
                 cu_seqlens=None, gate_scale: float = 0.0, Hk: int = 0, seq_split: int = 0):
        self.cu = None
        if cu_seqlens is not None:
            cu = torch.as_tensor(cu_seqlens, dtype=torch.int64).contiguous().cpu()
            self.cu = cu
        self.shape = Shape(B, T, H, D, D, N,
                           None if self.cu is None else ctypes.cast(self.cu.data_ptr(), ctypes.POINTER(ctypes.c_int64)),
                           gate, dtype, scale, gate_scale, Hk, seq_split)

    @staticmethod
    def from_inputs(inp: Dict, varlen: Optional[bool] = None, seq_split: int = 0) -> "Problem":
        lengths = inp["lengths"]
        if varlen is None:
            varlen = inp["B"] == 1 and (len(lengths) > 1 or lengths[0] != inp["T"])
        dtype = GDR_BF16 if inp["dtype"] == "bf16" else GDR_F32
        gs = float(inp.get("gate_scale", 0.0))
        hk = int(inp.get("Hk") or 0)
        if varlen:
            return Problem(1, inp["T"], inp["H"], inp["K"], inp["N"], inp["gate"], dtype, inp["scale"],
                           cu_seqlens=inp["cu_seqlens"], gate_scale=gs, Hk=hk, seq_split=seq_split)
        return Problem(inp["B"], inp["T"], inp["H"], inp["K"], inp["N"], inp["gate"], dtype, inp["scale"],
                       gate_scale=gs, Hk=hk, seq_split=seq_split)


def gdr_workspace_bytes(prob: Problem) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().gdr_workspace_bytes(ctypes.byref(prob.shape), ctypes.byref(out)))
    return out.value


def gdr_workspace_region(prob: Problem, which: int):
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load_library().gdr_workspace_region(ctypes.byref(prob.shape), which, ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


def _inputs(t: Dict) -> Inputs:
    return Inputs(_ptr(t["q"]), _ptr(t["k"]), _ptr(t["v"]), _ptr(t["g"]), _ptr(t["b"]),
                  _ptr(t.get("A_log")), _ptr(t.get("dt_bias")), _ptr(t.get("h0")))


def _grads(o: Dict) -> Grads:
    return Grads(_ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o["dg"]), _ptr(o["db"]),
                 _ptr(o.get("dh0")), _ptr(o.get("dA_log")), _ptr(o.get("ddt_bias")))


def gdr_fwd_recompute(prob: Problem, t: Dict, ws: torch.Tensor, ht: Optional[torch.Tensor] = None,
                      o: Optional[torch.Tensor] = None, stream=None) -> None:
    inp = _inputs(t)
    _check(load_library().gdr_fwd_recompute(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(ws),
                                            ws.numel() * ws.element_size(), _ptr(o), _ptr(ht), _stream(stream)))


def gdr_fwd(prob: Problem, t: Dict, ws: torch.Tensor, o: torch.Tensor, ht: Optional[torch.Tensor] = None,
            stream=None) -> None:
    inp = _inputs(t)
    _check(load_library().gdr_fwd(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(o), _ptr(ht), _stream(stream)))


def gdr_bwd(prob: Problem, t: Dict, dO: torch.Tensor, dht: Optional[torch.Tensor], ws: torch.Tensor,
            out: Dict, stream=None) -> None:
    inp, gr = _inputs(t), _grads(out)
    _check(load_library().gdr_bwd(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(dO), _ptr(dht), _ptr(ws),
                                  ws.numel() * ws.element_size(), ctypes.byref(gr), _stream(stream)))


def gdr_fwd_bwd(prob: Problem, t: Dict, dO: torch.Tensor, dht: Optional[torch.Tensor], ws: torch.Tensor,
                out: Dict, ht: Optional[torch.Tensor] = None, stream=None) -> None:
    inp, gr = _inputs(t), _grads(out)
    _check(load_library().gdr_fwd_bwd(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(dO), _ptr(dht),
                                      _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(gr), _ptr(ht),
                                      _stream(stream)))


def gdr_fwd_bwd_noalloc(prob: Problem, t: Dict, dO: torch.Tensor, dht: Optional[torch.Tensor], out: Dict,
                        ht: Optional[torch.Tensor] = None, stream=None) -> None:
    inp, gr = _inputs(t), _grads(out)
    _check(load_library().gdr_fwd_bwd_noalloc(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(dO), _ptr(dht),
                                              ctypes.byref(gr), _ptr(ht), _stream(stream)))


def gdr_run_stage(prob: Problem, t: Dict, dO: torch.Tensor, dht: Optional[torch.Tensor], ws: torch.Tensor,
                  out: Dict, stage: int, ht: Optional[torch.Tensor] = None, stream=None) -> None:
    inp, gr = _inputs(t), _grads(out)
    _check(load_library().gdr_run_stage(ctypes.byref(prob.shape), ctypes.byref(inp), _ptr(dO), _ptr(dht),
                                        _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(gr), _ptr(ht),
                                        stage, _stream(stream)))


# ---------------------------------------------------------------------------
# convenience for tests and the benchmark: device copies and output buffers
# ---------------------------------------------------------------------------

def to_device(inp: Dict, device="cuda") -> Dict:
    """Device copies of the generator's tensors (same bytes)."""
    out = {}
    for key in ("q", "k", "v", "g", "b", "dO", "A_log", "dt_bias", "h0", "dht"):
        x = inp.get(key)
        out[key] = None if x is None else x.to(device).contiguous()
    return out


def alloc_outputs(inp: Dict, dev: Dict, want_dh0: bool = True) -> Dict:
    """Output tensors of the right shapes/dtypes on the inputs' device."""
    q, g = dev["q"], dev["g"]
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(dev["k"]), "dv": torch.empty_like(dev["v"]),
           "dg": torch.empty_like(g), "db": torch.empty_like(dev["b"])}
    N, H, K, V = inp["N"], inp["H"], inp["K"], inp["V"]
    out["dh0"] = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device) if want_dh0 else None
    if inp["gate"] != GDR_GATE_SCALAR:
        out["dA_log"] = torch.empty((H,), dtype=torch.float32, device=q.device)
        out["ddt_bias"] = torch.empty((H, K), dtype=torch.float32, device=q.device)
    return out


def alloc_workspace(prob: Problem, device="cuda") -> torch.Tensor:
    n = gdr_workspace_bytes(prob)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
