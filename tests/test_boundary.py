"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol declared in include/gdr.h, sizes workspaces, and rejects bad arguments
before anything is enqueued (every case here fails validation, so no HIP call
is made).  If libgdr.so has not been built yet, it is built here (hipcc
cross-compiles for gfx950 without a GPU); a failed build fails these tests."""

import ctypes
import os
import re

import pytest
import torch

from chunked_gated_delta_bwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))



@pytest.fixture(scope="module", autouse=True)
def _library():
    if not os.path.exists(B.library_path()):
        from chunked_gated_delta_bwd_amd import build
        build.build()
    B.load_library()


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    return sorted(set(re.findall(r"^\s*(?:gdr_status|const char\*)\s+(gdr_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert _declared_symbols() == sorted(B.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.library_path())
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def _prob(**kw):
    args = dict(B=1, T=128, H=2, D=64, N=1, gate=0, dtype=0, scale=0.125, cu_seqlens=None)
    args.update(kw)
    return B.Problem(**args)


def test_workspace_bytes_scales_with_chunks():
    a = B.gdr_workspace_bytes(_prob(T=64))
    b = B.gdr_workspace_bytes(_prob(T=128))
    c = B.gdr_workspace_bytes(_prob(T=65))
    assert 0 < a < b and c == b  # 65 tokens need two chunks, like 128
    # lengths 1, 64, 65 need 1 + 1 + 2 chunks; 64, 64, 64 need 3
    v4 = B.gdr_workspace_bytes(_prob(B=1, T=130, N=3, cu_seqlens=[0, 1, 65, 130]))
    v3 = B.gdr_workspace_bytes(_prob(B=1, T=192, N=3, cu_seqlens=[0, 64, 128, 192]))
    assert v4 > v3


def test_sigmoid_gate_uses_the_per_channel_workspace():
    sig = B.gdr_workspace_bytes(_prob(gate=2, gate_scale=-1.0, D=128))
    assert sig == B.gdr_workspace_bytes(_prob(gate=1, D=128))


def test_grouped_heads_workspace_holds_per_value_head_dq_dk():
    full = B.gdr_workspace_bytes(_prob(H=4, D=64, T=128))
    assert B.gdr_workspace_bytes(_prob(H=4, Hk=4, D=64, T=128)) == full   # Hk == H: not grouped
    grouped = B.gdr_workspace_bytes(_prob(H=4, Hk=2, D=64, T=128))
    assert grouped >= full + 2 * 128 * 4 * 64 * 2                          # bf16 dq, dk per value head
    f32 = B.gdr_workspace_bytes(_prob(H=4, Hk=2, D=64, T=128, dtype=1))
    assert f32 - B.gdr_workspace_bytes(_prob(H=4, D=64, T=128, dtype=1)) >= 2 * 128 * 4 * 64 * 4


def test_workspace_regions_are_disjoint_and_inside():
    p = _prob(T=200, D=128, gate=1)
    total = B.gdr_workspace_bytes(p)
    spans = sorted(B.gdr_workspace_region(p, w) for w in range(5))
    for (o1, n1), (o2, _) in zip(spans, spans[1:]):
        assert o1 + n1 <= o2
    assert spans[-1][0] + spans[-1][1] <= total
    with pytest.raises(B.GdrError) as e:
        B.gdr_workspace_region(p, 99)
    assert e.value.status == B.GDR_EINVAL


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), B.GDR_EUNSUPPORTED),
    (dict(gate=7), B.GDR_EINVAL),
    (dict(dtype=5), B.GDR_EINVAL),
    (dict(N=2), B.GDR_EINVAL),                                  # dense needs N == B
    (dict(B=2, N=2, cu_seqlens=[0, 64, 128]), B.GDR_EINVAL),   # varlen needs B == 1
    (dict(N=2, cu_seqlens=[0, 100, 90]), B.GDR_EINVAL),        # decreasing
    (dict(N=2, cu_seqlens=[0, 50, 100]), B.GDR_EINVAL),        # last != T (128)
    (dict(N=1, cu_seqlens=[5, 128]), B.GDR_EINVAL),            # first != 0
    (dict(gate=2, gate_scale=0.5), B.GDR_EINVAL),               # the bound of a log decay is <= 0
    (dict(gate=2, gate_scale=float("nan")), B.GDR_EINVAL),
    (dict(gate=2, gate_scale=float("-inf")), B.GDR_EINVAL),
    (dict(H=4, Hk=3), B.GDR_EINVAL),                            # key heads must divide value heads
    (dict(H=2, Hk=4), B.GDR_EINVAL),
    (dict(Hk=-1), B.GDR_EINVAL),
])
def test_shape_validation(kw, status):
    with pytest.raises(B.GdrError) as e:
        B.gdr_workspace_bytes(_prob(**kw))
    assert e.value.status == status
    assert B.load_library().gdr_last_error().decode()


class _Fake:
    """Stands in for a device tensor: only its address is used by validation."""

    def __init__(self, addr, n=1 << 20):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _tensors(gate=0, **override):
    t = {k: _Fake(0x10000 * (i + 1)) for i, k in enumerate(("q", "k", "v", "g", "b"))}
    if gate:
        t["A_log"], t["dt_bias"] = _Fake(0x900000), _Fake(0xa00000)
    t.update(override)
    return t


def _outs(gate=0, **override):
    o = {k: _Fake(0x1000000 * (i + 1)) for i, k in enumerate(("dq", "dk", "dv", "dg", "db"))}
    if gate:
        o["dA_log"], o["ddt_bias"] = _Fake(0x8000000), _Fake(0x9000000)
    o.update(override)
    return o


@pytest.mark.parametrize("case,status", [
    ("null_q", B.GDR_EINVAL),
    ("misaligned_k", B.GDR_EINVAL),
    ("gdn_with_A_log", B.GDR_EINVAL),
    ("kda_without_dt_bias", B.GDR_EINVAL),
    ("small_workspace", B.GDR_EWORKSPACE),
    ("misaligned_workspace", B.GDR_EINVAL),
])
def test_fwd_recompute_rejects(case, status):
    gate = 1 if case.startswith("kda") else 0
    p = _prob(gate=gate)
    need = B.gdr_workspace_bytes(p)
    ws = _Fake(0x40000000, need)
    t = _tensors(gate)
    if case == "null_q":
        t["q"] = None
    elif case == "misaligned_k":
        t["k"] = _Fake(0x10008)
    elif case == "gdn_with_A_log":
        t["A_log"] = _Fake(0x900000)
    elif case == "kda_without_dt_bias":
        t["dt_bias"] = None
    elif case == "small_workspace":
        ws = _Fake(0x40000000, need - 1)
    elif case == "misaligned_workspace":
        ws = _Fake(0x40000010, need)
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd_recompute(p, t, ws, stream=0)
    assert e.value.status == status
    # the same with the optional output o given: the same status
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd_recompute(p, t, ws, o=_Fake(0x30000000), stream=0)
    assert e.value.status == status


def test_fwd_recompute_checks_the_optional_output():
    """o is optional in gdr_fwd_recompute: NULL passes its check (the call then
    fails on the next bad argument, not on o), a misaligned o is rejected."""
    p = _prob(gate=0)
    ws = _Fake(0x40000000, B.gdr_workspace_bytes(p))
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd_recompute(p, _tensors(0), ws, o=_Fake(0x30000008), stream=0)
    assert e.value.status == B.GDR_EINVAL and "o is not 16-byte aligned" in str(e.value)
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd_recompute(p, _tensors(0, q=None), ws, o=None, stream=0)
    assert e.value.status == B.GDR_EINVAL and "input q" in str(e.value)


@pytest.mark.parametrize("case", ["null_dO", "null_dg", "kda_missing_dA_log", "gdn_with_ddt_bias",
                                  "misaligned_dh0"])
def test_bwd_rejects(case):
    gate = 1 if case.startswith("kda") else 0
    p = _prob(gate=gate)
    ws = _Fake(0x40000000, B.gdr_workspace_bytes(p))
    dO = _Fake(0x20000000)
    o = _outs(gate)
    if case == "null_dO":
        dO = None
    elif case == "null_dg":
        o["dg"] = None
    elif case == "kda_missing_dA_log":
        o["dA_log"] = None
    elif case == "gdn_with_ddt_bias":
        o["ddt_bias"] = _Fake(0x9000000)
    elif case == "misaligned_dh0":
        o["dh0"] = _Fake(0x9000004)
    for fn in (B.gdr_bwd, B.gdr_fwd_bwd):
        with pytest.raises(B.GdrError) as e:
            fn(p, _tensors(gate), dO, None, ws, o, stream=0)
        assert e.value.status == B.GDR_EINVAL


@pytest.mark.parametrize("case", ["null_o", "misaligned_o", "misaligned_ht", "null_q", "small_workspace"])
def test_fwd_rejects(case):
    p = _prob(gate=0)
    need = B.gdr_workspace_bytes(p)
    ws = _Fake(0x40000000, need)
    t = _tensors(0)
    o, ht = _Fake(0x30000000), None
    if case == "null_o":
        o = None
    elif case == "misaligned_o":
        o = _Fake(0x30000008)
    elif case == "misaligned_ht":
        ht = _Fake(0x50000004)
    elif case == "null_q":
        t["q"] = None
    elif case == "small_workspace":
        ws = _Fake(0x40000000, need - 1)
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd(p, t, ws, o, ht=ht, stream=0)
    assert e.value.status == (B.GDR_EWORKSPACE if case == "small_workspace" else B.GDR_EINVAL)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.load_library()
    assert torch is not None


def test_sequence_split_workspace_and_validation():
    """A split adds the boundary-state buffers (2 roles x segments x H x (2D + D) x D
    fp32); the library's own choice splits a long sequence with few heads and
    leaves the full-width shapes alone; a negative seq_split is rejected."""
    long_few = dict(B=1, T=32768, H=2, D=128, N=1)
    plain = B.gdr_workspace_bytes(_prob(seq_split=1, **long_few))
    auto = B.gdr_workspace_bytes(_prob(seq_split=0, **long_few))
    forced = B.gdr_workspace_bytes(_prob(seq_split=4, **long_few))
    seg_bytes = 2 * 2 * 3 * 128 * 128 * 4      # per segment: 2 roles, H = 2, (2D + D) x D fp32
    assert forced - plain >= 4 * seg_bytes
    assert auto > plain                          # split by the library's choice
    wide = dict(B=1, T=32768, H=16, D=128, N=1)
    assert B.gdr_workspace_bytes(_prob(seq_split=0, **wide)) == B.gdr_workspace_bytes(_prob(seq_split=1, **wide))
    # a one-chunk sequence is never split
    one = dict(B=1, T=64, H=2, D=64, N=1)
    assert B.gdr_workspace_bytes(_prob(seq_split=8, **one)) == B.gdr_workspace_bytes(_prob(seq_split=1, **one))
    with pytest.raises(B.GdrError) as e:
        B.gdr_workspace_bytes(_prob(seq_split=-1))
    assert e.value.status == B.GDR_EINVAL


def _ws_split(H, seq_split, gate=0):
    prob = B.Problem(B=1, T=32768, H=H, D=128, N=1, gate=gate, dtype=0, scale=128 ** -0.5, cu_seqlens=None,
                     seq_split=seq_split)
    return B.gdr_workspace_bytes(prob)


@pytest.mark.parametrize("H,gate,segments", [(2, 0, 8), (4, 0, 8), (2, 1, 8), (8, 0, 1), (16, 0, 1)])
def test_automatic_sequence_split_choice(H, gate, segments):
    """The workspace holds the split's segment-end rows per segment, so its size
    shows the segment count the library chose.  At T = 32768, D = 128 the
    planner's time model (fitted to timings of 2 .. 16 segments) picks 8
    segments for 2 and 4 heads and no split once the unsplit recursions give
    every compute unit a workgroup (8 heads and more)."""
    auto = _ws_split(H, 0, gate)
    assert auto == _ws_split(H, segments, gate)
    for other in (1, 4, 16):
        if other != segments:
            assert auto != _ws_split(H, other, gate), other
