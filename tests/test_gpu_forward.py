"""GPU parity of the forward output path (gdr_fwd): the output o and the final
state ht from the HIP path through the C ABI against the float64 oracle's forward
(o_t = scale S_t qn_t, token by token) on the same seeded input bytes.  o is stored
in the input dtype and held to the bf16 bar |o - ref| / |ref| <= 2e-2; ht (fp32)
to the bar the backward tests hold it to; the worst (token, head) row within five
times those bars.  Every workload is compared in full (all heads)."""

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_bwd_amd import binding as B
from chunked_gated_delta_bwd_amd import synth
from gpu_common import TOL_BF16, TOL_FP32, compare, gpu_run, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def gpu_fwd(inp, ws=None):
    """o and ht of gdr_fwd (float64 host copies), and the device state for reuse."""
    dev = B.to_device(inp)
    prob = B.Problem.from_inputs(inp)
    ws = B.alloc_workspace(prob) if ws is None else ws
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    # NaN-filled, so that a row the kernel fails to write cannot pass
    o = torch.full((inp["B"], inp["T"], inp["H"], inp["V"]), float("nan"), dtype=dt, device="cuda")
    ht = torch.empty((inp["N"], inp["H"], inp["V"], inp["K"]), dtype=torch.float32, device="cuda")
    B.gdr_fwd(prob, dev, ws, o, ht=ht)
    torch.cuda.synchronize()
    return {"o": o.double().cpu().numpy(), "ht": ht.double().cpu().numpy()}, (dev, prob, ws)


def _check(inp, got, label):
    ref = oracle.run(inp, backward=False)
    assert np.isfinite(got["o"]).all(), f"{label}: output rows left unwritten"
    compare(got, ref, ("o",), TOL_BF16, label + " o")
    compare(got, ref, ("ht",), TOL_FP32 * 5, label + " ht")


SMALL = [
    ("gdn_bf16_varlen_edges_d128",
     synth.Spec("fe", 0, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1, seed=51)),
    ("gdn_f32_b2_t100_d64", synth.Spec("ff", 0, "f32", H=2, K=64, V=64, B=2, T=100, seed=52)),
    ("gdn_bf16_b1_t300_d64_h0", synth.Spec("fg", 0, "bf16", H=4, K=64, V=64, B=1, T=300, h0_std=0.5, seed=53)),
    ("kda_bf16_varlen_edges_d128",
     synth.Spec("fk", 1, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1, seed=54)),
    ("kda_f32_b2_t100_d128", synth.Spec("fl", 1, "f32", H=2, K=128, V=128, B=2, T=100, h0_std=0.2, seed=55)),
    ("kda_bf16_b1_t300_d64", synth.Spec("fm", 1, "bf16", H=4, K=64, V=64, B=1, T=300, seed=56)),
    ("kdas_bf16_varlen_edges_d128",
     synth.Spec("fs", 2, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1, seed=58)),
]


@pytest.mark.parametrize("name,spec", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small_against_oracle(name, spec):
    log(f"case {name}")
    inp = synth.generate(spec)
    got, _ = gpu_fwd(inp)
    _check(inp, got, name)


@pytest.mark.parametrize("wl", ["gdn_bf16_t32768_h16_d128", "gdn_varlen12_bf16_t32768_h32_d128",
                                "kda_bf16_t8192_h16_d128", "kda_bf16_t32768_h16_d128",
                                "gdn_gqa4_bf16_t32768_h32_d128"])
def test_forward_workloads(wl):
    log(f"case {wl}")
    inp = synth.generate(synth.workload(wl))
    got, _ = gpu_fwd(inp)
    _check(inp, got, wl)


@pytest.mark.parametrize("gate", [0, 1])
def test_forward_then_backward_equals_fused(gate):
    # gdr_fwd leaves the workspace gdr_bwd needs: its gradients are the fused call's, bit for bit
    spec = synth.Spec("fb", gate, "bf16", H=2, K=128, V=128, B=1, T=333, h0_std=0.3, dht_std=0.3, seed=57)
    log(f"case fwd+bwd gate {gate}")
    inp = synth.generate(spec)
    _, (dev, prob, ws) = gpu_fwd(inp)
    out = B.alloc_outputs(inp, dev)
    B.gdr_bwd(prob, dev, dev["dO"], dev["dht"], ws, out)
    torch.cuda.synchronize()
    fused = gpu_run(inp, mode="fused")
    for key, x in out.items():
        if x is not None:
            assert np.array_equal(x.double().cpu().numpy(), fused[key]), key


def test_forward_no_tokens():
    """T = 0: o has no storage (a NULL pointer), ht = h0 exactly."""
    inp = synth.generate(synth.Spec("z", 1, "bf16", H=2, K=64, V=64, lengths=[0, 0], h0_std=0.3, seed=92))
    got, _ = gpu_fwd(inp)
    assert got["o"].size == 0
    assert np.array_equal(got["ht"], inp["h0"].double().numpy())


@pytest.mark.parametrize("gate", [0, 1])
def test_fwd_recompute_optional_output(gate):
    """gdr_fwd_recompute with o given writes the same o as gdr_fwd (bit for bit);
    with o NULL it writes the same ht and leaves a workspace from which gdr_bwd
    gives the fused call's gradients."""
    spec = synth.Spec("fo", gate, "bf16", H=2, K=128, V=128, lengths=[190, 64, 7], h0_std=0.3, dht_std=0.3,
                      seed=59)
    log(f"case fwd_recompute o gate {gate}")
    inp = synth.generate(spec)
    ref, (dev, prob, _) = gpu_fwd(inp)
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    for with_o in (True, False):
        ws = B.alloc_workspace(prob)
        o = torch.full((inp["B"], inp["T"], inp["H"], inp["V"]), float("nan"), dtype=dt, device="cuda")
        ht = torch.empty((inp["N"], inp["H"], inp["V"], inp["K"]), dtype=torch.float32, device="cuda")
        B.gdr_fwd_recompute(prob, dev, ws, ht=ht, o=o if with_o else None)
        torch.cuda.synchronize()
        assert np.array_equal(ht.double().cpu().numpy(), ref["ht"])
        if with_o:
            assert np.array_equal(o.double().cpu().numpy(), ref["o"])
        else:
            assert torch.isnan(o.float()).all()   # untouched
        out = B.alloc_outputs(inp, dev)
        B.gdr_bwd(prob, dev, dev["dO"], dev["dht"], ws, out)
        torch.cuda.synchronize()
        fused = gpu_run(inp, mode="fused")
        for key, x in out.items():
            if x is not None:
                assert np.array_equal(x.double().cpu().numpy(), fused[key]), (with_o, key)
