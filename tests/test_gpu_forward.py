"""GPU parity of the forward output path (gdr_fwd): the output o and the final
state ht from the HIP path through the C ABI against the float64 oracle's forward
(o_t = scale S_t qn_t, token by token) on the same seeded input bytes.  o is stored
in the input dtype and held to the bf16 bar |o - ref| / |ref| <= 2e-2; ht (fp32)
to the bar the backward tests hold it to.  Full-size workloads are compared on
sampled heads (heads are independent)."""

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_bwd_amd import binding as B
from chunked_gated_delta_bwd_amd import synth
from gpu_common import TOL_BF16, TOL_FP32, compare, gpu_run, log, subset_heads

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


def _check(inp, got, label, heads=None):
    sub = inp if heads is None else subset_heads(inp, heads)
    ref = oracle.run(sub, backward=False)
    assert np.isfinite(got["o"]).all(), f"{label}: output rows left unwritten"
    compare(got, ref, ("o",), TOL_BF16, label + " o", heads)
    compare(got, ref, ("ht",), TOL_FP32 * 5, label + " ht", heads)


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


@pytest.mark.parametrize("wl,heads", [("gdn_bf16_t32768_h16_d128", [0, 15]),
                                      ("gdn_varlen12_bf16_t32768_h32_d128", [3, 30]),
                                      ("kda_bf16_t8192_h16_d128", [0, 9])])
def test_forward_workloads_sampled_heads(wl, heads):
    log(f"case {wl} heads {heads}")
    inp = synth.generate(synth.workload(wl))
    got, _ = gpu_fwd(inp)
    _check(inp, got, wl, heads=heads)


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
