"""GPU parity of the exact sequence split of the two chunk recursions.

Each segment of a split sequence first runs from a zero state (the first one of
each direction from h0 / dht) while carrying the transfer product of its
chunks; the true boundary states are then composed in order and every segment
runs again from its true state.  The result is the unsplit recursion's up to
rounding, so it is held to the same bars against the float64 oracle: forced
splits on small problems (every gate form, both dtypes, both head sizes,
ragged varlen packs with empty and one-token sequences, segments of one chunk),
the library's own choice at T = 32768 with H = 2 and H = 4, both gates (one GPU's
share of the H = 16 and H = 32 problems under 8-way head sharding, where the
unsplit recursions would use 32 or 64 of 256 compute units), and agreement with
the unsplit path."""

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_bwd_amd import binding as B
from chunked_gated_delta_bwd_amd import synth
from gpu_common import FP32_GRADS, TOKEN_GRADS, TOL_BF16, TOL_FP32, compare, gpu_run, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _check(inp, got, label):
    ref = oracle.run(inp)
    compare(got, ref, TOKEN_GRADS, TOL_BF16, label + " grads")
    compare(got, ref, FP32_GRADS, TOL_FP32, label + " fp32")
    compare(got, ref, ("ht",), TOL_FP32 * 5, label + " ht")


SMALL = [
    ("gdn_bf16_t1000_h2_d128_s3", 3, synth.Spec("sa", 0, "bf16", H=2, K=128, V=128, B=1, T=1000, h0_std=0.2,
                                                 dht_std=0.2, seed=401)),
    ("gdn_bf16_b2_t700_h3_d64_s5", 5, synth.Spec("sb", 0, "bf16", H=3, K=64, V=64, B=2, T=700, h0_std=0.3,
                                                  dht_std=0.3, seed=402)),
    ("gdn_f32_t333_h2_d64_s16", 16, synth.Spec("sc", 0, "f32", H=2, K=64, V=64, B=1, T=333, h0_std=0.2,
                                                dht_std=0.2, seed=403)),
    ("gdn_bf16_varlen_d128_s4", 4, synth.Spec("sd", 0, "bf16", H=2, K=128, V=128,
                                               lengths=[900, 1, 0, 130, 64, 65, 2000], h0_std=0.1, dht_std=0.1,
                                               seed=404)),
    ("kda_bf16_t800_h2_d128_s4", 4, synth.Spec("se", 1, "bf16", H=2, K=128, V=128, B=1, T=800, h0_std=0.2,
                                                dht_std=0.2, seed=405)),
    ("kda_f32_varlen_d64_s3", 3, synth.Spec("sf", 1, "f32", H=2, K=64, V=64, lengths=[300, 7, 450],
                                             h0_std=0.2, dht_std=0.2, seed=406)),
    ("kdas_bf16_t640_h2_d128_s2", 2, synth.Spec("sg", 2, "bf16", H=2, K=128, V=128, B=1, T=640, h0_std=0.2,
                                                 dht_std=0.2, seed=407)),
    ("gqa2_gdn_bf16_t600_d128_s3", 3, synth.Spec("sh", 0, "bf16", H=4, Hk=2, K=128, V=128, B=1, T=600,
                                                  h0_std=0.2, dht_std=0.2, seed=408)),
]


@pytest.mark.parametrize("name,P,spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_forced_split_against_oracle(name, P, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode, seq_split=P)
    if spec.gate == 2:
        ref = oracle.run(inp)
        compare(got, ref, TOKEN_GRADS, TOL_BF16, name + " grads")
        compare(got, ref, ("dh0", "ddt_bias"), TOL_FP32, name + " fp32")
        compare(got, ref, ("dA_log",), 2e-2, name + " dA_log")
        compare(got, ref, ("ht",), TOL_FP32 * 5, name + " ht")
    else:
        _check(inp, got, f"{name}/{mode}")


# The synthetic gates forget fast (about e^-4.4 per chunk for the scalar gate), so
# a segment's run from zero soon meets the true state bit for bit and the
# composed boundary state hardly matters.  With weak decay the transfer products
# carry the boundary state through whole segments: these cases check the
# composition itself.
# (fp32 inputs at D = 64: the materialised-tile steps with Khat and W in two parts,
# in both passes)
@pytest.mark.parametrize("gate,P,dtype,D", [(0, 4, "bf16", 128), (0, 16, "bf16", 128), (1, 5, "bf16", 128),
                                            (0, 4, "f32", 64)],
                         ids=["gdn_s4", "gdn_s16", "kda_s5", "gdn_f32_d64_s4"])
def test_forced_split_weak_decay(gate, P, dtype, D):
    log(f"case weak decay gate {gate} split {P} {dtype} D={D}")
    inp = synth.generate(synth.Spec("sw", gate, dtype, H=2, K=D, V=D, lengths=[1200, 333, 64], h0_std=0.3,
                                    dht_std=0.3, seed=411))
    if gate == 0:
        inp["g"] = torch.full_like(inp["g"], -0.002)
    else:
        inp["A_log"] = torch.full_like(inp["A_log"], -3.0)
    got = gpu_run(inp, seq_split=P)
    ref = oracle.run(inp)
    compare(got, ref, TOKEN_GRADS, TOL_BF16, f"weak decay s{P} grads")
    compare(got, ref, ("ht",), TOL_FP32 * 5, f"weak decay s{P} ht")
    plain = gpu_run(inp, seq_split=1)
    for key in FP32_GRADS + ("ht",):
        if key not in ref:
            continue
        d_split = np.linalg.norm(got[key] - ref[key]) / np.linalg.norm(ref[key])
        d_plain = np.linalg.norm(plain[key] - ref[key]) / np.linalg.norm(ref[key])
        log(f"[weak decay s{P}] {key}: split {d_split:.2e}, unsplit {d_plain:.2e}")
        # the split adds no error of its own beyond rounding
        assert d_split <= max(1.5 * d_plain, 2e-4), (key, d_split, d_plain)


def test_split_chunk_states_match_unsplit():
    """The per-chunk states and state gradients the final pass stores equal the
    unsplit recursion's up to rounding."""
    spec = synth.Spec("si", 0, "bf16", H=2, K=128, V=128, lengths=[1500, 333], h0_std=0.2, dht_std=0.2, seed=409)
    inp = synth.generate(spec)
    a = gpu_run(inp, exports=True, seq_split=1)
    b = gpu_run(inp, exports=True, seq_split=6)
    ref = oracle.run(inp, exports=True)
    compare(b, ref, ("S_chunk", "dS_chunk"), 1e-2, "split chunk states")
    for key in ("S_chunk", "dS_chunk"):
        err = np.linalg.norm(a[key] - b[key]) / np.linalg.norm(a[key])
        log(f"[split vs unsplit] {key} {err:.2e}")
        assert err < 1e-2, (key, err)


@pytest.mark.parametrize("wl", ["gdn_bf16_t32768_h2_d128", "gdn_bf16_t32768_h4_d128", "kda_bf16_t32768_h2_d128"])
def test_long_sequence_few_heads(wl):
    """The library's own choice (it splits these) against the oracle, every head,
    every token, and against the unsplit path."""
    log(f"case {wl}")
    inp = synth.generate(synth.workload(wl))
    got = gpu_run(inp)
    _check(inp, got, wl)
    plain = gpu_run(inp, seq_split=1)
    for key in TOKEN_GRADS + ("dh0",):
        err = np.linalg.norm(got[key] - plain[key]) / np.linalg.norm(plain[key])
        log(f"[{wl} split vs unsplit] {key} {err:.2e}")
        assert err < TOL_BF16, (key, err)


def test_split_is_deterministic():
    inp = synth.generate(synth.Spec("sj", 1, "bf16", H=2, K=128, V=128, B=1, T=900, h0_std=0.1, dht_std=0.1,
                                    seed=410))
    a = gpu_run(inp, seq_split=4)
    b = gpu_run(inp, seq_split=4)
    for key in TOKEN_GRADS + FP32_GRADS + ("ht",):
        assert (a[key] == b[key]).all(), key
