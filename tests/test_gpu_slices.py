"""GPU parity of the recursions with two V slices a workgroup.

When one 16-wide V slice a workgroup would need more recursion workgroups than
the GPU has compute units (one fits per CU), the scalar gate with bf16 inputs
runs two slices a workgroup, which share the chunk tiles.  The library picks
this by the grid size alone, so these cases are sized to cross that line at
small token counts (both head sizes, ragged varlen packs, forced sequence
splits whose local and final passes both take two slices, grouped heads) and
compared with the float64 oracle at the standard bars; the full-size workloads
with 32 heads run it as well."""

import pytest
import torch

import oracle
from chunked_gated_delta_bwd_amd import synth
from gpu_common import FP32_GRADS, TOKEN_GRADS, TOL_BF16, TOL_FP32, compare, gpu_run, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (name, forced segments per sequence (0: the library's choice), spec); every
# case has 2 x heads x D/16 x sequences (x 2 for a split's local pass) > 256
CASES = [
    ("gdn_bf16_t300_h17_d128", 0, synth.Spec("na", 0, "bf16", H=17, K=128, V=128, B=1, T=300, h0_std=0.2,
                                              dht_std=0.2, seed=501)),
    ("gdn_bf16_t260_h40_d64", 0, synth.Spec("nb", 0, "bf16", H=40, K=64, V=64, B=1, T=260, h0_std=0.2,
                                             dht_std=0.2, seed=502)),
    ("gdn_bf16_varlen_h9_d128", 0, synth.Spec("nc", 0, "bf16", H=9, K=128, V=128,
                                               lengths=[200, 1, 0, 64, 65, 130], h0_std=0.1, dht_std=0.1,
                                               seed=503)),
    ("gdn_bf16_t700_h12_d128_s2", 2, synth.Spec("nd", 0, "bf16", H=12, K=128, V=128, B=1, T=700, h0_std=0.2,
                                                 dht_std=0.2, seed=504)),
    ("gqa4_gdn_bf16_t300_h24_d128", 0, synth.Spec("ne", 0, "bf16", H=24, Hk=6, K=128, V=128, B=1, T=300,
                                                   h0_std=0.2, dht_std=0.2, seed=505)),
]


@pytest.mark.parametrize("name,P,spec", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_two_slices_against_oracle(name, P, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode, seq_split=P)
    ref = oracle.run(inp)
    compare(got, ref, TOKEN_GRADS, TOL_BF16, name + " grads")
    compare(got, ref, FP32_GRADS, TOL_FP32, name + " fp32")
    compare(got, ref, ("ht",), TOL_FP32 * 5, name + " ht")
