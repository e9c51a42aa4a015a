"""The no-allocation entry point gdr_fwd_bwd_noalloc (workspace in a device array
the library holds) against gdr_fwd_bwd on a workspace of the caller's, through
the C ABI: the same kernels on the same inputs, so every output must agree bit
for bit, on two calls in a row (the second smaller, so it runs over what the
first left in the array).  Shapes beyond the array are rejected before anything
is enqueued (no GPU needed)."""

import numpy as np
import pytest
import torch

from chunked_gated_delta_bwd_amd import binding as B
from chunked_gated_delta_bwd_amd import synth
from gpu_common import log


def _outputs(inp, dev, out, ht):
    res = {k: v.double().cpu().numpy() for k, v in out.items() if v is not None}
    res["ht"] = ht.double().cpu().numpy()
    return res


def _run(inp, noalloc):
    dev = B.to_device(inp)
    prob = B.Problem.from_inputs(inp)
    out = B.alloc_outputs(inp, dev)
    ht = torch.empty((inp["N"], inp["H"], inp["V"], inp["K"]), dtype=torch.float32, device="cuda")
    if noalloc:
        B.gdr_fwd_bwd_noalloc(prob, dev, dev["dO"], dev["dht"], out, ht=ht)
    else:
        ws = B.alloc_workspace(prob)
        B.gdr_fwd_bwd(prob, dev, dev["dO"], dev["dht"], ws, out, ht=ht)
    torch.cuda.synchronize()
    return _outputs(inp, dev, out, ht)


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_matches_fwd_bwd_on_two_calls():
    specs = [
        synth.Spec("na1", 1, "bf16", H=4, K=128, V=128, lengths=[700, 129, 63, 0, 200], h0_std=0.2, dht_std=0.2,
                   seed=81),
        synth.Spec("na2", 0, "bf16", H=2, K=128, V=128, B=1, T=190, h0_std=0.3, dht_std=0.3, seed=82),
    ]
    for spec in specs:
        log(f"case noalloc {spec.name}")
        inp = synth.generate(spec)
        prob = B.Problem.from_inputs(inp)
        assert B.gdr_workspace_bytes(prob) <= B.NOALLOC_WORKSPACE_BYTES
        got = _run(inp, noalloc=True)
        ref = _run(inp, noalloc=False)
        assert got.keys() == ref.keys()
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (spec.name, key)


def test_noalloc_rejects_shapes_beyond_its_array():
    B.load_library()
    prob = B.Problem(1, 32768, 16, 128, 1, 0, B.GDR_BF16, 128 ** -0.5)
    assert B.gdr_workspace_bytes(prob) > B.NOALLOC_WORKSPACE_BYTES
    with pytest.raises(B.GdrError) as e:
        B.gdr_fwd_bwd_noalloc(prob, {k: None for k in ("q", "k", "v", "g", "b")}, None, None,
                              {k: None for k in ("dq", "dk", "dv", "dg", "db")}, stream=0)
    assert e.value.status == B.GDR_EWORKSPACE
    assert "no-allocation" in str(e.value)
