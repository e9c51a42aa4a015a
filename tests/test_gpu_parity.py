"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded input bytes.  Normalised errors |X - ref| / |ref| must stay within
2e-2 for the per-token gradients (stored in bf16) and 1e-3 for dh0, dA_log and
ddt_bias (fp32), and the worst (token, head) row within five times those bars.
Every workload is compared in full: all heads, all tokens.""" 

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_bwd_amd import synth
from gpu_common import FP32_GRADS, TOKEN_GRADS, TOL_BF16, TOL_FP32, compare, gpu_run, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _check(inp, got, label, tol_fp32=TOL_FP32):
    ref = oracle.run(inp)
    compare(got, ref, TOKEN_GRADS, TOL_BF16, label + " grads")
    compare(got, ref, FP32_GRADS, tol_fp32, label + " fp32")
    compare(got, ref, ("ht",), TOL_FP32 * 5, label + " ht")


SMALL = [
    ("gdn_f32_t128_h2_d64", synth.workload("gdn_f32_t128_h2_d64")),
    ("gdn_bf16_varlen_edges_d128",
     synth.Spec("e", 0, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1,
                dht_std=0.1, seed=31)),
    ("gdn_f32_b2_t100_d64", synth.Spec("f", 0, "f32", H=2, K=64, V=64, B=2, T=100, seed=32)),
    ("gdn_bf16_b1_t300_d64_h0", synth.Spec("g", 0, "bf16", H=4, K=64, V=64, B=1, T=300, h0_std=0.5,
                                           dht_std=0.5, seed=33)),
]


@pytest.mark.parametrize("name,spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_small_against_oracle(name, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode)
    _check(inp, got, f"{name}/{mode}")


def test_chunk_boundary_states():
    """Stage check: states at chunk starts and state gradients at chunk ends."""
    spec = synth.Spec("s", 0, "bf16", H=2, K=128, V=128, lengths=[130, 64, 5], h0_std=0.2, dht_std=0.2,
                      seed=34)
    inp = synth.generate(spec)
    got = gpu_run(inp, exports=True)
    ref = oracle.run(inp, exports=True)
    compare(got, ref, ("S_chunk", "dS_chunk"), 1e-2, "chunk states")


# gdr_fwd_bwd against gdr_fwd_recompute + gdr_bwd, bit for bit: the recipe, and the
# two-part steps (the scalar gate without decay: reverse steps in the second launch;
# the per-channel gate with weak decay: forward steps in the common launch)
@pytest.mark.parametrize("case", ["recipe", "gdn_no_decay", "kda_weak_decay"])
def test_fused_and_split_agree(case):
    gate = 1 if case.startswith("kda") else 0
    inp = synth.generate(synth.Spec("a", gate, "bf16", H=4, K=128, V=128, B=1, T=512, h0_std=0.1,
                                    dht_std=0.1, seed=35))
    if case == "gdn_no_decay":
        inp["g"] = torch.zeros_like(inp["g"])
    elif case == "kda_weak_decay":
        inp["A_log"] = torch.full_like(inp["A_log"], -3.0)
    a = gpu_run(inp, mode="fused")
    b = gpu_run(inp, mode="split")
    for key in TOKEN_GRADS + FP32_GRADS + ("ht",):
        if key in a:
            assert (a[key] == b[key]).all(), key


def test_repeat_is_deterministic():
    inp = synth.generate(synth.Spec("r", 0, "bf16", H=2, K=128, V=128, B=2, T=256, seed=36))
    a = gpu_run(inp)
    b = gpu_run(inp)
    for key in TOKEN_GRADS + ("dh0",):
        assert (a[key] == b[key]).all(), key


def test_workload_b2_t4096_h16():
    inp = synth.generate(synth.workload("gdn_bf16_b2_t4096_h16_d128"))
    got = gpu_run(inp)
    _check(inp, got, "gdn_bf16_b2_t4096_h16_d128")


def test_workload_varlen12_h32():
    inp = synth.generate(synth.workload("gdn_varlen12_bf16_t32768_h32_d128"))
    assert any(L % 64 for L in inp["lengths"])
    got = gpu_run(inp)
    _check(inp, got, "gdn_varlen12_h32")


@pytest.mark.parametrize("H", [16, 32])
def test_workload_t32768(H):
    inp = synth.generate(synth.workload(f"gdn_bf16_t32768_h{H}_d128"))
    got = gpu_run(inp)
    _check(inp, got, f"gdn_t32768_h{H}")


# ---------------------------------------------------------------------------
# per-channel gate (KDA)
# ---------------------------------------------------------------------------
SMALL_KDA = [
    ("kda_f32_t128_h2_d64", synth.Spec("kf", 1, "f32", H=2, K=64, V=64, B=1, T=128, seed=41)),
    ("kda_bf16_varlen_edges_d128",
     synth.Spec("ke", 1, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1,
                dht_std=0.1, seed=42)),
    ("kda_f32_b2_t100_d128", synth.Spec("kg", 1, "f32", H=2, K=128, V=128, B=2, T=100, h0_std=0.2,
                                        dht_std=0.2, seed=43)),
    ("kda_bf16_b1_t300_d64", synth.Spec("kh", 1, "bf16", H=4, K=64, V=64, B=1, T=300, h0_std=0.5,
                                        dht_std=0.5, seed=44)),
]


@pytest.mark.parametrize("name,spec", SMALL_KDA, ids=[s[0] for s in SMALL_KDA])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_kda_small_against_oracle(name, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode)
    _check(inp, got, f"{name}/{mode}")


# Outside the synthetic recipe's A_log ~ U(0, 1.5): weak decay (e^A_log = 0.05,
# per-token log decays ~ -0.04) sends every 16-row diagonal block of the gradient
# and prologue kernels down the factored fp32-MFMA path (factored at the block's
# middle row); strong decay (e^A_log = 20, log decays ~ -15, in-block half-spans
# far above 60) sends every channel down the exact per-element path; in between
# (e^A_log = 9, half-spans of 60 and more in about half of the channels of every
# block) the prologue splits each diagonal block between the two paths by channel
# and the gradient kernel by 16-channel tile.  With almost no forgetting the chunk
# states' bf16 rounding is not damped between chunks: the forward state update
# then takes U and Khat in two parts (weak chunks), and all three regimes keep the
# standard bars (one part each: dA_log 1.7e-3, ddt_bias 1.2e-3 in the weak regime).
# The H = 17 case runs the same in a grid of more than one workgroup per CU.
@pytest.mark.parametrize("a_log,H,D,dtype", [(-3.0, 2, 128, "bf16"), (-3.0, 17, 128, "bf16"), (-3.0, 3, 64, "bf16"),
                                              (-3.0, 2, 128, "f32"), (2.2, 2, 128, "bf16"), (3.0, 2, 128, "bf16")],
                         ids=["weak_decay", "weak_decay_h17", "weak_decay_d64", "weak_decay_f32", "mixed_decay",
                              "strong_decay"])
def test_kda_decay_regimes(a_log, H, D, dtype):
    log(f"case kda decay regime A_log={a_log} H={H} D={D} {dtype}")
    inp = synth.generate(synth.Spec("kd", 1, dtype, H=H, K=D, V=D, lengths=[200, 77], h0_std=0.1,
                                    dht_std=0.1, seed=47))
    inp["A_log"] = torch.full_like(inp["A_log"], a_log)
    got = gpu_run(inp)
    _check(inp, got, f"kda_decay_{a_log}_h{H}_d{D}_{dtype}")


def test_kda_chunk_boundary_states():
    spec = synth.Spec("ks", 1, "bf16", H=2, K=128, V=128, lengths=[130, 64, 5], h0_std=0.2, dht_std=0.2,
                      seed=45)
    inp = synth.generate(spec)
    got = gpu_run(inp, exports=True)
    ref = oracle.run(inp, exports=True)
    compare(got, ref, ("S_chunk", "dS_chunk"), 1e-2, "kda chunk states")


def test_kda_repeat_is_deterministic():
    inp = synth.generate(synth.Spec("kr", 1, "bf16", H=2, K=128, V=128, B=2, T=256, seed=46))
    a = gpu_run(inp)
    b = gpu_run(inp)
    for key in TOKEN_GRADS + FP32_GRADS:
        assert (a[key] == b[key]).all(), key


def test_kda_workload_t8192_h16():
    inp = synth.generate(synth.workload("kda_bf16_t8192_h16_d128"))
    got = gpu_run(inp)
    _check(inp, got, "kda_bf16_t8192_h16_d128")


@pytest.mark.parametrize("H", [16, 32])
def test_kda_workload_t32768(H):
    inp = synth.generate(synth.workload(f"kda_bf16_t32768_h{H}_d128"))
    got = gpu_run(inp)
    _check(inp, got, f"kda_t32768_h{H}")


# ---------------------------------------------------------------------------
# per-channel gate, bounded sigmoid form: lambda = gate_scale sigma(e^A_log (g + dt_bias))
# ---------------------------------------------------------------------------
# dA_log = sum over tokens and channels of dg * (g + dt_bias): for this gate form
# the terms cancel 60-850x on the synthetic recipe (softplus form: 30-50x), so the
# per-term error of the bf16 pipeline (dg within 1e-3) is amplified by that much;
# dA_log is held to 2e-2 here and, separately, checked to be exactly the reduction
# of the kernel's own fp32 dg (which pins the reduction, not the precision).
TOL_KDAS_DA_LOG = 2e-2


def _check_kdas(inp, got, label):
    ref = oracle.run(inp)
    compare(got, ref, TOKEN_GRADS, TOL_BF16, label + " grads")
    compare(got, ref, ("dh0", "ddt_bias"), TOL_FP32, label + " fp32")
    compare(got, ref, ("dA_log",), TOL_KDAS_DA_LOG, label + " dA_log")
    compare(got, ref, ("ht",), TOL_FP32 * 5, label + " ht")
    if inp["dtype"] == "f32":
        x = inp["g"].double().numpy() + inp["dt_bias"].double().numpy()[None, None]
        own = np.einsum("bthk,bthk->h", got["dg"], x)
        scale = np.einsum("bthk,bthk->h", np.abs(got["dg"]), np.abs(x))
        assert np.all(np.abs(own - got["dA_log"]) <= 1e-5 * scale), (label, own, got["dA_log"])


SMALL_KDAS = [
    ("kdas_f32_t128_h2_d64", synth.Spec("sf", 2, "f32", H=2, K=64, V=64, B=1, T=128, seed=61)),
    ("kdas_bf16_varlen_edges_d128",
     synth.Spec("se", 2, "bf16", H=3, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1,
                dht_std=0.1, seed=62)),
    ("kdas_f32_b1_t300_d64_gs05", synth.Spec("sh", 2, "f32", H=4, K=64, V=64, B=1, T=300, h0_std=0.5,
                                             dht_std=0.5, seed=63, gate_scale=-0.5)),
]


@pytest.mark.parametrize("name,spec", SMALL_KDAS, ids=[s[0] for s in SMALL_KDAS])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_kdas_small_against_oracle(name, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode)
    _check_kdas(inp, got, f"{name}/{mode}")


def test_kdas_workload_t8192_h16():
    inp = synth.generate(synth.workload("kdas_bf16_t8192_h16_d128"))
    got = gpu_run(inp)
    _check_kdas(inp, got, "kdas_bf16_t8192_h16_d128")


# ---------------------------------------------------------------------------
# grouped heads: q, k with Hk heads, each read by H / Hk value heads; dq, dk are
# the group sums (every gate, both dtypes, dense and ragged varlen)
# ---------------------------------------------------------------------------
SMALL_GQA = [
    ("gqa2_gdn_bf16_b1_t300_d64", synth.Spec("qa", 0, "bf16", H=4, Hk=2, K=64, V=64, B=1, T=300,
                                             h0_std=0.3, dht_std=0.3, seed=71)),
    ("gqa3_gdn_f32_varlen_edges_d128",
     synth.Spec("qb", 0, "f32", H=6, Hk=2, K=128, V=128, lengths=[1, 63, 64, 65, 0, 200], h0_std=0.1,
                dht_std=0.1, seed=72)),
    ("gqa4_kda_bf16_varlen_d128", synth.Spec("qc", 1, "bf16", H=4, Hk=1, K=128, V=128,
                                             lengths=[130, 7, 64], h0_std=0.1, dht_std=0.1, seed=73)),
    ("gqa2_kda_f32_b2_t100_d64", synth.Spec("qd", 1, "f32", H=4, Hk=2, K=64, V=64, B=2, T=100, seed=74)),
]


@pytest.mark.parametrize("name,spec", SMALL_GQA, ids=[s[0] for s in SMALL_GQA])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_grouped_heads_small_against_oracle(name, spec, mode):
    log(f"case {name} mode {mode}")
    inp = synth.generate(spec)
    got = gpu_run(inp, mode=mode)
    assert got["dq"].shape[2] == spec.Hk
    _check(inp, got, f"{name}/{mode}")


def test_grouped_heads_sigmoid_gate():
    inp = synth.generate(synth.Spec("qe", 2, "f32", H=4, Hk=2, K=64, V=64, B=1, T=200, h0_std=0.2,
                                    dht_std=0.2, seed=75))
    _check_kdas(inp, gpu_run(inp), "gqa2_kdas_f32_t200_d64")


def test_grouped_heads_workload():
    """H = 32 value heads over Hk = 8 key heads at T = 32768, every group."""
    inp = synth.generate(synth.workload("gdn_gqa4_bf16_t32768_h32_d128"))
    got = gpu_run(inp)
    _check(inp, got, "gdn_gqa4_t32768_h32")


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_no_tokens(gate):
    """Every sequence empty (T = 0): the token tensors have no storage (NULL
    pointers), ht = h0 and dh0 = dht exactly, the parameter gradients are zero."""
    log(f"case no tokens, gate {gate}")
    inp = synth.generate(synth.Spec("z", gate, "bf16", H=2, K=64, V=64, lengths=[0, 0], h0_std=0.3,
                                    dht_std=0.3, seed=91))
    assert inp["T"] == 0
    got = gpu_run(inp)
    ref = oracle.run(inp)
    assert np.array_equal(got["dh0"], ref["dh0"]) and np.array_equal(got["ht"], ref["ht"])
    if gate:
        assert not got["dA_log"].any() and not got["ddt_bias"].any()


# ---------------------------------------------------------------------------
# mixed small configurations: every gate with both dtypes and head dims, grouped
# heads, dense batches and ragged varlen packs together (one seeded draw each)
# ---------------------------------------------------------------------------
def _mixed_specs():
    rng = np.random.default_rng(2024)
    specs = []
    for i in range(8):
        gate = i % 3
        dtype = "f32" if i % 4 == 3 else "bf16"
        D = 64 if i % 2 else 128
        Hk = int(rng.choice([1, 2]))
        H = Hk * int(rng.choice([1, 2, 3]))
        if i % 2:
            lengths = [int(x) for x in rng.integers(0, 150, size=int(rng.integers(1, 4)))]
            kw = dict(lengths=lengths)
        else:
            kw = dict(B=int(rng.integers(1, 3)), T=int(rng.integers(1, 200)))
        specs.append((f"mix{i}_g{gate}_{dtype}_d{D}_h{H}_hk{Hk}",
                      synth.Spec(f"m{i}", gate, dtype, H=H, Hk=Hk, K=D, V=D, h0_std=0.2, dht_std=0.2,
                                 seed=300 + i, **kw)))
    return specs


MIXED = _mixed_specs()


@pytest.mark.parametrize("name,spec", MIXED, ids=[s[0] for s in MIXED])
def test_mixed_small_against_oracle(name, spec):
    log(f"case {name}")
    inp = synth.generate(spec)
    got = gpu_run(inp)
    if spec.gate == 2:
        _check_kdas(inp, got, name)
    else:
        _check(inp, got, name)


# Many sequences in one pack: the chunk and segment tables are written on the device
# from batches of 56 sequence entries a launch, so 130 sequences take three batches
# (and, split, three batches of segment rows); lengths 0 .. 149, every head compared.
@pytest.mark.parametrize("gate,split", [(0, 1), (1, 1), (0, 3)], ids=["gdn", "kda", "gdn_split3"])
def test_many_sequences(gate, split):
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 150, size=130)]
    log(f"case many sequences gate {gate} split {split}: {len(lengths)} sequences, {sum(lengths)} tokens")
    inp = synth.generate(synth.Spec("ms", gate, "bf16", H=3, K=64, V=64, lengths=lengths, h0_std=0.2, dht_std=0.2,
                                    seed=78))
    got = gpu_run(inp, seq_split=split)
    _check(inp, got, f"many_sequences_g{gate}_s{split}")


# Scalar gate outside the synthetic recipe (g = -0.1 softplus(N(0, 1))): no decay at all
# (g = 0: the plain delta rule), weak decay (g = -0.01 a token: e^-0.64 a chunk) and very
# strong decay (g = -30 per token: e^Gamma underflows to zero inside a chunk, so every
# chunk forgets its past).  With little decay a reverse step's bf16 rounding is not damped
# between chunks; the recursion then takes dS, dU and Y in two bf16 parts, and dh0 keeps
# the standard 1e-3 bar (one bf16 part each: 1.6e-3 over five chunks).  The H = 17 cases
# run two V slices a workgroup.  With strong decay dg and dh0 are ~1e-13 in the oracle
# (every path to them carries e^-30 or less), so a relative bar is meaningless there:
# they are held to an absolute 1e-6 instead; every other output keeps the standard bars.
@pytest.mark.parametrize("gval,H,D,dtype", [(0.0, 2, 128, "bf16"), (-0.01, 2, 128, "bf16"), (0.0, 17, 128, "bf16"),
                                             (0.0, 3, 64, "bf16"), (0.0, 2, 64, "f32"), (-30.0, 2, 128, "bf16")],
                         ids=["no_decay", "weak_decay", "no_decay_h17", "no_decay_d64", "no_decay_f32", "strong_decay"])
def test_gdn_decay_extremes(gval, H, D, dtype):
    log(f"case gdn decay g={gval} H={H} D={D} {dtype}")
    inp = synth.generate(synth.Spec("ge", 0, dtype, H=H, K=D, V=D, lengths=[200, 77], h0_std=0.1,
                                    dht_std=0.1, seed=48))
    inp["g"] = torch.full_like(inp["g"], gval)
    got = gpu_run(inp)
    if gval > -1.0:
        _check(inp, got, f"gdn_decay_{gval}_h{H}_d{D}_{dtype}")
        return
    ref = oracle.run(inp)
    compare(got, ref, ("dq", "dk", "dv", "db"), TOL_BF16, f"gdn_decay_{gval} grads")
    compare(got, ref, ("ht",), TOL_FP32 * 5, f"gdn_decay_{gval} ht")
    for key in ("dg", "dh0"):
        worst = float(np.abs(got[key] - ref[key]).max())
        log(f"[gdn_decay_{gval}] {key} max abs error {worst:.2e} (oracle max {np.abs(ref[key]).max():.2e})")
        assert worst <= 1e-6, (key, worst)
