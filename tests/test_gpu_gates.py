"""GPU parity of the forget-gate variants: one decay per token and head
(Gated DeltaNet) and no gate (DeltaNet), through the *_gated entry points of
the C ABI, against the fp64 oracle fed the per-channel decays the gate stands
for (oracle.channel_gate).  Same error metric and bounds as the per-channel
tests: max |x_gpu - x_ref| / max |x_ref|, 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, gen
from test_gpu_parity import dvt_env, rel, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as lib
    lib.load_library()
    return lib


def dev():
    return torch.device("cuda:0")


def lead(d):
    return tuple(d["q"].shape[:3])


def ref(d):
    dk = d["q"].shape[-1]
    a = oracle.channel_gate(d["alpha"], d["gate"], dk, lead(d))
    return oracle.forward(d["q"], d["k"], d["v"], a, d["beta"], d["initial_state"],
                          cu_seqlens=d.get("cu_seqlens_host"))


def run(kda, d, **kw):
    return kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                   d["initial_state"], cu_seqlens=d.get("cu_seqlens"),
                                   cu_seqlens_host=d.get("cu_seqlens_host"), gate=d["gate"], **kw)


CASES = [
    # dtype, B, T, H, dk, dv, s0_std, dvt, gate
    ("f32", 1, 200, 2, 64, 64, None, 16, "head"),
    ("f32", 2, 77, 1, 64, 128, 0.1, 64, "none"),
    ("f32", 1, 100, 1, 128, 128, 0.1, 16, "head"),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 16, "head"),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "head"),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 64, "head"),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "none"),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 64, "none"),
    ("bf16", 1, 1, 2, 128, 128, 0.5, None, "head"),
    ("bf16", 1, 65, 2, 128, 128, 0.5, None, "head"),
    ("bf16", 1, 63, 2, 128, 128, 0.5, None, "none"),
    ("bf16", 3, 129, 2, 64, 64, 0.2, 16, "head"),
    ("bf16", 1, 200, 2, 64, 64, 0.2, 64, "none"),
    ("bf16", 1, 190, 2, 128, 64, 0.2, 32, "none"),
    ("bf16", 1, 190, 2, 64, 128, 0.2, 64, "head"),
]
IDS = ["-".join(str(x) for x in c) for c in CASES]


def draw(idx):
    dt, B, T, H, dk, dv, s0, dvt, gate = CASES[idx]
    return gen.draw_chunk(B, T, H, dk, dv, dt, alpha_mu=3.0, s0_std=s0, seed=300 + idx,
                          device=dev(), gate=gate)


@pytest.mark.parametrize("idx", range(len(CASES)), ids=IDS)
def test_gated_chunk_small(kda, idx):
    case = CASES[idx]
    print("case", case, flush=True)
    d = draw(idx)
    with dvt_env(case[7]):
        o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= TOL[case[0]]
    assert rel(s, rs) <= TOL[case[0]]


@pytest.mark.parametrize("idx", [i for i, c in enumerate(CASES) if c[0] == "bf16"],
                         ids=[i for i, c in zip(IDS, CASES) if c[0] == "bf16"])
def test_gated_chunk_small_generic_kernel(kda, idx):
    case = CASES[idx]
    print("case", case, flush=True)
    d = draw(idx)
    with dvt_env(case[7], generic=True):
        o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= TOL[case[0]]
    assert rel(s, rs) <= TOL[case[0]]


@pytest.mark.parametrize("gate", ["head", "none"])
def test_gate_equals_the_channel_path_with_repeated_decays(kda, gate):
    """A per-head decay repeated over the channels, or alpha = 1, through the
    per-channel entry point gives the same bits: every channel then runs the
    same products in the same order."""
    d = gen.draw_chunk(2, 333, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.2, seed=41,
                       device=dev(), gate=gate)
    a = (torch.ones((2, 333, 2, 128), device=dev()) if gate == "none"
         else d["alpha"][..., None].expand(2, 333, 2, 128).contiguous())
    o1, s1 = run(kda, d)
    o2, s2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], a, d["beta"], d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate", ["head", "none"])
def test_gated_chunk_varlen_small(kda, gate):
    lens = [0, 1, 64, 65, 200, 0, 7, 130]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = gen.draw_chunk(1, cu[-1], 3, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.1,
                       num_states=len(lens), seed=51, device=dev(), gate=gate)
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2
    assert rel(s, rs) <= 2e-2
    assert torch.equal(s[0], d["initial_state"][0]) and torch.equal(s[5], d["initial_state"][5])


@pytest.mark.parametrize("gate", ["head", "none"])
def test_gated_chunk_full_B4_H16_T4096(kda, gate):
    """The B4 H16 T4096 d128 workload with a per-head gate, or none: every
    output against the oracle."""
    d = gen.chunk_inputs(CONFIGS[1], device=dev(), gate=gate)
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    eo, es = rel(o, ro), rel(s, rs)
    print("B4 H16 T4096 gate %s: err o %.2e state %.2e" % (gate, eo, es))
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dt,dk,dv", [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128)])
def test_gated_step_small(kda, gate, dt, dk, dv):
    from workloads.configs import Config
    cfg = Config("t", "decode", dt, 3, 1, 5, dk, dv, 4.0, 0.3, steps=6, seed=61)
    d = gen.decode_inputs(cfg, device=dev(), gate=gate)
    st = d["state"].clone()
    ref_state = d["state"]
    for t in range(cfg.steps):
        a = None if gate == "none" else d["alpha"][t]
        args = [d[n][t] for n in ("q", "k", "v")]
        ro, ref_state = oracle.step(*args, oracle.channel_gate(a, gate, dk, (3, 5)),
                                    d["beta"][t], ref_state)
        o = kda.kda_recurrent_step_gated(*args, a, d["beta"][t], st, gate=gate)
        torch.cuda.synchronize()
        assert rel(o, ro) <= TOL[dt], t
    assert rel(st, ref_state) <= TOL[dt]
