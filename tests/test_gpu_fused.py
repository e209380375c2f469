"""GPU parity of in-kernel input preparation (kda_chunk_fwd_fused,
kda_recurrent_step_fused): gate logits (alpha = sigmoid), beta logits and
q/k L2 normalisation, against the fp64 oracle run on the inputs that
oracle.prepare derives from the same stored tensors.  Same error metric and
bounds as the other parity tests: max |x_gpu - x_ref| / max |x_ref|, 1e-4
for fp32 inputs and 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, gen
from test_gpu_parity import dvt_env, rel, TOL

pytestmark = pytest.mark.gpu

ALL = dict(gate_logits=True, beta_logits=True, qk_l2norm=True)


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as lib
    lib.load_library()
    return lib


def dev():
    return torch.device("cuda:0")


def ref(d, flags):
    q, k, a, b = oracle.prepare(d["q"], d["k"], d["alpha"], d["beta"], d["gate"],
                                lead=tuple(d["q"].shape[:3]), **flags)
    return oracle.forward(q, k, d["v"], a, b, d["initial_state"],
                          cu_seqlens=d.get("cu_seqlens_host"))


def run(kda, d, flags, **kw):
    return kda.kda_chunk_fwd_fused(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                   d["initial_state"], cu_seqlens=d.get("cu_seqlens"),
                                   cu_seqlens_host=d.get("cu_seqlens_host"),
                                   gate_kind=d["gate"], **flags, **kw)


def draw(dt, B, T, H, dk, dv, s0, gate, flags, seed):
    """Raw draws; the tensors a flag does not cover are stored prepared."""
    d = gen.draw_chunk(B, T, H, dk, dv, dt, alpha_mu=3.0, s0_std=s0, seed=seed, device=dev(),
                       gate=gate, raw=True)
    if gate != "none" and not flags["gate_logits"]:
        d["alpha"] = torch.sigmoid(d["alpha"].double()).float().contiguous()
    if not flags["beta_logits"]:
        d["beta"] = torch.sigmoid(d["beta"].double()).float().contiguous()
    if not flags["qk_l2norm"]:
        for n in ("q", "k"):
            x = d[n].double()
            d[n] = (x / x.norm(dim=-1, keepdim=True)).to(d[n].dtype).contiguous()
    return d


NONE_ = dict(gate_logits=False, beta_logits=False, qk_l2norm=False)
CASES = [
    # dtype, B, T, H, dk, dv, s0_std, dvt, gate, flags
    ("f32", 1, 200, 2, 64, 64, None, 16, "channel", ALL),
    ("f32", 2, 77, 1, 64, 128, 0.1, 64, "head", ALL),
    ("f32", 1, 100, 1, 128, 128, 0.1, 16, "none", dict(NONE_, qk_l2norm=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 16, "channel", ALL),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "channel", ALL),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 64, "channel", ALL),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "head", ALL),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 64, "head", ALL),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "none", dict(NONE_, qk_l2norm=True, beta_logits=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "channel", dict(NONE_, gate_logits=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "channel", dict(NONE_, beta_logits=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "channel", dict(NONE_, qk_l2norm=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "head", dict(NONE_, gate_logits=True)),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32, "head", dict(NONE_, qk_l2norm=True)),
    ("bf16", 1, 1, 2, 128, 128, 0.5, None, "channel", ALL),
    ("bf16", 1, 65, 2, 128, 128, 0.5, None, "head", ALL),
    ("bf16", 3, 129, 2, 64, 64, 0.2, 16, "channel", ALL),
    ("bf16", 1, 200, 2, 64, 64, 0.2, 64, "head", ALL),
    ("bf16", 1, 190, 2, 128, 64, 0.2, 32, "channel", ALL),
    ("bf16", 1, 190, 2, 64, 128, 0.2, 64, "none", dict(NONE_, qk_l2norm=True)),
]


def case_id(c):
    f = "".join(n[0] for n in ("gate_logits", "beta_logits", "qk_l2norm") if c[9][n])
    return "-".join(str(x) for x in c[:9]) + "-" + (f or "0")


IDS = [case_id(c) for c in CASES]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=IDS)
def test_fused_chunk_small(kda, idx):
    c = CASES[idx]
    print("case", IDS[idx], flush=True)
    d = draw(*c[:7], c[8], c[9], 500 + idx)
    with dvt_env(c[7]):
        o, s = run(kda, d, c[9])
    torch.cuda.synchronize()
    ro, rs = ref(d, c[9])
    assert rel(o, ro) <= TOL[c[0]]
    assert rel(s, rs) <= TOL[c[0]]


@pytest.mark.parametrize("idx", [i for i, c in enumerate(CASES) if c[0] == "bf16"],
                         ids=[i for i, c in zip(IDS, CASES) if c[0] == "bf16"])
def test_fused_chunk_small_generic_kernel(kda, idx):
    c = CASES[idx]
    print("case", IDS[idx], flush=True)
    d = draw(*c[:7], c[8], c[9], 500 + idx)
    with dvt_env(c[7], generic=True):
        o, s = run(kda, d, c[9])
    torch.cuda.synchronize()
    ro, rs = ref(d, c[9])
    assert rel(o, ro) <= TOL[c[0]]
    assert rel(s, rs) <= TOL[c[0]]


def test_fused_varlen_small(kda):
    lens = [0, 1, 64, 65, 200, 0, 7, 130]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = draw("bf16", 1, cu[-1], 3, 128, 128, 0.1, "channel", ALL, 61)
    d["initial_state"] = torch.randn((len(lens), 3, 128, 128), device=dev(),
                                     generator=torch.Generator(device=dev()).manual_seed(1)) * 0.1
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    o, s = run(kda, d, ALL)
    torch.cuda.synchronize()
    ro, rs = ref(d, ALL)
    assert rel(o, ro) <= 2e-2
    assert rel(s, rs) <= 2e-2
    assert torch.equal(s[0], d["initial_state"][0]) and torch.equal(s[5], d["initial_state"][5])


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_fused_chunk_full_B4_H16_T4096(kda, gate):
    """The B4 H16 T4096 d128 workload drawn raw (logits, unnormalised q and k):
    every output against the oracle."""
    d = gen.chunk_inputs(CONFIGS[1], device=dev(), gate=gate, raw=True)
    o, s = run(kda, d, ALL)
    torch.cuda.synchronize()
    ro, rs = ref(d, ALL)
    eo, es = rel(o, ro), rel(s, rs)
    print("B4 H16 T4096 fused, gate %s: err o %.2e state %.2e" % (gate, eo, es))
    assert eo <= 2e-2 and es <= 2e-2


def test_fused_equals_prepared_inputs(kda):
    """The fused call against the unfused one fed inputs prepared on the host
    in float32 (sigmoid, L2 norm, then rounded like the stored tensors): the
    two differ only by that rounding."""
    d = draw("bf16", 2, 200, 2, 128, 128, 0.1, "channel", ALL, 71)
    o1, s1 = run(kda, d, ALL)
    x = {n: d[n].double() for n in ("q", "k")}
    qn = (x["q"] / (x["q"].pow(2).sum(-1, keepdim=True) + 1e-6).sqrt()).to(torch.bfloat16)
    kn = (x["k"] / (x["k"].pow(2).sum(-1, keepdim=True) + 1e-6).sqrt()).to(torch.bfloat16)
    a = torch.sigmoid(d["alpha"].double()).float().contiguous()
    b = torch.sigmoid(d["beta"].double()).float().contiguous()
    o2, s2 = kda.kda_chunk_fwd(qn.contiguous(), kn.contiguous(), d["v"], a, b, d["initial_state"])
    torch.cuda.synchronize()
    assert rel(o1, o2.double().cpu().numpy()) <= 2e-2
    assert rel(s1, s2.double().cpu().numpy()) <= 2e-2


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dt,dk,dv", [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128)])
def test_fused_step_small(kda, gate, dt, dk, dv):
    from workloads.configs import Config
    cfg = Config("t", "decode", dt, 3, 1, 5, dk, dv, 4.0, 0.3, steps=6, seed=81)
    d = gen.decode_inputs(cfg, device=dev(), gate=gate, raw=True)
    flags = dict(ALL, gate_logits=gate != "none")
    st = d["state"].clone()
    ref_state = d["state"]
    for t in range(cfg.steps):
        a = None if gate == "none" else d["alpha"][t]
        q, k, v, b = d["q"][t], d["k"][t], d["v"][t], d["beta"][t]
        qn, kn, an, bn = oracle.prepare(q, k, a, b, gate, lead=(3, 5), **flags)
        ro, ref_state = oracle.step(qn, kn, v, an, bn, ref_state)
        o = kda.kda_recurrent_step_fused(q, k, v, a, b, st, gate_kind=gate, **flags)
        torch.cuda.synchronize()
        assert rel(o, ro) <= TOL[dt], t
    assert rel(st, ref_state) <= TOL[dt]
