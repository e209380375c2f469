"""GPU parity of the Gated DeltaNet-2 kernels (kda_gdn2_chunk_fwd and
kda_gdn2_recurrent_step, through the C ABI) against the fp64 oracle
(oracle.gdn2_*, pinned in test_oracle_gdn2.py).  Error metric and bounds as
for KDA: max |x_gpu - x_ref| / max |x_ref|, 2e-2 for bf16 inputs and 1e-4
for float32 inputs (decode), on o and on the final state; NaN fails."""
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as lib
    lib.load_library()
    return lib


def dev():
    return torch.device("cuda:0")


def rel(x, ref):
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x)
    assert not np.isnan(x).any(), "NaN in GPU output"
    return float(np.max(np.abs(x - ref), initial=0.0) / max(float(np.max(np.abs(ref), initial=0.0)), 1e-30))


def run(kda, d, **kw):
    return kda.kda_gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["erase"], d["write"],
                                  d["initial_state"], cu_seqlens=d.get("cu_seqlens"),
                                  cu_seqlens_host=d.get("cu_seqlens_host"), **kw)


def ref(d, heads=None):
    return oracle.gdn2_forward(d["q"], d["k"], d["v"], d["alpha"], d["erase"], d["write"],
                               d["initial_state"], cu_seqlens=d.get("cu_seqlens_host"),
                               heads=heads)


class dvt_env:
    def __init__(self, dvt):
        self.dvt = dvt

    def __enter__(self):
        self.old = os.environ.get("KDA_CHUNK_DVT")
        if self.dvt:
            os.environ["KDA_CHUNK_DVT"] = str(self.dvt)
        else:
            os.environ.pop("KDA_CHUNK_DVT", None)

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("KDA_CHUNK_DVT", None)
        else:
            os.environ["KDA_CHUNK_DVT"] = self.old


CASES = [
    # B, T, H, dk, dv, s0_std, dvt, forget
    (2, 300, 3, 128, 128, 0.02, 16, True),
    (2, 300, 3, 128, 128, 0.02, 32, True),
    (1, 1, 2, 128, 128, 0.5, None, True),
    (1, 63, 2, 128, 128, 0.5, None, True),
    (1, 64, 2, 128, 128, 0.5, None, True),
    (1, 65, 2, 128, 128, 0.5, None, True),
    (3, 129, 2, 64, 64, 0.2, 16, True),
    (1, 200, 2, 64, 64, 0.2, 64, True),
    (1, 190, 2, 64, 128, 0.2, 32, True),
    (1, 190, 2, 128, 64, 0.2, 32, True),
    (2, 150, 2, 128, 128, None, None, False),
]


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=["-".join(str(x) for x in c) for c in CASES])
def test_gdn2_chunk_small(kda, idx):
    B, T, H, dk, dv, s0, dvt, forget = CASES[idx]
    print("case", CASES[idx], flush=True)
    d = gen.draw_gdn2(B, T, H, dk, dv, "bf16", alpha_mu=3.0, s0_std=s0, seed=300 + idx,
                      device=dev(), forget=forget)
    with dvt_env(dvt):
        o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    eo, es = rel(o, ro), rel(s, rs)
    print("err o %.2e state %.2e" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("mode", ["kda", "no_erase", "no_write", "full_erase_write"])
def test_gdn2_chunk_special_gates(kda, mode):
    """Gates at the special cases the page's table names: e = w = beta (KDA:
    compared with the KDA chunk kernel and the oracle), e = 0 (gated linear
    attention), w = 0 (nothing written), e = w = 1."""
    d = gen.draw_gdn2(2, 257, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.3, seed=320,
                      device=dev())
    if mode == "kda":
        beta = torch.sigmoid(torch.randn((2, 257, 2), device=dev(), dtype=torch.float64)).float()
        d["erase"] = beta[..., None].expand(-1, -1, -1, 128).contiguous()
        d["write"] = d["erase"].clone()
    elif mode == "no_erase":
        d["erase"].zero_()
    elif mode == "no_write":
        d["write"].zero_()
    else:
        d["erase"].fill_(1.0)
        d["write"].fill_(1.0)
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2 and rel(s, rs) <= 2e-2
    if mode == "kda":
        ok, sk = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], beta, d["initial_state"])
        torch.cuda.synchronize()
        assert rel(o, ok.double().cpu().numpy()) <= 2e-2
        assert rel(s, sk.double().cpu().numpy()) <= 2e-2


def test_gdn2_chunk_varlen_small(kda):
    lens = [0, 1, 64, 65, 200, 0, 7, 130]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = gen.draw_gdn2(1, cu[-1], 3, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.1,
                      num_states=len(lens), seed=330, device=dev())
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2 and rel(s, rs) <= 2e-2
    assert torch.equal(s[0], d["initial_state"][0]) and torch.equal(s[5], d["initial_state"][5])


def test_gdn2_chunk_full_B4_H16_T4096(kda):
    """The benchmarked Gated DeltaNet-2 workload (the headline's shapes): every
    (batch, head) unit compared."""
    d = gen.draw_gdn2(4, 4096, 16, 128, 128, "bf16", alpha_mu=4.0, s0_std=0.02, seed=1,
                      device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    eo, es = rel(o, ro), rel(s, rs)
    print("GDN-2 B4 H16 T4096 all units: err o %.2e state %.2e" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2


def test_gdn2_chunk_deterministic_and_in_place(kda):
    d = gen.draw_gdn2(2, 500, 4, 128, 128, "bf16", alpha_mu=4.0, s0_std=0.05, seed=340,
                      device=dev())
    o1, s1 = run(kda, d)
    o2, s2 = run(kda, d)
    st = d["initial_state"].clone()
    o3, s3 = kda.kda_gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["erase"], d["write"],
                                    st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, st)


@pytest.mark.parametrize("dt,dk,dv,forget", [(torch.float32, 64, 64, True),
                                             (torch.float32, 128, 128, False),
                                             (torch.bfloat16, 128, 128, True),
                                             (torch.bfloat16, 64, 128, True),
                                             (torch.bfloat16, 128, 64, False)])
def test_gdn2_step_small(kda, dt, dk, dv, forget):
    N, H, steps = 3, 5, 6
    g = torch.Generator(device=dev())
    g.manual_seed(350 + dk + dv)
    st = (0.3 * torch.randn((N, H, dk, dv), generator=g, device=dev(), dtype=torch.float64)).float()
    ref_state = oracle._f64(st)
    for t in range(steps):
        d = gen.draw_gdn2(N, 1, H, dk, dv, "f32" if dt == torch.float32 else "bf16",
                          alpha_mu=3.0, seed=360 + t, device=dev(), forget=forget)
        args = [None if d[n] is None else d[n][:, 0].contiguous()
                for n in ("q", "k", "v", "alpha", "erase", "write")]
        ro, ref_state = oracle.gdn2_step(*args, ref_state, in_place=True)
        o = kda.kda_gdn2_recurrent_step(*args, st)
        torch.cuda.synchronize()
        assert rel(o, ro) <= TOL[dt], t
    assert rel(st, ref_state) <= TOL[dt]


def test_gdn2_step_full_N256_H32_100_steps(kda):
    """Decode at the KDA decode workload's shapes (N256 H32 d128, fp32 state
    ~ N(0, 0.05) in place, 100 steps): o of every unit at every step and all
    8192 final states."""
    N, H, d_ = 256, 32, 128
    g = torch.Generator(device=dev())
    g.manual_seed(3)
    st = (0.05 * torch.randn((N, H, d_, d_), generator=g, device=dev(), dtype=torch.float64)).float()
    ref_state = oracle._f64(st)
    num = den = 0.0
    for t in range(100):
        d = gen.draw_gdn2(N, 1, H, d_, d_, "bf16", alpha_mu=4.0, seed=1000 + t, device=dev())
        args = [d[n][:, 0].contiguous() for n in ("q", "k", "v", "alpha", "erase", "write")]
        o = kda.kda_gdn2_recurrent_step(*args, st)
        ro, ref_state = oracle.gdn2_step(*args, ref_state, in_place=True)
        go = o.double().cpu().numpy()
        assert not np.isnan(go).any()
        num = max(num, float(np.max(np.abs(go - ro))))
        den = max(den, float(np.max(np.abs(ro))))
    es = rel(st, ref_state)
    print("GDN-2 decode N256 H32 x100 all units: err o %.2e state %.2e" % (num / den, es))
    assert num / den <= 2e-2 and es <= 2e-2


def test_gdn2_chunk_equals_repeated_steps(kda):
    d = gen.draw_gdn2(2, 100, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.2, seed=370,
                      device=dev())
    o, s = run(kda, d)
    st = d["initial_state"].clone()
    outs = []
    for t in range(100):
        outs.append(kda.kda_gdn2_recurrent_step(*[d[n][:, t].contiguous() for n in
                                                  ("q", "k", "v", "alpha", "erase", "write")],
                                                st))
    torch.cuda.synchronize()
    o_steps = torch.stack(outs, 1)
    assert float((o.float() - o_steps.float()).abs().max()) / float(o.abs().max()) <= 2e-2
    assert float((s - st).abs().max()) / float(s.abs().max()) <= 2e-2
