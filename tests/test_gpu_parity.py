"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Error metric: max |x_gpu - x_ref| / max |x_ref| over the tensor, in fp64, for
o and for the final state separately.  Bounds: 1e-4 for fp32 inputs, 2e-2
for bf16 inputs.  Any NaN fails.  Full-size workloads compare every output:
the whole of the B4 H16 T4096 forward, every head of the T = 65536 forward,
every (sequence, head) unit of the packed varlen forward, and o of every unit
at each of the 100 decode steps together with all 8192 final states.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


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
    den = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(x - ref)) / den)


def run(kda, d, **kw):
    return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                             cu_seqlens=d.get("cu_seqlens"),
                             cu_seqlens_host=d.get("cu_seqlens_host"), **kw)


def ref(d, heads=None):
    return oracle.forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                          cu_seqlens=d.get("cu_seqlens_host"), heads=heads)


class dvt_env:
    """Force the value-column tile width of the chunk kernel and, optionally,
    route bf16 through the generic (fp32-capable) chunk kernel."""
    def __init__(self, dvt, generic=False):
        self.vals = {"KDA_CHUNK_DVT": str(dvt) if dvt else None,
                     "KDA_CHUNK_GENERIC": "1" if generic else None}

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.vals}
        for k, v in self.vals.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


# ------------------------------------------------------------ chunk forward

CASES = [
    # dtype, B, T, H, dk, dv, s0_std, dvt
    ("f32", 1, 200, 2, 64, 64, None, 16),
    ("f32", 1, 130, 2, 64, 64, 0.3, 32),
    ("f32", 2, 77, 1, 64, 128, 0.1, 64),
    ("f32", 1, 150, 2, 128, 64, 0.1, 16),
    ("f32", 1, 100, 1, 128, 128, 0.1, 16),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 16),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 32),
    ("bf16", 2, 300, 3, 128, 128, 0.02, 64),
    ("bf16", 1, 1, 2, 128, 128, 0.5, None),
    ("bf16", 1, 63, 2, 128, 128, 0.5, None),
    ("bf16", 1, 64, 2, 128, 128, 0.5, None),
    ("bf16", 1, 65, 2, 128, 128, 0.5, None),
    ("bf16", 3, 129, 2, 64, 64, 0.2, 16),
    ("bf16", 1, 200, 2, 64, 64, 0.2, 64),
    ("bf16", 1, 190, 2, 128, 64, 0.2, 32),
    ("bf16", 1, 190, 2, 64, 128, 0.2, 64),
]


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=["-".join(str(x) for x in c) for c in CASES])
def test_chunk_small(kda, idx):
    case = CASES[idx]
    dt, B, T, H, dk, dv, s0, dvt = case
    print("case", case, flush=True)
    d = gen.draw_chunk(B, T, H, dk, dv, dt, alpha_mu=3.0, s0_std=s0, seed=100 + idx,
                       device=dev())
    with dvt_env(dvt):
        o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= TOL[dt]
    assert rel(s, rs) <= TOL[dt]


@pytest.mark.parametrize("idx", [i for i, c in enumerate(CASES) if c[0] == "bf16"],
                         ids=["-".join(str(x) for x in c) for c in CASES if c[0] == "bf16"])
def test_chunk_small_generic_kernel(kda, idx):
    """The bf16 cases through the generic kernel too (both paths stay green)."""
    case = CASES[idx]
    dt, B, T, H, dk, dv, s0, dvt = case
    d = gen.draw_chunk(B, T, H, dk, dv, dt, alpha_mu=3.0, s0_std=s0, seed=100 + idx,
                       device=dev())
    with dvt_env(dvt, generic=True):
        o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= TOL[dt]
    assert rel(s, rs) <= TOL[dt]


def test_chunk_fp32_config(kda):
    """The fp32 workload: B1 H2 T256 d64, zero start."""
    d = gen.chunk_inputs(CONFIGS[0], device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    eo, es = rel(o, ro), rel(s, rs)
    print("fp32 B1 H2 T256 d64: err o %.2e state %.2e" % (eo, es))
    assert eo <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("mode", ["alpha_one", "beta_zero", "beta_one", "strong_decay",
                                  "zero_keys"])
def test_chunk_degenerate(kda, mode):
    """DeltaNet (alpha = 1), nothing written (beta = 0), full-strength writes
    (beta = 1), fast forgetting within the documented range, and zero keys."""
    d = gen.draw_chunk(2, 257, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.3, seed=5,
                       device=dev())
    if mode == "alpha_one":
        d["alpha"].fill_(1.0)
    elif mode == "beta_zero":
        d["beta"].zero_()
    elif mode == "beta_one":
        d["beta"].fill_(1.0)
    elif mode == "strong_decay":
        d = gen.draw_chunk(2, 257, 2, 128, 128, "bf16", alpha_mu=0.0, s0_std=0.3, seed=6,
                           device=dev())
    elif mode == "zero_keys":
        d["k"].zero_()
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2
    assert rel(s, rs) <= 2e-2


def test_chunk_varlen_small(kda):
    """Packed sequences with empty, one-token, exact-chunk and ragged lengths."""
    lens = [0, 1, 64, 65, 200, 0, 7, 130]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = gen.draw_chunk(1, cu[-1], 3, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.1,
                       num_states=len(lens), seed=9, device=dev())
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2
    assert rel(s, rs) <= 2e-2
    # empty sequences keep their initial state exactly
    assert torch.equal(s[0], d["initial_state"][0]) and torch.equal(s[5], d["initial_state"][5])


def test_chunk_varlen_reduced(kda):
    """The varlen workload with every length scaled down (same length mix)."""
    d = gen.chunk_inputs(CONFIGS[4], device=dev(), T=6000, H=4)
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    assert rel(o, ro) <= 2e-2
    assert rel(s, rs) <= 2e-2


def test_chunk_in_place_and_optional_state(kda):
    d = gen.draw_chunk(2, 150, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.2, seed=11,
                       device=dev())
    ro, rs = ref(d)
    st = d["initial_state"].clone()
    o1, s1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st,
                               final_state=st)
    o2, s2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                               output_final_state=False)
    torch.cuda.synchronize()
    assert s1.data_ptr() == st.data_ptr() and s2 is None
    assert rel(st, rs) <= 2e-2
    assert torch.equal(o1, o2)


# ------------------------------------------------------------ full sizes

def test_chunk_full_B4_H16_T4096(kda):
    d = gen.chunk_inputs(CONFIGS[1], device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    ro, rs = ref(d)
    eo, es = rel(o, ro), rel(s, rs)
    print("B4 H16 T4096: err o %.2e state %.2e" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2


def _heads(d, heads):
    out = {}
    for n in ("q", "k", "v", "alpha", "beta"):
        out[n] = d[n][:, :, heads].contiguous()
    out["initial_state"] = None if d["initial_state"] is None else \
        d["initial_state"][:, heads].contiguous()
    out["cu_seqlens_host"] = d.get("cu_seqlens_host")
    return out


def test_chunk_full_T65536_all_heads(kda):
    """The long-context workload, every head compared over all 65536 tokens,
    through both the two-segment path (the binding's default for this shape)
    and the single pass; the oracle runs 8 heads at a time to bound host
    memory."""
    d = gen.chunk_inputs(CONFIGS[2], device=dev())
    B, T, H, dk = d["q"].shape
    assert kda.kda_chunk_fwd_split_workspace_size(B, T, H, dk, d["v"].shape[-1]) > 0
    outs = {"split": run(kda, d), "single": run(kda, d, split=False)}
    torch.cuda.synchronize()
    num = {p: [0.0, 0.0] for p in outs}
    den_o = den_s = 0.0
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(H, h0 + 8)))
        ro, rs = ref(_heads(d, heads))
        den_o = max(den_o, float(np.max(np.abs(ro))))
        den_s = max(den_s, float(np.max(np.abs(rs))))
        for p, (o, s) in outs.items():
            go = o[:, :, heads].double().cpu().numpy()
            gs = s[:, heads].double().cpu().numpy()
            assert not np.isnan(go).any() and not np.isnan(gs).any()
            num[p][0] = max(num[p][0], float(np.max(np.abs(go - ro))))
            num[p][1] = max(num[p][1], float(np.max(np.abs(gs - rs))))
    for p in outs:
        eo, es = num[p][0] / den_o, num[p][1] / den_s
        print("B1 H32 T65536 all heads, %s: err o %.2e state %.2e" % (p, eo, es))
        assert eo <= 2e-2 and es <= 2e-2


def test_chunk_full_varlen_all_units(kda):
    """The packed workload (64 sequences of 128..8192 tokens, H16): every
    (sequence, head) unit compared, o over the whole packed tensor and all 64
    final states; per-sequence errors are printed for the worst sequences."""
    d = gen.chunk_inputs(CONFIGS[4], device=dev())
    o, s = run(kda, d)
    torch.cuda.synchronize()
    cu = d["cu_seqlens_host"]
    go_all = o.double().cpu().numpy()
    gs_all = s.double().cpu().numpy()
    assert not np.isnan(go_all).any() and not np.isnan(gs_all).any()
    num_o = num_s = den_o = den_s = 0.0
    per_seq = []
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        sub = {k: d[k][:, a:b].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        sub["initial_state"] = d["initial_state"][n:n + 1].contiguous()
        ro, rs = ref(sub)
        eo_n = float(np.max(np.abs(go_all[:, a:b] - ro), initial=0.0))
        es_n = float(np.max(np.abs(gs_all[n:n + 1] - rs)))
        num_o, num_s = max(num_o, eo_n), max(num_s, es_n)
        den_o = max(den_o, float(np.max(np.abs(ro), initial=0.0)))
        den_s = max(den_s, float(np.max(np.abs(rs))))
        per_seq.append((eo_n / max(float(np.max(np.abs(ro), initial=0.0)), 1e-30), b - a, n))
    eo, es = num_o / den_o, num_s / den_s
    worst = sorted(per_seq, reverse=True)[:3]
    print("varlen 64 seqs x H16, all units: err o %.2e state %.2e; worst sequences "
          "(err, len, index) %s" % (eo, es, [("%.1e" % e, L, n) for e, L, n in worst]))
    assert eo <= 2e-2 and es <= 2e-2


# ------------------------------------------------------------ decode

@pytest.mark.parametrize("dt,dk,dv", [("f32", 64, 64), ("f32", 128, 128), ("bf16", 128, 128),
                                      ("bf16", 64, 128), ("bf16", 128, 64), ("bf16", 64, 64)])
def test_step_small(kda, dt, dk, dv):
    from workloads.configs import Config
    cfg = Config("t", "decode", dt, 3, 1, 5, dk, dv, 4.0, 0.3, steps=6, seed=21)
    d = gen.decode_inputs(cfg, device=dev())
    st = d["state"].clone()
    ref_state = d["state"]
    for t in range(cfg.steps):
        args = [d[n][t] for n in ("q", "k", "v", "alpha", "beta")]
        ro, ref_state = oracle.step(*args, ref_state)
        o = kda.kda_recurrent_step(*args, st)
        torch.cuda.synchronize()
        assert rel(o, ro) <= TOL[dt], t
    assert rel(st, ref_state) <= TOL[dt]


def test_step_full_100_steps_all_units(kda):
    """The decode workload: N256 H32 d128, 100 steps in place; o of every
    (sequence, head) unit at every step and the final state of all 8192 units
    are compared with the oracle run over the same 100 steps."""
    cfg = CONFIGS[3]
    d = gen.decode_inputs(cfg, device=dev())
    st = d["state"].clone()
    outs = []
    for t in range(cfg.steps):
        args = [d[n][t] for n in ("q", "k", "v", "alpha", "beta")]
        outs.append(kda.kda_recurrent_step(*args, st))
    torch.cuda.synchronize()
    ref_state = oracle._f64(d["state"])
    num = den = 0.0
    for t in range(cfg.steps):
        args = [d[n][t] for n in ("q", "k", "v", "alpha", "beta")]
        ro, ref_state = oracle.step(*args, ref_state, in_place=True)
        go = outs[t].double().cpu().numpy()
        assert not np.isnan(go).any()
        num = max(num, float(np.max(np.abs(go - ro))))
        den = max(den, float(np.max(np.abs(ro))))
    worst = num / den
    es = rel(st, ref_state)
    print("decode N256 H32 d128 x100, all units: err o %.2e state %.2e" % (worst, es))
    assert worst <= 2e-2 and es <= 2e-2


# ------------------------------------------------------------ cross-checks

def test_chunk_equals_repeated_steps(kda):
    """The two compute modes agree: a chunk-wise pass over T tokens and T
    decode steps from the same start (both on the GPU, both near the oracle)."""
    d = gen.draw_chunk(2, 100, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.2, seed=13,
                       device=dev())
    o, s = run(kda, d)
    st = d["initial_state"].clone()
    outs = []
    for t in range(100):
        outs.append(kda.kda_recurrent_step(*[d[n][:, t].contiguous() for n in
                                             ("q", "k", "v", "alpha", "beta")], st))
    torch.cuda.synchronize()
    o_steps = torch.stack(outs, 1)
    scale = float(o.abs().max())
    assert float((o.float() - o_steps.float()).abs().max()) / scale <= 2e-2
    assert float((s - st).abs().max()) / float(s.abs().max()) <= 2e-2


def test_chunk_deterministic(kda):
    d = gen.chunk_inputs(CONFIGS[1], device=dev(), T=1000, H=4)
    o1, s1 = run(kda, d)
    o2, s2 = run(kda, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_chunk_resume(kda):
    """Running x1 then x2 from x1's final state matches the oracle on x1 || x2."""
    d = gen.draw_chunk(1, 333, 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.2, seed=17,
                       device=dev())
    ro, rs = ref(d)
    cut = 150
    part = lambda a, b: {n: d[n][:, a:b].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    o1, s1 = kda.kda_chunk_fwd(**part(0, cut), initial_state=d["initial_state"])
    o2, s2 = kda.kda_chunk_fwd(**part(cut, 333), initial_state=s1)
    torch.cuda.synchronize()
    assert rel(torch.cat([o1, o2], 1), ro) <= 2e-2
    assert rel(s2, rs) <= 2e-2


def test_varlen_equals_dense_per_sequence(kda):
    """With the same column tiling, each packed sequence is computed exactly as
    a dense call on that sequence alone (bitwise)."""
    lens = [100, 37, 256]
    cu = [0, 100, 137, 393]
    d = gen.draw_chunk(1, cu[-1], 2, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.1, num_states=3,
                       seed=19, device=dev())
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    with dvt_env(32):
        o, s = run(kda, d)
        for n in range(3):
            a, b = cu[n], cu[n + 1]
            on, sn = kda.kda_chunk_fwd(*[d[x][:, a:b].contiguous() for x in
                                         ("q", "k", "v", "alpha", "beta")],
                                       initial_state=d["initial_state"][n:n + 1].contiguous())
            torch.cuda.synchronize()
            assert torch.equal(on, o[:, a:b]) and torch.equal(sn, s[n:n + 1])
