"""GPU parity of kda_backward (gradients of the chunk-wise forward) against
the fp64 oracle's reverse sweep (oracle.backward, itself pinned by central
differences of the oracle's forward).  Error: max |g_gpu - g_ref| / max
|g_ref| per gradient.  bf16 inputs take the chunk form on the matrix cores
(bf16 operands, fp32 accumulation) and are held to the bf16 bound 2e-2;
float32 inputs take the token recurrence in fp32 and are held to 1e-4."""
import numpy as np
import pytest
import torch

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
NAMES = ["dq", "dk", "dv", "dalpha", "dbeta", "dinitial_state"]


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
    x = x.detach().double().cpu().numpy()
    assert not np.isnan(x).any(), "NaN in GPU output"
    den = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(x - ref)) / den)


def grads_inputs(dt, B, T, H, dk, dv, s0, with_dsT, seed, num_states=None):
    d = gen.draw_chunk(B, T, H, dk, dv, dt, alpha_mu=3.0, s0_std=s0, seed=seed, device=dev(),
                       num_states=num_states)
    g = torch.Generator(device=dev())
    g.manual_seed(seed + 7)
    d["dout"] = torch.randn((B, T, H, dv), generator=g, device=dev(), dtype=torch.float64).to(
        d["q"].dtype).contiguous()
    ns = B if num_states is None else num_states
    d["dsT"] = (torch.randn((ns, H, dk, dv), generator=g, device=dev(), dtype=torch.float64)
                .float().contiguous() if with_dsT else None)
    return d


def check(kda, d, cu=None):
    got = kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                           d["dout"], d["dsT"], cu_seqlens=d.get("cu_seqlens"),
                           cu_seqlens_host=cu)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                          d["dout"], d["dsT"], cu_seqlens=cu)
    errs = {n: rel(g, r) for n, g, r in zip(NAMES, got, ref)}
    print("errors", {n: "%.1e" % e for n, e in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[d["q"].dtype], (n, e)


CASES = [
    # dtype, B, T, H, dk, dv, s0_std, dS_T
    ("f32", 1, 37, 2, 64, 64, 0.3, True),
    ("f32", 2, 16, 1, 128, 128, None, False),
    ("f32", 1, 50, 2, 128, 64, 0.2, True),
    ("bf16", 2, 100, 2, 128, 128, 0.1, True),
    ("bf16", 1, 33, 3, 64, 128, 0.1, False),
    ("bf16", 1, 1, 2, 128, 128, 0.5, True),
    ("bf16", 1, 64, 2, 128, 128, None, True),
    ("bf16", 1, 65, 2, 64, 64, 0.3, True),
    ("bf16", 2, 190, 3, 128, 64, 0.2, True),
    ("bf16", 1, 130, 2, 64, 128, 0.2, False),
]


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=["-".join(str(x) for x in c) for c in CASES])
def test_backward_small(kda, idx):
    c = CASES[idx]
    print("case", c, flush=True)
    check(kda, grads_inputs(*c, seed=700 + idx))


def test_backward_varlen(kda):
    lens = [0, 1, 16, 17, 40, 0, 5]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = grads_inputs("bf16", 1, cu[-1], 2, 128, 128, 0.1, True, seed=790, num_states=len(lens))
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    check(kda, d, cu=cu)


def test_backward_longer(kda):
    """512 tokens, two heads, d128."""
    check(kda, grads_inputs("bf16", 1, 512, 2, 128, 128, 0.02, True, seed=795))


def test_backward_varlen_more_heads(kda):
    """Eight heads, lengths that are not multiples of 8 or 64 (and an empty
    sequence), dk = 128, dv = 64."""
    lens = [77, 3, 0, 130, 9, 200]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = grads_inputs("bf16", 1, cu[-1], 8, 128, 64, 0.1, True, seed=797, num_states=len(lens))
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    check(kda, d, cu=cu)


def test_backward_no_tokens(kda):
    """Units but no tokens (T = 0 dense, and varlen with every sequence empty):
    the initial-state gradient is the final-state gradient."""
    d = grads_inputs("bf16", 2, 0, 3, 128, 128, 0.1, True, seed=798)
    got = kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                           d["dout"], d["dsT"])
    torch.cuda.synchronize()
    assert torch.equal(got[5], d["dsT"])
    cu = [0, 0, 0]
    d = grads_inputs("bf16", 1, 0, 3, 64, 64, 0.1, True, seed=799, num_states=2)
    got = kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                           d["dout"], d["dsT"], cu_seqlens_host=cu)
    torch.cuda.synchronize()
    assert torch.equal(got[5], d["dsT"])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_bitwise_reproducible(kda, dt):
    """Two calls on the same inputs give the same gradients bit for bit (bf16:
    the value-column slices' partial sums are added in a fixed order)."""
    d = grads_inputs(dt, 2, 300 if dt == "bf16" else 70, 3, 128, 128, 0.1, True, seed=801)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"], d["dout"], d["dsT"])
    a = kda.kda_backward(*args)
    b = kda.kda_backward(*args)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, a, b):
        if dt == "bf16" or n in ("dv", "dinitial_state"):
            assert torch.equal(x, y), n


def test_backward_outputs_at_odd_offsets(kda):
    """Gradient tensors that start 4 bytes past a 16-byte boundary (views into
    larger buffers): the same values as freshly allocated outputs."""
    d = grads_inputs("bf16", 1, 150, 2, 128, 128, 0.1, True, seed=803)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"], d["dout"], d["dsT"])
    ref = kda.kda_backward(*args)
    out = []
    for i, x in enumerate(ref):
        if i == 5:  # the state gradient keeps its 16-byte alignment
            out.append(torch.empty_like(x))
        else:
            buf = torch.empty(x.numel() + 1, dtype=torch.float32, device=dev())
            out.append(buf[1:].view(x.shape))
    got = kda.kda_backward(*args, out=tuple(out))
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, got, ref):
        assert torch.equal(x, y), n


def test_backward_full_B4_H16_T4096(kda):
    """The benchmarked backward call (bf16 B4 H16 T4096 d128, S0 ~ N(0, 0.02),
    random dL/do and dL/dS_T): every (batch, head) unit compared with the
    oracle, four heads (16 units) at a time."""
    from workloads import CONFIGS
    cfg = CONFIGS[1]
    d = gen.chunk_inputs(cfg, device=dev())
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    g = torch.Generator(device=dev())
    g.manual_seed(11)
    dout = torch.randn((B, T, H, dv), generator=g, device=dev(), dtype=torch.float64).to(
        torch.bfloat16)
    dsT = torch.randn((B, H, dk, dv), generator=g, device=dev(), dtype=torch.float64).float()
    got = kda.kda_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                           dout, dsT)
    torch.cuda.synchronize()
    got = [x.double().cpu().numpy() for x in got]
    for x in got:
        assert not np.isnan(x).any(), "NaN in GPU output"
    num = [0.0] * 6
    den = [0.0] * 6
    for h0 in range(0, H, 4):
        heads = list(range(h0, h0 + 4))
        ref = oracle.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                              dout, dsT, heads=heads)
        for i in range(6):
            gx = got[i][:, heads] if i == 5 else got[i][:, :, heads]
            num[i] = max(num[i], float(np.max(np.abs(gx - ref[i]))))
            den[i] = max(den[i], float(np.max(np.abs(ref[i]))))
    errs = {n: num[i] / den[i] for i, n in enumerate(NAMES)}
    print("B4 H16 T4096 backward, all units:", {n: "%.1e" % e for n, e in errs.items()},
          flush=True)
    for n, e in errs.items():
        assert e <= TOL[torch.bfloat16], (n, e)
