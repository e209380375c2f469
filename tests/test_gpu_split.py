"""GPU parity of the two-segment path of the chunk-wise forward (dense bf16
calls with dk = dv = 128, at most 32 (batch, head) units and at least 64
chunks, given the workspace of kda_chunk_fwd_split_workspace_size): every
output against the fp64 oracle, with the same metric and bound as the other
parity tests (max |x_gpu - x_ref| / max |x_ref| <= 2e-2 for bf16 inputs), and
against the single pass of the same call.  The long-context workload itself
(B1 H32 T65536) is compared on every head in test_gpu_parity.py, through both
paths."""
import numpy as np
import pytest
import torch

import oracle
from workloads import gen
from test_gpu_parity import rel, TOL

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


def split_ws(kda, d):
    B, T, H, dk = d["q"].shape
    n = kda.kda_chunk_fwd_split_workspace_size(B, T, H, dk, d["v"].shape[-1])
    assert n > 0, "shape does not take the two-segment path"
    return torch.empty(n, dtype=torch.uint8, device=dev())


CASES = [
    # B, T, H, s0_std, alpha_mu, gate, fused
    (1, 5000, 4, 0.05, 4.0, "channel", False),   # ragged last chunk
    (2, 4500, 3, 0.05, 3.0, "channel", False),   # two sequences
    (1, 4096, 2, None, 5.0, "channel", False),   # zero start, whole chunks
    (1, 4160, 8, 0.05, 4.0, "head", False),      # Gated DeltaNet
    (1, 4200, 2, 0.05, 4.0, "none", False),      # DeltaNet
    (1, 4321, 3, 0.05, 3.0, "channel", True),    # gate and beta logits, q/k L2 norm in-kernel
    (1, 4300, 2, 0.1, -3.0, "channel", False),   # every chunk out of the chunk form's range
]


@pytest.mark.parametrize("B,T,H,s0,mu,gate,fused", CASES)
def test_split_matches_oracle_and_single_pass(kda, B, T, H, s0, mu, gate, fused):
    d = gen.draw_chunk(B, T, H, 128, 128, "bf16", alpha_mu=mu, s0_std=s0, seed=B * 7 + H,
                       device=dev(), gate=gate, raw=fused)
    ws = split_ws(kda, d)
    flags = dict(gate_logits=gate != "none", beta_logits=True, qk_l2norm=True)

    def call(split):
        if fused:
            return kda.kda_chunk_fwd_fused(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                           d["initial_state"], gate_kind=gate,
                                           workspace=ws if split else None, split=split, **flags)
        return kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                       d["initial_state"], gate=gate,
                                       workspace=ws if split else None, split=split)
    o, s = call(True)
    o1, s1 = call(False)
    torch.cuda.synchronize()
    if fused:
        q, k, a, b = oracle.prepare(d["q"], d["k"], d["alpha"], d["beta"], gate,
                                    lead=(B, T, H), **flags)
    else:
        q, k, b = d["q"], d["k"], d["beta"]
        a = oracle.channel_gate(d["alpha"], gate, 128, (B, T, H))
    ro, rs = oracle.forward(q, k, d["v"], a, b, d["initial_state"])
    eo, es = rel(o, ro), rel(s, rs)
    po, ps = rel(o, o1.double().cpu().numpy()), rel(s, s1.double().cpu().numpy())
    print("B%d T%d H%d gate %s fused %s: err o %.2e state %.2e; vs single pass %.2e %.2e"
          % (B, T, H, gate, fused, eo, es, po, ps))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert po <= TOL["bf16"] and ps <= TOL["bf16"]


def test_split_in_place_state_and_no_final_state(kda):
    """final_state == initial_state (in-place update) and a call that wants no
    final state, both through the two-segment path."""
    d = gen.draw_chunk(1, 4500, 2, 128, 128, "bf16", alpha_mu=4.0, s0_std=0.05, seed=5,
                       device=dev())
    ws = split_ws(kda, d)
    ro, rs = oracle.forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"])
    o2, none = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                 d["initial_state"], output_final_state=False, workspace=ws)
    st = d["initial_state"].clone()
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st, final_state=st,
                             workspace=ws)
    torch.cuda.synchronize()
    assert none is None and s.data_ptr() == st.data_ptr()
    assert rel(o, ro) <= TOL["bf16"] and rel(st, rs) <= TOL["bf16"]
    assert torch.equal(o, o2)


def test_split_deterministic(kda):
    d = gen.draw_chunk(1, 4500, 4, 128, 128, "bf16", alpha_mu=4.0, s0_std=0.05, seed=9,
                       device=dev())
    ws = split_ws(kda, d)
    o1, s1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                               d["initial_state"], workspace=ws)
    o2, s2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                               d["initial_state"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
