"""Decode steps captured in a HIP graph: kda_recurrent_step calls recorded with
torch.cuda.CUDAGraph on the capturing stream (the library launches on the
caller's stream and records no memset), then replayed several times with eager
work and synchronisations between the replays.  Every replay must give the
states and outputs of the same steps run eagerly, bit for bit, and the eager
steps match the fp64 oracle (max |x_gpu - x_ref| / max |x_ref| <= 2e-2 for bf16
inputs)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, gen
from test_gpu_parity import rel, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as lib
    lib.load_library()
    return lib


def test_decode_steps_replayed_from_a_graph(kda):
    dev = torch.device("cuda:0")
    steps = 12
    ddc = gen.decode_inputs(CONFIGS[3], device=dev, N=16, H=4, steps=steps)
    s0 = ddc["state"].clone()
    args = [[ddc[n][t] for n in ("q", "k", "v", "alpha", "beta")] for t in range(steps)]
    N, H, dk, dv = s0.shape

    st_e = s0.clone()
    o_e = torch.empty((steps, N, H, dv), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        kda.kda_recurrent_step(*args[t], st_e, o=o_e[t])
    torch.cuda.synchronize()

    st_g = s0.clone()
    o_g = torch.empty_like(o_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            kda.kda_recurrent_step(*args[t], st_g, o=o_g[t])
    for rep in range(3):
        st_g.copy_(s0)   # eager work between replays
        o_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st_g, st_e), "replay %d: state differs from the eager steps" % rep
        assert torch.equal(o_g, o_e), "replay %d: outputs differ from the eager steps" % rep

    st_r = s0.double().cpu().numpy()
    for t in range(steps):
        ro, st_r = oracle.step(*[a.cpu() for a in args[t]], st_r)
        assert rel(o_e[t], ro) <= TOL["bf16"]
    assert rel(st_e, st_r) <= TOL["bf16"]


def test_two_segment_forward_replayed_from_a_graph(kda):
    """The two-segment path forks onto the library's own streams with events and
    joins back; captured from the caller's stream it becomes one graph, whose
    replays give the eager call's outputs and final state bit for bit."""
    dev = torch.device("cuda:0")
    d = gen.draw_chunk(1, 4200, 2, 128, 128, "bf16", alpha_mu=4.0, s0_std=0.05, seed=21,
                       device=dev)
    n = kda.kda_chunk_fwd_split_workspace_size(1, 4200, 2, 128, 128)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    call = lambda o, fs: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                           d["initial_state"], o=o, final_state=fs, workspace=ws)
    o_e = torch.empty_like(d["v"])
    fs_e = torch.empty_like(d["initial_state"])
    call(o_e, fs_e)  # eager first: the library's streams and events exist before the capture
    torch.cuda.synchronize()

    o_g = torch.empty_like(o_e)
    fs_g = torch.empty_like(fs_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(o_g, fs_g)
    for rep in range(3):
        o_g.fill_(0)     # eager work between replays
        fs_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), "replay %d: outputs differ from the eager call" % rep
        assert torch.equal(fs_g, fs_e), "replay %d: final state differs from the eager call" % rep
    ro, rs = oracle.forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"])
    assert rel(o_e, ro) <= TOL["bf16"] and rel(fs_e, rs) <= TOL["bf16"]
