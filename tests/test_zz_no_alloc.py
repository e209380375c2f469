"""kda_chunk_fwd_noalloc (the entry point that allocates nothing, its scratch
in a fixed device array) against kda_chunk_fwd on the same inputs: packed
sequences twice in a row, the second call smaller, and a dense call; and the
size limit rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle
from workloads import gen

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


def rel(x, ref):
    x = x.detach().double().cpu().numpy()
    assert not np.isnan(x).any(), "NaN in GPU output"
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def packed(lens, H, seed):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    d = gen.draw_chunk(1, cu[-1], H, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.1,
                       num_states=len(lens), seed=seed, device=dev())
    d["cu_seqlens_host"] = cu
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=dev())
    return d


def both(kda, d):
    ns = d["initial_state"].shape[0]
    H = d["q"].shape[2]
    o_ref, s_ref = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                     d["initial_state"], cu_seqlens=d["cu_seqlens"],
                                     cu_seqlens_host=d["cu_seqlens_host"])
    o = torch.empty_like(d["v"])
    s = torch.empty((ns, H, 128, 128), dtype=torch.float32, device=dev())
    kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                              o, s, cu_seqlens=d["cu_seqlens"],
                              cu_seqlens_host=d["cu_seqlens_host"])
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


def test_noalloc_varlen_twice_then_smaller(kda):
    rng = np.random.default_rng(3)
    big = [int(x) for x in rng.integers(0, 300, 40)] + [0, 1, 64, 65]
    small = [130, 0, 7, 200, 64, 3]
    for i, lens in enumerate([big, small]):
        d = packed(lens, 3, seed=50 + i)
        o, s, o_ref, s_ref = both(kda, d)
        print("call %d: %d sequences, %d tokens" % (i, len(lens), sum(lens)), flush=True)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        ro, rs = oracle.forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                d["initial_state"], cu_seqlens=d["cu_seqlens_host"])
        assert rel(o, ro) <= 2e-2 and rel(s, rs) <= 2e-2


def test_noalloc_dense_matches(kda):
    d = gen.draw_chunk(2, 300, 4, 128, 128, "bf16", alpha_mu=3.0, s0_std=0.05, seed=61,
                       device=dev())
    o_ref, s_ref = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                     d["initial_state"])
    o = torch.empty_like(d["v"])
    s = torch.empty_like(s_ref)
    kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                              o, s)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_noalloc_rejects_too_many_sequences(kda):
    n = kda.KDA_NOALLOC_MAX_SEQS + 1
    cu = [0] * (n + 1)
    d = gen.draw_chunk(1, 0, 1, 64, 64, "bf16", s0_std=None, seed=0, device=dev())
    o = torch.empty_like(d["v"])
    with pytest.raises(kda.KDAError) as err:
        kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, o,
                                  cu_seqlens=torch.zeros(n + 1, dtype=torch.int32, device=dev()),
                                  cu_seqlens_host=cu)
    assert err.value.status == 2  # KDA_ERROR_NOT_SUPPORTED
