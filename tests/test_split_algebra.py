"""The two-segment form of the chunk-wise forward, checked on the CPU.

The update of "Kimi Delta Attention" (section "KDA 的更新式") is affine in the
state, so over a second segment of a sequence, from any start X,
S_t = Phi_t X + R_t and o_t = X^T z_t + o^R_t, where (z, Phi) is the
recurrence run from the identity with every value zero and (o^R, R) the
recurrence from the zero state.  These tests take every part from the fp64
oracle alone and check that they recombine to the oracle's single pass, so
that the decomposition the library's split path computes is pinned before
any GPU code runs; they also pin the host-side plan of that path (which
shapes qualify, how the tokens are divided, the workspace it needs).
"""
import numpy as np
import pytest

import oracle


def _draw(rng, U, T, dk, dv, alpha_mu):
    q = rng.standard_normal((U, T, dk))
    k = rng.standard_normal((U, T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((U, T, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((U, T))))
    alpha = 1 / (1 + np.exp(-(alpha_mu + rng.standard_normal((U, T, dk)))))
    s0 = 0.1 * rng.standard_normal((U, dk, dv))
    return q, k, v, alpha, beta, s0


@pytest.mark.parametrize("L0,alpha_mu", [(24, 4.0), (1, 2.0), (39, 0.0)])
def test_two_segments_recombine_to_single_pass(L0, alpha_mu):
    rng = np.random.default_rng(7 + L0)
    U, T, d = 3, 40, 8
    q, k, v, alpha, beta, s0 = _draw(rng, U, T, d, d, alpha_mu)
    o_ref, s_ref = oracle.forward_units(q, k, v, alpha, beta, s0)

    seg0 = lambda x: np.ascontiguousarray(x[:, :L0])
    seg1 = lambda x: np.ascontiguousarray(x[:, L0:])
    o0, sm = oracle.forward_units(seg0(q), seg0(k), seg0(v), seg0(alpha), seg0(beta), s0)
    o_r, r_T = oracle.forward_units(seg1(q), seg1(k), seg1(v), seg1(alpha), seg1(beta), None)
    ident = np.broadcast_to(np.eye(d), (U, d, d)).copy()
    z, phi_T = oracle.forward_units(seg1(q), seg1(k), np.zeros_like(seg1(v)), seg1(alpha),
                                    seg1(beta), ident)

    o1 = o_r + np.einsum("uij,uti->utj", sm, z)
    s_T = np.einsum("uim,umj->uij", phi_T, sm) + r_T
    np.testing.assert_allclose(o0, o_ref[:, :L0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o1, o_ref[:, L0:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s_T, s_ref, rtol=0, atol=1e-12)


def test_transition_part_is_the_product_of_token_transitions():
    """Phi_T from the oracle's zero-value, identity-start run equals the
    product of the per-token maps (I - beta k k^T) Diag(alpha), written out."""
    rng = np.random.default_rng(3)
    U, T, d = 1, 9, 6
    q, k, v, alpha, beta, _ = _draw(rng, U, T, d, d, 1.0)
    ident = np.eye(d)[None].copy()
    _, phi_T = oracle.forward_units(q, k, np.zeros_like(v), alpha, beta, ident)
    prod = np.eye(d)
    for t in range(T):
        kt = k[0, t][:, None]
        prod = (np.eye(d) - beta[0, t] * kt @ kt.T) @ np.diag(alpha[0, t]) @ prod
    np.testing.assert_allclose(phi_T[0], prod, rtol=0, atol=1e-13)


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_38_amd as kda
    kda.load_library()
    return kda


def test_split_plan_sizes(lib):
    import torch
    f = lib.kda_chunk_fwd_split_workspace_size
    # the long-context workload: 1024 chunks, 597 in the first segment
    l0 = 597 * 64
    l1 = 65536 - l0
    st = 32 * 128 * 128 * 4
    assert f(1, 65536, 32, 128, 128) == 3 * st + l1 * 32 * 128 * 2
    # two sequences: the transition outputs of both, rows seq * T + tau
    T = 5000
    nch = (T + 63) // 64
    l0 = (nch * 583 + 500) // 1000 * 64
    zrows = T + (T - l0)
    z = (zrows * 3 * 128 * 2 + 255) // 256 * 256
    assert f(2, T, 3, 128, 128) == 3 * ((6 * 128 * 128 * 4 + 255) // 256 * 256) + z
    # shapes that keep the single pass
    assert f(4, 4096, 16, 128, 128) == 0          # 64 units: eight workgroups each exceed the chip
    assert f(1, 4032, 32, 128, 128) == 0          # 63 chunks
    assert f(1, 4033, 32, 128, 128) > 0           # 64 chunks
    assert f(1, 65536, 32, 64, 64) == 0           # dk = dv = 128 only
    assert f(1, 65536, 32, 128, 64) == 0
    assert f(1, 65536, 32, 128, 128, torch.float32) == 0
    assert f(0, 65536, 32, 128, 128) == 0
    assert f(1, 65536, 0, 128, 128) == 0
    assert f(-1, 65536, 32, 128, 128) == 0
