"""Pins of the Gated DeltaNet-2 oracle (``oracle.gdn2_*``) against what the
page and the mathematics fix ("线性注意力机制：从标准注意力到 Gated
DeltaNet-2", jindou-blog, section 4 and its erase/write table: the method
splits the delta rule's one gate into a per-channel erase gate e_t and write
gate w_t and contains linear attention, Gated DeltaNet and KDA as special
cases).  Each pin maps one unit's inputs through ``impl(q, k, v, alpha, erase,
write, s0, scale) -> (o, S_T)``; every planted mistake below must fail at
least one pin."""
import numpy as np
import pytest

import brute
import oracle

TOL = 1e-11


def gdn2_impl(q, k, v, alpha, erase, write, s0, scale):
    o, s = oracle.gdn2_forward_units(q[None], k[None], v[None], alpha[None], erase[None],
                                     write[None], s0[None], scale=scale, threads=1)
    return o[0], s[0]


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def draw(rng, T, dk, dv):
    q = unit(rng.standard_normal((T, dk)))
    k = unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    alpha = sig(rng.normal(2.0, 1.0, (T, dk)))
    erase = sig(rng.standard_normal((T, dk)))
    write = sig(rng.standard_normal((T, dk)))
    s0 = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, alpha, erase, write, s0


def pin_kda(impl, rng, T=9, dk=6, dv=5):
    """e_t = w_t = beta_t 1: KDA's token step (the separately pinned KDA oracle)."""
    q, k, v, alpha, _, _, s0 = draw(rng, T, dk, dv)
    beta = sig(rng.standard_normal(T))
    bb = np.repeat(beta[:, None], dk, 1)
    o, s = impl(q, k, v, alpha, bb, bb, s0, 0.7)
    ro, rs = oracle.forward_units(q[None], k[None], v[None], alpha[None], beta[None], s0[None],
                                  scale=0.7, threads=1)
    return max(rel(o, ro[0]), rel(s, rs[0]))


def pin_gated_deltanet(impl, rng, T=8, dk=5, dv=4):
    """alpha_t = a_t 1 and e_t = w_t = beta_t 1: Gated DeltaNet in the transposed
    matrix form of bugfactory.tech news 3610, third paragraph (brute.py)."""
    q, k, v, _, _, _, s0 = draw(rng, T, dk, dv)
    a = sig(rng.normal(1.0, 1.0, T))
    beta = sig(rng.standard_normal(T))
    bb = np.repeat(beta[:, None], dk, 1)
    o, s = impl(q, k, v, np.repeat(a[:, None], dk, 1), bb, bb, s0, 0.6)
    ro, rs = brute.deltanet_matrix_form(q, k, v, beta, s0, 0.6, gate=a)
    return max(rel(o, ro), rel(s, rs))


def pin_linear_attention(impl, rng, T=7, dk=4, dv=3):
    """alpha = 1, e = 0, w = 1, S0 = 0: textbook causal linear attention
    S_T = K^T V, O = scale tril(Q K^T) V, for any keys (no orthogonality needed:
    nothing is erased)."""
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    one, zero = np.ones((T, dk)), np.zeros((T, dk))
    o, s = impl(q, k, v, one, zero, one, np.zeros((dk, dv)), 0.5)
    ro, rs = brute.causal_linear_attention(q, k, v, 0.5)
    return max(rel(o, ro), rel(s, rs))


def pin_no_erase_closed_form(impl, rng, T=8, dk=5, dv=4):
    """e = 0: a gated linear attention with a per-channel write gate, in closed
    form (weighted sums of k v^T with cumulative decays)."""
    q, k, v, alpha, _, write, s0 = draw(rng, T, dk, dv)
    k = k * rng.uniform(0.5, 2.0, (T, 1))
    o, s = impl(q, k, v, alpha, np.zeros((T, dk)), write, s0, 0.8)
    ro, rs = brute.gated_write_linear_attention(q, k, v, alpha, write, s0, 0.8)
    return max(rel(o, ro), rel(s, rs))


def pin_no_write(impl, rng, T=6, dk=5, dv=4):
    """w = 0: nothing of V reaches the state (two different V give the same
    result) and S_T is the product of the erase/forget transitions applied to S0."""
    q, k, v, alpha, erase, _, s0 = draw(rng, T, dk, dv)
    zero = np.zeros((T, dk))
    o1, s1 = impl(q, k, v, alpha, erase, zero, s0, 0.9)
    o2, s2 = impl(q, k, rng.standard_normal(v.shape), alpha, erase, zero, s0, 0.9)
    P = np.eye(dk)
    for t in range(T):
        P = brute.gdn2_transition(alpha[t], erase[t], k[t]) @ P
    return max(rel(o1, o2), rel(s1, s2), rel(s1, P @ s0))


def pin_brute_force(impl, rng, T=5, dk=4, dv=3):
    """General gates: the explicit product of transitions."""
    q, k, v, alpha, erase, write, s0 = draw(rng, T, dk, dv)
    k = k * rng.uniform(0.5, 1.5, (T, 1))
    o, s = impl(q, k, v, alpha, erase, write, s0, 0.7)
    ro, rs = brute.gdn2_product_of_transitions(q, k, v, alpha, erase, write, s0, 0.7)
    return max(rel(o, ro), rel(s, rs))


def pin_full_erase(impl, rng, T=6, dk=5, dv=4):
    """e = 1, w = 0 and a unit key: the association stored under the key is
    removed entirely, S_t^T k_t = 0, so reading with q_t = k_t gives 0; other
    directions keep their (decayed) content."""
    q, k, v, alpha, _, _, s0 = draw(rng, T, dk, dv)
    s0 = s0 + 1.0
    o, s = impl(k.copy(), k, v, alpha, np.ones((T, dk)), np.zeros((T, dk)), s0, 1.0)
    return float(np.max(np.abs(o))) / float(np.max(np.abs(s0)))


def pin_overwrite(impl, rng, T=6, dk=5, dv=4):
    """e = w = 1 and a unit key: the write replaces the value under the key,
    S_t^T k_t = v_t, so reading with q_t = k_t gives scale v_t."""
    q, k, v, alpha, _, _, s0 = draw(rng, T, dk, dv)
    one = np.ones((T, dk))
    o, s = impl(k.copy(), k, v, alpha, one, one, s0, 0.5)
    return rel(o, 0.5 * v)


def pin_superposition(impl, rng, T=7, dk=4, dv=3):
    """For fixed q, k and gates the result is linear in (S0, V)."""
    q, k, v, alpha, erase, write, s0 = draw(rng, T, dk, dv)
    v2, s02 = rng.standard_normal(v.shape), rng.standard_normal(s0.shape)
    o1, s1 = impl(q, k, v, alpha, erase, write, s0, 0.6)
    o2, s2 = impl(q, k, v2, alpha, erase, write, s02, 0.6)
    o3, s3 = impl(q, k, 2 * v - 3 * v2, alpha, erase, write, 2 * s0 - 3 * s02, 0.6)
    return max(rel(o3, 2 * o1 - 3 * o2), rel(s3, 2 * s1 - 3 * s2))


PINS = [pin_kda, pin_gated_deltanet, pin_linear_attention, pin_no_erase_closed_form,
        pin_no_write, pin_brute_force, pin_full_erase, pin_overwrite, pin_superposition]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gdn2_oracle_meets_pin(pin, seed):
    err = pin(gdn2_impl, np.random.default_rng(seed))
    assert err < TOL, (pin.__name__, err)


def mutant(mistake):
    """A NumPy token loop of the reading with one planted mistake."""
    def impl(q, k, v, alpha, erase, write, s0, scale):
        T, dk = k.shape
        S = s0.copy()
        o = np.zeros((T, v.shape[1]))
        for t in range(T):
            a, e, w, kt = alpha[t], erase[t], write[t], k[t]
            if mistake == "predict_before_forget":
                vh = S.T @ kt
                S = a[:, None] * S
            elif mistake == "no_forget":
                vh = S.T @ kt
            else:
                S = a[:, None] * S
                vh = S.T @ kt
            ev, wv = e * kt, w * kt
            if mistake == "erase_with_write_gate":
                ev = w * kt
            elif mistake == "write_with_erase_gate":
                wv = e * kt
            elif mistake == "gates_swapped":
                ev, wv = wv, ev
            elif mistake == "ungated_erase":
                ev = kt
            elif mistake == "literal_decay":  # (1 - e) . S + w . k v^T, no delta term
                S = (1.0 - e)[:, None] * S
                ev = np.zeros_like(kt)
            S = S - np.outer(ev, vh) + np.outer(wv, v[t])
            if mistake == "read_before_write":
                o[t] = scale * (S - np.outer(wv, v[t]) + np.outer(ev, vh)).T @ q[t]
            else:
                o[t] = scale * S.T @ q[t]
        return o, S
    return impl


MISTAKES = ["predict_before_forget", "no_forget", "erase_with_write_gate",
            "write_with_erase_gate", "gates_swapped", "ungated_erase", "literal_decay",
            "read_before_write"]


def test_correct_numpy_loop_meets_every_pin():
    """The mutant harness without a mistake is the reading itself (it must pass),
    so the failures below come from the planted mistakes alone."""
    for pin in PINS:
        assert pin(mutant(None), np.random.default_rng(5)) < 1e-10, pin.__name__


@pytest.mark.parametrize("mistake", MISTAKES)
def test_every_gdn2_mutant_fails_a_pin(mistake):
    worst = max(pin(mutant(mistake), np.random.default_rng(7)) for pin in PINS)
    assert worst > 1e-3, (mistake, worst)


def test_gdn2_layouts_match_units():
    """oracle.gdn2_forward in the [B, T, H, d] layout, varlen (with an empty
    sequence), a head sample, no forget gate (alpha None), and the decode step
    are re-arrangements of the unit loop."""
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 2, 7, 3, 4, 5
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    a, e, w = (rng.uniform(0.2, 1.0, (B, T, H, dk)) for _ in range(3))
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.gdn2_forward(q, k, v, a, e, w, s0, scale=0.4)
    for b in range(B):
        for h in range(H):
            ou, su = gdn2_impl(q[b, :, h], k[b, :, h], v[b, :, h], a[b, :, h], e[b, :, h],
                               w[b, :, h], s0[b, h], 0.4)
            assert rel(o[b, :, h], ou) < 1e-15 and rel(s[b, h], su) < 1e-15
    cu = [0, T, T, 2 * T]
    pk = lambda x: x.reshape((1, B * T) + x.shape[2:])
    s0v = np.concatenate([s0[:1], rng.standard_normal((1, H, dk, dv)), s0[1:]])
    ov, sv = oracle.gdn2_forward(pk(q), pk(k), pk(v), pk(a), pk(e), pk(w), s0v, cu_seqlens=cu,
                                 scale=0.4)
    assert rel(ov[0], pk(o)[0]) < 1e-15 and np.array_equal(sv[1], s0v[1])
    assert rel(sv[[0, 2]], s) < 1e-15
    oh, sh = oracle.gdn2_forward(q, k, v, a, e, w, s0, scale=0.4, heads=[2, 0])
    assert np.array_equal(oh, o[:, :, [2, 0]]) and np.array_equal(sh, s[:, [2, 0]])
    on, sn = oracle.gdn2_forward(q, k, v, None, e, w, s0, scale=0.4)
    o1, s1 = oracle.gdn2_forward(q, k, v, np.ones_like(a), e, w, s0, scale=0.4)
    assert np.array_equal(on, o1) and np.array_equal(sn, s1)
    os_, ss = oracle.gdn2_step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], e[:, 0], w[:, 0], s0,
                               scale=0.4)
    of, sf = oracle.gdn2_forward(q[:, :1], k[:, :1], v[:, :1], a[:, :1], e[:, :1], w[:, :1],
                                 s0, scale=0.4)
    assert np.array_equal(os_, of[:, 0]) and np.array_equal(ss, sf)


@pytest.mark.parametrize("T,dk,dv", [(64, 8, 4), (150, 16, 8), (1, 8, 8), (200, 32, 16)])
def test_gdn2_chunk_algebra_matches_the_oracle(T, dk, dv):
    """The chunk decomposition the HIP kernel uses (tests/chunk_ref.py, fp64)
    equals the oracle's token loop: full and partial chunks, mid-chunk decay
    references and the stacked [V; -Pred] products."""
    import chunk_ref
    rng = np.random.default_rng(T + dk)
    q, k = unit(rng.standard_normal((T, dk))), unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    alpha = sig(rng.normal(3.0, 1.0, (T, dk)))
    erase, write = sig(rng.standard_normal((T, dk))), sig(rng.standard_normal((T, dk)))
    s0 = 0.2 * rng.standard_normal((dk, dv))
    o, s = chunk_ref.gdn2_chunk_forward_unit(q, k, v, alpha, erase, write, s0, 0.5)
    ro, rs = gdn2_impl(q, k, v, alpha, erase, write, s0, 0.5)
    assert rel(o, ro) < 1e-12 and rel(s, rs) < 1e-12


def test_gdn2_step_in_place_matches_copy():
    rng = np.random.default_rng(11)
    N, H, dk, dv = 3, 2, 4, 5
    q, k, v = rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk)), \
        rng.standard_normal((N, H, dv))
    a, e, w = (rng.uniform(0.2, 1.0, (N, H, dk)) for _ in range(3))
    s = rng.standard_normal((N, H, dk, dv))
    o1, s1 = oracle.gdn2_step(q, k, v, a, e, w, s)
    s2 = s.copy()
    o2, s3 = oracle.gdn2_step(q, k, v, a, e, w, s2, in_place=True)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2) and s3 is s2
    assert not np.array_equal(s, s1)
