"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every pin is a function ``pin(impl, rng) -> error`` where ``impl`` maps one
unit's inputs (q, k, v, alpha, beta, s0, scale) to (o [T, dv], S_T [dk, dv]).
The oracle must meet each pin to ~1e-12; every planted mistake in
``mutants.py`` must fail at least one pin by a wide margin.
"""
import json
import os

import numpy as np
import pytest

import brute
import mutants
import oracle

TOL = 1e-11
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oracle_impl(q, k, v, alpha, beta, s0, scale):
    o, s = oracle.forward_units(q[None], k[None], v[None], alpha[None], beta[None],
                                s0[None], scale=scale, threads=1)
    return o[0], s[0]


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def draw(rng, T, dk, dv, s0_std=0.3):
    q = unit(rng.standard_normal((T, dk)))
    k = unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    alpha = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, (T, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    s0 = s0_std * rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, s0


# ---------------------------------------------------------------- the pins

def pin_requery(impl, rng, dk=6, dv=6, T=7):
    """beta = 1 and a unit-norm key: right after the write, querying the state
    with that key gives back the written value exactly (bugfactory.tech news
    3610, second paragraph).  The read uses q_t = k_t, so o_t = scale * v_t."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    beta[:] = 1.0
    q = k.copy()
    o, _ = impl(q, k, v, alpha, beta, s0, 0.5)
    return rel(o, 0.5 * v)


def pin_orthogonal(impl, rng, dk=6, dv=5, T=6):
    """Directions orthogonal to the current key are only decayed
    (bugfactory.tech news 3610, second paragraph, with the decay-first order of
    the third and fourth paragraphs): for x orthogonal to k_t,
    S_t^T x = S_{t-1}^T Diag(alpha_t) x.  S_{t-1} comes from the same
    implementation run on the prefix."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    x = rng.standard_normal(dk)
    x -= (x @ k[-1]) * k[-1]
    q[-1] = x
    o, _ = impl(q, k, v, alpha, beta, s0, 1.0)
    _, s_prev = impl(q[:-1], k[:-1], v[:-1], alpha[:-1], beta[:-1], s0, 1.0)
    return rel(o[-1], s_prev.T @ (alpha[-1] * x))


def pin_deltanet(impl, rng, dk=5, dv=4, T=9):
    """alpha = 1: the matrix form of DeltaNet in the |v><k| convention
    (bugfactory.tech news 3610, second paragraph)."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    alpha[:] = 1.0
    o, s = impl(q, k, v, alpha, beta, s0, 0.7)
    o_r, s_r = brute.deltanet_matrix_form(q, k, v, beta, s0, 0.7)
    return max(rel(o, o_r), rel(s, s_r))


def pin_gated_deltanet(impl, rng, dk=5, dv=4, T=9):
    """alpha_t constant across channels: Gated DeltaNet, the whole memory
    scaled by a scalar before the delta step (bugfactory.tech news 3610, third
    paragraph; the per-head scalar gate row of the table in "Kimi Delta
    Attention", section "一、Diag(α_t)：通道级遗忘")."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    g = 1.0 / (1.0 + np.exp(-rng.normal(1.0, 1.0, T)))
    alpha = np.repeat(g[:, None], dk, axis=1)
    o, s = impl(q, k, v, alpha, beta, s0, 0.7)
    o_r, s_r = brute.deltanet_matrix_form(q, k, v, beta, s0, 0.7, gate=g)
    return max(rel(o, o_r), rel(s, s_r))


def pin_brute_force(impl, rng, dk=4, dv=3, T=6):
    """Unrolled product of the per-token transitions A_t = (I - beta k k^T)
    Diag(alpha) ("Kimi Delta Attention", section "KDA 的更新式")."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    # non-unit keys and arbitrary beta, so no special structure helps
    k = k * rng.uniform(0.5, 1.5, (T, 1))
    o, s = impl(q, k, v, alpha, beta, s0, 0.9)
    o_r, s_r = brute.product_of_transitions(q, k, v, alpha, beta, s0, 0.9)
    return max(rel(o, o_r), rel(s, s_r))


def pin_linear_attention(impl, rng, dk=8, dv=5, T=6):
    """Orthonormal keys, beta = 1, alpha = 1, zero start: the delta rule never
    has anything to erase, so the result is plain causal linear attention,
    S_T = K^T V and O = scale tril(Q K^T) V (the additive update of "Kimi Delta
    Attention", section "先建立直觉：从缓存到状态")."""
    qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = qm[:T].copy()  # orthonormal rows
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    alpha = np.ones((T, dk))
    beta = np.ones(T)
    o, s = impl(q, k, v, alpha, beta, np.zeros((dk, dv)), 0.4)
    o_r, s_r = brute.causal_linear_attention(q, k, v, 0.4)
    return max(rel(o, o_r), rel(s, s_r))


def pin_no_write(impl, rng, dk=5, dv=4, T=7):
    """beta = 0: nothing is written, the state only decays per channel:
    S_t = Diag(prod_{i<=t} alpha_i) S0 and o_t = scale S_t^T q_t ("Kimi Delta
    Attention", section "一、Diag(α_t)：通道级遗忘")."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    beta[:] = 0.0
    o, s = impl(q, k, v, alpha, beta, s0, 1.3)
    cum = np.cumprod(alpha, axis=0)
    o_r = np.stack([1.3 * (cum[t][:, None] * s0).T @ q[t] for t in range(T)])
    return max(rel(o, o_r), rel(s, cum[-1][:, None] * s0))


def pin_gradient_step(impl, rng, dk=5, dv=4, T=5):
    """The delta write is one gradient-descent step of size beta on
    L(S) = 1/2 ||S^T k - v||^2, taken at the decayed state (bugfactory.tech news
    3610, second paragraph; the Widrow-Hoff / LMS view on the kongchang.com
    page, section "Delta规则如何解决这一问题？").  The gradient is taken by
    central differences, which are exact for a quadratic up to rounding."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    k = k * 1.7  # a non-unit key so the step size matters
    _, s_prev = impl(q[:-1], k[:-1], v[:-1], alpha[:-1], beta[:-1], s0, 1.0)
    _, s_t = impl(q, k, v, alpha, beta, s0, 1.0)
    s_tilde = alpha[-1][:, None] * s_prev

    def loss(S):
        r = S.T @ k[-1] - v[-1]
        return 0.5 * float(r @ r)

    h = 1e-3
    grad = np.zeros_like(s_tilde)
    for i in range(dk):
        for j in range(dv):
            e = np.zeros_like(s_tilde)
            e[i, j] = h
            grad[i, j] = (loss(s_tilde + e) - loss(s_tilde - e)) / (2 * h)
    return rel(s_t, s_tilde - beta[-1] * grad)


def pin_superposition(impl, rng, dk=5, dv=4, T=8):
    """For fixed (q, k, alpha, beta) the map (S0, V) -> (O, S_T) is linear: the
    update equation of "Kimi Delta Attention", section "KDA 的更新式", is
    affine in S and in v_t."""
    q, k, v1, alpha, beta, s1 = draw(rng, T, dk, dv)
    v2 = rng.standard_normal((T, dv))
    s2 = rng.standard_normal((dk, dv))
    c = -0.75
    o1, f1 = impl(q, k, v1, alpha, beta, s1, 1.0)
    o2, f2 = impl(q, k, v2, alpha, beta, s2, 1.0)
    o3, f3 = impl(q, k, v1 + c * v2, alpha, beta, s1 + c * s2, 1.0)
    return max(rel(o3, o1 + c * o2), rel(f3, f1 + c * f2))


def pin_resume(impl, rng, dk=5, dv=4, T=9, split=4):
    """The fixed-size state is all that is carried between segments (the
    chunk-wise form on the kongchang.com page, section "硬件效率的优化策略"):
    running x1 then x2 from x1's final state equals running x1 || x2."""
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    o, s = impl(q, k, v, alpha, beta, s0, 1.0)
    oa, sa = impl(q[:split], k[:split], v[:split], alpha[:split], beta[:split], s0, 1.0)
    ob, sb = impl(q[split:], k[split:], v[split:], alpha[split:], beta[split:], sa, 1.0)
    return max(rel(o, np.concatenate([oa, ob])), rel(s, sb))


def pin_rewrite(impl, rng, dk=6, dv=5):
    """The same key written twice with beta = 1, alpha = 1 keeps only the
    latest value; nothing accumulates ("Kimi Delta Attention", section
    "二、I − β_t k_t k_tᵀ：delta 规则")."""
    k1 = unit(rng.standard_normal(dk))
    k = np.stack([k1, k1])
    v = rng.standard_normal((2, dv))
    q = k.copy()
    o, _ = impl(q, k, v, np.ones((2, dk)), np.ones(2), rng.standard_normal((dk, dv)), 1.0)
    return rel(o[1], v[1])


PINS = [pin_requery, pin_orthogonal, pin_deltanet, pin_gated_deltanet, pin_brute_force,
        pin_linear_attention, pin_no_write, pin_gradient_step, pin_superposition,
        pin_resume, pin_rewrite]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_meets_pin(pin, seed):
    err = pin(oracle_impl, np.random.default_rng(seed))
    tol = 1e-8 if pin is pin_gradient_step else TOL
    assert err < tol, (pin.__name__, err)


@pytest.mark.parametrize("mistake", mutants.MISTAKES)
def test_every_mutant_fails_a_pin(mistake):
    impl = mutants.make(mistake)
    worst = 0.0
    for pin in PINS:
        try:
            worst = max(worst, pin(impl, np.random.default_rng(7)))
        except ValueError:  # a shape-breaking mistake fails outright
            worst = np.inf
    assert worst > 1e-3, (mistake, worst)


def test_worked_example():
    """A 2x2 two-token example worked by hand from the four steps (forget,
    predict, correct and write, read); see tests/golden/worked_2x2.json."""
    with open(os.path.join(GOLDEN, "worked_2x2.json")) as f:
        g = json.load(f)
    arr = {key: np.asarray(val, dtype=np.float64) for key, val in g["inputs"].items()}
    o, s = oracle_impl(arr["q"], arr["k"], arr["v"], arr["alpha"], arr["beta"], arr["s0"],
                       float(g["inputs"]["scale"]))
    assert rel(o, np.asarray(g["expected"]["o"])) < 1e-14
    assert rel(s, np.asarray(g["expected"]["state"])) < 1e-14


def test_empty_sequence_keeps_state():
    rng = np.random.default_rng(3)
    s0 = rng.standard_normal((1, 4, 3))
    e = np.zeros((1, 0, 4))
    o, s = oracle.forward_units(e, e, np.zeros((1, 0, 3)), e, np.zeros((1, 0)), s0)
    assert o.shape == (1, 0, 3)
    assert np.array_equal(s, s0)


def test_layouts_and_varlen_match_units():
    """The [B, T, H, d] wrapper, the varlen split and the decode step are
    re-arrangements of the same unit loop (units are independent; a decode step
    is one token)."""
    rng = np.random.default_rng(4)
    B, T, H, dk, dv = 2, 11, 3, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    a = rng.uniform(0.3, 1.0, (B, T, H, dk))
    b = rng.uniform(0.0, 1.0, (B, T, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.forward(q, k, v, a, b, s0)
    for bb in range(B):
        for h in range(H):
            o_u, s_u = oracle_impl(q[bb, :, h], k[bb, :, h], v[bb, :, h], a[bb, :, h],
                                   b[bb, :, h], s0[bb, h], dk ** -0.5)
            assert rel(o[bb, :, h], o_u) < 1e-15 and rel(s[bb, h], s_u) < 1e-15
    # varlen: pack both batch rows as two sequences plus an empty one
    cu = [0, T, T, 2 * T]
    pk = lambda x: x.reshape((1, B * T) + x.shape[2:])
    s0v = np.concatenate([s0[:1], rng.standard_normal((1, H, dk, dv)), s0[1:]])
    ov, sv = oracle.forward(pk(q), pk(k), pk(v), pk(a), pk(b), s0v, cu_seqlens=cu)
    assert rel(ov[0], pk(o)[0]) < 1e-15
    assert np.array_equal(sv[1], s0v[1])
    assert rel(sv[[0, 2]], s) < 1e-15
    # head sample
    oh, sh = oracle.forward(q, k, v, a, b, s0, heads=[2, 0])
    assert np.array_equal(oh, o[:, :, [2, 0]]) and np.array_equal(sh, s[:, [2, 0]])
    # one decode step == forward with T = 1
    o1, st1 = oracle.step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], s0)
    of, sf = oracle.forward(q[:, :1], k[:, :1], v[:, :1], a[:, :1], b[:, :1], s0)
    assert np.array_equal(o1, of[:, 0]) and np.array_equal(st1, sf)


@pytest.mark.parametrize("seed", [0, 1])
def test_head_and_no_gate_through_the_token_layout(seed):
    """oracle.channel_gate in the library's [B, T, H] layout: a per-head gate
    gives Gated DeltaNet and no gate gives DeltaNet, unit by unit, against the
    matrix forms written separately in brute.py (bugfactory.tech news 3610,
    second and third paragraphs)."""
    rng = np.random.default_rng(10 + seed)
    B, T, H, dk, dv = 2, 7, 3, 5, 4
    q = unit(rng.standard_normal((B, T, H, dk)))
    k = unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    g = 1.0 / (1.0 + np.exp(-rng.normal(1.0, 1.0, (B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    o_g, s_g = oracle.forward(q, k, v, oracle.channel_gate(g, "head", dk), beta, s0, scale=0.6)
    o_n, s_n = oracle.forward(q, k, v, oracle.channel_gate(None, "none", dk, (B, T, H)), beta,
                              s0, scale=0.6)
    for b in range(B):
        for h in range(H):
            args = (q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h], s0[b, h], 0.6)
            o_r, s_r = brute.deltanet_matrix_form(*args, gate=g[b, :, h])
            assert rel(o_g[b, :, h], o_r) < TOL and rel(s_g[b, h], s_r) < TOL
            o_r, s_r = brute.deltanet_matrix_form(*args)
            assert rel(o_n[b, :, h], o_r) < TOL and rel(s_n[b, h], s_r) < TOL
    with pytest.raises(ValueError):
        oracle.channel_gate(g, "scalar", dk)


def test_prepare_logistic_and_norm_fixed_points():
    """oracle.prepare: the logistic map at points where it is known exactly
    (1/2 at 0, 3/4 at ln 3, 1/4 at -ln 3), and the L2 normalisation: unit rows
    parallel to the stored ones, zero rows left zero."""
    z = np.array([[0.0, np.log(3.0), -np.log(3.0)]])
    q = np.array([[[3.0, 4.0, 0.0]], [[0.0, 0.0, 0.0]]])  # [2 tokens, 1 head, 3]
    k = np.array([[[1.0, 2.0, 2.0]], [[0.0, 5.0, 0.0]]])
    qn, kn, a, b = oracle.prepare(q, k, np.repeat(z, 2, 0)[:, None, :], z[:, :2].T,
                                  gate_logits=True, beta_logits=True, qk_l2norm=True)
    assert np.allclose(a[0, 0], [0.5, 0.75, 0.25], rtol=0, atol=1e-15)
    assert np.allclose(b[:, 0], [0.5, 0.75], rtol=0, atol=1e-15)
    e = 1e-6
    assert np.allclose(qn[0, 0], np.array([3.0, 4.0, 0.0]) / np.sqrt(25 + e), rtol=1e-15)
    assert np.array_equal(qn[1, 0], np.zeros(3))
    assert np.allclose(kn[:, 0], [[1 / 3, 2 / 3, 2 / 3], [0, 1, 0]], atol=1e-7)
    # per-head logits: one decay repeated over the channels
    _, _, ah, _ = oracle.prepare(q, k, z[:, :2].T, z[:, :2].T, gate="head", gate_logits=True)
    assert np.allclose(ah[:, 0], [[0.5] * 3, [0.75] * 3], atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1])
def test_prepared_forward_is_scale_invariant_in_q_and_k(seed):
    """With in-kernel normalisation the result depends on q and k only through
    their directions: positive per-token scalings of the stored q and k leave
    the prepared forward unchanged (the 1e-6 inside the root aside)."""
    rng = np.random.default_rng(20 + seed)
    B, T, H, dk, dv = 1, 9, 2, 6, 4
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    z = rng.normal(3.0, 1.0, (B, T, H, dk))
    bl = rng.standard_normal((B, T, H))
    s0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    cq = rng.uniform(5.0, 50.0, (B, T, H, 1))
    ck = rng.uniform(5.0, 50.0, (B, T, H, 1))
    flags = dict(gate_logits=True, beta_logits=True, qk_l2norm=True)
    o1, s1 = _fwd_kw(*_prep4(q, k, z, bl, flags), v, s0)
    o2, s2 = _fwd_kw(*_prep4(cq * q, ck * k, z, bl, flags), v, s0)
    assert rel(o2, o1) < 1e-6 and rel(s2, s1) < 1e-6
    # and without the map, logits are not decays: a different result
    o3, _ = _fwd_kw(*_prep4(q, k, np.clip(z, 0.0, 1.0), bl, dict(flags, gate_logits=False)),
                    v, s0)
    assert rel(o3, o1) > 1e-2


def _prep4(q, k, z, bl, flags):
    qn, kn, a, b = oracle.prepare(q, k, z, bl, **flags)
    return qn, kn, a, b


def _fwd_kw(qn, kn, a, b, v, s0):
    return oracle.forward(qn, kn, v, a, b, s0)


BACKWARD_IMPLS = {"c": oracle.backward_units, "numpy": oracle.backward_units_numpy}


@pytest.mark.parametrize("impl", sorted(BACKWARD_IMPLS))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(impl, seed):
    """Both backward implementations against central differences of the
    oracle's own forward (the C token loop, a separate implementation): L =
    <W, o> + <V, S_T> with random weights, every input perturbed in turn."""
    rng = np.random.default_rng(40 + seed)
    T, dk, dv = 5, 3, 2
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    k = k * rng.uniform(0.6, 1.3, (T, 1))          # no special structure
    W = rng.standard_normal((T, dv))
    V = rng.standard_normal((dk, dv))
    scale = 0.8
    inputs = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, s0=s0)

    def loss(x):
        o, s = oracle_impl(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"], scale)
        return float(np.sum(W * o) + np.sum(V * s))
    grads = BACKWARD_IMPLS[impl](q[None], k[None], v[None], alpha[None], beta[None], s0[None],
                                 W[None], V[None], scale=scale)
    names = ["q", "k", "v", "alpha", "beta", "s0"]
    h = 1e-6
    for name, g in zip(names, grads):
        x0 = inputs[name]
        fd = np.zeros_like(x0)
        for idx in np.ndindex(x0.shape):
            xp = {n: a.copy() for n, a in inputs.items()}
            xm = {n: a.copy() for n, a in inputs.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert rel(g[0], fd) < 1e-7, (name, rel(g[0], fd))


@pytest.mark.parametrize("impl", sorted(BACKWARD_IMPLS))
def test_backward_special_cases(impl):
    """beta = 0 and alpha = 1: nothing is written or forgotten, S_t = S0 for
    every t, so dq_t = scale S0 do_t, dS0 = dS_T + scale sum_t q_t do_t^T,
    dalpha_t = rows of (dS_t (.) S0) and dk = dv = 0 (closed forms)."""
    rng = np.random.default_rng(5)
    U, T, dk, dv = 2, 6, 4, 3
    q = rng.standard_normal((U, T, dk))
    k = rng.standard_normal((U, T, dk))
    v = rng.standard_normal((U, T, dv))
    s0 = rng.standard_normal((U, dk, dv))
    do = rng.standard_normal((U, T, dv))
    dsT = rng.standard_normal((U, dk, dv))
    g = BACKWARD_IMPLS[impl](q, k, v, np.ones((U, T, dk)), np.zeros((U, T)), s0, do, dsT,
                             scale=0.5)
    assert np.allclose(g[0], 0.5 * np.einsum("uij,utj->uti", s0, do), atol=1e-13)
    assert np.allclose(g[5], dsT + 0.5 * np.einsum("uti,utj->uij", q, do), atol=1e-12)
    assert np.abs(g[1]).max() == 0.0 and np.abs(g[2]).max() == 0.0
    # dS_t = dS_T + scale sum_{r > t} q_r do_r^T + scale q_t do_t^T, then rows against S0
    for t in range(T):
        dS_t = dsT + 0.5 * np.einsum("uri,urj->uij", q[:, t:], do[:, t:])
        assert np.allclose(g[3][:, t], np.sum(dS_t * s0, axis=-1), atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_c_and_numpy_agree(seed):
    """The C and NumPy backward implementations (written separately, each pinned
    by finite differences above) agree on larger random units, with and without
    an initial state and a final-state gradient, for dk != dv and for T = 0, 1."""
    rng = np.random.default_rng(60 + seed)
    for U, T, dk, dv, with_s0, with_dsT in [(3, 40, 8, 5, True, True), (2, 17, 4, 9, False, True),
                                            (2, 23, 6, 6, True, False), (1, 1, 5, 3, True, True),
                                            (2, 0, 4, 4, True, True)]:
        q = rng.standard_normal((U, T, dk))
        k = unit(rng.standard_normal((U, T, dk))) if T else np.zeros((U, 0, dk))
        v = rng.standard_normal((U, T, dv))
        a = rng.uniform(0.5, 1.0, (U, T, dk))
        b = rng.uniform(0.0, 1.0, (U, T))
        s0 = rng.standard_normal((U, dk, dv)) if with_s0 else None
        do = rng.standard_normal((U, T, dv))
        dsT = rng.standard_normal((U, dk, dv)) if with_dsT else None
        gc = oracle.backward_units(q, k, v, a, b, s0, do, dsT, scale=0.7, threads=2)
        gn = oracle.backward_units_numpy(q, k, v, a, b, s0, do, dsT, scale=0.7)
        for x, y in zip(gc, gn):
            assert x.shape == y.shape
            assert np.max(np.abs(x - y), initial=0.0) <= 1e-12 * max(1.0, np.max(np.abs(y), initial=0.0))
        if T == 0:  # nothing happens: dS0 = dS_T
            assert np.array_equal(gc[5], dsT)


def test_backward_layouts_and_varlen_match_units():
    """oracle.backward in the [B, T, H, d] layout, the varlen split (with empty and
    one-token sequences) and a head sample are re-arrangements of backward_units on
    independent units: each unit is compared with its own call."""
    rng = np.random.default_rng(70)
    B, T, H, dk, dv = 2, 9, 3, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    a = rng.uniform(0.3, 1.0, (B, T, H, dk))
    b = rng.uniform(0.0, 1.0, (B, T, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dsT = rng.standard_normal((B, H, dk, dv))
    g = oracle.backward(q, k, v, a, b, s0, do, dsT, scale=0.6)
    for bb in range(B):
        for h in range(H):
            gu = oracle.backward_units_numpy(q[bb, :, h][None], k[bb, :, h][None],
                                             v[bb, :, h][None], a[bb, :, h][None],
                                             b[bb, :, h][None], s0[bb, h][None],
                                             do[bb, :, h][None], dsT[bb, h][None], scale=0.6)
            for i in range(5):
                assert rel(g[i][bb, :, h], gu[i][0]) < 1e-13, (bb, h, i)
            assert rel(g[5][bb, h], gu[5][0]) < 1e-13
    # varlen: lengths 0, 4, 1, 0, 13 over the packed tokens of both batch rows
    lens = [0, 4, 1, 0, 13]
    cu = np.concatenate([[0], np.cumsum(lens)])
    pk = lambda x: x.reshape((1, B * T) + x.shape[2:])
    s0v = rng.standard_normal((len(lens), H, dk, dv))
    dsv = rng.standard_normal((len(lens), H, dk, dv))
    gv = oracle.backward(pk(q), pk(k), pk(v), pk(a), pk(b), s0v, pk(do), dsv, cu_seqlens=cu,
                         scale=0.6)
    for n, L in enumerate(lens):
        t0 = cu[n]
        for h in range(H):
            sl = lambda x: x[0, t0:t0 + L, h][None]
            gu = oracle.backward_units_numpy(sl(pk(q)), sl(pk(k)), sl(pk(v)), sl(pk(a)),
                                             sl(pk(b)), s0v[n, h][None], sl(pk(do)),
                                             dsv[n, h][None], scale=0.6)
            for i in range(5):
                got = gv[i][0, t0:t0 + L, h]
                assert got.shape == gu[i][0].shape
                if L:
                    assert rel(got, gu[i][0]) < 1e-13, (n, h, i)
            assert rel(gv[5][n, h], gu[5][0]) < 1e-13
            if L == 0:  # an empty sequence passes the state gradient through
                assert np.array_equal(gv[5][n, h], dsv[n, h])
    # head sample
    gh = oracle.backward(q, k, v, a, b, s0, do, dsT, scale=0.6, heads=[2, 0])
    for i in range(5):
        assert np.array_equal(gh[i], g[i][:, :, [2, 0]])
    assert np.array_equal(gh[5], g[5][:, [2, 0]])


def test_step_in_place_matches_copy():
    """oracle.step with in_place rewrites the given float64 state and returns the
    same values as the copying call."""
    rng = np.random.default_rng(80)
    N, H, dk, dv = 3, 2, 4, 5
    q, k = rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv))
    a, b = rng.uniform(0.3, 1.0, (N, H, dk)), rng.uniform(0.0, 1.0, (N, H))
    s = rng.standard_normal((N, H, dk, dv))
    o1, s1 = oracle.step(q, k, v, a, b, s)
    s2 = s.copy()
    o2, s3 = oracle.step(q, k, v, a, b, s2, in_place=True)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s3) and np.array_equal(s2, s1)
    assert not np.array_equal(s, s1)  # the copying call left its input alone


@pytest.mark.parametrize("T,dk,dv", [(64, 8, 4), (150, 16, 8), (1, 8, 8), (200, 32, 16)])
def test_backward_chunk_algebra_matches_the_oracle(T, dk, dv):
    """The chunk decomposition of the gradients the HIP backward uses
    (tests/chunk_ref.py, fp64) equals the oracle's reverse token sweep."""
    import chunk_ref
    rng = np.random.default_rng(90 + T)
    q, k, v, alpha, beta, s0 = draw(rng, T, dk, dv)
    alpha = 1.0 / (1.0 + np.exp(-rng.normal(3.0, 1.0, (T, dk))))
    do = rng.standard_normal((T, dv))
    dsT = rng.standard_normal((dk, dv))
    got = chunk_ref.chunk_backward_unit(q, k, v, alpha, beta, s0, do, dsT, 0.6)
    ref = oracle.backward_units(q[None], k[None], v[None], alpha[None], beta[None], s0[None],
                                do[None], dsT[None], scale=0.6)
    for name, g, r in zip(["dq", "dk", "dv", "dalpha", "dbeta", "ds0"], got, ref):
        assert rel(g, r[0]) < 1e-11, (name, rel(g, r[0]))
