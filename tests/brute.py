"""Brute-force forms of the KDA recurrence, used only to pin the oracle.

These are deliberately written in a different shape from the oracle's token
loop: explicit transition matrices multiplied out, and the textbook closed
forms the pages say the method reduces to.
"""
import numpy as np


def transition(alpha_t, beta_t, k_t):
    """A_t = (I - beta_t k_t k_t^T) Diag(alpha_t): the key-space transition of
    one token ("Kimi Delta Attention", section "KDA 的更新式"; the diagonal-
    minus-rank-one form of bugfactory.tech news 3610, fourth paragraph)."""
    d = k_t.shape[0]
    return (np.eye(d) - beta_t * np.outer(k_t, k_t)) @ np.diag(alpha_t)


def product_of_transitions(q, k, v, alpha, beta, s0, scale):
    """One unit: S_t = (A_t ... A_1) S0 + sum_{i<=t} (A_t ... A_{i+1}) beta_i k_i v_i^T,
    every product formed explicitly from scratch for each t (O(T^2) matrix
    products, tiny T only).  o_t = scale S_t^T q_t.
    q, k, alpha: [T, dk]; v: [T, dv]; beta: [T]; s0: [dk, dv]."""
    T, dk = k.shape
    dv = v.shape[1]
    A = [transition(alpha[t], beta[t], k[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S = s0.copy()
    for t in range(T):
        P = np.eye(dk)
        for i in range(t, -1, -1):  # P = A_t ... A_0
            P = P @ A[i]
        S = P @ s0
        for i in range(t + 1):
            Pi = np.eye(dk)
            for j in range(t, i, -1):  # A_t ... A_{i+1}
                Pi = Pi @ A[j]
            S = S + Pi @ (beta[i] * np.outer(k[i], v[i]))
        o[t] = scale * S.T @ q[t]
    return o, S


def deltanet_matrix_form(q, k, v, beta, s0, scale, gate=None):
    """The delta rule in the transposed |v><k| convention of bugfactory.tech
    news 3610, second paragraph: M_t = M_{t-1} (I - beta_t k_t k_t^T)
    + beta_t v_t k_t^T with M = S^T (dv x dk); read o_t = scale M_t q_t.
    With a per-token scalar gate a_t the old memory is scaled first
    (third paragraph, Gated DeltaNet): M_t = a_t M_{t-1} (I - ...) + ..."""
    T, dk = k.shape
    M = s0.T.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        a = 1.0 if gate is None else gate[t]
        M = a * M @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
        o[t] = scale * M @ q[t]
    return o, M.T


def causal_linear_attention(q, k, v, scale):
    """Textbook causal linear attention with no normalisation
    ("Kimi Delta Attention" (daiw.net), section "先建立直觉：从缓存到状态";
    the recurrent view of linear attention on the kongchang.com page,
    section "循环视角下的线性注意力"):
    S_T = K^T V and O = scale * tril(Q K^T) V."""
    T = q.shape[0]
    mask = np.tril(np.ones((T, T)))
    return scale * (mask * (q @ k.T)) @ v, k.T @ v


def gdn2_transition(alpha_t, erase_t, k_t):
    """A_t = (I - (e_t . k_t) k_t^T) Diag(alpha_t): the key-space transition of
    one Gated DeltaNet-2 token under the reading of the jindou-blog page,
    section 4 (erase along the key, gated per key channel)."""
    d = k_t.shape[0]
    return (np.eye(d) - np.outer(erase_t * k_t, k_t)) @ np.diag(alpha_t)


def gdn2_product_of_transitions(q, k, v, alpha, erase, write, s0, scale):
    """One unit: S_t = (A_t ... A_1) S0 + sum_{i<=t} (A_t ... A_{i+1}) (w_i . k_i) v_i^T,
    every product formed explicitly for each t (tiny T only); o_t = scale S_t^T q_t."""
    T, dk = k.shape
    dv = v.shape[1]
    A = [gdn2_transition(alpha[t], erase[t], k[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S = s0.copy()
    for t in range(T):
        P = np.eye(dk)
        for i in range(t, -1, -1):
            P = P @ A[i]
        S = P @ s0
        for i in range(t + 1):
            Pi = np.eye(dk)
            for j in range(t, i, -1):
                Pi = Pi @ A[j]
            S = S + Pi @ np.outer(write[i] * k[i], v[i])
        o[t] = scale * S.T @ q[t]
    return o, S


def gated_write_linear_attention(q, k, v, alpha, write, s0, scale):
    """Closed form with no erasing (e = 0): S_t = Diag(G_t) S0 +
    sum_{i<=t} Diag(G_t / G_i) (w_i . k_i) v_i^T with G_t the running product of
    alpha, written as one weighted sum per t rather than a recurrence."""
    T, dk = k.shape
    G = np.cumprod(alpha, axis=0)                  # [T, dk]
    o = np.zeros((T, v.shape[1]))
    S = s0.copy()
    for t in range(T):
        ratio = G[t][None, :] / G[: t + 1]         # [t+1, dk]: G_t / G_i
        S = G[t][:, None] * s0 + (ratio * write[: t + 1] * k[: t + 1]).T @ v[: t + 1]
        o[t] = scale * S.T @ q[t]
    return o, S
