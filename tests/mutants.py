"""Deliberately wrong variants of the token loop, planted on the CPU.

Each one carries a single plausible mistake (an order swap, a dropped term, a
wrong sign, a transposed operand).  ``tests/test_oracle.py`` runs every pin
against each mutant and requires that at least one pin rejects it, which shows
that the pins can tell the oracle's arithmetic from a near miss.  None of
these is used anywhere else.
"""
import numpy as np


def _loop(q, k, v, alpha, beta, s0, scale, mistake):
    T, dk = k.shape
    dv = v.shape[1]
    S = s0.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        a, kt, vt, qt, bt = alpha[t], k[t], v[t], q[t], beta[t]
        prev = S.copy()
        if mistake == "predict_before_forget":
            vh = S.T @ kt
            S = a[:, None] * S
        elif mistake == "decay_value_side":
            S = S * a[None, :dv]
            vh = S.T @ kt
        elif mistake == "forget_after_write":
            vh = S.T @ kt
        else:
            S = a[:, None] * S
            vh = S.T @ kt
        if mistake == "error_sign":
            S = S + bt * np.outer(kt, vh - vt)
        elif mistake == "no_beta":
            S = S + np.outer(kt, vt - vh)
        elif mistake == "swap_k_v":  # the garbled DeltaNet formula on the interview page
            S = S + bt * np.outer(kt - S @ vt, vt)
        elif mistake == "no_erase":  # plain gated linear attention
            S = S + bt * np.outer(kt, vt)
        else:
            S = S + bt * np.outer(kt, vt - vh)
        if mistake == "forget_after_write":
            S = a[:, None] * S
        if mistake == "read_before_write":
            o[t] = scale * (a[:, None] * prev).T @ qt
        elif mistake == "no_scale":
            o[t] = S.T @ qt
        elif mistake == "read_with_key":
            o[t] = scale * S.T @ kt
        elif mistake == "read_transposed":
            o[t] = scale * S @ qt
        else:
            o[t] = scale * S.T @ qt
    return o, S


MISTAKES = [
    "predict_before_forget",
    "decay_value_side",
    "forget_after_write",
    "error_sign",
    "no_beta",
    "swap_k_v",
    "no_erase",
    "read_transposed",
    "read_before_write",
    "no_scale",
    "read_with_key",
]


def make(mistake):
    def impl(q, k, v, alpha, beta, s0, scale):
        return _loop(q, k, v, alpha, beta, s0, scale, mistake)
    impl.__name__ = "mutant_" + mistake
    return impl
