"""fp64 CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it, and the two share no code.

The arithmetic lives in ``kda_oracle.c`` (plain C, double precision, a token
loop: forget, predict, correct and write, read; for Gated DeltaNet-2 forget,
predict, erase, write, read; and the chain rule of the KDA loop in reverse).  This module only converts
inputs to contiguous float64 arrays, reorders the [B, T, H, d] token layout
into per-unit blocks, and calls the C library through ctypes.

Pins: every function here is pinned by ``tests/test_oracle.py`` against
closed forms, brute force and invariants stated on the pages; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/libkda_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
             "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.kda_oracle_step.restype = ctypes.c_int
        lib.kda_oracle_step.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                        ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_int]
        lib.gdn2_oracle_forward.restype = ctypes.c_int
        lib.gdn2_oracle_forward.argtypes = [dp] * 9 + [ctypes.c_long, ctypes.c_long,
                                                       ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_double, ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [dp] * 14 + [ctypes.c_long, ctypes.c_long,
                                                        ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_double, ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    """Exact widening of a stored tensor/array (fp32, bf16, fp64) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def channel_gate(alpha, gate, dk, lead=None):
    """The per-channel decays a forget gate stands for, as float64 [..., dk].

    gate "channel": alpha already holds one decay per key channel (KDA,
    "Kimi Delta Attention", section "一、Diag(α_t)：通道级遗忘").
    gate "head": one decay per token and head scales the whole state,
    alpha_t S = Diag(alpha_t 1) S (Gated DeltaNet, bugfactory.tech news 3610,
    third paragraph): the value is repeated over the dk channels.
    gate "none": no forget gate (DeltaNet, the same page's second paragraph):
    every decay is 1; ``lead`` gives the leading shape.
    """
    if gate == "channel":
        return _f64(alpha)
    if gate == "head":
        a = _f64(alpha)
        return np.ascontiguousarray(np.repeat(a[..., None], dk, axis=-1))
    if gate == "none":
        return np.ones(tuple(lead) + (dk,), np.float64)
    raise ValueError("unknown gate %r" % (gate,))


def prepare(q, k, alpha, beta, gate="channel", gate_logits=False, beta_logits=False,
            qk_l2norm=False, lead=None):
    """The inputs the recurrence takes, from the stored tensors of a call with
    in-kernel input preparation, as float64 (q, k, per-channel alpha, beta).

    gate_logits: alpha holds logits z and the decay is the logistic function
    1 / (1 + exp(-z)), which maps any logit into (0, 1) as the per-channel
    decay of "Kimi Delta Attention", section "一、Diag(α_t)：通道级遗忘"
    requires; beta_logits: the same map for the write strength beta.
    qk_l2norm: q and k divided by sqrt(sum of squares + 1e-6) per token and
    head.  gate and lead as for channel_gate.
    """
    q, k = _f64(q), _f64(k)
    dk = q.shape[-1]
    if qk_l2norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    a = None if alpha is None else _f64(alpha)
    if gate_logits:
        a = 1.0 / (1.0 + np.exp(-a))
    a = channel_gate(a, gate, dk, q.shape[:-1] if lead is None else lead)
    b = _f64(beta)
    if beta_logits:
        b = 1.0 / (1.0 + np.exp(-b))
    return q, k, a, b


def forward_units(q, k, v, alpha, beta, initial_state=None, scale=None, threads=0,
                  want_o=True):
    """Token loop over independent units.

    q, k, alpha: [U, T, dk]; v: [U, T, dv]; beta: [U, T];
    initial_state: [U, dk, dv] or None (zero state).
    Returns (o [U, T, dv] or None, final_state [U, dk, dv]), float64.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    s0 = _f64(initial_state)
    U, T, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (U, T, dk) and alpha.shape == (U, T, dk)
    assert v.shape == (U, T, dv) and beta.shape == (U, T)
    if s0 is not None:
        assert s0.shape == (U, dk, dv)
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((U, T, dv), np.float64) if want_o else None
    sT = np.zeros((U, dk, dv), np.float64)
    rc = _load().kda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(s0), _ptr(o), _ptr(sT), U, T, dk, dv,
                                    float(scale), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_forward failed with %d" % rc)
    return o, sT


def forward(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, scale=None,
            threads=0, heads=None):
    """Oracle in the library's token layout.

    Dense:  q, k, alpha [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
            initial_state [B, H, dk, dv] or None.
    Varlen: B == 1, cu_seqlens (length N+1, host ints) splits T into N
            sequences; initial_state [N, H, dk, dv] or None.
    heads:  optional list of head indices to evaluate (a sample); the result
            then holds only those heads, in that order.
    Returns (o [B, T, Hs, dv], final_state [B or N, Hs, dk, dv]), float64.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    s0 = _f64(initial_state)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    hs = list(range(H)) if heads is None else list(heads)
    sel = np.asarray(hs, dtype=np.int64)
    if cu_seqlens is None:
        starts = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = [int(c) for c in cu_seqlens]
        starts = [(0, cu[n], cu[n + 1] - cu[n]) for n in range(len(cu) - 1)]
    o_all = np.zeros((B, T, len(hs), dv), np.float64)
    s_all = np.zeros((len(starts), len(hs), dk, dv), np.float64)
    for n, (b, t0, L) in enumerate(starts):
        def units(x):  # [L, Hs, d] -> [Hs, L, d]
            return np.ascontiguousarray(np.moveaxis(x[b, t0:t0 + L][:, sel], 1, 0))
        init = None if s0 is None else s0[n][sel]
        o_u, s_u = forward_units(units(q), units(k), units(v), units(alpha),
                                 np.ascontiguousarray(beta[b, t0:t0 + L][:, sel].T),
                                 init, scale=scale, threads=threads)
        o_all[b, t0:t0 + L] = np.moveaxis(o_u, 0, 1)
        s_all[n] = s_u
    return o_all, s_all


def gdn2_forward_units(q, k, v, alpha, erase, write, initial_state=None, scale=None,
                       threads=0):
    """Gated DeltaNet-2 token loop over independent units (``run_unit_gdn2`` in
    ``kda_oracle.c``): forget with alpha, predict, erase along e . k, write
    along w . k, read ("线性注意力机制：从标准注意力到 Gated DeltaNet-2",
    jindou-blog, section 4, with the reading stated in the C source).

    q, k, alpha, erase, write: [U, T, dk]; v: [U, T, dv]; initial_state
    [U, dk, dv] or None.  Returns (o [U, T, dv], final_state [U, dk, dv])."""
    q, k, v, alpha, erase, write = (_f64(x) for x in (q, k, v, alpha, erase, write))
    s0 = _f64(initial_state)
    U, T, dk = q.shape
    dv = v.shape[2]
    for x in (k, alpha, erase, write):
        assert x.shape == (U, T, dk)
    assert v.shape == (U, T, dv)
    if s0 is not None:
        assert s0.shape == (U, dk, dv)
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((U, T, dv), np.float64)
    sT = np.zeros((U, dk, dv), np.float64)
    rc = _load().gdn2_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
                                     _ptr(write), _ptr(s0), _ptr(o), _ptr(sT), U, T, dk, dv,
                                     float(scale), int(threads))
    if rc != 0:
        raise RuntimeError("gdn2_oracle_forward failed with %d" % rc)
    return o, sT


def gdn2_forward(q, k, v, alpha, erase, write, initial_state=None, cu_seqlens=None,
                 scale=None, threads=0, heads=None):
    """gdn2_forward_units in the library's token layout: q, k, alpha, erase,
    write [B, T, H, dk] (alpha None: no forget gate, alpha = 1); v [B, T, H, dv];
    initial_state [B or N, H, dk, dv] or None; cu_seqlens and heads as for
    ``forward``.  Returns (o [B, T, Hs, dv], final_state [B or N, Hs, dk, dv])."""
    q, k, v, erase, write = (_f64(x) for x in (q, k, v, erase, write))
    alpha = np.ones_like(k) if alpha is None else _f64(alpha)
    s0 = _f64(initial_state)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    hs = list(range(H)) if heads is None else list(heads)
    sel = np.asarray(hs, dtype=np.int64)
    if cu_seqlens is None:
        starts = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = [int(c) for c in cu_seqlens]
        starts = [(0, cu[n], cu[n + 1] - cu[n]) for n in range(len(cu) - 1)]
    o_all = np.zeros((B, T, len(hs), dv), np.float64)
    s_all = np.zeros((len(starts), len(hs), dk, dv), np.float64)
    for n, (b, t0, L) in enumerate(starts):
        def units(x):  # [L, Hs, d] -> [Hs, L, d]
            return np.ascontiguousarray(np.moveaxis(x[b, t0:t0 + L][:, sel], 1, 0))
        init = None if s0 is None else s0[n][sel]
        o_u, s_u = gdn2_forward_units(units(q), units(k), units(v), units(alpha), units(erase),
                                      units(write), init, scale=scale, threads=threads)
        o_all[b, t0:t0 + L] = np.moveaxis(o_u, 0, 1)
        s_all[n] = s_u
    return o_all, s_all


def gdn2_step(q, k, v, alpha, erase, write, state, scale=None, threads=0, in_place=False):
    """One Gated DeltaNet-2 decode step: q, k, alpha, erase, write [N, H, dk]
    (alpha None: no forget gate); v [N, H, dv]; state [N, H, dk, dv].  Returns
    (o [N, H, dv], new_state), float64.  The input state is not modified unless
    in_place is set and it is a contiguous float64 array, which is then
    rewritten and returned (each unit reads its state before writing it)."""
    q, k, v, erase, write = (_f64(x) for x in (q, k, v, erase, write))
    alpha = np.ones_like(k) if alpha is None else _f64(alpha)
    N, H, dk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = dk ** -0.5
    if in_place and isinstance(state, np.ndarray) and state.dtype == np.float64 \
            and state.flags.c_contiguous:
        st = state
    else:
        st = _f64(state).copy()
    o = np.zeros((N, H, dv), np.float64)
    c = lambda x: np.ascontiguousarray(x)
    rc = _load().gdn2_oracle_forward(_ptr(c(q)), _ptr(c(k)), _ptr(c(v)), _ptr(c(alpha)),
                                     _ptr(c(erase)), _ptr(c(write)), _ptr(st), _ptr(o), _ptr(st),
                                     N * H, 1, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise RuntimeError("gdn2_oracle_forward failed with %d" % rc)
    return o, st


def backward_units(q, k, v, alpha, beta, initial_state, do, dfinal_state=None, scale=None,
                   threads=0):
    """Gradients of the token loop, float64: ``kda_oracle_backward`` in
    ``kda_oracle.c``, the chain rule through the four steps of each token
    (forget, predict, correct and write, read; the update equation of "Kimi
    Delta Attention", section "KDA 的更新式", with the order of
    bugfactory.tech news 3610, second to fourth paragraphs) in reverse token
    order, threaded over the independent units.

    q, k, alpha: [U, T, dk]; v: [U, T, dv]; beta: [U, T]; initial_state
    [U, dk, dv] or None; do: [U, T, dv] (gradient of o); dfinal_state
    [U, dk, dv] or None (gradient of the final state).
    Returns dq, dk, dv, dalpha, dbeta, dinitial_state (same shapes as the
    inputs).  Each thread keeps one unit's T forward states (T * dk * dv
    doubles).
    """
    q, k, v, alpha, beta, do = (_f64(x) for x in (q, k, v, alpha, beta, do))
    s0, dsT = _f64(initial_state), _f64(dfinal_state)
    U, T, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (U, T, dk) and alpha.shape == (U, T, dk) and beta.shape == (U, T)
    assert v.shape == (U, T, dv) and do.shape == (U, T, dv)
    if scale is None:
        scale = dk ** -0.5
    g = [np.zeros_like(x) for x in (q, k, v, alpha, beta)] + [np.zeros((U, dk, dv))]
    rc = _load().kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(s0), _ptr(do), _ptr(dsT), *[_ptr(x) for x in g],
                                     U, T, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_backward failed with %d" % rc)
    return tuple(g)


def backward_units_numpy(q, k, v, alpha, beta, initial_state, do, dfinal_state=None,
                         scale=None):
    """The same gradients written a second time, in NumPy with the steps as
    whole-array operations (small cases only: the forward states of every
    unit are kept).  It serves to pin ``backward_units``; both are pinned by
    central differences of the forward."""
    q, k, v, alpha, beta, do = (_f64(x) for x in (q, k, v, alpha, beta, do))
    U, T, dk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = dk ** -0.5
    S = np.zeros((U, dk, dv)) if initial_state is None else _f64(initial_state).copy()
    s_prev = np.empty((T, U, dk, dv))
    resid = np.empty((T, U, dv))  # v_t - vhat_t
    for t in range(T):
        s_prev[t] = S
        st = alpha[:, t, :, None] * S                                 # forget
        vhat = np.einsum("uij,ui->uj", st, k[:, t])                   # predict
        resid[t] = v[:, t] - vhat
        S = st + beta[:, t, None, None] * k[:, t, :, None] * resid[t][:, None, :]  # write
    dS = np.zeros((U, dk, dv)) if dfinal_state is None else _f64(dfinal_state).copy()
    g_q, g_k, g_v = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    g_a, g_b = np.zeros_like(alpha), np.zeros_like(beta)
    for t in reversed(range(T)):
        st = alpha[:, t, :, None] * s_prev[t]
        e = beta[:, t, None] * resid[t]
        s_t = st + k[:, t, :, None] * e[:, None, :]
        # read: o_t = scale S_t^T q_t
        g_q[:, t] = scale * np.einsum("uij,uj->ui", s_t, do[:, t])
        dS = dS + scale * q[:, t, :, None] * do[:, t, None, :]
        # write: S_t = S~ + k_t e^T
        g_k[:, t] = np.einsum("uij,uj->ui", dS, e)
        de = np.einsum("uij,ui->uj", dS, k[:, t])
        # correct: e = beta_t (v_t - vhat)
        g_b[:, t] = np.sum(de * resid[t], axis=-1)
        g_v[:, t] = beta[:, t, None] * de
        dvhat = -beta[:, t, None] * de
        # predict: vhat = S~^T k_t
        dst = dS + k[:, t, :, None] * dvhat[:, None, :]
        g_k[:, t] += np.einsum("uij,uj->ui", st, dvhat)
        # forget: S~ = Diag(alpha_t) S_{t-1}
        g_a[:, t] = np.sum(dst * s_prev[t], axis=-1)
        dS = alpha[:, t, :, None] * dst
    return g_q, g_k, g_v, g_a, g_b, dS


def backward(q, k, v, alpha, beta, initial_state, do, dfinal_state=None, cu_seqlens=None,
             scale=None, threads=0, heads=None):
    """backward_units in the library's token layout (dense [B, T, H, d], or
    B == 1 with cu_seqlens); returns dq, dk, dv, dalpha, dbeta, dinitial_state
    ([B or N, H, dk, dv]).  heads: optional list of head indices (a sample);
    the results then hold only those heads, in that order."""
    q, k, v, alpha, beta, do = (_f64(x) for x in (q, k, v, alpha, beta, do))
    s0 = _f64(initial_state)
    ds = _f64(dfinal_state)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    hs = list(range(H)) if heads is None else list(heads)
    sel = np.asarray(hs, dtype=np.int64)
    if cu_seqlens is None:
        starts = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = [int(c) for c in cu_seqlens]
        starts = [(0, cu[n], cu[n + 1] - cu[n]) for n in range(len(cu) - 1)]
    Hs = len(hs)
    outs = [np.zeros((B, T, Hs) + x.shape[3:]) for x in (q, k, v, alpha, beta)]
    g_s0 = np.zeros((len(starts), Hs, dk, dv))
    for n, (b, t0, L) in enumerate(starts):
        def units(x):  # [L, H, ...] -> [Hs, L, ...]
            return np.ascontiguousarray(np.moveaxis(x[b, t0:t0 + L][:, sel], 1, 0))
        res = backward_units(units(q), units(k), units(v), units(alpha), units(beta),
                             None if s0 is None else s0[n][sel], units(do),
                             None if ds is None else ds[n][sel], scale=scale, threads=threads)
        for i in range(5):
            outs[i][b, t0:t0 + L] = np.moveaxis(res[i], 0, 1)
        g_s0[n] = res[5]
    return tuple(outs) + (g_s0,)


def step(q, k, v, alpha, beta, state, scale=None, threads=0, in_place=False):
    """One decode step.  q, k, alpha [N, H, dk]; v [N, H, dv]; beta [N, H];
    state [N, H, dk, dv].  Returns (o [N, H, dv], new_state), float64.  The
    input state is not modified unless in_place is set and it is already a
    contiguous float64 array, which is then rewritten and returned."""
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = dk ** -0.5
    if in_place and isinstance(state, np.ndarray) and state.dtype == np.float64 \
            and state.flags.c_contiguous:
        st = state.reshape(N * H, dk, dv)
    else:
        st = _f64(state).reshape(N * H, dk, dv).copy()
    o = np.zeros((N * H, dv), np.float64)
    rc = _load().kda_oracle_step(_ptr(np.ascontiguousarray(q.reshape(N * H, dk))),
                                 _ptr(np.ascontiguousarray(k.reshape(N * H, dk))),
                                 _ptr(np.ascontiguousarray(v.reshape(N * H, dv))),
                                 _ptr(np.ascontiguousarray(alpha.reshape(N * H, dk))),
                                 _ptr(np.ascontiguousarray(beta.reshape(N * H))),
                                 _ptr(st), _ptr(o), N * H, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_step failed with %d" % rc)
    return o.reshape(N, H, dv), st.reshape(N, H, dk, dv)
