"""fp64 NumPy model of the chunk decomposition the HIP kernel uses.

Test-side only: it checks the chunk algebra (and, with ``bf16=True``, how
much bf16 rounding of the matrix-core operands costs) against the oracle
before and independently of the GPU code.  It is not the oracle and the HIP
library does not use it.

Per chunk of C = 64 tokens with start state S0 (dk x dv), zero-padded past
the end of the sequence with k = v = q = 0, beta = 0, alpha = 1 (an exact
no-op), and P_r = prod_{t <= r} alpha_t per key channel:

  Pm = P_31 (a mid-chunk reference), Pn = P_63
  Kr = K * P / Pm,  Qr = Q * P / Pm,  Kc = K * Pm / P
  A  = strict_lower(Kr Kc^T),  M = lower(Qr Kc^T)
  T  = (I + Diag(beta) A)^{-1} Diag(beta)        (blocked over 16 rows)
  X  = V - Kr (Pm * S0)                           (Pm scales the rows of S0)
  U  = T X
  O  = scale * (Qr (Pm * S0) + M U)
  S  = Pn * S0 + (Pn / Pm) * (Kc^T U)
"""
import numpy as np
import torch

C = 64
BLK = 16


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32).to(
        torch.bfloat16).to(torch.float64).numpy()


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def blocked_unit_lower_inverse(L, rnd):
    """Inverse of a unit lower-triangular 64x64 matrix: 16x16 diagonal blocks
    by forward substitution, then T_ab = -D_a sum_{j=b}^{a-1} L_aj T_jb."""
    n = L.shape[0]
    nb = n // BLK
    T = np.zeros_like(L)
    for a in range(nb):
        s = slice(a * BLK, (a + 1) * BLK)
        Laa = L[s, s]
        D = np.zeros((BLK, BLK))
        for j in range(BLK):  # column j of the block inverse
            x = np.zeros(BLK)
            for r in range(BLK):
                x[r] = (1.0 if r == j else 0.0) - Laa[r, :r] @ x[:r]
            D[:, j] = x
        T[s, s] = D
    for d in range(1, nb):
        for a in range(d, nb):
            b = a - d
            sa, sb = slice(a * BLK, (a + 1) * BLK), slice(b * BLK, (b + 1) * BLK)
            acc = np.zeros((BLK, BLK))
            for j in range(b, a):
                sj = slice(j * BLK, (j + 1) * BLK)
                acc += rnd(L[sa, sj]) @ rnd(T[sj, sb])
            T[sa, sb] = -(rnd(T[sa, sa]) @ rnd(acc))
    return T


def chunk_forward_unit(q, k, v, alpha, beta, s0, scale, bf16_ops=False):
    """One unit.  q, k, alpha: [T, dk]; v: [T, dv]; beta: [T]; s0: [dk, dv]."""
    rnd = bf16 if bf16_ops else (lambda x: x)
    T_, dk = k.shape
    dv = v.shape[1]
    S = s0.astype(np.float64).copy()
    o = np.zeros((T_, dv))
    for c0 in range(0, T_, C):
        n = min(C, T_ - c0)
        Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
        Al = np.ones((C, dk)); Be = np.zeros(C)
        Q[:n], K[:n], V[:n], Al[:n], Be[:n] = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n], \
            alpha[c0:c0 + n], beta[c0:c0 + n]
        P = np.cumprod(Al, axis=0)
        if bf16_ops:
            P = f32(np.cumprod(f32(Al), axis=0))
        Pm, Pn = P[31], P[C - 1]
        Kr, Qr, Kc = K * P / Pm, Q * P / Pm, K * Pm / P
        A = np.tril(rnd(Kr) @ rnd(Kc).T, -1)
        M = np.tril(rnd(Qr) @ rnd(Kc).T, 0)
        L = np.eye(C) + Be[:, None] * A
        Tm = blocked_unit_lower_inverse(L, rnd) * Be[None, :]
        SP = rnd(Pm[:, None] * S)
        X = V - rnd(Kr) @ SP
        U = rnd(Tm) @ rnd(X)
        O = scale * (rnd(Qr) @ SP + rnd(M) @ rnd(U))
        S = Pn[:, None] * S + (Pn / Pm)[:, None] * (rnd(Kc).T @ rnd(U))
        if bf16_ops:
            S = f32(S)
        o[c0:c0 + n] = O[:n]
    return o, S
