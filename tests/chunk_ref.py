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


def gdn2_chunk_forward_unit(q, k, v, alpha, erase, write, s0, scale, bf16_ops=False):
    """Gated DeltaNet-2, one unit, in the chunk decomposition of the HIP kernel
    (erase vectors a = e . k, write vectors c = w . k; Pred = the predictions
    S~_r^T k_r of the chunk's tokens):

      Kr = K * P / Pm, Qr = Q * P / Pm, Ec = (E.K) * Pm / P, Wc = (W.K) * Pm / P
      Y    = Kr (Pm * S0) + strict_lower(Kr Wc^T) V
      Pred = (I + strict_lower(Kr Ec^T))^{-1} Y                (blocked over 16 rows)
      O    = scale (Qr (Pm * S0) + [lower(Qr Wc^T) | lower(Qr Ec^T)] [V; -Pred])
      S    = Pn * S0 + (Pn / Pm) * ([Wc; Ec]^T [V; -Pred])
    """
    rnd = bf16 if bf16_ops else (lambda x: x)
    T_, dk = k.shape
    dv = v.shape[1]
    S = s0.astype(np.float64).copy()
    o = np.zeros((T_, dv))
    for c0 in range(0, T_, C):
        n = min(C, T_ - c0)
        Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
        Al = np.ones((C, dk)); E = np.zeros((C, dk)); W = np.zeros((C, dk))
        Q[:n], K[:n], V[:n] = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n]
        Al[:n], E[:n], W[:n] = alpha[c0:c0 + n], erase[c0:c0 + n], write[c0:c0 + n]
        P = np.cumprod(Al, axis=0)
        if bf16_ops:
            P = f32(np.cumprod(f32(Al), axis=0))
        Pm, Pn = P[31], P[C - 1]
        Kr, Qr = K * P / Pm, Q * P / Pm
        Ec, Wc = E * K * Pm / P, W * K * Pm / P
        La = np.tril(rnd(Kr) @ rnd(Ec).T, -1)
        Lc = np.tril(rnd(Kr) @ rnd(Wc).T, -1)
        Ma = np.tril(rnd(Qr) @ rnd(Ec).T, 0)
        Mc = np.tril(rnd(Qr) @ rnd(Wc).T, 0)
        SP = rnd(Pm[:, None] * S)
        Y = rnd(Kr) @ SP + rnd(Lc) @ rnd(V)
        Tm = blocked_unit_lower_inverse(np.eye(C) + La, rnd)
        Pred = rnd(Tm) @ rnd(Y)
        Z = np.concatenate([V, -Pred])
        O = scale * (rnd(Qr) @ SP + rnd(np.concatenate([Mc, Ma], 1)) @ rnd(Z))
        F = np.concatenate([Wc, Ec])
        S = Pn[:, None] * S + (Pn / Pm)[:, None] * (rnd(F).T @ rnd(Z))
        if bf16_ops:
            S = f32(S)
        o[c0:c0 + n] = O[:n]
    return o, S


def chunk_backward_unit(q, k, v, alpha, beta, s0, do, dsT, scale, bf16_ops=False):
    """Gradients of one unit in the chunk form the HIP backward uses (fp64; the
    decays referenced to the middle of each chunk as in the forward).

    Per chunk, with the chunk-start states S0 of a forward sweep and dS the
    gradient of the chunk-end state (from the next chunk, or dS_T):
      T' = (I + Diag(beta) A)^{-1},  Y = beta X,  U = T' Y
      dW   = (Pn/Pm) dS;            dU = scale M^T dO + Kc dW
      dY   = T'^T dU;               dX = beta dY;  dV = dX
      G    = dY U^T;  dA = -Diag(beta) G (strictly lower);  dM = scale dO U^T (lower)
      dbeta = rowsum(dY X) - rowsum(G A)           (strictly lower part of G)
      dQr  = scale dO SP^T + dM Kc;  dKr = -dX SP^T + dA Kc
      dKc  = U dW^T + dA^T Kr + dM^T Qr
      dq = dQr P/Pm,  dk = dKr P/Pm + dKc Pm/P
      dlogP_r = dKr Kr - dKc Kc + dQr Qr  (+ rowsum(dS S_C) at the last row)
      dalpha_t = (sum_{r >= t} dlogP_r) / alpha_t
      dS0  = Pn dS + Pm (scale Qr^T dO - Kr^T dX)
    Returns dq, dk, dv, dalpha, dbeta, dS0."""
    rnd = bf16 if bf16_ops else (lambda x: x)
    T_, dk = k.shape
    dv = v.shape[1]
    nch = (T_ + C - 1) // C
    # forward sweep: chunk-start states
    S = s0.astype(np.float64).copy()
    starts = []
    pieces = []
    for ch in range(nch):
        c0 = ch * C
        n = min(C, T_ - c0)
        Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
        Al = np.ones((C, dk)); Be = np.zeros(C); dO = np.zeros((C, dv))
        Q[:n], K[:n], V[:n], Al[:n], Be[:n], dO[:n] = q[c0:c0 + n], k[c0:c0 + n], \
            v[c0:c0 + n], alpha[c0:c0 + n], beta[c0:c0 + n], do[c0:c0 + n]
        P = np.cumprod(Al, axis=0)
        Pm, Pn = P[31], P[C - 1]
        Kr, Qr, Kc = K * P / Pm, Q * P / Pm, K * Pm / P
        A = np.tril(rnd(Kr) @ rnd(Kc).T, -1)
        M = np.tril(rnd(Qr) @ rnd(Kc).T, 0)
        Tp = blocked_unit_lower_inverse(np.eye(C) + Be[:, None] * A, rnd)
        starts.append(S.copy())
        SP = rnd(Pm[:, None] * S)
        X = V - rnd(Kr) @ SP
        U = rnd(Tp) @ rnd(Be[:, None] * X)
        S = Pn[:, None] * S + (Pn / Pm)[:, None] * (rnd(Kc).T @ rnd(U))
        pieces.append((n, Q, K, V, Al, Be, dO, P, Pm, Pn, Kr, Qr, Kc, A, M, Tp, SP, X, U))
    starts.append(S.copy())
    g_q, g_k, g_v = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    g_a, g_b = np.zeros_like(alpha), np.zeros_like(beta)
    dS = np.zeros((dk, dv)) if dsT is None else dsT.astype(np.float64).copy()
    for ch in reversed(range(nch)):
        n, Q, K, V, Al, Be, dO, P, Pm, Pn, Kr, Qr, Kc, A, M, Tp, SP, X, U = pieces[ch]
        SC = starts[ch + 1]
        dW = (Pn / Pm)[:, None] * dS
        dU = scale * rnd(M).T @ rnd(dO) + rnd(Kc) @ rnd(dW)
        dY = rnd(Tp).T @ rnd(dU)
        dX = Be[:, None] * dY
        G = rnd(dY) @ rnd(U).T
        dA = -Be[:, None] * np.tril(G, -1)
        dM = np.tril(scale * rnd(dO) @ rnd(U).T, 0)
        db = np.sum(dY * X, axis=1) - np.sum(np.tril(G, -1) * A, axis=1)
        dQr = scale * rnd(dO) @ SP.T + rnd(dM) @ rnd(Kc)
        dKr = -rnd(dX) @ SP.T + rnd(dA) @ rnd(Kc)
        dKc = rnd(U) @ rnd(dW).T + rnd(dA).T @ rnd(Kr) + rnd(dM).T @ rnd(Qr)
        ratio = P / Pm
        dlogP = dKr * Kr - dKc * Kc + dQr * Qr
        dlogP[C - 1] += np.sum(dS * SC, axis=1)
        dloga = np.cumsum(dlogP[::-1], axis=0)[::-1]
        c0 = ch * C
        g_q[c0:c0 + n] = (dQr * ratio)[:n]
        g_k[c0:c0 + n] = (dKr * ratio + dKc / ratio)[:n]
        g_v[c0:c0 + n] = dX[:n]
        g_a[c0:c0 + n] = (dloga / Al)[:n]
        g_b[c0:c0 + n] = db[:n]
        dSP = scale * rnd(Qr).T @ rnd(dO) - rnd(Kr).T @ rnd(dX)
        dS = Pn[:, None] * dS + Pm[:, None] * dSP
    return g_q, g_k, g_v, g_a, g_b, dS
