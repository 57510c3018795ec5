"""NumPy float64 forms of the bounded-decay KDA forward, for the oracle's self-checks.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU-baseline leg).

Sources on the pages:
  * gate g = g_min * sigmoid(.) with g_min = -5, and the unbounded log-sigmoid
    (negative softplus) form it replaces: "Trillion-Scale MoE Multimodal Models:
    Practical Techniques ...", sec. 3.2; "Breaking Through Trillion-Parameter
    Multimodal MoE", sec. 2.1.
  * chunked computation that scales by the cumulative decay Gamma and its
    inverse: first page sec. 3.1, third page sec. 2.1; the 16-token tile within
    which the inverse stays representable: first page sec. 3.2, third page
    sec. 2.1.
  * the incrementally updated constant-size state carried chunk to chunk:
    "Trillion-Parameter MoE Multimodal Models: Engineering Long-Context ...",
    sec. 3.2; the delta rule ("Delta Net"): third page sec. 2.1.

The state convention is S (dv x dk):
    S_t = S_{t-1} diag(exp g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.

Functions here:
  gate                -- the two gate forms, float64
  lowrank_preactivation -- the gate pre-activation from a rank-R factor
  recurrent           -- the same token recurrence as kda_oracle.c, vectorised
                         over rows (a second, independent transcription)
  brute_force         -- unrolled products of dense per-token transition matrices
  decayed_linear_attention -- quadratic (parallel) form of the erase-free case
  chunked             -- the chunk-parallel WY/UT form, three ways of applying
                         the within-chunk decay (pairwise, whole-chunk Gamma and
                         1/Gamma, 16-token sub-tile references)
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0  # the pages' fixed lower bound of the log-decay
SUBTILE = 16  # tokens per tile inside which 1/Gamma stays representable


def gate(a, g_min=G_MIN, mode="bounded"):
    """Log-decay g from the pre-activation a (float64)."""
    a = np.asarray(a, dtype=np.float64)
    if mode == "bounded":
        with np.errstate(over="ignore"):
            return g_min / (1.0 + np.exp(-a))
    if mode == "logsigmoid":
        # log sigmoid(a) = -softplus(-a), written so that no exp overflows
        return -(np.maximum(-a, 0.0) + np.log1p(np.exp(-np.abs(a))))
    raise ValueError(mode)


def lowrank_preactivation(h, z, A_log):
    """Gate pre-activation from a rank-R factor (the e^A h z of "Trillion-Scale MoE
    Multimodal Models: Practical Techniques ...", sec. 3.2), read as
        a[b, hd, t, c] = exp(A_log[hd, c]) * sum_j h[b, t, j] z[hd, c, j]
    with h [B,T,R] the per-token low-rank gate input shared by all heads, z [H,dk,R] each
    head's map from it to the key channels and A_log [H,dk] a per-channel log-scale.
    Returns a [B,H,T,dk] float64, the input of gate()."""
    h, z, A_log = _f64(h, z, A_log)
    lin = np.matmul(h[:, None, :, :], np.swapaxes(z, 1, 2)[None, :, :, :])  # [B,H,T,dk]
    return np.exp(A_log)[None, :, None, :] * lin


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def recurrent(q, k, v, a, beta, g_min=G_MIN, gate_mode="bounded", erase=True, S0=None):
    """Token-by-token recurrence; rows of S vectorised.  Returns (out, final_state)."""
    q, k, v, a, beta = _f64(q, k, v, a, beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = gate(a, g_min, gate_mode)
    S = np.zeros((B, H, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.empty((B, H, T, dv))
    for t in range(T):
        kt = k[:, :, t, :]                                   # [B,H,dk]
        S = S * np.exp(g[:, :, t, None, :])                  # S diag(exp g_t)
        if erase:
            Sk = np.einsum("bhij,bhj->bhi", S, kt)           # S k_t
            S = S - beta[:, :, t, None, None] * Sk[..., None] * kt[:, :, None, :]
        S = S + beta[:, :, t, None, None] * v[:, :, t, :, None] * kt[:, :, None, :]
        out[:, :, t, :] = np.einsum("bhij,bhj->bhi", S, q[:, :, t, :])
    return out, S


def brute_force(q, k, v, a, beta, g_min=G_MIN, gate_mode="bounded", S0=None):
    """Unrolled form: S_t = S0 P_1..P_t + sum_{s<=t} beta_s v_s k_s^T P_{s+1}..P_t,
    with dense P_r = diag(exp g_r)(I - beta_r k_r k_r^T).  Tiny inputs only."""
    q, k, v, a, beta = _f64(q, k, v, a, beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = gate(a, g_min, gate_mode)
    out = np.empty((B, H, T, dv))
    fin = np.empty((B, H, dv, dk))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            P = [np.diag(np.exp(g[b, h, r])) @ (eye - beta[b, h, r] * np.outer(k[b, h, r], k[b, h, r]))
                 for r in range(T)]
            for t in range(T):
                S = np.zeros((dv, dk))
                if S0 is not None:
                    M = np.asarray(S0[b, h], dtype=np.float64)
                    for r in range(t + 1):
                        M = M @ P[r]
                    S += M
                for s in range(t + 1):
                    M = beta[b, h, s] * np.outer(v[b, h, s], k[b, h, s])
                    for r in range(s + 1, t + 1):
                        M = M @ P[r]
                    S += M
                out[b, h, t] = S @ q[b, h, t]
                if t == T - 1:
                    fin[b, h] = S
    return out, fin


def decayed_linear_attention(q, k, v, a, beta, g_min=G_MIN, gate_mode="bounded", S0=None):
    """Quadratic form of the erase-free recurrence:
    o_t = S0 diag(e^{G_t}) q_t + sum_{s<=t} beta_s v_s (q_t . (e^{G_t - G_s} * k_s)),
    G = inclusive cumulative sum of g from the sequence start."""
    q, k, v, a, beta = _f64(q, k, v, a, beta)
    B, H, T, dk = q.shape
    G = np.cumsum(gate(a, g_min, gate_mode), axis=2)
    out = np.zeros(v.shape[:3] + (v.shape[-1],))
    for t in range(T):
        w = np.exp(G[:, :, t:t + 1, :] - G[:, :, :t + 1, :])            # [B,H,t+1,dk]
        s = np.einsum("bhc,bhsc->bhs", q[:, :, t, :], w * k[:, :, :t + 1, :])
        out[:, :, t, :] = np.einsum("bhs,bhsv->bhv", s * beta[:, :, :t + 1], v[:, :, :t + 1, :])
        if S0 is not None:
            out[:, :, t, :] += np.einsum("bhij,bhj->bhi", S0, np.exp(G[:, :, t, :]) * q[:, :, t, :])
    return out


def _pair_decay_products(X, Y, G, mode):
    """P[r, s] = sum_c X[r,c] Y[s,c] exp(G[r,c] - G[s,c]) for one chunk, three ways."""
    C = X.shape[0]
    if mode == "pairwise":       # explicit position-pair path
        return np.einsum("rc,sc,rsc->rs", X, Y, np.exp(G[:, None, :] - G[None, :, :]))
    if mode == "chunk":          # Gamma and 1/Gamma referenced to the chunk start
        return (X * np.exp(G)) @ (Y * np.exp(-G)).T
    if mode == "subtile":        # each 16-token row tile referenced to its own start
        P = np.zeros((C, C))
        for i0 in range(0, C, SUBTILE):
            rows = slice(i0, min(i0 + SUBTILE, C))
            rho = G[i0]
            P[rows, :] = (X[rows] * np.exp(G[rows] - rho)) @ (Y * np.exp(rho - G)).T
        return P
    raise ValueError(mode)


def chunked(q, k, v, a, beta, chunk, g_min=G_MIN, gate_mode="bounded", S0=None,
            decay_ref="subtile", return_parts=False):
    """Chunk-parallel (WY/UT) form, float64.  With S = state^T (dk x dv), per chunk:
        A_rs = beta_r sum_c k_rc k_sc e^{G_rc-G_sc} (s<r),  M_rs = sum_c q_rc k_sc e^{G_rc-G_sc} (s<=r)
        T = (I + A)^-1,  W = T diag(beta) (K*e^G),  U~ = T diag(beta) V
        U = U~ - W S,  O = (Q*e^G) S + M U,  S <- diag(e^{G_last}) S + (K*e^{G_last-G})^T U
    G is the inclusive cumulative sum of g restarted at every chunk.  The last
    chunk may be shorter than `chunk`."""
    q, k, v, a, beta = _f64(q, k, v, a, beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = gate(a, g_min, gate_mode)
    out = np.empty((B, H, T, dv))
    fin = np.empty((B, H, dv, dk))
    parts = []
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64).T
            for n0 in range(0, T, chunk):
                sl = slice(n0, min(n0 + chunk, T))
                Q, K, V, bt = q[b, h, sl], k[b, h, sl], v[b, h, sl], beta[b, h, sl]
                G = np.cumsum(g[b, h, sl], axis=0)
                C = Q.shape[0]
                A = np.tril(_pair_decay_products(K, K, G, decay_ref), -1) * bt[:, None]
                M = np.tril(_pair_decay_products(Q, K, G, decay_ref), 0)
                Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
                Kt, Qt = K * np.exp(G), Q * np.exp(G)
                Kh = K * np.exp(G[-1] - G)
                W = Tm @ (bt[:, None] * Kt)
                Ut = Tm @ (bt[:, None] * V)
                U = Ut - W @ S
                out[b, h, sl] = Qt @ S + M @ U
                if return_parts:
                    parts.append(dict(b=b, h=h, n0=n0, G=G, A=A, M=M, T=Tm, W=W, Ut=Ut,
                                      Kt=Kt, Qt=Qt, Kh=Kh, U=U, S_in=S.copy()))
                S = np.exp(G[-1])[:, None] * S + Kh.T @ U
            fin[b, h] = S.T
    if return_parts:
        return out, fin, parts
    return out, fin


def _gate_derivative(a, g_min, mode):
    s = 1.0 / (1.0 + np.exp(-a))
    return g_min * s * (1.0 - s) if mode == "bounded" else 1.0 - s


def chunked_backward(q, k, v, a, beta, dout, chunk, g_min=G_MIN, gate_mode="bounded", S0=None, dfinal=None):
    """Gradients of L = sum(dout * out) + sum(dfinal * final_state) by the chunk form (the
    algorithm the GPU backward follows), float64.  A forward pass keeps each chunk's start
    state S_n (S = state^T, dk x dv); a reverse pass over the chunks carries
    dS' = dL/d(state at the chunk's end), and for each chunk, with the quantities of chunked()
    and E_rsc = e^{G_rc - G_sc}:
        dU  = M^T dO + K^ dS'          dQ~ = dO S^T      dK^ = U dS'^T     dW = -dU S^T
        dM  = tril(dO U^T)             dgamma_c = sum_j S_cj dS'_cj
        dT  = dW (b K~)^T + dU (b V)^T dX = T^T dW       dY = T^T dU       dA = -strict_tril(T^T dT T^T)
        dv  = b dY                     dbeta = rowsum(dX K~ + dY V + dA P)   (P = A / b)
        dq  = sum_s dM_rs k_s E_rs + dQ~ e^G
        dk  = sum_r dM_rs q_r E_rs + sum_s' (b dA)_ss' k_s' E_ss' + sum_r (b dA)_rs k_r E_rs
              + b dX e^G + dK^ e^{G_last - G}
        dG  = q (first dq term) - k (first dk term) + k (second) - k (third) + dQ~ Q~ + b dX K~ - dK^ K^,
              and dG_last += sum_r dK^ K^ + dgamma e^{G_last}
        dg  = reverse cumulative sum of dG within the chunk,  da = dg * dg/da
        dS  = diag(gamma) dS' + Q~^T dO - W^T dU          (carried to the previous chunk)
    Returns the same dict as the oracle's adjoint: dq, dk, dv, da, dbeta, dS0."""
    q, k, v, a, beta, dout = _f64(q, k, v, a, beta, dout)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = gate(a, g_min, gate_mode)
    gp = _gate_derivative(a, g_min, gate_mode)
    res = {n: np.zeros(s) for n, s in (("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("da", q.shape),
                                        ("dbeta", beta.shape), ("dS0", (B, H, dv, dk)))}
    for b in range(B):
        for h in range(H):
            starts = list(range(0, T, chunk))
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64).T
            S_in = []
            for n0 in starts:                      # forward: chunk start states
                sl = slice(n0, min(n0 + chunk, T))
                S_in.append(S.copy())
                Q, K, V, bt = q[b, h, sl], k[b, h, sl], v[b, h, sl], beta[b, h, sl]
                G = np.cumsum(g[b, h, sl], axis=0)
                C = Q.shape[0]
                E = np.exp(G[:, None, :] - G[None, :, :])
                A = np.tril(np.einsum("rc,sc,rsc->rs", K, K, E), -1) * bt[:, None]
                Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
                W = Tm @ (bt[:, None] * K * np.exp(G))
                U = Tm @ (bt[:, None] * V) - W @ S
                S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1] - G)).T @ U
            dSp = np.zeros((dk, dv)) if dfinal is None else np.array(dfinal[b, h], dtype=np.float64).T
            for n0, S in zip(starts[::-1], S_in[::-1]):   # reverse over the chunks
                sl = slice(n0, min(n0 + chunk, T))
                Q, K, V, bt, dO = q[b, h, sl], k[b, h, sl], v[b, h, sl], beta[b, h, sl], dout[b, h, sl]
                G = np.cumsum(g[b, h, sl], axis=0)
                C = Q.shape[0]
                E = np.exp(G[:, None, :] - G[None, :, :])
                P = np.tril(np.einsum("rc,sc,rsc->rs", K, K, E), -1)
                A = P * bt[:, None]
                M = np.tril(np.einsum("rc,sc,rsc->rs", Q, K, E), 0)
                Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
                Kt, Qt, Kh, gam = K * np.exp(G), Q * np.exp(G), K * np.exp(G[-1] - G), np.exp(G[-1])
                X, Y = bt[:, None] * Kt, bt[:, None] * V
                W = Tm @ X
                U = Tm @ Y - W @ S
                dU = M.T @ dO + Kh @ dSp
                dQt = dO @ S.T
                dKh = U @ dSp.T
                dW = -dU @ S.T
                dM = np.tril(dO @ U.T, 0)
                dgam = np.sum(S * dSp, axis=1)
                dT = dW @ X.T + dU @ Y.T
                dX = Tm.T @ dW
                dY = Tm.T @ dU
                dA = np.tril(-Tm.T @ dT @ Tm.T, -1)
                dP = bt[:, None] * dA
                dqM = np.einsum("rs,sc,rsc->rc", dM, K, E)
                dkM = np.einsum("rs,rc,rsc->sc", dM, Q, E)
                dkR = np.einsum("rs,sc,rsc->rc", dP, K, E)
                dkC = np.einsum("rs,rc,rsc->sc", dP, K, E)
                res["dv"][b, h, sl] = bt[:, None] * dY
                res["dbeta"][b, h, sl] = np.sum(dX * Kt, 1) + np.sum(dY * V, 1) + np.sum(dA * P, 1)
                res["dq"][b, h, sl] = dqM + dQt * np.exp(G)
                res["dk"][b, h, sl] = dkM + dkR + dkC + dX * bt[:, None] * np.exp(G) + dKh * np.exp(G[-1] - G)
                dG = Q * dqM - K * dkM + K * dkR - K * dkC + dQt * Qt + bt[:, None] * dX * Kt - dKh * Kh
                dG[-1] += np.sum(dKh * Kh, 0) + dgam * gam
                dg = np.cumsum(dG[::-1], axis=0)[::-1]
                res["da"][b, h, sl] = dg * gp[b, h, sl]
                dSp = gam[:, None] * dSp + Qt.T @ dO - W.T @ dU
            res["dS0"][b, h] = dSp.T
    return res
