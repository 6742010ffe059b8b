"""The chunked algebra of the pages, in float64, for validation only.

TEST INFRASTRUCTURE ONLY.  None of these is used for GPU parity: parity is
always against the sequential rule in :mod:`oracle`.  They exist so that the
tests can show that the chunked reformulations the pages describe reach the
sequential result (up to float association) at every chunk size, tail and
decay, which is the property the GPU kernel relies on.

All decay ratios are formed as products of decays, never as quotients (the
ferrox-core ``gdn_chunk.rs`` page, "The algebra": a product that underflows
means the state has really been forgotten).

Each function takes one (batch, value-head) slot:
``S0`` [Dv,Dk], ``q, k`` [T,Dk], ``v`` [T,Dv], ``g, beta`` [T] (float64) and
the chunk size ``C``; it returns ``(y [T,Dv], S_end [Dv,Dk])``.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _gates(gc):
    """Chunk-local gate products for decays ``gc`` [c].

    Returns ``G`` [c] with G[t] = g_0 ... g_t and ``R`` [c,c] with
    R[t,j] = g_{j+1} ... g_t for j <= t (R[t,t] = 1) and 0 above the
    diagonal, each entry built by multiplying, never by dividing.
    """
    c = gc.shape[0]
    G = np.empty(c)
    acc = 1.0
    for t in range(c):
        acc *= gc[t]
        G[t] = acc
    R = np.zeros((c, c))
    for t in range(c):
        r = 1.0
        R[t, t] = 1.0
        for j in range(t - 1, -1, -1):
            r *= gc[j + 1]
            R[t, j] = r
    return G, R


def _unit_lower_solve(M, rhs):
    """Solve (I + M) X = rhs for strictly lower triangular M."""
    return solve_triangular(np.eye(M.shape[0]) + M, rhs, lower=True,
                            unit_diagonal=True)


def two_solve_wy(S0, q, k, v, g, beta, C):
    """The nine steps of the metaltile-std page ("Algorithm"), per chunk.

    Steps 4 and 5 are the two forward substitutions (I+L)p = K and
    (I+A)u = beta*V; step 9 uses K in the correction term, as the page's
    derivation in its header states.  The chunk outputs are scaled by
    1/sqrt(Dk) to match the rule's read-out.
    """
    T, Dk = k.shape
    S = S0.copy()
    y = np.empty((T, v.shape[1]))
    scale = 1.0 / np.sqrt(Dk)
    for t0 in range(0, T, C):
        sl = slice(t0, min(t0 + C, T))
        K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
        G, Gam = _gates(gc)                              # step 2
        KKT = K @ K.T                                    # step 3
        QKT = Q @ K.T
        L = np.tril(KKT, -1) * bc[None, :]               # L[t,j] = b_j KKT[t,j]
        p = _unit_lower_solve(L, K)                      # step 4
        A = np.tril(KKT, -1) * Gam * bc[:, None]         # A[t,j] = b_t Gam KKT
        uv = _unit_lower_solve(A, bc[:, None] * V)       # step 5
        y_local = (np.tril(QKT) * Gam) @ uv              # step 6
        S0p = S @ p.T                                    # [Dv, c]
        corr = (np.tril(QKT) * bc[None, :]) @ S0p.T      # sum_{i<=t} b_i QKT S0 p_i
        y_pass = G[:, None] * (Q @ S.T - corr)           # step 7
        y[sl] = (y_pass + y_local) * scale               # step 8
        Gc = G[-1]                                       # step 9 (with K)
        S = Gc * (S - (S0p * bc[None, :]) @ K) + (uv * Gam[-1][:, None]).T @ K
    return y, S


def per_row(S0, q, k, v, g, beta, C):
    """The ferrox-core page's chunk body: one forward substitution per row.

    m = S0 K^T and n = S0 Q^T against the chunk's keys and queries, the two
    triangles k_u.k_t and k_u.q_t, then d_t row by row, then the state once
    per chunk (the page's ``delta_chunk``), with A_t = g_0...g_t.
    """
    T, Dk = k.shape
    S = S0.copy()
    y = np.empty((T, v.shape[1]))
    scale = 1.0 / np.sqrt(Dk)
    for t0 in range(0, T, C):
        sl = slice(t0, min(t0 + C, T))
        K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
        c = K.shape[0]
        a, R = _gates(gc)
        m = S @ K.T                                      # [Dv, c]
        n = S @ Q.T
        gram = K @ K.T
        qk = Q @ K.T                                     # qk[t,u] = q_t.k_u
        d = np.zeros((c, v.shape[1]))
        for t in range(c):
            pred = a[t] * m[:, t] + (R[t, :t] * gram[t, :t]) @ d[:t]
            d[t] = bc[t] * (V[t] - pred)
            read = a[t] * n[:, t] + (R[t, :t + 1] * qk[t, :t + 1]) @ d[:t + 1]
            y[t0 + t] = read * scale
        S = a[-1] * S + (d * R[-1][:, None]).T @ K
    return y, S


def unified_wy(S0, q, k, v, g, beta, C):
    """One unit-lower-triangular system for both of the page's solves.

    With A[t,j] = b_t R[t,j] k_t.k_j (j < t), (I+A)[W | U] = [b G K | b V]
    gives W = (b G) p (the metaltile page's step 4 up to row scaling) and
    U = u (its step 5).  Then D = U - W S0^T are the true per-token deltas
    (the ferrox page's d), Y = G (Q S0^T) + (QK^T * R, causal) D and
    S_end = G_last S0 + D^T diag(R[last,:]) K.
    """
    T, Dk = k.shape
    S = S0.copy()
    y = np.empty((T, v.shape[1]))
    scale = 1.0 / np.sqrt(Dk)
    for t0 in range(0, T, C):
        sl = slice(t0, min(t0 + C, T))
        K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
        G, R = _gates(gc)
        A = np.tril(K @ K.T, -1) * R * bc[:, None]
        rhs = np.concatenate([(bc * G)[:, None] * K, bc[:, None] * V], axis=1)
        WU = _unit_lower_solve(A, rhs)
        W, U = WU[:, :Dk], WU[:, Dk:]
        D = U - W @ S.T
        y[sl] = (G[:, None] * (Q @ S.T) + (np.tril(Q @ K.T) * R) @ D) * scale
        S = G[-1] * S + (D * R[-1][:, None]).T @ K
    return y, S


FORMS = {"two_solve_wy": two_solve_wy, "per_row": per_row,
         "unified_wy": unified_wy}


def run(form, q, k, v, g, beta, state, C):
    """Apply one chunk form to every (b, hv) slot of a full input set."""
    fn = FORMS[form] if isinstance(form, str) else form
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    y = np.empty((B, T, Hv, Dv))
    S_out = np.empty((B, Hv, Dv, Dk))
    for b in range(B):
        for hv in range(Hv):
            hk = hv // (Hv // Hk)
            S0 = np.zeros((Dv, Dk)) if state is None else np.asarray(state[b, hv], dtype=np.float64)
            yy, ss = fn(S0, q[b, :, hk], k[b, :, hk], v[b, :, hv], g[b, :, hv], beta[b, :, hv], C)
            y[b, :, hv] = yy
            S_out[b, hv] = ss
    return y, S_out
