"""The chunked algebra of the pages reaches the sequential rule.

The ferrox-core gdn_chunk.rs page states that the chunked rule is identical
to the sequential one up to float association and tests it at shapes where
the chunk boundary falls short of, at, and past a chunk, with decays from
"barely decays" to "forgets almost at once" (its tests
``a_chunk_is_the_sequential_recurrence`` and
``a_vanishing_decay_is_forgetting_and_not_a_division``).  Here the three
float64 chunk forms of :mod:`oracle.chunk_forms` are checked the same way at
many chunk sizes, which pins both the forms and the sequential oracle (they
are independent derivations), and two wrong forms are shown to fail.
"""
import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle
from oracle import chunk_forms as cf

CS = [1, 2, 3, 4, 5, 8, 16, 32, 64]


def case(seed, B, T, Hk, Hv, Dk, Dv, g_lo=0.05, g_hi=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    g = rng.uniform(g_lo, g_hi, (B, T, Hv))
    beta = rng.uniform(0.0, 1.0, (B, T, Hv))
    S0 = rng.standard_normal((B, Hv, Dv, Dk)) * 0.4
    return q, k, v, g, beta, S0


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("form", list(cf.FORMS))
@pytest.mark.parametrize("C", CS)
def test_form_equals_sequential(form, C):
    for T in sorted({3, 7, C, C + 5, 2 * C + 1}):
        args = case(C * 100 + T, 1, T, 2, 4, 8, 6)
        y, S = oracle.forward(*args)
        yc, Sc = cf.run(form, *args, C)
        assert rel(yc, y) < 1e-12, (form, C, T)
        assert rel(Sc, S) < 1e-12, (form, C, T)


@pytest.mark.parametrize("form", list(cf.FORMS))
def test_long_memory_many_chunks(form):
    # decays in [0.95, 1): the state carries across many chunk boundaries
    args = case(7, 1, 200, 1, 2, 16, 16, g_lo=0.95, g_hi=1.0)
    y, S = oracle.forward(*args)
    for C in (16, 64):
        yc, Sc = cf.run(form, *args, C)
        assert rel(yc, y) < 1e-11 and rel(Sc, S) < 1e-11


@pytest.mark.parametrize("form", list(cf.FORMS))
@pytest.mark.parametrize("gval", [0.0, 1e-20, 1e-45])
def test_vanishing_decay_is_a_product(form, gval):
    q, k, v, g, beta, S0 = case(3, 1, 37, 1, 2, 8, 8)
    g[:] = gval
    y, S = oracle.forward(q, k, v, g, beta, S0)
    yc, Sc = cf.run(form, q, k, v, g, beta, S0, 16)
    assert np.all(np.isfinite(yc)) and np.all(np.isfinite(Sc))
    assert np.max(np.abs(yc - y)) < 1e-12 and np.max(np.abs(Sc - S)) < 1e-12


def test_independent_of_chunk_size():
    args = case(9, 2, 70, 2, 4, 16, 8, g_lo=0.5)
    outs = [cf.run("unified_wy", *args, C) for C in (16, 32, 64)]
    for yc, Sc in outs[1:]:
        assert rel(yc, outs[0][0]) < 1e-12 and rel(Sc, outs[0][1]) < 1e-12


# --------------------------------------------------------- wrong forms
def _step9_with_p(S0, q, k, v, g, beta, C):
    """The metaltile page's chunk with its step 9 correction using p in place
    of k (the form its kernel body codes); a negative control."""
    T, Dk = k.shape
    S = S0.copy()
    y = np.empty((T, v.shape[1]))
    for t0 in range(0, T, C):
        sl = slice(t0, min(t0 + C, T))
        K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
        G, Gam = cf._gates(gc)
        KKT, QKT = K @ K.T, Q @ K.T
        p = cf._unit_lower_solve(np.tril(KKT, -1) * bc[None, :], K)
        uv = cf._unit_lower_solve(np.tril(KKT, -1) * Gam * bc[:, None], bc[:, None] * V)
        S0p = S @ p.T
        corr = (np.tril(QKT) * bc[None, :]) @ S0p.T
        y[sl] = (G[:, None] * (Q @ S.T - corr) + (np.tril(QKT) * Gam) @ uv) / np.sqrt(Dk)
        S = G[-1] * (S - (S0p * bc[None, :]) @ p) + (uv * Gam[-1][:, None]).T @ K
    return y, S


def _ratios_by_division(S0, q, k, v, g, beta, C):
    """The unified form with R[t,j] = G_t / G_j; a negative control."""
    T, Dk = k.shape
    S = S0.copy()
    y = np.empty((T, v.shape[1]))
    with np.errstate(all="ignore"):
        for t0 in range(0, T, C):
            sl = slice(t0, min(t0 + C, T))
            K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
            G = np.cumprod(gc)
            R = np.tril(G[:, None] / G[None, :])
            A = np.tril(K @ K.T, -1) * R * bc[:, None]
            WU = solve_triangular(np.eye(A.shape[0]) + A,
                                  np.concatenate([(bc * G)[:, None] * K, bc[:, None] * V], 1),
                                  lower=True, unit_diagonal=True, check_finite=False)
            D = WU[:, Dk:] - WU[:, :Dk] @ S.T
            y[sl] = (G[:, None] * (Q @ S.T) + (np.tril(Q @ K.T) * R) @ D) / np.sqrt(Dk)
            S = G[-1] * S + (D * R[-1][:, None]).T @ K
    return y, S


def test_step9_with_p_is_wrong():
    args = case(21, 1, 16, 1, 1, 8, 8, g_lo=0.6)
    y, S = oracle.forward(*args)
    yc, Sc = cf.run(cf.unified_wy, *args, 1)
    assert rel(Sc, S) < 1e-12            # C = 1: p = k, no difference
    yc, Sc = cf.run(_step9_with_p, *args, 4)
    assert rel(Sc, S) > 1e-3 or rel(yc, y) > 1e-3


def test_division_ratios_break_on_vanished_decay():
    q, k, v, g, beta, S0 = case(22, 1, 20, 1, 1, 8, 8)
    g[:] = 0.0
    yc, Sc = cf.run(_ratios_by_division, q, k, v, g, beta, S0, 8)
    assert not (np.all(np.isfinite(yc)) and np.all(np.isfinite(Sc)))
