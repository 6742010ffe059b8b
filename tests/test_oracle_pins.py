"""Pins of the CPU oracle to facts other than itself.

Every check takes a forward callable ``fwd(q, k, v, g, beta, state) ->
(y, state_out)`` over float64 arrays in the pages' layouts, so that the same
checks run on both oracles (C and NumPy) and on planted mistakes.  Each
planted mistake below (a plausible error in the rule: a dropped term, a wrong
sign, a wrong index, a transposed operand, a pre-update read-out) must fail
at least one check; the real oracles must pass all of them.

Sources of the pinned facts:
* the hand-worked example in ``tests/golden/worked_example_t2.json``;
* the rule as the ferrox-core gdn_chunk.rs page states it ("The algebra"):
  with b = 0 nothing is written and the state only decays; with b = 1 and a
  unit key the written value is read back exactly; the component of the
  state orthogonal to k_t only decays;
* linearity in (V, S0), continuation across calls ("state at chunk N+1 is
  S_end of chunk N", metaltile-std gated_delta_wy.rs, "Algorithm"),
  independence of (b, hv) slots and the grouped head map hk = hv / (Hv/Hk)
  (metaltile-std page, "Layouts");
* vanishing decays stay finite (ferrox-core page's underflow test).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=1, T=6, Hk=1, Hv=1, Dk=4, Dv=3, unit_k=True):
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    g = rng.uniform(0.3, 1.0, (B, T, Hv))
    beta = rng.uniform(0.1, 1.0, (B, T, Hv))
    S0 = rng.standard_normal((B, Hv, Dv, Dk)) * 0.5
    return q, k, v, g, beta, S0


# ----------------------------------------------------------------- checks
def check_worked_example(fwd):
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_t2.json")))
    q = np.array(ex["q"])[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    g = np.array(ex["g"])[None, :, None]
    beta = np.array(ex["beta"])[None, :, None]
    S0 = np.array(ex["S0"])[None, None]
    y, S = fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], S0)
    ok = np.allclose(S[0, 0], ex["S_after_t1"], rtol=0, atol=1e-14)
    ok &= np.allclose(y[0, 0, 0] * np.sqrt(2), ex["y_times_sqrt2"][0], rtol=0, atol=1e-13)
    y, S = fwd(q, k, v, g, beta, S0)
    ok &= np.allclose(S[0, 0], ex["S_final"], rtol=0, atol=1e-14)
    ok &= np.allclose(y[0, :, 0] * np.sqrt(2), ex["y_times_sqrt2"], rtol=0, atol=1e-13)
    return bool(ok)


def check_beta_zero(fwd):
    """b = 0: S_T = (prod g) S0 and y_t = G_t S0 q_t / sqrt(Dk)."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=7, Hk=1, Hv=2, Dk=5, Dv=3)
    beta[:] = 0.0
    y, S = fwd(q, k, v, g, beta, S0)
    G = np.cumprod(g, axis=1)                                  # [B,T,Hv]
    ok = np.allclose(S, G[:, -1][..., None, None] * S0, rtol=1e-12, atol=1e-14)
    for t in range(q.shape[1]):
        ref = G[:, t][..., None] * np.einsum("bhjd,bd->bhj", S0, q[:, t, 0]) / np.sqrt(5)
        ok &= np.allclose(y[:, t], ref, rtol=1e-12, atol=1e-14)
    return bool(ok)


def check_orthonormal_write(fwd):
    """g = 1, b = 1, orthonormal keys, S0 = 0: S_T = sum v_t k_t^T and
    reading with q_t = k_t returns v_t / sqrt(Dk) exactly."""
    rng = np.random.default_rng(12)
    Dk, Dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:T]                                              # orthonormal rows
    k = keys[None, :, None, :]
    q = k.copy()
    v = rng.standard_normal((1, T, 1, Dv))
    g = np.ones((1, T, 1))
    beta = np.ones((1, T, 1))
    y, S = fwd(q, k, v, g, beta, np.zeros((1, 1, Dv, Dk)))
    ok = np.allclose(S[0, 0], v[0, :, 0].T @ keys, atol=1e-13)
    ok &= np.allclose(y[0, :, 0], v[0, :, 0] / np.sqrt(Dk), atol=1e-13)
    ok &= np.allclose(S[0, 0] @ keys.T, v[0, :, 0].T, atol=1e-13)
    return bool(ok)


def check_write_readback(fwd):
    """b = 1, unit keys, any decay and initial state: S_t k_t = v_t, so the
    read-out with q_t = k_t is v_t / sqrt(Dk) at every step."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=9, Hk=1, Hv=1, Dk=6, Dv=4)
    beta[:] = 1.0
    q = k.copy()
    y, S = fwd(q, k, v, g, beta, S0)
    ok = np.allclose(y[0, :, 0], v[0, :, 0] / np.sqrt(6), atol=1e-12)
    ok &= np.allclose(S[0, 0] @ k[0, -1, 0], v[0, -1, 0], atol=1e-12)
    return bool(ok)


def check_orthogonal_complement(fwd):
    """One step: for x orthogonal to k, S_1 x = g S_0 x (only the key
    direction is rewritten); along k, S_1 k = (1-b) g S_0 k + b v for unit k."""
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=1, Hk=1, Hv=1, Dk=7, Dv=3)
    _, S = fwd(q, k, v, g, beta, S0)
    kk = k[0, 0, 0]
    x = rng.standard_normal(7)
    x -= (x @ kk) * kk
    gg, bb = g[0, 0, 0], beta[0, 0, 0]
    ok = np.allclose(S[0, 0] @ x, gg * (S0[0, 0] @ x), atol=1e-13)
    ok &= np.allclose(S[0, 0] @ kk, (1 - bb) * gg * (S0[0, 0] @ kk) + bb * v[0, 0, 0], atol=1e-13)
    return bool(ok)


def check_linearity(fwd):
    """(y, S_T) is linear in (V, S0) for fixed q, k, g, b."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=6, Hk=1, Hv=2, Dk=4, Dv=3)
    _, _, v2, _, _, S02 = rand_case(rng, B=1, T=6, Hk=1, Hv=2, Dk=4, Dv=3)
    a, c = 0.7, -1.3
    y1, s1 = fwd(q, k, v, g, beta, S0)
    y2, s2 = fwd(q, k, v2, g, beta, S02)
    y3, s3 = fwd(q, k, a * v + c * v2, g, beta, a * S0 + c * S02)
    return bool(np.allclose(y3, a * y1 + c * y2, atol=1e-12) and
                np.allclose(s3, a * s1 + c * s2, atol=1e-12))


def check_split(fwd):
    """run(T1) then run(T2) from its state equals run(T1 + T2)."""
    rng = np.random.default_rng(16)
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=10, Hk=1, Hv=2, Dk=4, Dv=3)
    y, S = fwd(q, k, v, g, beta, S0)
    ya, Sa = fwd(q[:, :4], k[:, :4], v[:, :4], g[:, :4], beta[:, :4], S0)
    yb, Sb = fwd(q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], Sa)
    return bool(np.allclose(np.concatenate([ya, yb], 1), y, atol=1e-12) and
                np.allclose(Sb, S, atol=1e-12))


def check_grouped_heads(fwd):
    """Value head hv reads key head hv // (Hv/Hk); slots are independent."""
    rng = np.random.default_rng(17)
    Hk, Hv = 2, 6
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=5, Hk=Hk, Hv=Hv, Dk=4, Dv=3)
    y, S = fwd(q, k, v, g, beta, S0)
    ok = True
    for b in range(2):
        for hv in range(Hv):
            hk = hv // (Hv // Hk)
            sl = np.s_[b:b + 1, :, hk:hk + 1]
            vs = np.s_[b:b + 1, :, hv:hv + 1]
            y1, S1 = fwd(q[sl], k[sl], v[vs], g[b:b + 1, :, hv:hv + 1],
                         beta[b:b + 1, :, hv:hv + 1], S0[b:b + 1, hv:hv + 1])
            ok &= np.allclose(y1[0, :, 0], y[b, :, hv], atol=1e-13)
            ok &= np.allclose(S1[0, 0], S[b, hv], atol=1e-13)
    return bool(ok)


def check_value_permutation(fwd):
    """Permuting the value index permutes y and the state rows alike."""
    rng = np.random.default_rng(18)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=5, Hk=1, Hv=1, Dk=4, Dv=6)
    p = rng.permutation(6)
    y, S = fwd(q, k, v, g, beta, S0)
    yp, Sp = fwd(q, k, v[..., p], g, beta, S0[:, :, p])
    return bool(np.allclose(yp, y[..., p], atol=1e-13) and np.allclose(Sp, S[:, :, p], atol=1e-13))


def check_zero_decay(fwd):
    """g = 0: the state is forgotten each step, S_t = b_t v_t k_t^T and
    y_t = b_t v_t (k_t . q_t) / sqrt(Dk); g = 1e-20 stays finite."""
    rng = np.random.default_rng(19)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=5, Hk=1, Hv=1, Dk=4, Dv=3)
    g[:] = 0.0
    y, S = fwd(q, k, v, g, beta, S0)
    kq = np.einsum("td,td->t", k[0, :, 0], q[0, :, 0])
    ok = np.allclose(y[0, :, 0], beta[0, :, 0, None] * v[0, :, 0] * kq[:, None] / 2.0, atol=1e-14)
    ok &= np.allclose(S[0, 0], beta[0, -1, 0] * np.outer(v[0, -1, 0], k[0, -1, 0]), atol=1e-14)
    g[:] = 1e-20
    y, S = fwd(q, k, v, g, beta, S0 * 1e30)
    ok &= bool(np.all(np.isfinite(y)) and np.all(np.isfinite(S)))
    return bool(ok)


def check_no_initial_state(fwd):
    """state=None is the zero initial state."""
    rng = np.random.default_rng(20)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=4, Hk=1, Hv=2, Dk=4, Dv=3)
    y1, s1 = fwd(q, k, v, g, beta, None)
    y2, s2 = fwd(q, k, v, g, beta, np.zeros_like(S0))
    return bool(np.array_equal(y1, y2) and np.array_equal(s1, s2))


CHECKS = [check_worked_example, check_beta_zero, check_orthonormal_write,
          check_write_readback, check_orthogonal_complement, check_linearity,
          check_split, check_grouped_heads, check_value_permutation,
          check_zero_decay, check_no_initial_state]

ORACLES = {"c": oracle.forward, "numpy": oracle.forward_numpy}


@pytest.mark.parametrize("name", list(ORACLES))
@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(name, check):
    assert check(ORACLES[name])


# ------------------------------------------------------ planted mistakes
def _mutant(kind):
    """A sequential rule with one planted mistake (NumPy, float64)."""
    def fwd(q, k, v, g, beta, state=None):
        B, T, Hk, Dk = q.shape
        Hv, Dv = v.shape[2], v.shape[3]
        if kind == "tiled_heads":
            head_of = np.arange(Hv) % Hk
        else:
            head_of = np.arange(Hv) // (Hv // Hk)
        S = np.zeros((B, Hv, Dv, Dk)) if state is None else np.array(state, dtype=np.float64)
        y = np.empty((B, T, Hv, Dv))
        scale = 1.0 if kind == "no_scale" else 1.0 / np.sqrt(Dk)
        for t in range(T):
            kt, qt = k[:, t][:, head_of], q[:, t][:, head_of]
            gt, bt = g[:, t][..., None, None], beta[:, t][..., None]
            Sk = np.einsum("bhjd,bhd->bhj", S, kt)
            if kind == "transposed_state":
                Sk = np.einsum("bhdj,bhd->bhj", S, kt)
            if kind == "raw_prediction":
                d = bt * (v[:, t] - Sk)
            elif kind == "sign":
                d = bt * (v[:, t] + gt[..., 0] * Sk)
            elif kind == "beta_on_value_only":
                d = bt * v[:, t] - gt[..., 0] * Sk
            else:
                d = bt * (v[:, t] - gt[..., 0] * Sk)
            S_prev = S
            if kind == "undecayed_update":
                S = S + d[..., :, None] * kt[..., None, :]
            else:
                S = gt * S + d[..., :, None] * kt[..., None, :]
            R = S_prev if kind == "pre_update_readout" else S
            y[:, t] = np.einsum("bhjd,bhd->bhj", R, qt) * scale
        return y, S
    return fwd


MUTANTS = ["tiled_heads", "no_scale", "transposed_state", "raw_prediction",
           "sign", "beta_on_value_only", "undecayed_update", "pre_update_readout"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    fwd = _mutant(kind)
    failed = []
    for c in CHECKS:
        try:
            ok = c(fwd)
        except ValueError:          # e.g. a transposed state of the wrong shape
            ok = False
        if not ok:
            failed.append(c.__name__)
    assert failed, f"mutant {kind} passed every pin"
    # the mistake must also show on square shapes, where it cannot raise
    if kind == "transposed_state":
        assert not check_worked_example(fwd)


def test_unmutated_numpy_rule_passes():
    # the mutant harness itself, with no mutation, must pass every check
    fwd = _mutant("none")
    assert all(c(fwd) for c in CHECKS)


# ------------------------------------------------------ C vs NumPy
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 4, 4), (2, 9, 2, 4, 8, 5),
                                   (1, 33, 3, 6, 16, 16), (3, 4, 1, 3, 5, 7)])
def test_c_matches_numpy(shape):
    B, T, Hk, Hv, Dk, Dv = shape
    rng = np.random.default_rng(sum(shape))
    q, k, v, g, beta, S0 = rand_case(rng, B, T, Hk, Hv, Dk, Dv)
    for s in (S0, None):
        y1, s1 = oracle.forward(q, k, v, g, beta, s)
        y2, s2 = oracle.forward_numpy(q, k, v, g, beta, s)
        assert np.allclose(y1, y2, rtol=1e-12, atol=1e-14)
        assert np.allclose(s1, s2, rtol=1e-12, atol=1e-14)


def test_c_slot_mask_and_empty():
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=3, Hk=1, Hv=2, Dk=4, Dv=3)
    mask = np.array([[True, False], [False, True]])
    y, s = oracle.forward(q, k, v, g, beta, S0, slot_mask=mask)
    yf, sf = oracle.forward(q, k, v, g, beta, S0)
    assert np.array_equal(y[0, :, 0], yf[0, :, 0]) and np.array_equal(s[1, 1], sf[1, 1])
    assert np.isnan(y[0, :, 1]).all() and np.isnan(s[1, 0]).all()
    # T = 0: the state passes through
    y0, s0 = oracle.forward(q[:, :0], k[:, :0], v[:, :0], g[:, :0], beta[:, :0], S0)
    assert y0.shape == (2, 0, 2, 3) and np.array_equal(s0, S0)


# ------------------------------------------- head maps and the log gate
# The ferrox-core page's host body selects the key head of a value head
# through one of two head maps, "Tiled" or "Grouped", and takes the gate as
# the logarithm of the decay (it applies exp before use).  The grouped map is
# pinned above; the tiled map is pinned to it through the cases where the two
# coincide and through a relabelling of the value heads.

def _tiled_to_grouped_perm(Hk, Hv):
    """Position p[hv] that value head hv takes so that the grouped map of
    position p[hv] is the key head the tiled reading gives hv (hv mod Hk):
    the value heads of key head h are listed together, in head order."""
    grp = Hv // Hk
    return np.array([(hv % Hk) * grp + hv // Hk for hv in range(Hv)])


def check_tiled_heads(fwd):
    rng = np.random.default_rng(31)
    ok = True
    # Hk == Hv and Hk == 1: the two maps agree
    for Hk, Hv in ((3, 3), (1, 4)):
        q, k, v, g, beta, S0 = rand_case(rng, B=2, T=5, Hk=Hk, Hv=Hv, Dk=4, Dv=3)
        yt, st = fwd(q, k, v, g, beta, S0, head_map="tiled")
        yg, sg = fwd(q, k, v, g, beta, S0, head_map="grouped")
        ok &= np.allclose(yt, yg, rtol=0, atol=1e-14) and np.allclose(st, sg, rtol=0, atol=1e-14)
    # Hk = 2, Hv = 6: tiled == grouped after moving value head hv to p[hv]
    Hk, Hv = 2, 6
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=6, Hk=Hk, Hv=Hv, Dk=4, Dv=3)
    p = _tiled_to_grouped_perm(Hk, Hv)
    assert sorted(p) == list(range(Hv))
    vp, gp, bp, sp = (np.empty_like(a) for a in (v, g, beta, S0))
    vp[:, :, p], gp[:, :, p], bp[:, :, p], sp[:, p] = v, g, beta, S0
    yt, st = fwd(q, k, v, g, beta, S0, head_map="tiled")
    yg, sg = fwd(q, k, vp, gp, bp, sp, head_map="grouped")
    ok &= np.allclose(yt, yg[:, :, p], rtol=0, atol=1e-13) and np.allclose(st, sg[:, p], rtol=0, atol=1e-13)
    # and the maps really differ there
    yg0, _ = fwd(q, k, v, g, beta, S0, head_map="grouped")
    ok &= not np.allclose(yt, yg0, atol=1e-6)
    return bool(ok)


def check_log_gate(fwd):
    rng = np.random.default_rng(32)
    q, k, v, g, beta, S0 = rand_case(rng, B=1, T=6, Hk=1, Hv=2, Dk=4, Dv=3)
    ok = True
    # a log gate of log(g) is the decay g
    yl, sl = fwd(q, k, v, np.log(g), beta, S0, gate="log")
    yd, sd = fwd(q, k, v, g, beta, S0, gate="decay")
    ok &= np.allclose(yl, yd, rtol=1e-13, atol=1e-14) and np.allclose(sl, sd, rtol=1e-13, atol=1e-14)
    # log gate 0 is decay 1 (no forgetting), exactly
    yl, sl = fwd(q, k, v, np.zeros_like(g), beta, S0, gate="log")
    yd, sd = fwd(q, k, v, np.ones_like(g), beta, S0, gate="decay")
    ok &= np.array_equal(yl, yd) and np.array_equal(sl, sd)
    # log gate -inf is decay 0: y_t = b_t v_t (k_t . q_t) / sqrt(Dk)
    yl, sl = fwd(q, k, v, np.full_like(g, -np.inf), beta, S0, gate="log")
    kq = np.einsum("td,td->t", k[0, :, 0], q[0, :, 0])
    want = beta[0, :, :, None] * v[0] * kq[:, None, None] / 2.0
    ok &= np.allclose(yl[0], want, rtol=0, atol=1e-14)
    return bool(ok)


@pytest.mark.parametrize("name", list(ORACLES))
@pytest.mark.parametrize("check", [check_tiled_heads, check_log_gate], ids=lambda c: c.__name__)
def test_oracle_options(name, check):
    assert check(ORACLES[name])


def _option_mutant(kind):
    """The NumPy oracle with a planted mistake in one option."""
    def fwd(q, k, v, g, beta, state=None, *, head_map="grouped", gate="decay"):
        if gate == "log":
            g = {"log_negated": lambda x: np.exp(-x), "log_ignored": lambda x: x}.get(kind, np.exp)(g)
        if head_map == "tiled" and kind == "tiled_as_block":
            head_map = "grouped"
        if head_map == "tiled" and kind == "tiled_wrong_index":
            # value head hv reads key head (hv // Hk) mod Hk: give every value
            # head its own copy of that key head and map them one to one
            Hk, Hv = q.shape[2], v.shape[2]
            sel = (np.arange(Hv) // Hk) % Hk
            return oracle.forward_numpy(q[:, :, sel], k[:, :, sel], v, g, beta, state)
        return oracle.forward_numpy(q, k, v, g, beta, state, head_map=head_map)
    return fwd


@pytest.mark.parametrize("kind,check", [("tiled_as_block", check_tiled_heads),
                                        ("tiled_wrong_index", check_tiled_heads),
                                        ("log_negated", check_log_gate),
                                        ("log_ignored", check_log_gate)])
def test_option_mistake_is_caught(kind, check):
    with np.errstate(all="ignore"):
        assert not check(_option_mutant(kind))


# ----------------------------------------------------- per-key-dimension gate
# A gate g [B,T,Hv,Dk] decays each key column of the state by its own factor
# (the 4-D "vector" gate the MLX pull request page names).  Pins: a vector of
# equal entries is the scalar gate; with beta = 0 nothing is written and the
# state's columns decay by the running products of their gates (closed form);
# with beta = 1 and a unit key the written value is read back exactly, for
# any gate; relabelling the key dimensions relabels the state's columns.

def check_vector_gate(fwd):
    rng = np.random.default_rng(41)
    ok = True
    q, k, v, g, beta, S0 = rand_case(rng, B=2, T=6, Hk=1, Hv=2, Dk=5, Dv=3)
    gv = np.repeat(g[..., None], 5, axis=-1)
    y1, s1 = fwd(q, k, v, gv, beta, S0)
    y2, s2 = fwd(q, k, v, g, beta, S0)
    ok &= np.allclose(y1, y2, rtol=1e-13, atol=1e-14) and np.allclose(s1, s2, rtol=1e-13, atol=1e-14)
    # beta = 0: S_t = S0 diag(prod_{s<=t} g_s), y_t = S_t q_t / sqrt(Dk)
    gv = rng.uniform(0.0, 1.0, (2, 6, 2, 5))
    gv[0, 2, 1, 3] = 0.0
    y, s = fwd(q, k, v, gv, np.zeros_like(beta), S0)
    cum = np.cumprod(gv, axis=1)                                # [B,T,Hv,Dk]
    want_s = S0 * cum[:, -1][:, :, None, :]
    want_y = np.einsum("bhji,bthi,bti->bthj", S0, cum, q[:, :, 0]) / np.sqrt(5)
    ok &= np.allclose(s, want_s, rtol=0, atol=1e-14) and np.allclose(y, want_y, rtol=0, atol=1e-14)
    # beta = 1, unit key: S_t k_t = v_t whatever the gate
    _, k1, v1, _, _, S1 = rand_case(rng, B=1, T=1, Hk=1, Hv=1, Dk=5, Dv=3)
    g1 = rng.uniform(0.1, 1.0, (1, 1, 1, 5))
    _, st = fwd(q[:1, :1, :1], k1, v1, g1, np.ones((1, 1, 1)), S1)
    ok &= np.allclose(st[0, 0] @ k1[0, 0, 0], v1[0, 0, 0], rtol=0, atol=1e-14)
    # relabelling key dimensions
    p = rng.permutation(5)
    y, s = fwd(q, k, v, gv, beta, S0)
    yp, sp = fwd(q[..., p], k[..., p], v, gv[..., p], beta, S0[..., p])
    ok &= np.allclose(yp, y, rtol=0, atol=1e-13) and np.allclose(sp, s[..., p], rtol=0, atol=1e-13)
    return bool(ok)


@pytest.mark.parametrize("name", list(ORACLES))
def test_oracle_vector_gate(name):
    assert check_vector_gate(ORACLES[name])


def _vector_gate_mutant(kind):
    def fwd(q, k, v, g, beta, state=None):
        if g.ndim == 3:
            return oracle.forward_numpy(q, k, v, g, beta, state)
        B, T, Hk, Dk = q.shape
        Hv, Dv = v.shape[2], v.shape[3]
        S = np.zeros((B, Hv, Dv, Dk)) if state is None else np.array(state, dtype=np.float64)
        y = np.empty((B, T, Hv, Dv))
        for t in range(T):
            kt, qt = k[:, t][:, [0] * Hv], q[:, t][:, [0] * Hv]
            gt = g[:, t]
            if kind == "gate_on_value_rows":
                Sd = S * gt[..., :Dv, None] if Dv <= Dk else S
            elif kind == "gate_mean":
                Sd = S * gt.mean(-1)[..., None, None]
            else:
                Sd = S * gt[..., None, :]
            pred = np.einsum("bhji,bhi->bhj", S if kind == "undecayed_prediction" else Sd, kt)
            d = beta[:, t][..., None] * (v[:, t] - pred)
            S = Sd + d[..., :, None] * kt[..., None, :]
            y[:, t] = np.einsum("bhji,bhi->bhj", S, qt) / np.sqrt(Dk)
        return y, S
    return fwd


@pytest.mark.parametrize("kind", ["gate_on_value_rows", "gate_mean", "undecayed_prediction"])
def test_vector_gate_mistake_is_caught(kind):
    assert not check_vector_gate(_vector_gate_mutant(kind))


def test_vector_gate_harness_passes_unmutated():
    assert check_vector_gate(_vector_gate_mutant("none"))
