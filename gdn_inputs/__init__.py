"""Seeded synthetic inputs for the gated delta rule forward pass.

This module is shared by the tests, the bench and the oracle's callers. It
draws random numbers and stores them in the dtypes the kernels read; it holds
none of the method's arithmetic (no state, no decay products, no solve).

Layouts follow the metaltile-std page (``gated_delta_wy.rs``, "Layouts"
section) and the ferrox-core ``gdn_chunk.rs`` page:

    q, k   [B, T, Hk, Dk]      v      [B, T, Hv, Dv]
    g, beta [B, T, Hv] (f32)   state  [B, Hv, Dv, Dk] (f32)

Recipe (one ``numpy.random.default_rng(seed)`` per call, PCG64):

* draws in the order q, k, v, x_g, x_beta, state, each one
  ``standard_normal`` (or ``random`` for uniform gates) call over the full
  shape, in float64;
* q and k are L2-normalised per (b, t, head) in float64, without an epsilon;
* g is the decay itself (the state is multiplied by g):
  ``"softplus"``  g = exp(-softplus(x)), x ~ N(2, 1)   (the formula as printed)
  ``"sigmoid"``   g = sigmoid(x),        x ~ N(2, 1)   (decays 0.73..0.95)
  ``"uniform"``   g ~ U[lo, hi)
  ``"const"``     g = a given constant (used for underflow cases)
* beta = sigmoid(N(0, 1)), or a given constant;
* with ``key_corr = rho``, every key of a (batch, key head) is
  normalise(k_0 + rho * n_t): one shared direction k_0 (drawn from a second
  generator, ``default_rng([seed, 1])``, so that the main draws are the same
  as without it) plus the usual per-token draw n_t scaled by rho.  Small rho
  gives nearly parallel keys, the hard case of the chunk's triangular system
  (with beta near 1 and g = 1 its rows nearly cancel);
* state_in ~ N(0, sigma) with sigma the standard deviation, or zeros, or None;
* float64 values are stored as float32 (round to nearest even, numpy's
  cast), then as bf16 (round to nearest even on the float32 bits) or as
  float16 (numpy's cast, round to nearest even).

bf16 arrays are carried as ``uint16`` bit patterns; :func:`decode` turns any
stored array back into exact float64 values.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS", "make_inputs", "workload_inputs", "decode", "encode",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
]

DTYPES = ("f32", "bf16", "f16")

# The five workloads.  "T" of the decode workload is the number of chained
# single-token steps.  "gate" / "gate_args" name the decay draw, "state" the
# initial state draw.
WORKLOADS = {
    "tiny_f32": dict(B=1, T=64, Hk=2, Hv=2, Dk=32, Dv=32, C=16, dtype="f32",
                     gate="softplus", state_std=0.1),
    "bonsai_prefill": dict(B=1, T=128, Hk=48, Hv=48, Dk=128, Dv=128, C=32,
                           dtype="bf16", gate="softplus", state_std=0.05),
    "gqa_ragged": dict(B=2, T=1111, Hk=16, Hv=32, Dk=128, Dv=128, C=64,
                       dtype="bf16", gate="softplus", state_std=0.0),
    "long_prefill": dict(B=8, T=8192, Hk=16, Hv=32, Dk=128, Dv=128, C=64,
                         dtype="bf16", gate="uniform", gate_lo=0.95,
                         gate_hi=1.0, state_std=0.05),
    "decode": dict(B=64, T=256, Hk=16, Hv=32, Dk=128, Dv=128, C=None,
                   dtype="f16", gate="softplus", state_std=0.05),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN.  Written from the IEEE-754 definition of
    the binary32 layout: bf16 keeps the upper 16 bits of the float32 word;
    adding 0x7FFF plus the lowest kept bit rounds the dropped half to nearest
    even.  (The 32-bit sum cannot wrap for any non-NaN input.)
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> stored array: float32, bf16 bits (uint16) or float16."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f16":
        return np.asarray(x64, dtype=np.float64).astype(np.float16)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    if dtype in ("f32", "f16"):
        return np.asarray(stored).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def make_inputs(B, T, Hk, Hv, Dk, Dv, dtype="bf16", *, gate="softplus",
                gate_lo=0.95, gate_hi=1.0, gate_const=None, state_std=0.05,
                state=True, normalise_qk=True, key_corr=None, beta_const=None,
                seed=0, **_ignored):
    """Draw one seeded input set.

    Returns a dict with ``q, k, v`` (stored dtype), ``g, beta`` (float32),
    ``state`` (float32 or None) and ``dtype``.  ``state=False`` returns
    ``state=None`` (the "no initial state" case); ``state_std=0`` returns a
    zero buffer.
    """
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    if key_corr is not None:
        k0 = np.random.default_rng([seed, 1]).standard_normal((B, 1, Hk, Dk))
        k = k0 / np.sqrt(np.sum(k0 * k0, axis=-1, keepdims=True)) * np.sqrt(Dk) + float(key_corr) * k
    if normalise_qk:
        q = _l2_normalise(q)
        k = _l2_normalise(k)
    qs, ks = encode(q, dtype), encode(k, dtype)
    del q, k
    vs = encode(rng.standard_normal((B, T, Hv, Dv)), dtype)
    if gate == "uniform":
        g = gate_lo + (gate_hi - gate_lo) * rng.random((B, T, Hv))
    else:
        x_g = rng.standard_normal((B, T, Hv)) + 2.0
        if gate == "softplus":
            g = np.exp(-_softplus(x_g))
        elif gate == "sigmoid":
            g = _sigmoid(x_g)
        elif gate == "const":
            g = np.full((B, T, Hv), float(gate_const))
        else:
            raise ValueError(f"unknown gate {gate!r}")
    beta = _sigmoid(rng.standard_normal((B, T, Hv)))
    if beta_const is not None:
        beta = np.full((B, T, Hv), float(beta_const))
    s = rng.standard_normal((B, Hv, Dv, Dk)) * state_std
    if state_std == 0:
        s = np.zeros_like(s)
    out = dict(q=qs, k=ks, v=vs,
               g=g.astype(np.float32), beta=beta.astype(np.float32),
               state=(s.astype(np.float32) if state else None), dtype=dtype)
    return out


def vector_gate(B, T, Hv, Dk, *, seed=0, kind="sigmoid"):
    """A decay per key dimension, float32 [B,T,Hv,Dk] (seeded).

    ``sigmoid``: sigmoid(N(0,1) + 2) per entry (mean about 0.85, some
    entries near 0.3); ``near_one``: U[0.95, 1), the slow decays of long
    contexts; ``mixed``: half the key dimensions near 1, half small
    (U[0.05, 0.5]), so that some columns of the state are forgotten within a
    few tokens while others persist.
    """
    rng = np.random.default_rng(seed)
    if kind == "sigmoid":
        g = _sigmoid(rng.standard_normal((B, T, Hv, Dk)) + 2.0)
    elif kind == "near_one":
        g = 0.95 + 0.05 * rng.random((B, T, Hv, Dk))
    elif kind == "mixed":
        g = 0.95 + 0.05 * rng.random((B, T, Hv, Dk))
        small = rng.random(Dk) < 0.5
        g[..., small] = 0.05 + 0.45 * rng.random((B, T, Hv, int(small.sum())))
    else:
        raise ValueError(f"unknown vector gate {kind!r}")
    return g.astype(np.float32)


def workload_inputs(name: str, *, seed=0, gate=None, **overrides):
    """Inputs of one named workload (see ``WORKLOADS``)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    if gate is not None:
        cfg["gate"] = gate
    return make_inputs(**cfg, seed=seed)
