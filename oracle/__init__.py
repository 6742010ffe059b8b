"""CPU oracle of the gated delta rule forward pass (float64).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package's
``smoke()`` check and by the bench's CPU-baseline leg, never by the product
path.  It shares no code with the HIP library.

Two independent implementations of the sequential rule, which the
ferrox-core ``gdn_chunk.rs`` page gives as the definition ("The algebra";
its test comment calls the sequential step the definition):

* :func:`forward`        -- plain C, float64, OpenMP over (b, hv) slots
                            (``oracle/gdn_ref.c``); used for GPU parity;
* :func:`forward_numpy`  -- NumPy, float64, token loop vectorised over slots;
                            for tiny cases and as a cross-check of the C one.

The chunked algebra of the pages, written out in float64 for validation only,
is in :mod:`oracle.chunk_forms`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_ref.c")
_LIB = os.path.join(_HERE, "libgdn_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``gdn_ref.c`` with gcc into ``oracle/libgdn_ref.so``."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_ref_forward.argtypes = [dp] * 8 + [ctypes.c_long] * 6 + [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.gdn_ref_forward.restype = ctypes.c_int
        lib.gdn_ref_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn_ref_max_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


HEAD_MAPS = ("grouped", "tiled")
GATES = ("decay", "log")


def key_heads(Hk: int, Hv: int, head_map: str = "grouped") -> np.ndarray:
    """Key head of every value head: ``hv // (Hv // Hk)`` (grouped, the
    metaltile-std page's "Layouts") or ``hv % Hk`` (tiled, the other map the
    ferrox-core page's host body selects)."""
    if head_map not in HEAD_MAPS:
        raise ValueError(f"head_map must be one of {HEAD_MAPS}")
    hv = np.arange(Hv)
    return hv % Hk if head_map == "tiled" else hv // (Hv // Hk)


def forward(q, k, v, g, beta, state=None, *, slot_mask=None, nthreads=0,
            head_map="grouped", gate="decay"):
    """Sequential rule in C, float64.

    ``q, k`` [B,T,Hk,Dk], ``v`` [B,T,Hv,Dv], ``g, beta`` [B,T,Hv] and
    ``state`` [B,Hv,Dv,Dk] (or None for a zero initial state) are float64
    arrays (use :func:`gdn_inputs.decode` on stored inputs).  Returns
    ``(y, state_out)`` in float64.  ``slot_mask`` (bool [B,Hv]) restricts
    the work to some slots; the others come back as NaN.  ``head_map``
    picks the key head of each value head (:func:`key_heads`); ``gate`` says
    whether ``g`` is the decay or its natural logarithm.  ``g`` may also be
    [B,T,Hv,Dk]: one decay per key dimension, scaling the state's key
    columns.
    """
    if head_map not in HEAD_MAPS or gate not in GATES:
        raise ValueError("head_map / gate")
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    vector_gate = g.ndim == 4
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, Hv) \
            or g.shape != ((B, T, Hv, Dk) if vector_gate else (B, T, Hv)):
        raise ValueError("inconsistent shapes")
    s_in = None if state is None else _f64(state)
    if s_in is not None and s_in.shape != (B, Hv, Dv, Dk):
        raise ValueError("state shape")
    y = np.full((B, T, Hv, Dv), np.nan)
    s_out = np.full((B, Hv, Dv, Dk), np.nan)
    mask = None
    if slot_mask is not None:
        mask = np.ascontiguousarray(np.asarray(slot_mask, dtype=np.uint8).reshape(B * Hv))
    rc = _load().gdn_ref_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s_in), _ptr(s_out),
        _ptr(y), B, T, Hk, Hv, Dk, Dv, HEAD_MAPS.index(head_map), GATES.index(gate),
        int(vector_gate),
        None if mask is None else mask.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"gdn_ref_forward failed ({rc})")
    return y, s_out


def forward_numpy(q, k, v, g, beta, state=None, *, head_map="grouped", gate="decay"):
    """Sequential rule in NumPy, float64 (tiny cases).

    Same contract as :func:`forward`.  Token loop; every slot advances at
    once: the value head ``hv`` reads key head ``key_heads(...)[hv]``; a
    [B,T,Hv,Dk] gate decays each key column of the state by its own factor.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if Hv % Hk:
        raise ValueError("Hv must be a multiple of Hk")
    head_of = key_heads(Hk, Hv, head_map)
    if gate not in GATES:
        raise ValueError("gate")
    if gate == "log":
        g = np.exp(g)
    S = np.zeros((B, Hv, Dv, Dk)) if state is None else _f64(state).copy()
    y = np.empty((B, T, Hv, Dv))
    scale = 1.0 / np.sqrt(Dk)
    for t in range(T):
        kt = k[:, t][:, head_of]                  # [B,Hv,Dk]
        qt = q[:, t][:, head_of]
        gt = g[:, t][..., None, :] if g.ndim == 4 else g[:, t][..., None, None]   # [B,Hv,1,Dk|1]
        bt = beta[:, t][..., None]                # [B,Hv,1]
        S = gt * S                                # decay first
        d = bt * (v[:, t] - np.einsum("bhjd,bhd->bhj", S, kt))
        S = S + d[..., :, None] * kt[..., None, :]
        y[:, t] = np.einsum("bhjd,bhd->bhj", S, qt) * scale
    return y, S
