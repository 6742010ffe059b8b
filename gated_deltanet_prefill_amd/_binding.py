"""ctypes binding of ``libgdn.so`` (argument marshalling only).

Tensors supply device memory and the stream; every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is
not built or not loadable, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
DTYPE_CODE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}
SUPPORTED_DIMS = (32, 64, 128)
SUPPORTED_CHUNKS = (0, 16, 32, 64)     # 0: the library chooses
GDN_HEADS_TILED, GDN_GATE_LOG, GDN_GATE_VECTOR = 1, 2, 4
HEAD_MAPS = ("grouped", "tiled")
GATES = ("decay", "log")

_lib = None


class GDNError(RuntimeError):
    """A non-zero status from libgdn."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m gated_deltanet_prefill_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 8 + [vp]
        lib.gdn_chunk_fwd.restype = i
        lib.gdn_seq_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [vp]
        lib.gdn_seq_fwd.restype = i
        lib.gdn_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 6 + [vp]
        lib.gdn_step.restype = i
        lib.gdn_chunk_fwd_ex.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 9 + [vp]
        lib.gdn_chunk_fwd_ex.restype = i
        lib.gdn_seq_fwd_ex.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 8 + [vp]
        lib.gdn_seq_fwd_ex.restype = i
        lib.gdn_step_ex.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [vp]
        lib.gdn_step_ex.restype = i
        lib.gdn_status_string.argtypes = [i]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_version.restype = i
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _flags(heads, gate, vector=False):
    if heads not in HEAD_MAPS:
        raise ValueError(f"heads must be one of {HEAD_MAPS}")
    if gate not in GATES:
        raise ValueError(f"gate must be one of {GATES}")
    return ((GDN_HEADS_TILED if heads == "tiled" else 0) | (GDN_GATE_LOG if gate == "log" else 0)
            | (GDN_GATE_VECTOR if vector else 0))


def _prefill_args(q, k, v, g, beta, state_in, state_out, y):
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    _check_tensor("q", q, (B, T, Hk, Dk), dt, dev)
    _check_tensor("k", k, (B, T, Hk, Dk), dt, dev)
    _check_tensor("v", v, (B, T, Hv, Dv), dt, dev)
    _check_tensor("g", g, (B, T, Hv, Dk) if g.dim() == 4 else (B, T, Hv), torch.float32, dev)
    _check_tensor("beta", beta, (B, T, Hv), torch.float32, dev)
    if state_in is not None:
        _check_tensor("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if state_out is None:
        state_out = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    _check_tensor("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, Hv, Dv), dtype=dt, device=dev)
    _check_tensor("y", y, (B, T, Hv, Dv), dt, dev)
    return (B, T, Hk, Hv, Dk, Dv, dev, dt), state_out, y


def seq_fwd(q, k, v, g, beta, state_in=None, *, state_out=None, y=None, stream=None,
            heads="grouped", gate="decay"):
    """``gdn_seq_fwd_ex`` on torch tensors (token by token, the state read
    once).  Arguments and result as for :func:`chunk_fwd` (without ``C``)."""
    lib = load()
    flags = _flags(heads, gate, g.dim() == 4)
    (B, T, Hk, Hv, Dk, Dv, dev, dt), state_out, y = _prefill_args(q, k, v, g, beta, state_in, state_out, y)
    rc = lib.gdn_seq_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                            _ptr(state_out), _ptr(y), B, T, Hk, Hv, Dk, Dv, flags,
                            DTYPE_CODE[dt], _stream_handle(stream, dev))
    if rc != 0:
        raise GDNError("gdn_seq_fwd_ex", rc, status_string(rc))
    return y, state_out


def chunk_fwd(q, k, v, g, beta, state_in=None, *, C=64, state_out=None, y=None,
              stream=None, heads="grouped", gate="decay"):
    """``gdn_chunk_fwd`` on torch tensors.  Returns ``(y, state_out)``.

    q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv] (float32, bfloat16 or float16); g, beta
    [B,T,Hv] float32; state_in [B,Hv,Dv,Dk] float32 or None.  Outputs are
    allocated when not given; ``state_out`` may be ``state_in`` (in place).
    ``C = 0`` lets the library choose the kernel and the chunk length.
    ``heads`` is the head map ("grouped": key head hv // (Hv // Hk);
    "tiled": hv % Hk) and ``gate`` says whether ``g`` is the decay or its
    natural logarithm ("decay" / "log").  ``g`` [B,T,Hv,Dk] is a decay per
    key dimension (each key column of the state decays by its own factor).
    """
    lib = load()
    flags = _flags(heads, gate, g.dim() == 4)
    (B, T, Hk, Hv, Dk, Dv, dev, dt), state_out, y = _prefill_args(q, k, v, g, beta, state_in, state_out, y)
    rc = lib.gdn_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                              _ptr(state_out), _ptr(y), B, T, Hk, Hv, Dk, Dv, int(C), flags,
                              DTYPE_CODE[dt], _stream_handle(stream, dev))
    if rc != 0:
        raise GDNError("gdn_chunk_fwd_ex", rc, status_string(rc))
    return y, state_out


def step(q, k, v, g, beta, state_in=None, *, state_out=None, y=None, stream=None,
         heads="grouped", gate="decay"):
    """``gdn_step_ex`` on torch tensors (one token).  Returns ``(y, state_out)``.

    q, k [B,Hk,Dk]; v [B,Hv,Dv]; g, beta [B,Hv] float32; state_in
    [B,Hv,Dv,Dk] float32 or None; ``state_out`` may be ``state_in``.
    ``heads`` and ``gate`` as for :func:`chunk_fwd`; ``g`` [B,Hv,Dk] is a
    decay per key dimension.
    """
    lib = load()
    flags = _flags(heads, gate, g.dim() == 3)
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    dev, dt = q.device, q.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    _check_tensor("q", q, (B, Hk, Dk), dt, dev)
    _check_tensor("k", k, (B, Hk, Dk), dt, dev)
    _check_tensor("v", v, (B, Hv, Dv), dt, dev)
    _check_tensor("g", g, (B, Hv, Dk) if g.dim() == 3 else (B, Hv), torch.float32, dev)
    _check_tensor("beta", beta, (B, Hv), torch.float32, dev)
    if state_in is not None:
        _check_tensor("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if state_out is None:
        state_out = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    _check_tensor("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    if y is None:
        y = torch.empty((B, Hv, Dv), dtype=dt, device=dev)
    _check_tensor("y", y, (B, Hv, Dv), dt, dev)
    rc = lib.gdn_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                         _ptr(state_out), _ptr(y), B, Hk, Hv, Dk, Dv, flags, DTYPE_CODE[dt],
                         _stream_handle(stream, dev))
    if rc != 0:
        raise GDNError("gdn_step_ex", rc, status_string(rc))
    return y, state_out
