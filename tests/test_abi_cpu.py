"""The C ABI on the host, without a GPU: the library loads, exports every
function ``include/gdn.h`` declares, and rejects invalid arguments with the
documented codes before anything is launched (no call here reaches a
kernel: each one fails a host-side check).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, UNSUP, ALIAS, ALIGN, HIP, DTYPE = 0, -1, -2, -3, -4, -5, -6, -7


@pytest.fixture(scope="module")
def lib():
    from gated_deltanet_prefill_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from gated_deltanet_prefill_amd import build
        build.build_library()
    return _binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdn_chunk_fwd", "gdn_seq_fwd", "gdn_step", "gdn_chunk_fwd_ex", "gdn_seq_fwd_ex",
            "gdn_step_ex", "gdn_status_string", "gdn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdn.h but not exported"


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, UNSUP, ALIAS, ALIGN, HIP, DTYPE, 12345):
        s = lib.gdn_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.gdn_version() >= 100


P = ctypes.c_void_p
A = 1 << 20            # fake, 16-byte aligned "device" addresses; never dereferenced


def chunk(lib, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=6 * A, so=7 * A, y=8 * A,
          B=1, T=4, Hk=1, Hv=1, Dk=32, Dv=32, C=16, dtype=1):
    return lib.gdn_chunk_fwd(P(q), P(k), P(v), P(g), P(b), P(si), P(so), P(y),
                             B, T, Hk, Hv, Dk, Dv, C, dtype, None)


def seq(lib, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=6 * A, so=7 * A, y=8 * A,
        B=1, T=4, Hk=1, Hv=1, Dk=32, Dv=32, dtype=1):
    return lib.gdn_seq_fwd(P(q), P(k), P(v), P(g), P(b), P(si), P(so), P(y),
                           B, T, Hk, Hv, Dk, Dv, dtype, None)


def step(lib, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=6 * A, so=7 * A, y=8 * A,
         B=1, Hk=1, Hv=1, Dk=32, Dv=32, dtype=1):
    return lib.gdn_step(P(q), P(k), P(v), P(g), P(b), P(si), P(so), P(y),
                        B, Hk, Hv, Dk, Dv, dtype, None)


def test_shape_errors(lib):
    assert chunk(lib, B=-1) == SHAPE
    assert chunk(lib, T=-2) == SHAPE
    assert chunk(lib, Hk=0) == SHAPE
    assert chunk(lib, Hk=2, Hv=3) == SHAPE
    assert step(lib, Hk=3, Hv=4) == SHAPE
    assert seq(lib, T=-1) == SHAPE
    assert seq(lib, Hk=2, Hv=3) == SHAPE


def test_unsupported(lib):
    assert chunk(lib, Dk=48) == UNSUP
    assert chunk(lib, Dv=256) == UNSUP
    assert chunk(lib, C=8) == UNSUP
    assert chunk(lib, C=128) == UNSUP
    assert chunk(lib, C=-16) == UNSUP
    assert seq(lib, Dv=96) == UNSUP
    assert step(lib, Dk=16) == UNSUP


def test_dtype(lib):
    assert chunk(lib, dtype=3) == DTYPE
    assert step(lib, dtype=-1) == DTYPE
    assert seq(lib, dtype=7) == DTYPE


def test_null(lib):
    assert chunk(lib, so=0) == NULL
    for name in ("q", "k", "v", "g", "b", "y"):
        assert chunk(lib, **{name: 0}) == NULL, name
    assert step(lib, q=0) == NULL
    assert seq(lib, so=0) == NULL
    assert seq(lib, k=0) == NULL


def test_alignment(lib):
    assert chunk(lib, q=A + 8) == ALIGN
    assert chunk(lib, so=7 * A + 4) == ALIGN
    assert chunk(lib, g=4 * A + 2) == ALIGN
    assert step(lib, y=8 * A + 2) == ALIGN
    assert seq(lib, v=3 * A + 4) == ALIGN


def test_aliasing(lib):
    # y on top of v
    assert chunk(lib, y=3 * A) == ALIAS
    # state_out inside k
    assert chunk(lib, so=2 * A) == ALIAS
    # state_out partly overlapping state_in (but not equal)
    assert chunk(lib, si=6 * A, so=6 * A + 16) == ALIAS
    # y overlapping state_out
    assert chunk(lib, y=7 * A + 64) == ALIAS
    assert step(lib, y=2 * A) == ALIAS
    assert seq(lib, so=5 * A) == ALIAS


def test_empty_batch_is_a_no_op(lib):
    # B = 0: nothing to do, and no pointer is needed
    assert chunk(lib, B=0, q=0, k=0, v=0, g=0, b=0, si=0, so=0, y=0) == OK
    assert step(lib, B=0, q=0, k=0, v=0, g=0, b=0, si=0, so=0, y=0) == OK
    assert seq(lib, B=0, q=0, k=0, v=0, g=0, b=0, si=0, so=0, y=0) == OK
    assert chunk(lib, B=0, C=0, q=0, k=0, v=0, g=0, b=0, si=0, so=0, y=0) == OK


def chunk_ex(lib, flags, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=6 * A, so=7 * A, y=8 * A,
             B=1, T=4, Hk=1, Hv=1, Dk=32, Dv=32, C=16, dtype=1):
    return lib.gdn_chunk_fwd_ex(P(q), P(k), P(v), P(g), P(b), P(si), P(so), P(y),
                                B, T, Hk, Hv, Dk, Dv, C, flags, dtype, None)


def test_ex_flags(lib):
    """Unknown flag bits are rejected; known ones pass the host checks (B = 0
    stops before any launch); the _ex calls check arguments like the plain
    ones."""
    for bad in (8, 16, 1 << 30, -1):
        assert chunk_ex(lib, bad) == UNSUP
        assert lib.gdn_seq_fwd_ex(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A),
                                  P(8 * A), 1, 4, 1, 1, 32, 32, bad, 1, None) == UNSUP
        assert lib.gdn_step_ex(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A),
                               P(8 * A), 1, 1, 1, 32, 32, bad, 1, None) == UNSUP
    for good in (0, 1, 2, 3):
        assert chunk_ex(lib, good, B=0, q=0, k=0, v=0, g=0, b=0, si=0, so=0, y=0) == OK
        assert chunk_ex(lib, good, Hk=2, Hv=3) == SHAPE
        assert chunk_ex(lib, good, C=8) == UNSUP
        assert chunk_ex(lib, good, y=2 * A) == ALIAS


def test_vector_gate_checks(lib):
    """A per-key-dimension gate (flag 4) is [B,T,Hv,Dk] and 16-byte aligned:
    the alignment and overlap checks use that size."""
    VEC = 4
    assert chunk_ex(lib, VEC, g=4 * A + 4) == ALIGN
    # a scalar gate needs 4 bytes only: the call gets past the pointer
    # checks and stops at the (invalid) chunk length, before any launch
    assert chunk_ex(lib, 0, g=4 * A + 4, C=8) == UNSUP
    # y 256 bytes after g: clear of a scalar gate (16 bytes), inside a vector one (512)
    assert chunk_ex(lib, VEC, y=4 * A + 256) == ALIAS
    assert chunk_ex(lib, 0, y=4 * A + 256, C=8) == UNSUP
    assert lib.gdn_step_ex(P(A), P(2 * A), P(3 * A), P(4 * A + 4), P(5 * A), P(6 * A), P(7 * A),
                           P(8 * A), 1, 1, 1, 32, 32, VEC, 1, None) == ALIGN
