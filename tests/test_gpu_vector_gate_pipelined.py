"""GPU parity of the pipelined kernel for a decay per key dimension (16-bit
inputs, Dk = Dv = 128, chunks of 32 tokens, grids of more than 128 slots)
against the f64 oracle, on sampled slots: ragged lengths across chunk and
block boundaries, both dtypes, grouped and tiled heads, log gates with
-inf entries, zero and tiny decays per column, absent and in-place state,
gates near one and mixed, and continuation over two calls.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def vg_inputs(B, T, Hk, Hv, dtype, seed, kind="sigmoid", state=True):
    inp = gi.make_inputs(B, T, Hk, Hv, 128, 128, dtype, gate="sigmoid", state_std=0.2, state=state, seed=seed)
    inp["g"] = gi.vector_gate(B, T, Hv, 128, seed=seed + 1, kind=kind)
    return inp


def sampled(B, Hv, seed, n=6):
    rng = np.random.default_rng(seed)
    mask = np.zeros((B, Hv), bool)
    mask.reshape(-1)[rng.choice(B * Hv, n, replace=False)] = True
    mask[0, 0] = mask[-1, -1] = True
    return mask


def check(y, s, inp, mask, dtype, what, **kw):
    yr, sr = oracle_run(inp, slot_mask=mask, **kw)
    assert np.isfinite(y).all() and np.isfinite(s).all()
    assert_parity(y, s, yr, sr, dtype, what,
                  np.broadcast_to(mask[:, None, :, None], yr.shape),
                  np.broadcast_to(mask[:, :, None, None], sr.shape))


def run(gdn, inp, state="given", C=32, **kw):
    d = upload(inp, state=state != "absent")
    st_out = d["state"] if state == "in_place" else None
    y, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C, state_out=st_out, **kw)
    torch.cuda.synchronize()
    if st_out is not None:
        assert s.data_ptr() == st_out.data_ptr()
    return to_host_f64(y), to_host_f64(s)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [1, 5, 16, 17, 31, 32, 33, 64, 100, 257])
def test_vgp_lengths(gpu_lib, dtype, T):
    B, Hk, Hv = 3, 43, 43
    inp = vg_inputs(B, T, Hk, Hv, dtype, seed=700 + T)
    y, s = run(gpu_lib, inp)
    check(y, s, inp, sampled(B, Hv, T), dtype, f"pipelined vector gate {dtype} T={T}")


@pytest.mark.parametrize("heads", ["grouped", "tiled"])
@pytest.mark.parametrize("kind", ["near_one", "mixed"])
def test_vgp_heads_and_kinds(gpu_lib, heads, kind):
    """256 slots of grouped key heads (the XCD-grouped order) and tiled."""
    B, Hk, Hv = 8, 16, 32
    inp = vg_inputs(B, 150, Hk, Hv, "bf16", seed=11, kind=kind)
    y, s = run(gpu_lib, inp, heads=heads)
    check(y, s, inp, sampled(B, Hv, 11), "bf16", f"pipelined vector gate {heads} {kind}", head_map=heads)


def test_vgp_log_and_extremes(gpu_lib):
    """Log-space gates with -inf (a zero decay) and very negative entries in
    some key columns, and decays of exactly 0 and 1e-30 in others."""
    B, Hk, Hv = 3, 43, 43
    inp = dict(vg_inputs(B, 77, Hk, Hv, "bf16", seed=5))
    g = inp["g"].astype(np.float64)
    g[:, 10, :, 3] = 0.0
    g[:, 40, :, 70:80] = 1e-30
    lg = np.log(np.maximum(g, 0.0), where=g > 0, out=np.full_like(g, -np.inf))
    lg[:, 50, :, 100] = -200.0
    inp["g"] = lg.astype(np.float32)
    mask = sampled(B, Hv, 5)
    y, s = run(gpu_lib, inp, gate="log")
    check(y, s, inp, mask, "bf16", "pipelined vector gate log/extremes", gate="log")


@pytest.mark.parametrize("state", ["absent", "in_place"])
def test_vgp_state(gpu_lib, state):
    B, Hk, Hv = 3, 43, 43
    inp = vg_inputs(B, 70, Hk, Hv, "f16", seed=13, state=state != "absent")
    y, s = run(gpu_lib, inp, state=state)
    check(y, s, inp, sampled(B, Hv, 13), "f16", f"pipelined vector gate state {state}",
          state=state != "absent")


def test_vgp_continuation(gpu_lib):
    """Two calls (T = 45, then 58) equal one call over all 103 tokens."""
    B, Hk, Hv = 3, 43, 43
    inp = vg_inputs(B, 103, Hk, Hv, "bf16", seed=17)
    d = upload(inp)
    cut = 45
    part = lambda t: tuple(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta"))
    y1, s1 = gpu_lib.chunk_fwd(*part(slice(0, cut)), d["state"], C=32)
    y2, s2 = gpu_lib.chunk_fwd(*part(slice(cut, None)), s1, C=32)
    torch.cuda.synchronize()
    y = to_host_f64(torch.cat([y1, y2], 1))
    check(y, to_host_f64(s2), inp, sampled(B, Hv, 17), "bf16", "pipelined vector gate continuation")
