"""GPU parity of the per-wave chunk kernel against the f64 oracle.

gdn_chunk_fwd at C = 16 (and the automatic choice from a few tokens on)
runs it for one chunk of 1..16 tokens with 16-bit inputs, Dk = 128 and Dv a
multiple of 64: one wave per 16 value rows, state and K/Q staged through
LDS, the chunk's 16 x 16 matrices formed per wave, transposed operands from
a product with the identity.  Covered here: every token count to the
boundary with the generic kernel (17 tokens), both value widths, head maps,
gate forms, absent / given / in-place state, extreme gates, nearly parallel
keys, grids with and without the XCD regrouping, and the decode-shaped grid
at full size (sampled slots).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def run_c16(lib, inp, state="given", C=16, **kw):
    d = upload(inp, state=state != "absent")
    st_in = d["state"]
    st_out = st_in if state == "in_place" else None
    y, s = lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st_in, C=C, state_out=st_out, **kw)
    torch.cuda.synchronize()
    if st_out is not None:
        assert s.data_ptr() == st_out.data_ptr()
    return to_host_f64(y), to_host_f64(s)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 8, 9, 13, 15, 16, 17])
def test_wave_tokens(gpu_lib, dtype, T):
    """Every length class up to the chunk (16 tokens), and 17 (the generic
    kernel, two chunks) on the other side of the boundary."""
    inp = gi.make_inputs(2, T, 2, 4, 128, 128, dtype, gate="sigmoid", state_std=0.2, seed=1300 + T)
    y, s = run_c16(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, dtype, f"wave {dtype} T={T}")


@pytest.mark.parametrize("Dv", [64, 128])
@pytest.mark.parametrize("heads,gate", [("grouped", "decay"), ("tiled", "decay"), ("grouped", "log"), ("tiled", "log")])
@pytest.mark.parametrize("state", ["given", "absent", "in_place"])
def test_wave_options(gpu_lib, Dv, heads, gate, state):
    T = 11
    inp = gi.make_inputs(3, T, 2, 6, 128, Dv, "bf16", gate="softplus", state_std=0.2,
                         state=state != "absent", seed=Dv + len(heads) + len(gate) + len(state))
    if gate == "log":
        inp = dict(inp)
        inp["g"] = np.log(inp["g"].astype(np.float64)).astype(np.float32)
    y, s = run_c16(gpu_lib, inp, state=state, heads=heads, gate=gate)
    yr, sr = oracle_run(inp, state=state != "absent", head_map=heads, gate=gate)
    assert_parity(y, s, yr, sr, "bf16", f"wave Dv={Dv} {heads} {gate} {state}")


@pytest.mark.parametrize("gval", [0.0, 1e-20, 1.0])
def test_wave_extreme_gates(gpu_lib, gval):
    """A zero decay (the state and every earlier token forgotten), one that
    underflows in products, and no decay at all."""
    inp = gi.make_inputs(2, 16, 2, 4, 128, 128, "f16", gate="const", gate_const=gval, state_std=0.1, seed=17)
    y, s = run_c16(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "f16", f"wave g={gval}")


def test_wave_log_gate_minus_inf(gpu_lib):
    inp = dict(gi.make_inputs(2, 12, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=23))
    g = np.log(inp["g"].astype(np.float64)).astype(np.float32)
    g[:, 5] = -np.inf
    g[:, 9] = -100.0
    inp["g"] = g
    y, s = run_c16(gpu_lib, inp, gate="log")
    yr, sr = oracle_run(inp, gate="log")
    assert_parity(y, s, yr, sr, "bf16", "wave log gates -inf / -100")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_wave_parallel_keys(gpu_lib, dtype):
    """Nearly parallel keys with beta near 1 and no decay: the 16 x 16
    system far from the identity."""
    inp = gi.make_inputs(2, 16, 2, 4, 128, 128, dtype, gate="const", gate_const=1.0, beta_const=0.99,
                         key_corr=0.1, state_std=0.05, seed=41)
    y, s = run_c16(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, dtype, f"wave parallel keys {dtype}")


@pytest.mark.parametrize("B,Hk,Hv,Dv", [(4, 4, 8, 128), (3, 5, 5, 128), (8, 2, 8, 64), (1, 3, 3, 64)],
                         ids=["regrouped", "dealt", "dv64_regrouped", "dv64_dealt"])
def test_wave_grids(gpu_lib, B, Hk, Hv, Dv):
    """Grids whose workgroup count is a multiple of 8 x the workgroups per
    q/k stream (renumbered onto one XCD per stream) and grids where it is
    not (dealt as launched)."""
    inp = gi.make_inputs(B, 6, Hk, Hv, 128, Dv, "f16", gate="uniform", gate_lo=0.8, state_std=0.2, seed=B * Hv + Dv)
    y, s = run_c16(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "f16", f"wave B={B} Hk={Hk} Hv={Hv} Dv={Dv}")


@pytest.mark.parametrize("T", [2, 8, 16])
def test_wave_decode_grid(gpu_lib, T):
    """The decode-shaped grid (B = 64, Hk = 16, Hv = 32, f16) at C = 16 and
    with the automatic choice, sampled slots."""
    B, Hk, Hv = 64, 16, 32
    inp = gi.make_inputs(B, T, Hk, Hv, 128, 128, "f16", gate="sigmoid", state_std=0.2, seed=2000 + T)
    rng = np.random.default_rng(T)
    mask = np.zeros((B, Hv), bool)
    mask.reshape(-1)[rng.choice(B * Hv, 8, replace=False)] = True
    mask[0, 0] = mask[-1, -1] = True
    yr, sr = oracle_run(inp, slot_mask=mask)
    ym = np.broadcast_to(mask[:, None, :, None], yr.shape)
    sm = np.broadcast_to(mask[:, :, None, None], sr.shape)
    for C in (16, 0):
        y, s = run_c16(gpu_lib, inp, C=C)
        assert np.isfinite(y).all() and np.isfinite(s).all()
        assert_parity(y, s, yr, sr, "f16", f"wave decode grid T={T} C={C}", y_mask=ym, s_mask=sm)
