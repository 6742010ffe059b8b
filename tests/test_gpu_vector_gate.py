"""GPU parity of the per-key-dimension gate (g [B,T,Hv,Dk], GDN_GATE_VECTOR)
against the f64 oracle: the chunked kernel for vector gates at C = 16 and
32 (16 for float32), the sequential kernel and the decode step; every dtype
and head size, grouped and tiled heads, log gates, ragged lengths, gate
extremes (zero, tiny and unit decays per column), in-place state and the
automatic kernel choice, and Dv = 128 on both sides of the value-slice threshold.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def vg_inputs(B, T, Hk, Hv, Dk, Dv, dtype, seed, kind="sigmoid", state_std=0.2):
    inp = gi.make_inputs(B, T, Hk, Hv, Dk, Dv, dtype, gate="sigmoid", state_std=state_std, seed=seed)
    inp["g"] = gi.vector_gate(B, T, Hv, Dk, seed=seed + 1, kind=kind)
    return inp


def run(gdn, inp, how, **kw):
    d = upload(inp)
    if how == "seq":
        y, s = gdn.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], **kw)
    else:
        y, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=how, **kw)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(s)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("how", [16, 32, "seq"])
def test_vector_gate_lengths(gpu_lib, dtype, how):
    for T in (1, 5, 16, 17, 31, 32, 33, 100):
        inp = vg_inputs(2, T, 2, 4, 128, 128, dtype, seed=200 + T)
        y, s = run(gpu_lib, inp, how)
        yr, sr = oracle_run(inp)
        assert_parity(y, s, yr, sr, dtype, f"vector gate {dtype} {how} T={T}")


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (64, 64), (128, 32), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vector_gate_head_dims(gpu_lib, dk, dv, dtype):
    inp = vg_inputs(1, 70, 1, 3, dk, dv, dtype, seed=dk + dv)
    for how in (32, "seq"):
        y, s = run(gpu_lib, inp, how)
        yr, sr = oracle_run(inp)
        assert_parity(y, s, yr, sr, dtype, f"vector gate Dk={dk} Dv={dv} {how}")


@pytest.mark.parametrize("kind", ["near_one", "mixed"])
@pytest.mark.parametrize("heads", ["grouped", "tiled"])
def test_vector_gate_kinds_and_heads(gpu_lib, kind, heads):
    inp = vg_inputs(2, 150, 4, 16, 128, 128, "bf16", seed=9, kind=kind)
    yr, sr = oracle_run(inp, head_map=heads)
    for how in (16, 32, "seq"):
        y, s = run(gpu_lib, inp, how, heads=heads)
        assert_parity(y, s, yr, sr, "bf16", f"vector gate {kind} {heads} {how}")


def test_vector_gate_log_and_extremes(gpu_lib):
    """Log-space vector gates, with whole columns at decay 1 (log 0), single
    entries at 0 (log -inf) and 1e-30, and a run of small decays."""
    inp = vg_inputs(2, 80, 2, 4, 64, 64, "f32", seed=17)
    g = inp["g"].astype(np.float64)
    g[:, :, :, :8] = 1.0
    g[:, 10, :, 20:30] = 0.0
    g[:, 11, :, 30:40] = 1e-30
    g[:, 40:60, :, 40:] = 0.02
    with np.errstate(divide="ignore"):
        inp["g"] = np.log(g).astype(np.float32)
    yr, sr = oracle_run(inp, gate="log")
    for how in (16, "seq"):
        y, s = run(gpu_lib, inp, how, gate="log")
        assert_parity(y, s, yr, sr, "f32", f"vector log gate extremes {how}")


def test_vector_gate_equal_entries_match_scalar(gpu_lib):
    """A vector gate whose entries are all equal gives the scalar gate's
    result (both kernels against the same oracle value)."""
    inp = gi.make_inputs(2, 90, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=23)
    yr, sr = oracle_run(inp)
    vin = dict(inp)
    vin["g"] = np.repeat(inp["g"][..., None], 128, axis=-1)
    for how in (32, "seq"):
        y, s = run(gpu_lib, vin, how)
        assert_parity(y, s, yr, sr, "bf16", f"equal-entry vector gate {how}")


def test_vector_gate_step_and_in_place(gpu_lib):
    inp = vg_inputs(3, 6, 2, 6, 128, 64, "f16", seed=31)
    d = upload(inp)
    st = d["state"].clone()
    ys = []
    for t in range(6):
        y, st = gpu_lib.step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), st,
                             state_out=st)
        ys.append(y)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(torch.stack(ys, 1)), to_host_f64(st), yr, sr, "f16", "vector gate steps")
    st = d["state"].clone()
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, C=32, state_out=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "f16", "vector gate chunk in place")


def test_vector_gate_auto_and_continuation(gpu_lib):
    """C = 0 on both sides of the sequential/chunked switch, and a split
    call (70 + 80 tokens) equal to the whole."""
    for T in (3, 40):
        inp = vg_inputs(2, T, 2, 4, 128, 128, "bf16", seed=40 + T)
        y, s = run(gpu_lib, inp, 0)
        yr, sr = oracle_run(inp)
        assert_parity(y, s, yr, sr, "bf16", f"vector gate auto T={T}")
    inp = vg_inputs(1, 150, 2, 4, 128, 128, "bf16", seed=5, state_std=0.05)
    d = upload(inp)
    part = lambda x, sl: x[:, sl].contiguous()
    s1, s2 = slice(0, 70), slice(70, 150)
    y1, st = gpu_lib.chunk_fwd(*(part(d[n], s1) for n in ("q", "k", "v", "g", "beta")), d["state"], C=32)
    y2, st = gpu_lib.chunk_fwd(*(part(d[n], s2) for n in ("q", "k", "v", "g", "beta")), st, C=16)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(torch.cat([y1, y2], 1)), to_host_f64(st), yr, sr, "bf16", "vector gate split")


def test_vector_gate_deterministic(gpu_lib):
    inp = vg_inputs(2, 200, 2, 4, 128, 128, "bf16", seed=8)
    d = upload(inp)
    outs = [gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=32)
            for _ in range(3)]
    torch.cuda.synchronize()
    for y, s in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(s, outs[0][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hk,Hv", [(4, 16, 32), (3, 43, 43)], ids=["128slots", "129slots"])
def test_vector_gate_value_slices(gpu_lib, dtype, B, Hk, Hv):
    """Dv = 128 runs two 64-column value slices per slot up to B Hv = 128
    slots and one workgroup per slot above: both sides of the threshold, on
    sampled slots."""
    inp = vg_inputs(B, 45, Hk, Hv, 128, 128, dtype, seed=B * Hv)
    y, s = run(gpu_lib, inp, 16 if dtype == "f32" else 32)
    rng = np.random.default_rng(B * Hv)
    mask = np.zeros((B, Hv), bool)
    mask.reshape(-1)[rng.choice(B * Hv, 12, replace=False)] = True
    mask[-1, -1] = True
    yr, sr = oracle_run(inp, slot_mask=mask)
    assert_parity(y, s, yr, sr, dtype, f"vector gate {B * Hv} slots {dtype}",
                  np.broadcast_to(mask[:, None, :, None], yr.shape),
                  np.broadcast_to(mask[:, :, None, None], sr.shape))
