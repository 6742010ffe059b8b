"""GPU parity of gdn_chunk_fwd against the f64 oracle (through the C ABI).

Covers the four prefill workloads at full size (the long prefill on sampled
slots, which the oracle can finish in seconds), both readings of the gate
draw, every chunk size on ragged lengths, grouped heads, Dk != Dv, the zero
and absent initial state, in-place state, T = 0 / B = 0, vanishing decays,
continuation across calls and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def run_chunk(gdn, inp, C, state=True, **kw):
    d = upload(inp, state=state)
    y, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C, **kw)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(s)


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_tiny_f32(gpu_lib, gate, C):
    inp = gi.workload_inputs("tiny_f32", gate=gate, seed=0 if gate == "softplus" else 1)
    y, s = run_chunk(gpu_lib, inp, C)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "f32", f"tiny_f32 gate={gate} C={C}")
    if C == 64:
        # float32 inputs are served in chunks of at most 32 tokens: C = 64
        # runs the C = 32 kernel, bit for bit
        y32, s32 = run_chunk(gpu_lib, inp, 32)
        assert np.array_equal(y, y32) and np.array_equal(s, s32)


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
def test_bonsai_prefill(gpu_lib, gate):
    inp = gi.workload_inputs("bonsai_prefill", gate=gate, seed=0 if gate == "softplus" else 1)
    y, s = run_chunk(gpu_lib, inp, 32)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "bf16", f"bonsai_prefill gate={gate}")


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("state", ["zeros", "null"])
def test_gqa_ragged(gpu_lib, gate, state):
    inp = gi.workload_inputs("gqa_ragged", gate=gate, seed=0 if gate == "softplus" else 1)
    y, s = run_chunk(gpu_lib, inp, 64, state=(state == "zeros"))
    yr, sr = oracle_run(inp, state=(state == "zeros"))
    assert_parity(y, s, yr, sr, "bf16", f"gqa_ragged gate={gate} state={state}")


def test_long_prefill_sampled(gpu_lib):
    """Full-size long prefill, in the launch configuration the bench times;
    the oracle checks four (batch, head) slots over all 8192 tokens."""
    inp = gi.workload_inputs("long_prefill")
    y, s = run_chunk(gpu_lib, inp, 64)
    B, Hv = 8, 32
    mask = np.zeros((B, Hv), bool)
    for b, hv in [(0, 0), (3, 17), (5, 30), (7, 31)]:
        mask[b, hv] = True
    yr, sr = oracle_run(inp, slot_mask=mask)
    ymask = np.broadcast_to(mask[:, None, :, None], y.shape)
    smask = np.broadcast_to(mask[:, :, None, None], s.shape)
    assert_parity(y, s, yr, sr, "bf16", "long_prefill (4 sampled slots)", ymask, smask)
    # every output finite
    assert np.isfinite(y).all() and np.isfinite(s).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_ragged_lengths(gpu_lib, dtype, C):
    for T in (1, 7, 15, 16, 17, 63, 64, 65, 129):
        inp = gi.make_inputs(2, T, 2, 4, 64, 64, dtype, gate="sigmoid", state_std=0.1, seed=T)
        y, s = run_chunk(gpu_lib, inp, C)
        yr, sr = oracle_run(inp)
        assert_parity(y, s, yr, sr, dtype, f"{dtype} C={C} T={T}")


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (128, 32), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims(gpu_lib, dk, dv, dtype):
    inp = gi.make_inputs(1, 100, 1, 3, dk, dv, dtype, gate="sigmoid", state_std=0.1, seed=dk + dv)
    y, s = run_chunk(gpu_lib, inp, 32)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, dtype, f"{dtype} Dk={dk} Dv={dv}")


@pytest.mark.parametrize("hk,hv", [(1, 1), (1, 4), (4, 4), (2, 6)])
def test_grouped_heads(gpu_lib, hk, hv):
    inp = gi.make_inputs(2, 77, hk, hv, 64, 64, "bf16", gate="sigmoid", state_std=0.1, seed=hk * 10 + hv)
    y, s = run_chunk(gpu_lib, inp, 64)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "bf16", f"Hk={hk} Hv={hv}")


@pytest.mark.parametrize("gval", [0.0, 1e-20])
def test_vanishing_decay(gpu_lib, gval):
    inp = gi.make_inputs(1, 80, 1, 2, 64, 64, "bf16", gate="const", gate_const=gval, state_std=0.1, seed=5)
    y, s = run_chunk(gpu_lib, inp, 64)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "bf16", f"g={gval}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_no_decay_repeated(gpu_lib, dtype):
    """g = 1 (the plain delta rule): no decay shrinks the couplings between
    distant tokens, so an error in any block of the triangular solve shows up
    at full size.  Several chunks and a ragged tail, the 128-dimensional
    heads of the pipelined kernel, three runs that must agree bit for bit."""
    inp = gi.make_inputs(2, 200, 2, 4, 128, 128, dtype, gate="const", gate_const=1.0,
                         state_std=0.05, seed=4)
    d = upload(inp)
    outs = []
    for _ in range(3):
        y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
        torch.cuda.synchronize()
        outs.append((y.clone(), s.clone()))
    for y, s in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(s, outs[0][1])
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(outs[0][0]), to_host_f64(outs[0][1]), yr, sr, dtype, f"g=1 {dtype}")


def test_in_place_state(gpu_lib):
    inp = gi.make_inputs(2, 90, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=9)
    d = upload(inp)
    st = d["state"].clone()
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, C=64, state_out=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "bf16", "in-place state")


def test_empty(gpu_lib):
    inp = gi.make_inputs(2, 0, 1, 2, 64, 64, "bf16", state_std=0.1, seed=1)
    d = upload(inp)
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 2, 64)
    assert torch.equal(s, d["state"])                       # T = 0 passes the state through
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, C=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s) == 0
    inp = gi.make_inputs(0, 5, 1, 2, 64, 64, "bf16", seed=1)
    d = upload(inp)
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
    assert y.shape[0] == 0 and s.shape[0] == 0


def test_continuation(gpu_lib):
    """chunk(T1) then chunk(T2) from its state matches chunk(T1 + T2)."""
    inp = gi.make_inputs(1, 150, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.05, seed=3)
    d = upload(inp)
    y_all, s_all = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
    sl1, sl2 = slice(0, 70), slice(70, 150)
    part = lambda x, sl: x[:, sl].contiguous()
    y1, s1 = gpu_lib.chunk_fwd(*(part(d[n], sl1) for n in ("q", "k", "v", "g", "beta")), d["state"], C=64)
    y2, s2 = gpu_lib.chunk_fwd(*(part(d[n], sl2) for n in ("q", "k", "v", "g", "beta")), s1, C=32)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(torch.cat([y1, y2], 1)), to_host_f64(s2), yr, sr, "bf16", "split 70+80")
    assert_parity(to_host_f64(y_all), to_host_f64(s_all), yr, sr, "bf16", "whole 150")


def test_deterministic(gpu_lib):
    inp = gi.make_inputs(2, 200, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.05, seed=4)
    d = upload(inp)
    outs = [gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
            for _ in range(3)]
    torch.cuda.synchronize()
    for y, s in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(s, outs[0][1])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("heads", [(16, 32), (32, 32)])
def test_sweep(gpu_lib, dtype, heads):
    """Lengths 1, 7, 16, 257, 1111 and batch 1 and 2 at Dk = Dv = 128 (the
    validation matrix of the MLX page's "Validation" section: heads x dtype
    x length x batch); at 1111 tokens on sampled slots."""
    hk, hv = heads
    for T in (1, 7, 16, 257, 1111):
        for B in (1, 2):
            inp = gi.make_inputs(B, T, hk, hv, 128, 128, dtype, gate="sigmoid", state_std=0.3,
                                 seed=1000 + T + B)
            y, s = run_chunk(gpu_lib, inp, 64)
            mask = ym = sm = None
            if T > 1000:
                mask = np.zeros((B, hv), bool)
                mask[0, 0] = mask[-1, hv - 1] = mask[B // 2, hv // 3] = True
                ym = np.broadcast_to(mask[:, None, :, None], y.shape)
                sm = np.broadcast_to(mask[:, :, None, None], s.shape)
            yr, sr = oracle_run(inp, slot_mask=mask)
            assert_parity(y, s, yr, sr, dtype, f"sweep {dtype} H={heads} T={T} B={B}", ym, sm)


# (dtype, B, Hk, Hv, C): the pipelined kernel with four state waves (more
# than 64 slots) and with the value split (up to 64), the generic kernel
@pytest.mark.parametrize("case", [("bf16", 1, 35, 70, 64), ("f16", 1, 35, 70, 64),
                                  ("bf16", 1, 2, 4, 64), ("f16", 2, 2, 2, 64),
                                  ("bf16", 1, 2, 4, 32), ("f16", 1, 2, 4, 32)],
                         ids=lambda c: f"{c[0]}-B{c[1]}-Hk{c[2]}-Hv{c[3]}-C{c[4]}")
def test_correlated_keys(gpu_lib, case):
    """Nearly parallel keys (every key of a head within a few degrees of one
    direction), beta = 0.99 and no decay over 1111 tokens: the rows of each
    chunk's triangular system nearly cancel and the state keeps everything
    it is told, the case where a solve carried in 16-bit precision loses
    most."""
    dt, B, Hk, Hv, C = case
    inp = gi.make_inputs(B, 1111, Hk, Hv, 128, 128, dt, gate="const", gate_const=1.0, beta_const=0.99,
                         key_corr=0.1, state_std=0.05, seed=31 + Hv + C)
    y, s = run_chunk(gpu_lib, inp, C)
    mask = ym = sm = None
    if B * Hv > 8:
        mask = np.zeros((B, Hv), bool)
        mask[0, 0] = mask[0, 37] = mask[-1, Hv - 1] = True
        ym = np.broadcast_to(mask[:, None, :, None], y.shape)
        sm = np.broadcast_to(mask[:, :, None, None], s.shape)
    yr, sr = oracle_run(inp, slot_mask=mask)
    assert_parity(y, s, yr, sr, dt, f"correlated keys {dt} B={B} Hk={Hk} Hv={Hv} C={C}", ym, sm)
    assert np.isfinite(y).all() and np.isfinite(s).all()
