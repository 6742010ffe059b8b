"""GPU parity of gdn_seq_fwd (the token-by-token prefill kernel) and of
gdn_chunk_fwd with C = 0 (the library picks the kernel) against the f64
oracle, through the C ABI.

Covers short and ragged lengths (T = 0 included), every dtype and head size,
grouped heads, the absent and the in-place state, the decode workload's 256
tokens on sampled slots, agreement with the chunked kernel, and a long
sequence in one call (error growth over many recurrent steps).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def run_seq(gdn, inp, state=True, **kw):
    d = upload(inp, state=state)
    y, s = gdn.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], **kw)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(s)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_seq_lengths(gpu_lib, dtype):
    for T in (1, 2, 7, 16, 33):
        inp = gi.make_inputs(2, T, 2, 4, 128, 128, dtype, gate="sigmoid", state_std=0.3, seed=70 + T)
        y, s = run_seq(gpu_lib, inp)
        yr, sr = oracle_run(inp)
        assert_parity(y, s, yr, sr, dtype, f"seq {dtype} T={T}")


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (128, 32), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_seq_head_dims(gpu_lib, dk, dv, dtype):
    inp = gi.make_inputs(2, 9, 1, 3, dk, dv, dtype, gate="softplus", state_std=0.1, seed=dk + 3 * dv)
    y, s = run_seq(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, dtype, f"seq {dtype} Dk={dk} Dv={dv}")


@pytest.mark.parametrize("hk,hv", [(1, 1), (1, 4), (2, 6), (16, 32)])
def test_seq_grouped_heads(gpu_lib, hk, hv):
    inp = gi.make_inputs(3, 6, hk, hv, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=hk * 7 + hv)
    y, s = run_seq(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "bf16", f"seq Hk={hk} Hv={hv}")


@pytest.mark.parametrize("B,hv,dv,dtype", [(8, 32, 128, "bf16"), (16, 32, 128, "f32"), (16, 32, 64, "f16")])
def test_seq_rows_per_lane(gpu_lib, B, hv, dv, dtype):
    """Grids large enough for two and four value rows per lane (the kernel
    packs more rows per lane when the grid has waves to spare)."""
    inp = gi.make_inputs(B, 3, 16, hv, 128, dv, dtype, gate="sigmoid", state_std=0.2, seed=B + dv)
    y, s = run_seq(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, dtype, f"seq B={B} Hv={hv} Dv={dv}")


def test_seq_gate_extremes(gpu_lib):
    """Zero, tiny and unit gates, and a run of small ones whose product
    leaves the float range: the kernel's deferred decay must fold and
    restart without loss."""
    inp = gi.make_inputs(2, 40, 1, 2, 64, 64, "f32", gate="sigmoid", state_std=0.3, seed=41)
    g = inp["g"]
    g[:, 0:3] = 1.0
    g[:, 3] = 0.0
    g[:, 4:9] = 1e-20
    g[:, 9:30] = 0.05
    g[0, 35] = 0.0
    y, s = run_seq(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "f32", "seq gate extremes")


def test_seq_null_and_in_place_state(gpu_lib):
    inp = gi.make_inputs(2, 5, 2, 4, 128, 128, "f16", gate="sigmoid", state_std=0.2, seed=11)
    y, s = run_seq(gpu_lib, inp, state=False)
    yr, sr = oracle_run(inp, state=False)
    assert_parity(y, s, yr, sr, "f16", "seq null state")
    d = upload(inp)
    st = d["state"].clone()
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "f16", "seq in-place state")


def test_seq_empty(gpu_lib):
    inp = gi.make_inputs(2, 0, 1, 2, 64, 64, "bf16", state_std=0.1, seed=1)
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 2, 64)
    assert torch.equal(s, d["state"])
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s) == 0


def test_seq_decode_tokens_sampled(gpu_lib):
    """The decode workload's 256 tokens in one call, checked on six slots."""
    inp = gi.workload_inputs("decode")
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    torch.cuda.synchronize()
    B, Hv = 64, 32
    mask = np.zeros((B, Hv), bool)
    for b, hv in [(0, 0), (2, 3), (19, 7), (40, 16), (51, 29), (63, 31)]:
        mask[b, hv] = True
    yr, sr = oracle_run(inp, slot_mask=mask)
    yg, sg = to_host_f64(y), to_host_f64(s)
    assert_parity(yg, sg, yr, sr, "f16", "seq over decode tokens (6 slots)",
                  np.broadcast_to(mask[:, None, :, None], yg.shape),
                  np.broadcast_to(mask[:, :, None, None], sg.shape))
    assert np.isfinite(yg).all() and np.isfinite(sg).all()


def test_seq_matches_chunk_and_step(gpu_lib):
    """Three kernels, one recurrence: seq, chunk and chained steps agree."""
    inp = gi.make_inputs(2, 24, 2, 4, 128, 128, "f32", gate="sigmoid", state_std=0.2, seed=21)
    d = upload(inp)
    ys, ss = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    yc, sc = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=16)
    st = d["state"].clone()
    ysteps = []
    for t in range(24):
        y, st = gpu_lib.step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")),
                             st, state_out=st)
        ysteps.append(y)
    torch.cuda.synchronize()
    yt = torch.stack(ysteps, 1)
    # seq and step run the same per-token arithmetic; chunk reorders it
    assert torch.allclose(ys, yt, rtol=1e-5, atol=1e-6) and torch.allclose(ss, st, rtol=1e-5, atol=1e-6)
    yr, sr = oracle_run(inp)
    for y, s, what in ((ys, ss, "seq"), (yc, sc, "chunk C=16"), (yt, st, "steps")):
        assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "f32", what)


def test_seq_long_sequence(gpu_lib):
    """600 recurrent steps in one call (state error compounds over steps)."""
    inp = gi.make_inputs(1, 600, 1, 2, 128, 128, "bf16", gate="softplus", state_std=0.1, seed=31)
    y, s = run_seq(gpu_lib, inp)
    yr, sr = oracle_run(inp)
    assert_parity(y, s, yr, sr, "bf16", "seq T=600")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_auto_chunk(gpu_lib, dtype, D):
    """C = 0: the library's own choice of kernel and chunk length is right
    on both sides of every switch (token-by-token to chunked, C = 16 / 32 /
    64)."""
    for T in (1, 3, 8, 12, 13, 15, 16, 17, 31, 32, 40, 47, 48, 63, 64, 95, 96, 100, 300):
        inp = gi.make_inputs(2, T, 2, 4, D, D, dtype, gate="sigmoid", state_std=0.2, seed=500 + T + D)
        d = upload(inp)
        y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=0)
        torch.cuda.synchronize()
        yr, sr = oracle_run(inp)
        assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, dtype, f"auto {dtype} T={T}")


@pytest.mark.parametrize("B,Hk,Hv", [(2, 16, 32), (5, 13, 13), (4, 16, 32), (1, 43, 129), (8, 16, 32), (1, 257, 257)],
                         ids=["64slots", "65slots", "128slots", "129slots", "256slots", "257slots"])
def test_auto_chunk_slots(gpu_lib, B, Hk, Hv):
    """C = 0 with 16-bit inputs and 128-dimensional heads on both sides of
    the slot-count switches of the chunk length (64 / 65, 128 / 129, 256 /
    257 slots) at lengths where the choice depends on them; sampled slots."""
    for T in (48, 96, 128):
        inp = gi.make_inputs(B, T, Hk, Hv, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=B * Hv + T)
        d = upload(inp)
        y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=0)
        torch.cuda.synchronize()
        rng = np.random.default_rng(B * Hv + T)
        mask = np.zeros((B, Hv), bool)
        mask.reshape(-1)[rng.choice(B * Hv, 6, replace=False)] = True
        mask[-1, -1] = True
        yr, sr = oracle_run(inp, slot_mask=mask)
        ym = np.broadcast_to(mask[:, None, :, None], yr.shape)
        sm = np.broadcast_to(mask[:, :, None, None], sr.shape)
        assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "bf16", f"auto B={B} Hk={Hk} Hv={Hv} T={T}",
                      y_mask=ym, s_mask=sm)


def sampled_slots(B, Hv, seed, n=8):
    """A few slots at random plus the first and the last (the last tiles of
    a persistent workgroup's loop)."""
    rng = np.random.default_rng(seed)
    mask = np.zeros((B, Hv), bool)
    mask.reshape(-1)[rng.choice(B * Hv, n, replace=False)] = True
    mask[0, 0] = mask[-1, -1] = True
    return mask


def check_sampled(y, s, inp, mask, dtype, what, **kw):
    yr, sr = oracle_run(inp, slot_mask=mask, **kw)
    yg, sg = to_host_f64(y), to_host_f64(s)
    assert_parity(yg, sg, yr, sr, dtype, what,
                  np.broadcast_to(mask[:, None, :, None], yg.shape),
                  np.broadcast_to(mask[:, :, None, None], sg.shape))
    assert np.isfinite(yg).all() and np.isfinite(sg).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 6, 7, 8, 9])
def test_seq_persistent(gpu_lib, dtype, T):
    """Grids of 768 slots and more with 16-bit inputs and 128-dimensional
    keys: up to 8 tokens gdn_seq_fwd runs the persistent form of the kernel
    (each workgroup walks tiles of 64 value rows, loading the next tile's
    inputs and state while it runs the current one); 9 tokens take the
    other form.  Also through gdn_chunk_fwd with C = 0 (at this grid the
    sequential kernel for one token, the per-wave chunk kernel from 2)."""
    B, Hk, Hv = 24, 16, 32
    inp = gi.make_inputs(B, T, Hk, Hv, 128, 128, dtype, gate="sigmoid", state_std=0.2, seed=900 + T)
    mask = sampled_slots(B, Hv, 900 + T)
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    yc, sc = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=0)
    torch.cuda.synchronize()
    check_sampled(y, s, inp, mask, dtype, f"seq persistent {dtype} T={T}")
    check_sampled(yc, sc, inp, mask, dtype, f"auto persistent {dtype} T={T}")


@pytest.mark.parametrize("B,Hk,Hv,Dv", [(48, 16, 32, 64), (767, 1, 1, 128), (3, 256, 256, 128)],
                         ids=["dv64_1536slots", "767slots", "768slots"])
def test_seq_persistent_grids(gpu_lib, B, Hk, Hv, Dv):
    """On both sides of the grid-size switch (767 and 768 slots of 128 value
    rows), and with 64 value rows per slot; absent and in-place state."""
    T = 4
    inp = gi.make_inputs(B, T, Hk, Hv, 128, Dv, "bf16", gate="softplus", state_std=0.2, seed=B + Hv + Dv)
    mask = sampled_slots(B, Hv, B * Hv)
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    torch.cuda.synchronize()
    check_sampled(y, s, inp, mask, "bf16", f"seq B={B} Hv={Hv} Dv={Dv} null state", state=False)
    st = d["state"].clone()
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    check_sampled(y, s, inp, mask, "bf16", f"seq B={B} Hv={Hv} Dv={Dv} in place")


@pytest.mark.parametrize("heads,gate", [("tiled", "decay"), ("grouped", "log"), ("tiled", "log")])
def test_seq_persistent_options(gpu_lib, heads, gate):
    """The tiled head map and log-space gates on the persistent form."""
    B, Hk, Hv, T = 24, 16, 32, 5
    inp = gi.make_inputs(B, T, Hk, Hv, 128, 128, "f16", gate="sigmoid", state_std=0.2, seed=77)
    if gate == "log":
        inp = dict(inp)
        inp["g"] = np.log(inp["g"].astype(np.float64)).astype(np.float32)
    mask = sampled_slots(B, Hv, 77)
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], heads=heads, gate=gate)
    torch.cuda.synchronize()
    check_sampled(y, s, inp, mask, "f16", f"seq persistent {heads} {gate}", head_map=heads, gate=gate)
