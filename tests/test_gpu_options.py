"""GPU parity of the _ex entry points' options against the f64 oracle: the
tiled head map (key head hv mod Hk) and log-space gates (decay = exp(g)),
alone and together, on every kernel: the pipelined chunk kernel (bf16,
Dk = Dv = 128, C = 64, with the XCD-grouped slot order), the generic chunk
kernel (other sizes, f32), the sequential kernel and the decode step.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu

OPTIONS = [("tiled", "decay"), ("grouped", "log"), ("tiled", "log")]


def with_log_gate(inp):
    inp = dict(inp)
    with np.errstate(divide="ignore"):
        inp["g"] = np.log(inp["g"].astype(np.float64)).astype(np.float32)
    return inp


def prepare(inp, gate):
    return with_log_gate(inp) if gate == "log" else inp


@pytest.mark.parametrize("heads,gate", OPTIONS)
@pytest.mark.parametrize("case", ["pipe", "generic_c16", "generic_dk64", "f32"])
def test_chunk_options(gpu_lib, heads, gate, case):
    shape = {"pipe": (2, 150, 4, 16, 128, 128, "bf16", 64),
             "generic_c16": (2, 70, 2, 6, 128, 128, "bf16", 16),
             "generic_dk64": (3, 45, 2, 4, 64, 128, "f16", 32),
             "f32": (2, 40, 2, 4, 64, 64, "f32", 16)}[case]
    B, T, Hk, Hv, Dk, Dv, dt, C = shape
    inp = prepare(gi.make_inputs(B, T, Hk, Hv, Dk, Dv, dt, gate="sigmoid", state_std=0.1,
                                 seed=7 + T), gate)
    d = upload(inp)
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C,
                             heads=heads, gate=gate)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp, head_map=heads, gate=gate)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, dt, f"chunk {case} {heads} {gate}")


@pytest.mark.parametrize("heads,gate", OPTIONS)
@pytest.mark.parametrize("B", [2, 16])
def test_seq_options(gpu_lib, heads, gate, B):
    inp = prepare(gi.make_inputs(B, 9, 4, 16, 128, 128, "bf16", gate="sigmoid", state_std=0.1,
                                 seed=B), gate)
    d = upload(inp)
    y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                           heads=heads, gate=gate)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp, head_map=heads, gate=gate)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "bf16", f"seq B={B} {heads} {gate}")


@pytest.mark.parametrize("heads,gate", OPTIONS)
def test_step_options(gpu_lib, heads, gate):
    inp = prepare(gi.make_inputs(3, 6, 2, 6, 64, 128, "f16", gate="sigmoid", state_std=0.1,
                                 seed=3), gate)
    d = upload(inp)
    st = d["state"].clone()
    ys = []
    for t in range(6):
        y, st = gpu_lib.step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), st,
                             state_out=st, heads=heads, gate=gate)
        ys.append(y)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp, head_map=heads, gate=gate)
    assert_parity(to_host_f64(torch.stack(ys, 1)), to_host_f64(st), yr, sr, "f16",
                  f"step {heads} {gate}")


def test_log_gate_limits(gpu_lib):
    """Log gates of 0 (keep the state), -inf (forget it) and -100 (a decay
    that underflows float32) through every kernel."""
    inp = gi.make_inputs(2, 70, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=12)
    inp = with_log_gate(inp)
    inp["g"][:, 0:10] = 0.0
    inp["g"][:, 10] = -np.inf
    inp["g"][:, 20:23] = -100.0
    inp["g"][1, 40:] = 0.0
    d = upload(inp)
    yr, sr = oracle_run(inp, gate="log")
    for name, fn in (("chunk64", lambda: gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                           d["state"], C=64, gate="log")),
                     ("chunk16", lambda: gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                           d["state"], C=16, gate="log")),
                     ("seq", lambda: gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                     d["state"], gate="log"))):
        y, s = fn()
        torch.cuda.synchronize()
        assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, "bf16", f"log limits {name}")


def test_tiled_equals_grouped_when_maps_agree(gpu_lib):
    """Hk == Hv: both maps are the identity, and the kernels give bitwise
    the same results."""
    inp = gi.make_inputs(2, 100, 4, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=2)
    d = upload(inp)
    for C in (16, 64):
        a = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C)
        b = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C,
                              heads="tiled")
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
