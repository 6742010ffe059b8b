"""GPU parity of gdn_step (decode) against the f64 oracle (through the C ABI).

The decode workload chains 256 single-token steps with the state carried in
HBM (state_out of one step is state_in of the next, in place); y of every
step and the final state are compared with the oracle run over the same 256
tokens, on sampled slots.  Also: every dtype and head size, the absent
initial state, and the prefill -> decode hand-over (chunk over T tokens
then one step equals T + 1 tokens).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def chained_steps(gdn, d, state_inplace=True):
    B, T = d["q"].shape[:2]
    st = d["state"].clone() if d["state"] is not None else None
    ys = []
    for t in range(T):
        args = [d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")]
        if st is None:
            y, st = gdn.step(*args, None)
        else:
            y, st = gdn.step(*args, st, state_out=st if state_inplace else None)
        ys.append(y)
    torch.cuda.synchronize()
    return torch.stack(ys, 1), st


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
def test_decode_chained(gpu_lib, gate):
    """The decode workload (256 chained steps, state in HBM) with both
    readings of the printed gate draw: g = exp(-softplus(x)) as printed and
    g = sigmoid(x)."""
    inp = gi.workload_inputs("decode", gate=gate, seed=0 if gate == "softplus" else 1)
    d = upload(inp)
    y, s = chained_steps(gpu_lib, d)
    B, Hv = 64, 32
    mask = np.zeros((B, Hv), bool)
    for b, hv in [(0, 0), (1, 1), (17, 5), (33, 16), (48, 30), (63, 31)]:
        mask[b, hv] = True
    yr, sr = oracle_run(inp, slot_mask=mask)
    yg, sg = to_host_f64(y), to_host_f64(s)
    ymask = np.broadcast_to(mask[:, None, :, None], yg.shape)
    smask = np.broadcast_to(mask[:, :, None, None], sg.shape)
    assert_parity(yg, sg, yr, sr, "f16", f"decode 256 chained steps (6 slots) gate={gate}", ymask, smask)
    assert np.isfinite(yg).all() and np.isfinite(sg).all()
    # the chunk kernel over the same 256 tokens agrees with the oracle too
    yc, sc = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=64)
    torch.cuda.synchronize()
    assert_parity(to_host_f64(yc), to_host_f64(sc), yr, sr, "f16", f"chunk over decode tokens gate={gate}",
                  ymask, smask)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
def test_step_shapes(gpu_lib, dtype, dk, dv):
    inp = gi.make_inputs(3, 5, 2, 4, dk, dv, dtype, gate="sigmoid", state_std=0.1, seed=dk * dv)
    d = upload(inp)
    y, s = chained_steps(gpu_lib, d, state_inplace=False)
    yr, sr = oracle_run(inp)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, dtype, f"step {dtype} Dk={dk} Dv={dv}")


def test_step_null_state(gpu_lib):
    inp = gi.make_inputs(2, 1, 1, 2, 128, 128, "f16", state_std=0.1, seed=2)
    d = upload(inp, state=False)
    y, s = gpu_lib.step(*(d[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta")), None)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp, state=False)
    assert_parity(to_host_f64(y)[:, None], to_host_f64(s), yr, sr, "f16", "step, no initial state")


def test_prefill_then_decode(gpu_lib):
    inp = gi.make_inputs(2, 101, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.05, seed=8)
    d = upload(inp)
    part = lambda x: x[:, :100].contiguous()
    y1, s1 = gpu_lib.chunk_fwd(*(part(d[n]) for n in ("q", "k", "v", "g", "beta")), d["state"], C=64)
    y2, s2 = gpu_lib.step(*(d[n][:, 100].contiguous() for n in ("q", "k", "v", "g", "beta")), s1)
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp)
    y = torch.cat([y1, y2[:, None]], 1)
    assert_parity(to_host_f64(y), to_host_f64(s2), yr, sr, "bf16", "chunk(100) then step")
