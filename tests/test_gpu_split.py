"""GPU parity of the chunk kernels' value-slice split against the f64
oracle.  With few (batch, value-head) slots the generic kernel runs Dv / DVS
workgroups per slot (4 or 2 slices of the value columns, each recomputing
the chunk's C x C work), and the pipelined 64-token kernel (16-bit inputs,
Dk = Dv = 128) four workgroups of 32 value rows; the cases sit on both
sides of every slot-count threshold of the split, with ragged lengths,
grouped and tiled heads, Dk != Dv and every dtype.  Large grids are checked
on sampled slots.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu

# (dtype, B, Hk, Hv, Dk, Dv, C, T, value slices expected)
CASES = [
    ("bf16", 1, 8, 8, 128, 128, 32, 45, 4),
    ("bf16", 3, 4, 8, 128, 128, 32, 70, 4),     # 24 slots, grouped heads
    ("bf16", 5, 5, 5, 128, 128, 32, 45, 2),     # 25 slots
    ("bf16", 12, 16, 32, 128, 128, 32, 40, 2),  # 384 slots
    ("bf16", 5, 7, 77, 128, 128, 32, 40, 1),    # 385 slots
    ("bf16", 2, 4, 8, 128, 128, 16, 37, 4),     # 16 slots
    ("bf16", 1, 17, 17, 128, 128, 16, 37, 2),   # 17 slots
    ("bf16", 4, 8, 32, 128, 128, 16, 50, 2),    # 128 slots
    ("bf16", 3, 43, 43, 128, 128, 16, 20, 1),   # 129 slots
    ("f16", 2, 3, 3, 64, 128, 32, 33, 4),       # Dk != Dv
    ("f16", 4, 16, 16, 64, 64, 16, 41, 2),      # Dv = 64, 64 slots
    ("f16", 5, 13, 13, 64, 64, 16, 41, 1),      # 65 slots
    ("f32", 2, 8, 64, 128, 128, 16, 35, 2),     # 128 slots
    ("f32", 1, 3, 129, 128, 128, 16, 35, 1),    # 129 slots (Hv / Hk = 43)
    ("f32", 1, 4, 8, 128, 128, 32, 35, 1),      # C = 32 is not split in f32
    # the pipelined kernel (C = 64)
    ("bf16", 1, 8, 8, 128, 128, 64, 150, 4),    # 8 slots
    ("bf16", 2, 16, 32, 128, 128, 64, 200, 4),  # 64 slots, grouped heads
    ("bf16", 5, 13, 13, 128, 128, 64, 130, 1),  # 65 slots
    ("bf16", 3, 11, 22, 128, 128, 64, 70, 1),   # 66 slots, grouped heads
    ("f16", 1, 3, 3, 128, 128, 64, 129, 4),     # 3 slots
    ("f16", 4, 8, 16, 128, 128, 64, 77, 4),     # 64 slots
    ("f16", 1, 5, 65, 128, 128, 64, 64, 1),     # 65 slots (Hv / Hk = 13)
]


def expected_split(dt, Dk, Dv, C, slots):
    """The slot-count rule of the dispatcher, restated for the cases above."""
    if C == 64 and dt != "f32" and Dk == 128 and Dv == 128:
        return 4 if slots <= 64 else 1
    if Dv == 128:
        if dt == "f32":
            return 2 if (C == 16 and slots <= 128) else 1
        if C == 32:
            return 4 if slots <= 24 else 2 if slots <= 384 else 1
        if C == 16:
            return 4 if slots <= 16 else 2 if slots <= 128 else 1
        return 1
    return 2 if (Dv == 64 and dt != "f32" and C == 16 and slots <= 64) else 1


@pytest.mark.parametrize("heads", ["grouped", "tiled"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}-Hk{c[2]}-Hv{c[3]}-D{c[4]}x{c[5]}-C{c[6]}-T{c[7]}")
def test_split(gpu_lib, case, heads):
    dt, B, Hk, Hv, Dk, Dv, C, T, nsplit = case
    assert expected_split(dt, Dk, Dv, C, B * Hv) == nsplit
    if heads == "tiled" and Hk == Hv:
        pytest.skip("the two head maps coincide when Hk = Hv")
    inp = gi.make_inputs(B, T, Hk, Hv, Dk, Dv, dt, gate="sigmoid", state_std=0.1, seed=B * 1000 + Hv + T)
    d = upload(inp)
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C, heads=heads)
    torch.cuda.synchronize()
    mask = None
    if B * Hv > 64:
        rng = np.random.default_rng(B * Hv)
        mask = np.zeros((B, Hv), bool)
        mask.reshape(-1)[rng.choice(B * Hv, 12, replace=False)] = True
        mask[-1, -1] = True
    yr, sr = oracle_run(inp, slot_mask=mask, head_map=heads)
    ym = None if mask is None else np.broadcast_to(mask[:, None, :, None], yr.shape)
    sm = None if mask is None else np.broadcast_to(mask[:, :, None, None], sr.shape)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, dt,
                  f"split x{nsplit} {dt} B={B} Hk={Hk} Hv={Hv} D={Dk}x{Dv} C={C} T={T} {heads}",
                  y_mask=ym, s_mask=sm)
