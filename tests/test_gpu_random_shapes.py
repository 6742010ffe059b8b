"""GPU parity against the f64 oracle over seeded random combinations of
the options, so that they are also checked together: batch, length (ragged
tails included), head counts with grouped or tiled maps, head sizes, dtype,
chunk length (0 = the library's choice, which may pick the sequential
kernel), gate form (decay, log-decay, per key dimension) and the presence
of an initial state.  The combinations are drawn once from a fixed seed.
"""
import zlib

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def draw_cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = str(rng.choice(["bf16", "f16", "f32"]))
        Dk, Dv = (int(x) for x in rng.choice([32, 64, 128], 2))
        Hk = int(rng.choice([1, 2, 3, 4]))
        Hv = Hk * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 4))
        T = int(rng.choice([1, 2, 5, 13, 16, 31, 33, 64, 77, 130, 200]))
        C = int(rng.choice([0, 16, 32, 64]))
        heads = str(rng.choice(["grouped", "tiled"]))
        gate = str(rng.choice(["decay", "log", "vector"]))
        state = bool(rng.random() < 0.8)
        if B * Hv * T * Dk * Dv > 3e7:
            continue
        cases.append((dt, B, T, Hk, Hv, Dk, Dv, C, heads, gate, state))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_random_shape(gpu_lib, case):
    dt, B, T, Hk, Hv, Dk, Dv, C, heads, gate, state = case
    seed = zlib.crc32(repr(case).encode()) % (2 ** 31)
    inp = gi.make_inputs(B, T, Hk, Hv, Dk, Dv, dt, gate="sigmoid", state_std=0.1, state=state,
                         seed=seed)
    oracle_gate = "decay"
    if gate == "vector":
        inp["g"] = gi.vector_gate(B, T, Hv, Dk, seed=seed + 1, kind="mixed")
    elif gate == "log":
        inp["g"] = np.log(inp["g"].astype(np.float64)).astype(np.float32)
        oracle_gate = "log"
    d = upload(inp)
    y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], C=C, heads=heads,
                             gate="log" if gate == "log" else "decay")
    torch.cuda.synchronize()
    yr, sr = oracle_run(inp, head_map=heads, gate=oracle_gate)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, dt, f"random {case}")
