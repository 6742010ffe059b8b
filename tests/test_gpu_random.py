"""GPU parity on a seeded random sweep of the option space, against the f64
oracle: 96 cases, each drawn from a fixed seed, mixing entry point
(gdn_chunk_fwd at C = 0, 16, 32, 64, gdn_seq_fwd, chained gdn_step), dtype,
head sizes, grouped-query ratios, head map, gate form (decay or its log,
one per head or one per key dimension), gate distribution, initial state
(given, absent, updated in place), batch and length (ragged tails, chunk
boundaries, lengths the automatic choice sends to either kernel).  Slots
are sampled on the larger grids.  Each case prints its parameters before it
runs.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu

NCASES = 96


def draw_case(i):
    rng = np.random.default_rng([20261, i])
    how = rng.choice(["auto", "c16", "c32", "c64", "seq", "steps"], p=[0.25, 0.15, 0.15, 0.2, 0.15, 0.1])
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.35, 0.2]))
    dk = int(rng.choice([32, 64, 128], p=[0.2, 0.2, 0.6]))
    dv = int(rng.choice([32, 64, 128], p=[0.2, 0.2, 0.6]))
    hk = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 4]))
    b = int(rng.integers(1, 4))
    vector = bool(rng.random() < 0.2)
    if how == "c64" and vector:
        how = "c32"                                  # the vector gate runs chunks of at most 32
    if how == "steps":
        t = int(rng.integers(1, 12))
    elif how == "seq":
        t = int(rng.integers(1, 40))
    else:
        t = int(rng.choice([1, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 129, 200, 333]))
    return dict(
        i=i, how=str(how), dtype=dtype, Dk=dk, Dv=dv, Hk=hk, Hv=hk * group, B=b, T=t,
        heads=str(rng.choice(["grouped", "tiled"])), log=bool(rng.random() < 0.25), vector=vector,
        gate=str(rng.choice(["sigmoid", "softplus", "uniform"])),
        state=str(rng.choice(["given", "absent", "in_place"], p=[0.6, 0.2, 0.2])),
        seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i", range(NCASES))
def test_random_case(gpu_lib, i):
    c = draw_case(i)
    print(f"[case] {c}", flush=True)
    inp = gi.make_inputs(c["B"], c["T"], c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["dtype"], gate=c["gate"],
                         gate_lo=0.9, gate_hi=1.0, state_std=0.2, state=c["state"] != "absent", seed=c["seed"])
    if c["vector"]:
        inp["g"] = gi.vector_gate(c["B"], c["T"], c["Hv"], c["Dk"], seed=c["seed"] + 1, kind="mixed")
    gate = "decay"
    if c["log"]:
        with np.errstate(divide="ignore"):
            inp["g"] = np.log(inp["g"].astype(np.float64)).astype(np.float32)
        gate = "log"
    d = upload(inp, state=c["state"] != "absent")
    kw = dict(heads=c["heads"], gate=gate)
    st_in = d["state"]
    st_out = st_in if c["state"] == "in_place" else None
    how = c["how"]
    if how == "seq":
        y, s = gpu_lib.seq_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st_in, state_out=st_out, **kw)
    elif how == "steps":
        st = st_in.clone() if st_in is not None else None
        ys = []
        for t in range(c["T"]):
            yt, st = gpu_lib.step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")),
                                  st, state_out=st if st is not None else None, **kw)
            ys.append(yt)
        y, s = torch.stack(ys, 1), st
    else:
        C = {"auto": 0, "c16": 16, "c32": 32, "c64": 64}[how]
        y, s = gpu_lib.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st_in, C=C, state_out=st_out, **kw)
    torch.cuda.synchronize()
    if st_out is not None and how != "steps":
        assert s.data_ptr() == st_out.data_ptr()
    yr, sr = oracle_run(inp, state=c["state"] != "absent", head_map=c["heads"], gate=gate)
    assert_parity(to_host_f64(y), to_host_f64(s), yr, sr, c["dtype"], f"random case {i} ({how})")
