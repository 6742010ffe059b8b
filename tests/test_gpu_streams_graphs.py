"""The entry points on non-default HIP streams and under HIP graph capture.

Every launch is enqueued on the caller's stream; the library allocates
nothing and issues no memset, so the calls can be captured in a graph.
Two independent prefills run concurrently on two streams; a graph holding a
prefill and two decode steps is replayed several times, with eager work and
synchronisations between the replays, and every replay is checked.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_testlib import assert_parity, oracle_run, to_host_f64, upload

pytestmark = pytest.mark.gpu


def test_two_streams(gpu_lib):
    a = gi.make_inputs(2, 300, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=61)
    b = gi.make_inputs(1, 77, 2, 6, 64, 64, "f16", gate="softplus", state_std=0.1, seed=62)
    da, db = upload(a), upload(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        ya, sa = gpu_lib.chunk_fwd(da["q"], da["k"], da["v"], da["g"], da["beta"], da["state"], C=64,
                                   stream=s1)
    with torch.cuda.stream(s2):
        yb, sb = gpu_lib.chunk_fwd(db["q"], db["k"], db["v"], db["g"], db["beta"], db["state"], C=0,
                                   stream=s2)
    torch.cuda.synchronize()
    yr, sr = oracle_run(a)
    assert_parity(to_host_f64(ya), to_host_f64(sa), yr, sr, "bf16", "stream 1")
    yr, sr = oracle_run(b)
    assert_parity(to_host_f64(yb), to_host_f64(sb), yr, sr, "f16", "stream 2")


def test_graph_replay(gpu_lib):
    inp = gi.make_inputs(2, 66, 2, 4, 128, 128, "bf16", gate="sigmoid", state_std=0.1, seed=63)
    d = upload(inp)
    T = 64
    pre = {n: d[n][:, :T].contiguous() for n in ("q", "k", "v", "g", "beta")}
    tok = [{n: d[n][:, T + i].contiguous() for n in ("q", "k", "v", "g", "beta")} for i in range(2)]
    s_in = d["state"].clone()
    st = torch.empty_like(s_in)
    y = torch.empty((2, T, 4, 128), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((2, 4, 128), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)

    def work(stream):
        gpu_lib.chunk_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], s_in, C=64,
                          state_out=st, y=y, stream=stream)
        gpu_lib.step(*(tok[0][n] for n in ("q", "k", "v", "g", "beta")), st, state_out=st, y=y1,
                     stream=stream)
        gpu_lib.step(*(tok[1][n] for n in ("q", "k", "v", "g", "beta")), st, state_out=st, y=y2,
                     stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(side)                                  # eager run on the capture stream
    torch.cuda.synchronize()
    y_e, y1_e, y2_e, st_e = y.clone(), y1.clone(), y2.clone(), st.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(torch.cuda.current_stream())
    yr, sr = oracle_run(inp)
    for rep in range(3):
        y.zero_(); y1.zero_(); y2.zero_(); st.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e) and torch.equal(y1, y1_e) and torch.equal(y2, y2_e) and torch.equal(st, st_e), \
            f"replay {rep} differs from the eager run"
        yall = torch.cat([y, y1[:, None], y2[:, None]], 1)
        assert_parity(to_host_f64(yall), to_host_f64(st), yr, sr, "bf16", f"graph replay {rep}")
        _ = (s_in * 2).sum().item()                   # eager work between replays
