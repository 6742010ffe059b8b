"""GPU parity at sizes whose element offsets pass 2^31 (64-bit indexing):
the long-prefill shape at B = 64 (y and v hold 2^31 elements, 4 GiB each in
bf16) through the pipelined chunk kernel, and the decode shapes at B = 4096
through the sequential kernel and the step (an 8 GiB state); and the long
prefill at its full size with a decay per key dimension, and with nearly
parallel keys.  Inputs are drawn on the device from a seeded generator; the
oracle checks the last (batch, head) slots, whose offsets are the largest,
and one early slot.
"""
import numpy as np
import pytest
import torch

import oracle
from gdn_testlib import assert_parity

pytestmark = pytest.mark.gpu


def device_inputs(B, T, Hk, Hv, D, dtype, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = torch.nn.functional.normalize(torch.randn((B, T, Hk, D), generator=gen, device="cuda"), dim=-1).to(dtype)
    k = torch.nn.functional.normalize(torch.randn((B, T, Hk, D), generator=gen, device="cuda"), dim=-1).to(dtype)
    v = torch.randn((B, T, Hv, D), generator=gen, device="cuda").to(dtype)
    g = 0.95 + 0.05 * torch.rand((B, T, Hv), generator=gen, device="cuda")
    beta = torch.sigmoid(torch.randn((B, T, Hv), generator=gen, device="cuda"))
    s0 = 0.05 * torch.randn((B, Hv, D, D), generator=gen, device="cuda")
    return q, k, v, g, beta, s0


def check_slots(q, k, v, g, beta, s0, y, s, slots, dt):
    B, T, Hk, D = q.shape
    Hv = v.shape[2]
    for b, hv in slots:
        hk = hv // (Hv // Hk)
        f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
        yr, sr = oracle.forward(f64(q[b:b + 1, :, hk:hk + 1]), f64(k[b:b + 1, :, hk:hk + 1]),
                                f64(v[b:b + 1, :, hv:hv + 1]), f64(g[b:b + 1, :, hv:hv + 1]),
                                f64(beta[b:b + 1, :, hv:hv + 1]), f64(s0[b:b + 1, hv:hv + 1]))
        assert_parity(f64(y[b:b + 1, :, hv:hv + 1]), f64(s[b:b + 1, hv:hv + 1]), yr, sr, dt,
                      f"B={B} T={T} slot ({b}, {hv})")


def test_long_prefill_b64(gpu_lib):
    B, T, Hk, Hv, D = 64, 8192, 16, 32, 128
    q, k, v, g, beta, s0 = device_inputs(B, T, Hk, Hv, D, torch.bfloat16, seed=11)
    assert v.numel() == 2 ** 31
    y, s = gpu_lib.chunk_fwd(q, k, v, g, beta, s0, C=64)
    torch.cuda.synchronize()
    assert torch.isfinite(s).all()
    check_slots(q, k, v, g, beta, s0, y, s, [(63, 31), (63, 17), (2, 5)], "bf16")
    del q, k, v, g, beta, s0, y, s
    torch.cuda.empty_cache()


def test_decode_b4096(gpu_lib):
    B, T, Hk, Hv, D = 4096, 3, 16, 32, 128
    q, k, v, g, beta, s0 = device_inputs(B, T, Hk, Hv, D, torch.float16, seed=12)
    assert s0.numel() >= 2 ** 31
    y, s = gpu_lib.seq_fwd(q, k, v, g, beta, s0)
    st = s0.clone()
    ys = []
    for t in range(T):
        yt, st = gpu_lib.step(*(x[:, t].contiguous() for x in (q, k, v, g, beta)), st, state_out=st)
        ys.append(yt)
    torch.cuda.synchronize()
    slots = [(4095, 31), (4095, 0), (7, 9)]
    check_slots(q, k, v, g, beta, s0, y, s, slots, "f16")
    check_slots(q, k, v, g, beta, s0, torch.stack(ys, 1), st, slots, "f16")
    del q, k, v, g, beta, s0, y, s, st, ys
    torch.cuda.empty_cache()


def test_vector_gate_long_prefill(gpu_lib):
    """The long prefill with a decay per key dimension in the launch
    configuration the bench times (C = 32, one workgroup per slot), checked
    on sampled slots over all 8192 tokens."""
    B, T, Hk, Hv, D = 8, 8192, 16, 32, 128
    q, k, v, g, beta, s0 = device_inputs(B, T, Hk, Hv, D, torch.bfloat16, seed=13)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(14)
    gvec = 0.95 + 0.05 * torch.rand((B, T, Hv, D), generator=gen, device="cuda")
    y, s = gpu_lib.chunk_fwd(q, k, v, gvec, beta, s0, C=32)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(s).all()
    check_slots(q, k, v, gvec, beta, s0, y, s, [(7, 31), (3, 16), (0, 1)], "bf16")
    del q, k, v, g, gvec, beta, s0, y, s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_long_prefill_correlated_keys(gpu_lib, dtype):
    """The long prefill (B = 8, T = 8192, Hk = 16, Hv = 32, C = 64, the
    launch configuration the bench times) with nearly parallel keys: every
    key of a (batch, key head) is normalise(k_0 sqrt(Dk) + 0.1 n_t) with one
    shared unit direction k_0, beta = 0.99 and no decay, so each chunk's
    triangular system nearly cancels and nothing is forgotten over 128
    chunks.  Whatever error the chunk solve leaves would build up here; the
    sampled slots must still meet the tolerance of their dtype over all
    8192 tokens."""
    B, T, Hk, Hv, D = 8, 8192, 16, 32, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    q = torch.nn.functional.normalize(torch.randn((B, T, Hk, D), generator=gen, device="cuda"), dim=-1).to(dtype)
    k0 = torch.nn.functional.normalize(torch.randn((B, 1, Hk, D), generator=gen, device="cuda"), dim=-1) * D ** 0.5
    k = torch.nn.functional.normalize(k0 + 0.1 * torch.randn((B, T, Hk, D), generator=gen, device="cuda"),
                                      dim=-1).to(dtype)
    del k0
    v = torch.randn((B, T, Hv, D), generator=gen, device="cuda").to(dtype)
    g = torch.ones((B, T, Hv), device="cuda")
    beta = torch.full((B, T, Hv), 0.99, device="cuda")
    s0 = 0.05 * torch.randn((B, Hv, D, D), generator=gen, device="cuda")
    y, s = gpu_lib.chunk_fwd(q, k, v, g, beta, s0, C=64)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(s).all()
    dt = "bf16" if dtype == torch.bfloat16 else "f16"
    check_slots(q, k, v, g, beta, s0, y, s, [(7, 31), (3, 16), (0, 1)], dt)
    del q, k, v, g, beta, s0, y, s
    torch.cuda.empty_cache()
