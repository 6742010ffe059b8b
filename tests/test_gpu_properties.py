"""Properties of the method that hold at any size, checked on the GPU
without the oracle, bitwise:

- permuting the value index (columns of v, rows of the initial state)
  permutes y and the final state the same way: each value row of the state
  evolves on its own, from the shared keys, queries and gates;
- every (batch, value-head) slot is computed on its own: the first batch
  element of a B = 3 call equals a B = 1 call on its inputs, even where the
  grid, the value-slice split or the slot order differ.

Every kernel is covered: pipelined (C = 64), generic (C = 16 and 32, with
and without value slices), vector gate, sequential, decode step.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def inputs(B, T, Hk, Hv, D, dtype, vector=False, seed=0):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = torch.nn.functional.normalize(torch.randn((B, T, Hk, D), generator=gen, device="cuda"), dim=-1).to(dtype)
    k = torch.nn.functional.normalize(torch.randn((B, T, Hk, D), generator=gen, device="cuda"), dim=-1).to(dtype)
    v = torch.randn((B, T, Hv, D), generator=gen, device="cuda").to(dtype)
    gshape = (B, T, Hv, D) if vector else (B, T, Hv)
    g = 0.8 + 0.2 * torch.rand(gshape, generator=gen, device="cuda")
    beta = torch.sigmoid(torch.randn((B, T, Hv), generator=gen, device="cuda"))
    s0 = 0.1 * torch.randn((B, Hv, D, D), generator=gen, device="cuda")
    return q, k, v, g, beta, s0


def run(gdn, how, q, k, v, g, beta, s0):
    if how == "seq":
        return gdn.seq_fwd(q, k, v, g, beta, s0)
    if how == "step":
        return gdn.step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(),
                        g[:, 0].contiguous(), beta[:, 0].contiguous(), s0)
    return gdn.chunk_fwd(q, k, v, g, beta, s0, C=how)


KERNELS = [
    # (how, B, T, Hk, Hv, D, dtype, vector gate)
    (64, 3, 150, 2, 4, 128, torch.bfloat16, False),    # pipelined
    (32, 3, 70, 2, 4, 128, torch.bfloat16, False),     # generic, value slices (12 slots)
    (16, 3, 70, 4, 64, 128, torch.float16, False),     # generic, 192 slots: no slices
    (16, 3, 45, 2, 4, 64, torch.float32, False),       # generic f32
    (32, 3, 70, 2, 4, 128, torch.bfloat16, True),      # vector gate, value slices
    ("seq", 3, 9, 2, 4, 128, torch.float16, False),
    ("seq", 3, 5, 2, 4, 128, torch.bfloat16, True),
    ("step", 3, 1, 2, 4, 128, torch.float16, False),
    ("step", 3, 1, 2, 4, 64, torch.float32, True),
]


@pytest.mark.parametrize("case", KERNELS, ids=lambda c: f"{c[0]}-Hv{c[4]}-D{c[5]}-{str(c[6])[6:]}{'-vg' if c[7] else ''}")
def test_value_permutation(gpu_lib, case):
    how, B, T, Hk, Hv, D, dtype, vector = case
    q, k, v, g, beta, s0 = inputs(B, T, Hk, Hv, D, dtype, vector, seed=1)
    perm = torch.randperm(D, generator=torch.Generator().manual_seed(2)).cuda()
    y, s = run(gpu_lib, how, q, k, v, g, beta, s0)
    yp, sp = run(gpu_lib, how, q, k, v[..., perm].contiguous(), g, beta, s0[:, :, perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(yp, y[..., perm]), f"{case}: y does not follow the value permutation"
    assert torch.equal(sp, s[:, :, perm]), f"{case}: state does not follow the value permutation"


@pytest.mark.parametrize("case", KERNELS, ids=lambda c: f"{c[0]}-Hv{c[4]}-D{c[5]}-{str(c[6])[6:]}{'-vg' if c[7] else ''}")
def test_slot_independence(gpu_lib, case):
    how, B, T, Hk, Hv, D, dtype, vector = case
    q, k, v, g, beta, s0 = inputs(B, T, Hk, Hv, D, dtype, vector, seed=3)
    y, s = run(gpu_lib, how, q, k, v, g, beta, s0)
    one = [x[:1].contiguous() for x in (q, k, v, g, beta, s0)]
    y1, s1 = run(gpu_lib, how, *one)
    torch.cuda.synchronize()
    assert torch.equal(y1, y[:1]), f"{case}: batch element 0 depends on the others"
    assert torch.equal(s1, s[:1]), f"{case}: batch element 0 depends on the others"
