"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the oracle, and measure the gap.

The parity metric is max|got - ref| / max|ref|, taken separately on y and on
the final state; the bar is 1e-4 for float32 inputs and 2e-2 for bf16 /
float16 inputs.
"""
from __future__ import annotations

import numpy as np
import torch

import gdn_inputs as gi
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_device(stored: np.ndarray, dtype: str, device="cuda"):
    """Stored numpy array (bf16 carried as uint16) -> torch tensor on device."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(stored)).to(device)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(inp, device="cuda", state=True):
    dt = inp["dtype"]
    d = dict(q=to_device(inp["q"], dt, device), k=to_device(inp["k"], dt, device),
             v=to_device(inp["v"], dt, device),
             g=torch.from_numpy(inp["g"]).to(device),
             beta=torch.from_numpy(inp["beta"]).to(device))
    d["state"] = (torch.from_numpy(inp["state"]).to(device)
                  if (state and inp["state"] is not None) else None)
    return d


def oracle_run(inp, slot_mask=None, state=True, head_map="grouped", gate="decay"):
    """The oracle on stored inputs; with ``gate="log"`` the stored ``g`` is
    taken as the logarithm of the decay."""
    dt = inp["dtype"]
    q, k, v = (gi.decode(inp[n], dt) for n in ("q", "k", "v"))
    s = inp["state"].astype(np.float64) if (state and inp["state"] is not None) else None
    return oracle.forward(q, k, v, inp["g"].astype(np.float64), inp["beta"].astype(np.float64),
                          s, slot_mask=slot_mask, head_map=head_map, gate=gate)


def gap(got: np.ndarray, ref: np.ndarray, mask=None) -> float:
    if mask is not None:
        got, ref = got[mask], ref[mask]
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)


def assert_parity(y_got, s_got, y_ref, s_ref, dtype, what="", y_mask=None, s_mask=None):
    tol = TOL[dtype]
    assert np.all(np.isfinite(y_got)) and np.all(np.isfinite(s_got)), f"{what}: non-finite output"
    ey, es = gap(y_got, y_ref, y_mask), gap(s_got, s_ref, s_mask)
    print(f"[parity] {what}: y {ey:.3e}  state {es:.3e}  (tol {tol:g})", flush=True)
    assert ey <= tol, f"{what}: y gap {ey:.3e} > {tol}"
    assert es <= tol, f"{what}: state gap {es:.3e} > {tol}"
    return ey, es
