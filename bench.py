#!/usr/bin/env python
"""Throughput of the gated delta rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one ``gdn_chunk_fwd`` over the long-prefill workload (B=8,
T=8192, Hk=16, Hv=32, Dk=Dv=128, C=64, bf16 q/k/v/y, f32 g/beta/state), with
seeded synthetic inputs already resident in HBM.  W untimed steps, then K
timed steps bracketed by ``torch.cuda.synchronize()``.  The secondary
measurements below (the vector-gate prefill on the same resident inputs,
then decode, a few tokens per call and the small workloads) run first, so
that the timed steps do not start on an idle GPU (its first dozen launches
run about 10-20% slower).  The vector-gate prefill goes first: timed right
before the prefill, its heat made the timed launches about 10% slower at
W = 5.  One JSON line is printed with:

* ``value``       prefill tokens/s (B*T per step);
* ``roofline``    the chunk kernel against the HBM roofline (it is
                  bandwidth-bound at this intensity): algorithmic bytes per
                  launch / average launch time (HIP events on the launch
                  stream), against 8 TB/s; ``traffic`` is the measured HBM
                  bytes per launch from the committed counter summary when it
                  was taken on the current kernel source, else null;
* ``roofline_mfma`` the same launch as algorithmic FLOP/s against the dense
                  bf16 MFMA peak;
* ``decode``      256 ``gdn_step`` launches on the decode workload (B=64,
                  Hk=16, Hv=32, Dk=Dv=128, fp16 I/O, f32 state): state GB/s
                  and total GB/s against 8 TB/s, the roofline from
                  back-to-back steps over 8 state buffers in rotation, so
                  that every state read comes from HBM (each buffer is read
                  once every 8 steps, after some 1.9 GB of other state
                  traffic), and the in-place chain;
* ``vector_gate`` the long prefill with a decay per key dimension (g
                  [B,T,Hv,Dk], seeded U[0.95, 1) on the device): launch time
                  of the pipelined vector-gate chunk kernel (C = 32; 5
                  untimed launches, then 20 timed) and its HBM rate;
* ``multi_token`` T = 2, 4, 8 tokens per call on the decode shapes: the
                  sequential kernel (``gdn_seq_fwd``), the chunked kernel at
                  C = 16 and the library's own choice (C = 0), back to back
                  over 8 state buffers in rotation (state from HBM);
* ``cpu_baseline`` the float64 CPU oracle timed on the same workload (all
                  8 batch elements, all heads, all 8192 tokens: about 40
                  thread-seconds), with the thread count it used; the
                  tiny, Bonsai-shaped and GQA ragged workloads are also
                  timed on one thread.

``--copy-calibration N`` instead times a plain device copy of N MiB (used to
scale the HBM byte counters); it prints its own JSON line.

``--summarize-traffic FETCH WRITE COPY_FETCH COPY_WRITE`` reads four
``rocprofv3 --pmc ... --output-format csv`` result directories (FETCH_SIZE and
WRITE_SIZE of a bench run, and of a ``--copy-calibration 1024`` run), scales
each counter by what it reads for the copy of known size, and writes the
measured HBM bytes per chunk launch to ``profiles/`` together with a hash of
the chunk kernel's source (the figure is only reported for that source).

``--decode-only KIND`` and ``--multi-only T`` run only the decode loop, or
only T tokens per call on the decode shapes with the library's own choice,
for counter collection; ``--summarize-step-traffic`` and
``--summarize-multi-traffic`` turn FETCH_SIZE / WRITE_SIZE runs of them into
HBM bytes per dispatch in ``profiles/`` the same way.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + TFLOP/s (chunk) and state GB/s (step), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
ROTATE = 8                       # state buffers cycled through by the back-to-back timings
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA, TFLOP/s
F32_PEAK_TFLOPS = 157.3          # MI355X dense fp32 MFMA, TFLOP/s
PREFILL = dict(B=8, T=8192, Hk=16, Hv=32, Dk=128, Dv=128, C=64, dtype="bf16")
DECODE = dict(B=64, T=256, Hk=16, Hv=32, Dk=128, Dv=128, dtype="f16")
CHUNK_KERNEL_SOURCES = ["gdn_chunk_wy.h", "gdn_chunk_impl.h", "gdn_chunk_dispatch.h", "gdn_internal.h",
                        "gdn_device.h", "gdn_chunk_bf16.hip"]
# the kernel that runs the long-prefill workload (bf16, Dk = Dv = 128, C = 64)
CHUNK_KERNEL = "chunk_wy_kernel"
CHUNK_KERNEL_LABEL = "chunk_wy_kernel<bf16, 4 state waves> (Dk=Dv=128, C=64)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_long_prefill_hbm_traffic.json")


def chunk_source_hash() -> str:
    h = hashlib.sha256()
    for n in CHUNK_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_deltanet_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_bytes(B, T, Hk, Hv, Dk, Dv, es=2, **_):
    """Algorithmic HBM bytes of one launch: q, k once per key head, v, y,
    g, beta, and the state read once and written once."""
    return (2 * B * T * Hk * Dk * es + 2 * B * T * Hv * Dv * es + 2 * B * T * Hv * 4
            + 2 * B * Hv * Dv * Dk * 4)


def prefill_flops(B, T, Hv, Dk, Dv, C, **_):
    """Algorithmic FLOPs: per token and value head, the three state-sized
    products (6 Dk Dv), the causal halves of K K^T and Q K^T (2 C Dk) and the
    value-side solve plus the intra-chunk term (2 C Dv)."""
    return B * T * Hv * (6 * Dk * Dv + 2 * C * Dk + 2 * C * Dv)


def step_bytes(B, Hk, Hv, Dk, Dv, es=2, **_):
    state = 2 * B * Hv * Dv * Dk * 4
    return state, state + 2 * B * Hk * Dk * es + 2 * B * Hv * Dv * es + 2 * B * Hv * 4


def load_traffic():
    """Measured HBM bytes per chunk launch, if taken on the current source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != chunk_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _counter_means(result_dir, counter):
    """Mean counter value per kernel name from a rocprofv3 csv directory."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(result_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def summarize_traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib=1024):
    kib = copy_mib * 1024.0

    def pick(means, needle):
        hits = [v for k, v in means.items() if needle in k]
        if not hits:
            raise SystemExit(f"no kernel matching {needle!r} in counter results")
        return max(hits)

    copy_fetch = pick(_counter_means(cfetch_dir, "FETCH_SIZE"), "copyBuffer")
    copy_write = pick(_counter_means(cwrite_dir, "WRITE_SIZE"), "copyBuffer")
    f_scale, w_scale = kib / copy_fetch, kib / copy_write
    fetch = pick(_counter_means(fetch_dir, "FETCH_SIZE"), CHUNK_KERNEL)
    write = pick(_counter_means(write_dir, "WRITE_SIZE"), CHUNK_KERNEL)
    rec = {
        "kernel": CHUNK_KERNEL_LABEL + ", long prefill",
        "source_hash": chunk_source_hash(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "copy_calibration_mib": copy_mib,
        "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "read_bytes_per_launch": fetch * f_scale * 1024,
        "write_bytes_per_launch": write * w_scale * 1024,
        "bytes_per_launch": (fetch * f_scale + write * w_scale) * 1024,
        "algorithmic_bytes_per_launch": prefill_bytes(**PREFILL),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


STEP_KERNEL = "step_kernel"
STEP_SOURCES = ["gdn_step.hip", "gdn_device.h", "gdn_internal.h"]


def step_source_hash() -> str:
    h = hashlib.sha256()
    for n in STEP_SOURCES:
        with open(os.path.join(ROOT, "gated_deltanet_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize_step_traffic(kind, fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib=1024):
    """HBM bytes per decode-step dispatch from FETCH_SIZE / WRITE_SIZE runs of
    ``bench.py --decode-only KIND``, each counter scaled by what it reads for a
    plain copy of known size."""
    kib = copy_mib * 1024.0

    def pick(means, needle):
        hits = [v for k, v in means.items() if needle in k]
        if not hits:
            raise SystemExit(f"no kernel matching {needle!r} in counter results")
        return max(hits)

    copy_fetch = pick(_counter_means(cfetch_dir, "FETCH_SIZE"), "copyBuffer")
    copy_write = pick(_counter_means(cwrite_dir, "WRITE_SIZE"), "copyBuffer")
    f_scale, w_scale = kib / copy_fetch, kib / copy_write
    fetch = pick(_counter_means(fetch_dir, "FETCH_SIZE"), STEP_KERNEL)
    write = pick(_counter_means(write_dir, "WRITE_SIZE"), STEP_KERNEL)
    sbytes, tbytes = step_bytes(**DECODE)
    rec = {
        "kernel": "step_kernel<f16>, decode (B=64, Hk=16, Hv=32, Dk=Dv=128)",
        "kind": kind, "source_hash": step_source_hash(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "copy_calibration_mib": copy_mib, "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "read_bytes_per_step": fetch * f_scale * 1024,
        "write_bytes_per_step": write * w_scale * 1024,
        "bytes_per_step": (fetch * f_scale + write * w_scale) * 1024,
        "algorithmic_bytes_per_step": tbytes, "algorithmic_state_bytes_per_step": sbytes,
    }
    path = os.path.join(ROOT, "profiles", f"step_decode_{kind}_hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


WAVE_KERNEL = "chunk_wave_kernel"
WAVE_SOURCES = ["gdn_chunk_wave.h", "gdn_chunk_wy.h", "gdn_chunk_impl.h", "gdn_chunk_dispatch.h",
                "gdn_device.h", "gdn_internal.h", "gdn_chunk_f16.hip"]


def wave_source_hash() -> str:
    h = hashlib.sha256()
    for n in WAVE_SOURCES:
        with open(os.path.join(ROOT, "gated_deltanet_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def multi_bytes(T: int) -> int:
    """Algorithmic HBM bytes of one call of T tokens on the decode shapes: the
    state read and written once, q, k, v, y, g, beta of T tokens."""
    sbytes, tbytes = step_bytes(**DECODE)
    return sbytes + (tbytes - sbytes) * T


def summarize_multi_traffic(T, fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib=1024):
    """HBM bytes per dispatch of the per-wave chunk kernel from FETCH_SIZE /
    WRITE_SIZE runs of ``bench.py --multi-only T``, each counter scaled by what
    it reads for a plain copy of known size."""
    T = int(T)
    kib = copy_mib * 1024.0

    def pick(means, needle):
        hits = [v for k, v in means.items() if needle in k]
        if not hits:
            raise SystemExit(f"no kernel matching {needle!r} in counter results")
        return max(hits)

    copy_fetch = pick(_counter_means(cfetch_dir, "FETCH_SIZE"), "copyBuffer")
    copy_write = pick(_counter_means(cwrite_dir, "WRITE_SIZE"), "copyBuffer")
    f_scale, w_scale = kib / copy_fetch, kib / copy_write
    fetch = pick(_counter_means(fetch_dir, "FETCH_SIZE"), WAVE_KERNEL)
    write = pick(_counter_means(write_dir, "WRITE_SIZE"), WAVE_KERNEL)
    rec = {
        "kernel": f"chunk_wave_kernel<f16>, {T} tokens per call on the decode shapes "
                  "(B=64, Hk=16, Hv=32, Dk=Dv=128), back to back over 8 rotating state buffers",
        "T": T, "source_hash": wave_source_hash(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "copy_calibration_mib": copy_mib, "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "read_bytes_per_call": fetch * f_scale * 1024,
        "write_bytes_per_call": write * w_scale * 1024,
        "bytes_per_call": (fetch * f_scale + write * w_scale) * 1024,
        "algorithmic_bytes_per_call": multi_bytes(T),
    }
    path = os.path.join(ROOT, "profiles", f"wave_multi_token_T{T}_hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def multi_only(T: int, ncalls: int = 256):
    """T tokens per call on the decode shapes with the library's own choice
    (C = 0), back to back over ROTATE state buffers in rotation: every call
    reads its state from HBM and writes it back while later calls run."""
    import numpy as np
    import torch

    import gated_deltanet_prefill_amd as gdn
    import gdn_inputs as gi

    gdn.load()
    dev = torch.device("cuda", 0)
    D = DECODE
    dinp = gi.workload_inputs("decode")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tq, tk, tv, tg, tb = (up(dinp[n][:, :T]) for n in ("q", "k", "v", "g", "beta"))
    st0 = up(dinp["state"])
    ty = torch.empty((D["B"], T, D["Hv"], D["Dv"]), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    rins = [st0.clone() for _ in range(ROTATE)]
    routs = [torch.empty_like(st0) for _ in range(ROTATE)]
    call = lambda i: gdn.chunk_fwd(tq, tk, tv, tg, tb, rins[i % ROTATE], C=0, state_out=routs[i % ROTATE],
                                   y=ty, stream=stream)
    for i in range(ROTATE):                      # warm-up pass
        call(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(ncalls):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / ncalls
    nbytes = multi_bytes(T)
    print(json.dumps({"multi_only": T, "calls": ncalls, "us_per_call": us,
                      "total_GBps": nbytes / (us * 1e-6) / 1e9,
                      "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}), flush=True)


def decode_only(kind: str, nsteps: int):
    """The decode loop alone: 256 chained steps with the state in place, or
    back to back over ROTATE state buffers in rotation (every step then reads
    its state from HBM and its output is written back while later steps
    run)."""
    import numpy as np
    import torch

    import gated_deltanet_prefill_amd as gdn
    import gdn_inputs as gi

    gdn.load()
    dev = torch.device("cuda", 0)
    D = DECODE
    dinp = gi.workload_inputs("decode")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dq, dk, dv, dg, db = (up(dinp[n]) for n in ("q", "k", "v", "g", "beta"))
    st0 = up(dinp["state"])
    nsteps = min(nsteps, D["T"])
    toks = [tuple(t[:, i].contiguous() for t in (dq, dk, dv, dg, db)) for i in range(nsteps)]
    ys = [torch.empty((D["B"], D["Hv"], D["Dv"]), dtype=torch.float16, device=dev) for _ in range(nsteps)]
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if kind == "inplace":
        st = st0.clone()
        for i in range(nsteps):                  # warm-up pass
            gdn.step(*toks[i], st, state_out=st, y=ys[i], stream=stream)
        st.copy_(st0)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(nsteps):
            gdn.step(*toks[i], st, state_out=st, y=ys[i], stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / nsteps
    else:                                        # rotating: every state read from HBM
        rins = [st0.clone() for _ in range(ROTATE)]
        routs = [torch.empty_like(st0) for _ in range(ROTATE)]
        for i in range(nsteps):                  # warm-up pass
            gdn.step(*toks[i], rins[i % ROTATE], state_out=routs[i % ROTATE], y=ys[i], stream=stream)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(nsteps):
            gdn.step(*toks[i], rins[i % ROTATE], state_out=routs[i % ROTATE], y=ys[i], stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / nsteps
    sbytes, tbytes = step_bytes(**D)
    print(json.dumps({"decode_only": kind, "steps": nsteps, "us_per_step": us,
                      "total_GBps": tbytes / (us * 1e-6) / 1e9,
                      "frac": tbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}), flush=True)


def copy_calibration(mib: int):
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    ev0.record()
    for _ in range(reps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    print(json.dumps({"copy_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": ms, "GB/s": 2 * n * 4 / ms / 1e6}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-multi", action="store_true")
    ap.add_argument("--no-vector-gate", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="DIR")
    ap.add_argument("--decode-only", choices=["inplace", "rotating"],
                    help="run only the decode loop of that kind (for counter collection)")
    ap.add_argument("--multi-only", type=int, choices=[2, 4, 8, 16],
                    help="run only T tokens per call on the decode shapes, back to back over rotating "
                         "state buffers (for counter collection)")
    ap.add_argument("--summarize-multi-traffic", nargs=5, metavar=("T", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="summarise FETCH_SIZE / WRITE_SIZE of the per-wave chunk kernel for a "
                         "--multi-only T run")
    ap.add_argument("--summarize-step-traffic", nargs=5, metavar=("KIND", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="summarise FETCH_SIZE / WRITE_SIZE of the decode step kernel for a "
                         "--decode-only KIND run")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_step_traffic:
        summarize_step_traffic(*args.summarize_step_traffic)
        return
    if args.summarize_multi_traffic:
        summarize_multi_traffic(*args.summarize_multi_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); every (batch, head) "
              "slot is independent, so more GPUs would each run this same kernel on their share.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.decode_only:
        decode_only(args.decode_only, args.decode_steps)
        return
    if args.multi_only:
        multi_only(args.multi_only)
        return

    import numpy as np
    import torch

    import gated_deltanet_prefill_amd as gdn
    import gdn_inputs as gi

    gdn.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def upload(arr, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    # ---------------- prefill
    P = PREFILL
    inp = gi.workload_inputs("long_prefill")
    q, k, v = (upload(inp[n], "bf16") for n in ("q", "k", "v"))
    g, beta = upload(inp["g"], "f32"), upload(inp["beta"], "f32")
    s_in = upload(inp["state"], "f32")
    s_out = torch.empty_like(s_in)
    y = torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)

    out = {}
    # ---------------- the long prefill with a decay per key dimension (first:
    # run just before the timed prefill, its heat slowed the first timed
    # launches by some 10%)
    if not args.no_vector_gate:
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        gvec = 0.95 + 0.05 * torch.rand((P["B"], P["T"], P["Hv"], P["Dk"]), generator=gen, device=dev)
        s_vg = torch.empty_like(s_in)
        call = lambda: gdn.chunk_fwd(q, k, v, gvec, beta, s_in, C=32, state_out=s_vg, y=y, stream=stream)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        n = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us_vg = e0.elapsed_time(e1) * 1e3 / n
        vg_bytes = prefill_bytes(**P) + 4 * P["B"] * P["T"] * P["Hv"] * (P["Dk"] - 1)
        out["vector_gate"] = {
            "workload": "long prefill with a decay per key dimension (g [B,T,Hv,Dk] f32, U[0.95,1))",
            "kernel": "chunk_vgp_kernel<bf16>", "C": 32,
            "us_per_launch": us_vg, "tokens_per_s": P["B"] * P["T"] / (us_vg * 1e-6),
            "hbm_GBps": vg_bytes / (us_vg * 1e-6) / 1e9,
            "hbm_frac": vg_bytes / (us_vg * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_launch": vg_bytes,
        }
        del gvec, s_vg
        torch.cuda.empty_cache()

    # ---------------- decode
    if not args.no_decode:
        D = DECODE
        dinp = gi.workload_inputs("decode")
        dq, dk, dv = (upload(dinp[n], "f16") for n in ("q", "k", "v"))
        dg, db = upload(dinp["g"], "f32"), upload(dinp["beta"], "f32")
        st0 = upload(dinp["state"], "f32")
        nsteps = min(args.decode_steps, D["T"])
        toks = [tuple(t[:, i].contiguous() for t in (dq, dk, dv, dg, db)) for i in range(nsteps)]
        ys = [torch.empty((D["B"], D["Hv"], D["Dv"]), dtype=torch.float16, device=dev)
              for _ in range(nsteps)]
        st = st0.clone()

        def run_decode():
            for i in range(nsteps):
                gdn.step(*toks[i], st, state_out=st, y=ys[i], stream=stream)

        run_decode()
        st.copy_(st0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_decode()
        e1.record(stream)
        torch.cuda.synchronize()
        us_step = e0.elapsed_time(e1) * 1e3 / nsteps
        sbytes, tbytes = step_bytes(**D)

        # Back-to-back steps over ROTATE state pairs: step i reads state
        # i % ROTATE and writes its own output buffer, so each state is read
        # once every ROTATE steps, after (ROTATE - 1) x 256 MiB of other state
        # traffic, far more than the 256 MB last-level cache: every read comes
        # from HBM, with no per-step event or flush around the launches.
        rins = [st0.clone() for _ in range(ROTATE)]
        routs = [torch.empty_like(st0) for _ in range(ROTATE)]

        def run_rotating():
            for i in range(nsteps):
                gdn.step(*toks[i], rins[i % ROTATE], state_out=routs[i % ROTATE], y=ys[i], stream=stream)

        run_rotating()
        torch.cuda.synchronize()
        e0.record(stream)
        run_rotating()
        e1.record(stream)
        torch.cuda.synchronize()
        us_rot = e0.elapsed_time(e1) * 1e3 / nsteps
        del rins, routs
        out["decode"] = {
            "workload": "decode", "B": D["B"], "Hk": D["Hk"], "Hv": D["Hv"], "Dk": D["Dk"],
            "Dv": D["Dv"], "dtype": "f16", "chained_steps": nsteps,
            "us_per_step": us_rot,
            "state_GBps": sbytes / (us_rot * 1e-6) / 1e9,
            "total_GBps": tbytes / (us_rot * 1e-6) / 1e9,
            "roofline": {"bound": "hbm", "achieved": tbytes / (us_rot * 1e-6) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": tbytes / (us_rot * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "method": f"{nsteps} back-to-back steps over {ROTATE} state buffers in rotation "
                      "(each state read once every %d steps, after about %.1f GB of other "
                      "state traffic: from HBM), timed together with HIP events"
                      % (ROTATE, (ROTATE - 1) * 2 * sbytes / 1e9),
            "in_place": {
                "us_per_step": us_step,
                "state_GBps": sbytes / (us_step * 1e-6) / 1e9,
                "total_GBps": tbytes / (us_step * 1e-6) / 1e9,
                "frac": tbytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "launches": "plain back-to-back launches, state updated in place",
                "note": "the 128 MiB state fits in the 256 MB last-level cache between steps",
            },
        }
        del toks, ys, st, st0, dq, dk, dv, dg, db

    # ---------------- a few tokens per call (speculative or batched decode)
    if not args.no_multi:
        D = DECODE
        dinp = gi.workload_inputs("decode")
        st0 = upload(dinp["state"], "f32")
        rows = []
        for T in (2, 4, 8):
            tq, tk, tv = (upload(dinp[n][:, :T], "f16") for n in ("q", "k", "v"))
            tg, tb = upload(dinp["g"][:, :T], "f32"), upload(dinp["beta"][:, :T], "f32")
            ty = torch.empty((D["B"], T, D["Hv"], D["Dv"]), dtype=torch.float16, device=dev)
            calls = {"seq": lambda a, b: gdn.seq_fwd(tq, tk, tv, tg, tb, a, state_out=b, y=ty,
                                                     stream=stream),
                     "chunk16": lambda a, b: gdn.chunk_fwd(tq, tk, tv, tg, tb, a, C=16, state_out=b,
                                                           y=ty, stream=stream),
                     "auto": lambda a, b: gdn.chunk_fwd(tq, tk, tv, tg, tb, a, C=0, state_out=b,
                                                        y=ty, stream=stream)}
            row = {"T": T}
            rins = [st0.clone() for _ in range(ROTATE)]
            routs = [torch.empty_like(st0) for _ in range(ROTATE)]
            for name, call in calls.items():
                # back to back over ROTATE state pairs (each state from HBM)
                nr = 4 * ROTATE
                for i in range(ROTATE):
                    call(rins[i], routs[i])
                r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                r0.record(stream)
                for i in range(nr):
                    call(rins[i % ROTATE], routs[i % ROTATE])
                r1.record(stream)
                torch.cuda.synchronize()
                row[f"{name}_us"] = r0.elapsed_time(r1) * 1e3 / nr
            del rins, routs
            sbytes, tbytes = step_bytes(**D)
            ibytes = (tbytes - sbytes) * T             # per-token inputs and outputs
            best = min(row[f"{n}_us"] for n in calls)
            row["tokens_per_s"] = D["B"] * T / (row["auto_us"] * 1e-6)
            row["hbm_frac_auto"] = (sbytes + ibytes) / (row["auto_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
            row["auto_vs_best"] = row["auto_us"] / best
            rows.append(row)
            del tq, tk, tv, tg, tb, ty
        del st0
        out["multi_token"] = {
            "workload": "decode shapes, T tokens per call", "B": D["B"], "Hk": D["Hk"],
            "Hv": D["Hv"], "Dk": D["Dk"], "Dv": D["Dv"], "dtype": "f16",
            "rows": rows,
            "method": f"{4 * ROTATE} back-to-back calls over {ROTATE} state buffers in rotation "
                      "(each state read from HBM once every %d calls, each output written back "
                      "while later calls run), timed together with HIP events" % ROTATE,
            "hbm_bytes": "state read + write once per call plus q, k, v, y, g, beta of T tokens",
        }

    # ---------------- the other prefill workloads (parity-test cases): times only
    if not args.no_configs:
        rows = []
        for name in ("tiny_f32", "bonsai_prefill", "gqa_ragged"):
            W = gi.WORKLOADS[name]
            winp = gi.workload_inputs(name)
            dt = W["dtype"]
            wq, wk, wv = (upload(winp[n], dt) for n in ("q", "k", "v"))
            wg, wb = upload(winp["g"], "f32"), upload(winp["beta"], "f32")
            ws = upload(winp["state"], "f32") if winp["state"] is not None else None
            wso = torch.empty((W["B"], W["Hv"], W["Dv"], W["Dk"]), dtype=torch.float32, device=dev)
            wy = torch.empty_like(wv)
            es = 4 if dt == "f32" else 2
            row = {"workload": name, "B": W["B"], "T": W["T"], "Hk": W["Hk"], "Hv": W["Hv"],
                   "Dk": W["Dk"], "Dv": W["Dv"], "dtype": dt}
            for label, C in (("named_C", W["C"]), ("auto", 0)):
                # 50 launches captured in one HIP graph and replayed, so that the
                # time is the GPU's and not the host's per-call overhead
                call = lambda: gdn.chunk_fwd(wq, wk, wv, wg, wb, ws, C=C, state_out=wso, y=wy)
                side = torch.cuda.Stream(dev)
                side.wait_stream(torch.cuda.current_stream(dev))
                with torch.cuda.stream(side):
                    for _ in range(3):
                        call()
                torch.cuda.current_stream(dev).wait_stream(side)
                torch.cuda.synchronize()
                n = 50
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for _ in range(n):
                        call()
                for _ in range(3):
                    graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                row[f"{label}_us"] = e0.elapsed_time(e1) * 1e3 / n
                del graph
            row["C"] = W["C"]
            sec = row["named_C_us"] * 1e-6
            nb = prefill_bytes(**W, es=es)
            nf = prefill_flops(**W)
            row["tokens_per_s"] = W["B"] * W["T"] / sec
            row["hbm_frac"] = nb / sec / 1e9 / HBM_PEAK_GBS
            row["mfma_frac"] = nf / sec / 1e12 / (F32_PEAK_TFLOPS if dt == "f32" else BF16_PEAK_TFLOPS)
            rows.append(row)
            del wq, wk, wv, wg, wb, ws, wso, wy
        out["configs"] = {
            "rows": rows,
            "method": "50 launches captured in a HIP graph, replayed after 3 warm-up replays, "
                      "HIP events around one replay; at the workload's named C and with the automatic choice (C = 0); fractions at "
                      "the named C against HBM and against the MFMA peak of the input dtype",
        }

    # ---------------- the timed long prefill (last, on a settled clock)
    def step():
        gdn.chunk_fwd(q, k, v, g, beta, s_in, C=P["C"], state_out=s_out, y=y, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms_per_step = wall * 1e3 / args.steps
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    tokens = P["B"] * P["T"]
    nbytes = prefill_bytes(**P)
    nflops = prefill_flops(**P)
    achieved_gbs = nbytes / avg_launch_s / 1e9
    traffic = load_traffic()

    out.update({
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), g U[0.95,1), "
                "beta sigmoid(N(0,1)), state N(0,0.05))",
        "config": {"workload": "long_prefill", "B": P["B"], "T": P["T"], "Hk": P["Hk"],
                   "Hv": P["Hv"], "Dk": P["Dk"], "Dv": P["Dv"], "C": P["C"]},
        "roofline": {
            "kernel": CHUNK_KERNEL_LABEL,
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes,
            "launch_us_avg": avg_launch_s * 1e6,
            "launch_us_min": min(launch_ms) * 1e3,
        },
        "roofline_mfma": {
            "achieved": nflops / avg_launch_s / 1e12,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": nflops / avg_launch_s / 1e12 / BF16_PEAK_TFLOPS,
            "algorithmic_flops_per_launch": nflops,
        },
    })
    if "vector_gate" in out:
        out["vector_gate"]["vs_scalar_gate"] = out["vector_gate"]["us_per_launch"] / out["roofline"]["launch_us_avg"]
    del q, k, v, g, beta, y, s_out
    torch.cuda.empty_cache()

    # ---------------- CPU oracle on a bounded sample
    if not args.no_cpu_baseline:
        import oracle
        nthreads = len(os.sched_getaffinity(0))
        nb = P["B"]                              # the whole long prefill
        qs, ks, vs = (gi.decode(inp[n][:nb], "bf16") for n in ("q", "k", "v"))
        gs, bs = inp["g"][:nb].astype(np.float64), inp["beta"][:nb].astype(np.float64)
        ss = inp["state"][:nb].astype(np.float64)
        t0 = time.perf_counter()
        oracle.forward(qs, ks, vs, gs, bs, ss, nthreads=nthreads)
        cpu_s = time.perf_counter() - t0
        # the three small prefill workloads on one thread each
        single = []
        for name in ("tiny_f32", "bonsai_prefill", "gqa_ragged"):
            W = gi.WORKLOADS[name]
            winp = gi.workload_inputs(name)
            wq, wk, wv = (gi.decode(winp[n], W["dtype"]) for n in ("q", "k", "v"))
            ws = winp["state"].astype(np.float64) if winp["state"] is not None else None
            t1 = time.perf_counter()
            oracle.forward(wq, wk, wv, winp["g"].astype(np.float64), winp["beta"].astype(np.float64),
                           ws, nthreads=1)
            sec = time.perf_counter() - t1
            single.append({"workload": name, "threads": 1, "seconds": sec,
                           "tokens_per_s": W["B"] * W["T"] / sec})
        out["cpu_baseline"] = {
            "value": nb * P["T"] / cpu_s, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"the whole long prefill, {nb} x {P['T']} tokens x {P['Hv']} value heads "
                      f"(float64 sequential rule, OpenMP over (batch, head) slots), {cpu_s:.2f} s "
                      f"on {nthreads} threads",
            "single_thread": single,
        }
    head = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")
    ordered = {key: out[key] for key in head if key in out}
    ordered.update({key: val for key, val in out.items() if key not in ordered})
    print(json.dumps(ordered), flush=True)


if __name__ == "__main__":
    main()
