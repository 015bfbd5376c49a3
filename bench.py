#!/usr/bin/env python3
"""Throughput of the BRA forward pass on one MI355X.

A step is one bra_forward call (region pooling, routing, gather-attention,
LePE) over one batch of seeded synthetic input of the BiFormer stage-1 shape
(B=64, 56x56, C=64, 2 heads of 32, S=7, topk=1, 5x5 LePE) unless --workload
says otherwise.  Inputs are resident in HBM before timing starts.  Several
copies of the batch are rotated so that a step does not find its inputs in
the 256 MB Infinity Cache left there by the previous step.

Prints one JSON line: tokens/s of the whole pass, the attention kernel's
roofline (HIP events on the launch stream), and the fp64 CPU oracle's
throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BRA fwd tokens/s + attention TFLOP/s (% of MI355X bf16 MFMA peak), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20         # Infinity Cache
# sources of the attention kernels (the traffic record is void once they change)
KERNEL_SOURCES = [
    "vision_transformer_dynamic_region_amd/csrc/region_kernels.hip",
    "vision_transformer_dynamic_region_amd/csrc/image_kernels.hip",
    "vision_transformer_dynamic_region_amd/csrc/attend_kernels.hip",
    "vision_transformer_dynamic_region_amd/csrc/device_common.h",
    "vision_transformer_dynamic_region_amd/csrc/fastdiv.h",
]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_traffic.json")
ATTEND_KERNELS = ("attend_region_kernel", "attend_image_kernel", "attend_image_mask_kernel",
                  "attend_stream_kernel", "attend_kernel")
# measured beside the headline workload on the default line
OTHER_WORKLOADS = ("dense", "st2", "st3")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="st1",
                   choices=["tiny", "st1", "st2", "st3", "dense", "video", "video_tiny"])
    p.add_argument("--path", default="bra", choices=["bra", "module", "block", "backward", "video"],
                   help="bra: the BRA forward pass on given Q, K, V (the default line); module: "
                        "the module around it (Q/K/V projections of x, BRA, output projection); "
                        "block: one BiFormer block (position conv, LN, module, LN, MLP); "
                        "backward: gradients of the BRA forward (with LePE) for a fixed index; "
                        "video: BRA on clips of T frames (--workload video)")
    p.add_argument("--sets", type=int, default=0,
                   help="input copies rotated across steps (0: enough to exceed the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="with the default workload, skip the other shapes and the module and block "
                        "timings measured beside it")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of this bench, "
                        "then of --copy-probe-mb 256); writes the attention kernel's HBM traffic "
                        "record and exits (no GPU needed)")
    return p.parse_args()


def _pmc_rows(folder: str):
    """(kernel name, counter, value) of every dispatch in a rocprofv3 csv folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    with open(files[0]) as f:
        return [(r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]))
                for r in csv.DictReader(f)]


def _mean(rows, counter, match):
    vals = [v for k, c, v in rows if c == counter and match(k)]
    if not vals:
        raise SystemExit(f"no {counter} dispatch matched")
    return sum(vals) / len(vals), len(vals)


def write_traffic(a) -> int:
    """HBM bytes per launch of the attention kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a plain
    device copy of 256 MiB (bytes moved / counter bytes)."""
    fetch_dir, write_dir, cf_dir, cw_dir = a.traffic_from
    is_attn = lambda k: any(n in k for n in ATTEND_KERNELS)
    is_copy = lambda k: "copyBuffer" in k or "copy" in k.lower()
    f_kib, nf = _mean(_pmc_rows(fetch_dir), "FETCH_SIZE", is_attn)
    w_kib, nw = _mean(_pmc_rows(write_dir), "WRITE_SIZE", is_attn)
    cf_kib, _ = _mean(_pmc_rows(cf_dir), "FETCH_SIZE", is_copy)
    cw_kib, _ = _mean(_pmc_rows(cw_dir), "WRITE_SIZE", is_copy)
    moved = 256 * 1024 * 1024
    f_scale, w_scale = moved / (cf_kib * 1024), moved / (cw_kib * 1024)
    rec = {
        "workload": a.workload,
        "kernel_sha": kernel_sha(),
        "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib, "dispatches": [nf, nw],
        "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": f_kib * 1024 * f_scale + w_kib * 1024 * w_scale,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def attend_kernel_name(wl) -> str:
    """The attention kernel the library launches for this workload: the
    whole-image 2x2-region kernel (grouped or masked form) for bf16 2x2 /
    top-16 regions (up to 64 of them), the whole-image gather kernel for
    bf16 4x4 regions with top-2, 4 or 8, the per-region kernel for bf16 8x8 regions
    (C 32..128 in heads of 32, top-1, 2 or 4: the stage-1 and dense shapes
    among them), else the pipelined general kernel or, when its routed keys
    or LePE halo do not fit that one, the chunked general kernel."""
    R = wl.S * wl.S
    if (wl.lepe_ks == 5 and wl.dtype == "bf16" and wl.C % 32 == 0 and wl.H // wl.S == 2
            and wl.topk == 16 and R <= 64):
        return "attend_image_mask_kernel"
    if (wl.lepe_ks == 5 and wl.dtype == "bf16" and wl.H // wl.S == 4 and wl.topk in (2, 4, 8)
            and wl.C % 32 == 0):
        return "attend_image_kernel"
    region = (wl.dtype == "bf16" and wl.H // wl.S == 8 and wl.C in (32, 64, 96, 128, 192, 256)
              and wl.C == 32 * wl.heads and wl.topk in (1, 2, 4))
    return "attend_region_kernel" if region and wl.lepe_ks == 5 \
        else "attend_stream_kernel|attend_kernel"


def copy_probe(mb: int) -> None:
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}))


_ORACLE_X = {}


def _oracle_init(name: str) -> None:
    """Oracle baseline process start-up: the same seeded inputs the GPU got
    (the generator is deterministic), BLAS limited to one thread."""
    from threadpoolctl import threadpool_limits

    from vision_transformer_dynamic_region_amd.workloads import WORKLOADS, make_inputs
    threadpool_limits(1)
    wl = WORKLOADS[name]
    _ORACLE_X["wl"], _ORACLE_X["x"] = wl, make_inputs(wl)


def _oracle_images(b: int) -> float:
    """The fp64 oracle on image b of the batch; returns its seconds."""
    import oracle
    wl, x = _ORACLE_X["wl"], _ORACLE_X["x"]
    t0 = time.perf_counter()
    oracle.bra_forward(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], wl.heads, wl.S, wl.topk,
                       x["w"])
    return time.perf_counter() - t0


def cpu_baseline(wl, target_s: float):
    """Time the fp64 oracle as it stands on the host's cores: one process per
    usable core (spawned, each single-threaded, each with its own copy of the
    seeded batch), taking whole images, to about target_s seconds of wall
    time."""
    import concurrent.futures as cf
    import multiprocessing as mp

    cores = max(1, len(os.sched_getaffinity(0)))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx, initializer=_oracle_init,
                                initargs=(wl.name,)) as pool:
        # start-up (interpreter, imports, inputs) outside the timed part
        t_one = max(pool.map(_oracle_images, [b % wl.B for b in range(cores)]))
        n = max(cores, int(target_s * cores / max(t_one, 1e-3)))
        images = [b % wl.B for b in range(n)]
        t0 = time.perf_counter()
        busy = sum(pool.map(_oracle_images, images, chunksize=max(1, n // (4 * cores))))
        dt = time.perf_counter() - t0
    tokens = len(images) * wl.H * wl.W
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{wl.name}: {len(images)} images of the batch (cycling through its {wl.B}), "
                   f"{tokens} tokens, full fp64 oracle in {dt:.1f} s wall on {cores} "
                   f"single-threaded processes ({busy / max(dt * cores, 1e-9):.0%} busy)"),
    }


def module_cpu_baseline(wl, m, target_s: float) -> dict:
    """The fp64 oracle's module_forward as it stands, on the first images of
    the same batch, repeated to about target_s seconds."""
    import oracle

    def run(nb):
        ru0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        oracle.module_forward(m["x"][:nb], m["w_qkv"], m["b_qkv"], wl.heads, wl.S, wl.topk,
                              m["w"], None, m["w_out"], m["b_out"], storage=wl.dtype)
        dt = time.perf_counter() - t0
        ru1 = resource.getrusage(resource.RUSAGE_SELF)
        return dt, (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)

    t1, _ = run(1)
    nb = int(max(1, min(wl.B, target_s / max(t1, 1e-3))))
    dt, cpu, reps = 0.0, 0.0, 0
    while reps == 0 or (nb == wl.B and dt < target_s and reps < 20):
        d, c = run(nb)
        dt, cpu, reps = dt + d, cpu + c, reps + 1
    tokens = nb * wl.H * wl.W * reps
    return {"value": tokens / dt, "unit": "tokens/s", "cores": max(1, int(round(cpu / dt))),
            "kind": "oracle",
            "sample": (f"{wl.name} module: first {nb} of {wl.B} images x {reps} passes "
                       f"({tokens} tokens), fp64 oracle module_forward in {dt:.1f} s")}


def run_module(a, wl) -> int:
    print(json.dumps(module_result(a, wl, cpu=not a.no_cpu_baseline)), flush=True)
    return 0


def module_result(a, wl, cpu: bool) -> dict:
    """One step = bra_module_forward over one batch: pooling of x, float64
    projection of the means, routing, the Q/K/V projection, attention with
    LePE, the output projection."""
    import numpy as np
    import torch

    import vision_transformer_dynamic_region_amd as bra
    from vision_transformer_dynamic_region_amd.workloads import bf16_bits, make_module_inputs

    dev = torch.device("cuda:0")
    m = make_module_inputs(wl)
    if wl.dtype == "bf16":
        up = lambda arr: torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        up = lambda arr: torch.from_numpy(arr).to(dev)
    f32 = lambda arr: torch.from_numpy(arr).to(dev)
    w_qkv, w_out = up(m["w_qkv"]), up(m["w_out"])
    b_qkv, b_out, lw = f32(m["b_qkv"]), f32(m["b_out"]), f32(m["w"])
    x0 = up(m["x"])
    code = 1 if wl.dtype == "bf16" else 0
    wsb = bra.module_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.S, code, True)
    set_bytes = 2 * wl.tensor_bytes + wsb
    sets = a.sets or max(1, -(-3 * MALL_BYTES // set_bytes))
    bufs = [dict(x=x0.clone(), out=torch.empty_like(x0),
                 idx=torch.empty((wl.B, wl.S * wl.S, wl.topk), dtype=torch.int32, device=dev),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=dev)) for _ in range(sets)]
    torch.cuda.synchronize()
    log(f"module: {sets} sets of {set_bytes / 1e6:.1f} MB (x, out, workspace) rotated per step")

    def step(i):
        b = bufs[i % sets]
        bra.module_forward(b["x"], w_qkv, b_qkv, wl.heads, wl.S, wl.topk, lw, None, w_out, b_out,
                           out=b["out"], idx=b["idx"], workspace=b["ws"])

    for i in range(a.warmup):
        step(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    log(f"module: {ms:.4f} ms/step")

    # the Q/K/V projection alone: x read once, Q, K, V written once
    qkv_views = []
    for b in bufs:
        qkv_views.append(torch.empty((wl.B, wl.H, wl.W, 3 * wl.C), dtype=x0.dtype, device=dev))

    def lin_step(i):
        b = bufs[i % sets]
        bra.linear(b["x"], w_qkv, b_qkv, out=qkv_views[i % sets])

    for i in range(a.warmup):
        lin_step(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        lin_step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_lin = e0.elapsed_time(e1) / a.steps
    lin_bytes = 4 * wl.tensor_bytes
    lin_gbs = lin_bytes / (t_lin * 1e-3) / 1e9
    res = {
        "metric": "BRA module fwd tokens/s (x -> QKV projection -> BRA -> output projection), 1 GPU",
        "value": wl.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} module: B={wl.B} H=W={wl.H} C={wl.C} "
                               f"heads={wl.heads} S={wl.S} topk={wl.topk} LePE "
                               f"{wl.lepe_ks}x{wl.lepe_ks}, w_qkv [3C,C], w_out [C,C]",
                   "tokens_per_step": wl.tokens, "input_sets_rotated": sets},
        "stages_ms": {"qkv_linear": t_lin},
        "roofline": {"kernel": "linear_kernel (Q/K/V projection)", "bound": "hbm",
                     "achieved": lin_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": lin_gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes": lin_bytes},
    }
    if cpu:
        log("timing the fp64 oracle module on the host")
        res["cpu_baseline"] = module_cpu_baseline(wl, m, a.cpu_seconds)
    return res


def run_block(a, wl) -> int:
    print(json.dumps(block_result(a, wl, cpu=not a.no_cpu_baseline)), flush=True)
    return 0


def block_result(a, wl, cpu: bool) -> dict:
    """One step = bra_block_forward over one batch."""
    import numpy as np
    import torch

    import vision_transformer_dynamic_region_amd as bra
    from vision_transformer_dynamic_region_amd.workloads import bf16_bits, make_block_inputs

    dev = torch.device("cuda:0")
    p = make_block_inputs(wl)
    if wl.dtype == "bf16":
        up = lambda arr: torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        up = lambda arr: torch.from_numpy(arr).to(dev)
    wdt = {"w_qkv", "w_out", "w_fc1", "w_fc2"}
    params = {n: (up(p[n]) if n in wdt else torch.from_numpy(p[n]).to(dev))
              for n in bra.BLOCK_PARAMS if n != "lepe_ks" and p.get(n) is not None}
    x0 = up(p["x"])
    code = 1 if wl.dtype == "bf16" else 0
    wsb = bra.block_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.S, code)
    set_bytes = 2 * wl.tensor_bytes + wsb
    sets = a.sets or max(1, -(-3 * MALL_BYTES // set_bytes))
    bufs = [dict(x=x0.clone(), out=torch.empty_like(x0),
                 idx=torch.empty((wl.B, wl.S * wl.S, wl.topk), dtype=torch.int32, device=dev),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=dev)) for _ in range(sets)]
    torch.cuda.synchronize()
    log(f"block: {sets} sets of {set_bytes / 1e6:.1f} MB (x, out, workspace) rotated per step")

    def step(i):
        b = bufs[i % sets]
        bra.block_forward(b["x"], params, wl.heads, wl.S, wl.topk, out=b["out"], idx=b["idx"],
                          workspace=b["ws"])

    for i in range(a.warmup):
        step(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    log(f"block: {ms:.4f} ms/step")

    # the largest launch alone: the fused MLP (fc1, GELU, fc2 and the
    # residual; x and r read once, out written once) where it covers the
    # shape, else fc1 with the GELU epilogue ([tokens, C] -> [tokens, 3C])
    fused = wl.dtype == "bf16" and wl.C in (64, 128, 256)
    if fused:
        outs = [torch.empty_like(x0) for _ in range(sets)]

        def big_step(i):
            b = bufs[i % sets]
            bra.mlp(b["x"], params["w_fc1"], params.get("b_fc1"), params["w_fc2"],
                    params.get("b_fc2"), b["x"], out=outs[i % sets])
        big_bytes = 3 * wl.tensor_bytes
        big_name = "mlp_kernel (fc1, GELU, fc2, residual)"
    else:
        hid = [torch.empty((wl.B, wl.H, wl.W, 3 * wl.C), dtype=x0.dtype, device=dev)
               for _ in range(sets)]

        def big_step(i):
            bra.linear(bufs[i % sets]["x"], params["w_fc1"], params["b_fc1"], out=hid[i % sets],
                       act="gelu")
        big_bytes = 4 * wl.tensor_bytes      # x (C) read, hidden (3C) written
        big_name = "linear_kernel (fc1 with GELU)"

    for i in range(a.warmup):
        big_step(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        big_step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_big = e0.elapsed_time(e1) / a.steps
    big_gbs = big_bytes / (t_big * 1e-3) / 1e9
    res = {
        "metric": "BiFormer block fwd tokens/s (pos conv, LN, BRA module, LN, MLP ratio 3), 1 GPU",
        "value": wl.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} block: B={wl.B} H=W={wl.H} C={wl.C} "
                               f"heads={wl.heads} S={wl.S} topk={wl.topk}, MLP 3C",
                   "tokens_per_step": wl.tokens, "input_sets_rotated": sets},
        "stages_ms": {("mlp" if fused else "fc1_gelu"): t_big},
        "roofline": {"kernel": big_name, "bound": "hbm",
                     "achieved": big_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": big_gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes": big_bytes},
    }
    if cpu:
        import oracle as O
        log("timing the fp64 oracle block on the host")
        ru0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        nb, reps = 1, 0
        while time.perf_counter() - t0 < a.cpu_seconds and reps < 50:
            O.block_forward(p["x"][:nb], p, wl.heads, wl.S, wl.topk, storage=wl.dtype)
            reps += 1
        dt = time.perf_counter() - t0
        ru1 = resource.getrusage(resource.RUSAGE_SELF)
        cpu = (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)
        tokens = nb * wl.H * wl.W * reps
        res["cpu_baseline"] = {"value": tokens / dt, "unit": "tokens/s",
                               "cores": max(1, int(round(cpu / dt))), "kind": "oracle",
                               "sample": (f"{wl.name} block: 1 image x {reps} passes ({tokens} "
                                          f"tokens), fp64 oracle block_forward in {dt:.1f} s")}
    return res


def run_backward(a, wl) -> int:
    """One step = bra_attend_backward over one batch (bf16): dQ, dK, dV with
    the LePE term, dw and db, for the routing index that bra_route computes
    from the same Q and K (so the inverse lists see the forward's skew)."""
    import numpy as np
    import torch

    import vision_transformer_dynamic_region_amd as bra
    from vision_transformer_dynamic_region_amd.workloads import bf16_bits, make_backward_inputs

    dev = torch.device("cuda:0")
    x = make_backward_inputs(wl)
    up = lambda arr: torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    q0, k0, v0, g0 = (up(x[n]) for n in ("q", "k", "v", "dout"))
    w = torch.from_numpy(x["w"]).to(dev)
    idx = bra.route(q0, k0, wl.S, wl.topk)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    wsb = int(bra.load().bra_backward_workspace_bytes(B, H, W, C, wl.heads, wl.S, wl.topk,
                                                      wl.lepe_ks))
    tb = B * H * W * C * 2
    set_bytes = 7 * tb + wsb
    sets = a.sets or max(1, -(-3 * MALL_BYTES // set_bytes))
    bufs = [dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), g=g0.clone(),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=dev)) for _ in range(sets)]
    outs = [(torch.empty_like(q0), torch.empty_like(q0), torch.empty_like(q0),
             torch.empty_like(w), torch.empty(C, dtype=torch.float32, device=dev))
            for _ in range(sets)]
    torch.cuda.synchronize()
    log(f"backward: {sets} sets of {set_bytes / 1e6:.1f} MB (q, k, v, dout, dq, dk, dv, "
        f"workspace) rotated per step")
    L = bra.load()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i):
        b, o = bufs[i % sets], outs[i % sets]
        st = L.bra_attend_backward(b["q"].data_ptr(), b["k"].data_ptr(), b["v"].data_ptr(),
                                   idx.data_ptr(), b["g"].data_ptr(), B, H, W, C, wl.heads, wl.S,
                                   wl.topk, 1, wl.d ** -0.5, w.data_ptr(), wl.lepe_ks,
                                   o[0].data_ptr(), o[1].data_ptr(), o[2].data_ptr(),
                                   o[3].data_ptr(), o[4].data_ptr(), b["ws"].data_ptr(), wsb, sp)
        if st != 0:
            raise RuntimeError(L.bra_last_error().decode())

    for i in range(a.warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    log(f"backward: {ms:.4f} ms/step")
    # minimum traffic of the whole pass: q, k, v, dout read once, dq, dk, dv
    # written once (dw, db and the saved statistics are small)
    alg = 7 * tb
    gbs = alg / (ms * 1e-3) / 1e9
    res = {
        "metric": "BRA backward tokens/s (dQ, dK, dV, LePE dw/db; fixed routing), 1 GPU",
        "value": wl.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} backward: B={B} H=W={H} C={C} heads={wl.heads} "
                               f"S={wl.S} topk={wl.topk} LePE {wl.lepe_ks}x{wl.lepe_ks}",
                   "tokens_per_step": wl.tokens, "input_sets_rotated": sets},
        "roofline": {"kernel": "bra_attend_backward (all launches)", "bound": "hbm",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": alg},
    }
    if not a.no_cpu_baseline:
        import oracle as O
        log("timing the fp64 oracle backward on the host")
        idx_h = idx.cpu().numpy()
        ru0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        nb, reps = 1, 0
        while time.perf_counter() - t0 < a.cpu_seconds and reps < 50:
            O.bra_backward(x["q"][:nb], x["k"][:nb], x["v"][:nb], idx_h[:nb], wl.heads, wl.S,
                           x["dout"][:nb], x["w"])
            reps += 1
        dt = time.perf_counter() - t0
        ru1 = resource.getrusage(resource.RUSAGE_SELF)
        cpu = (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)
        tokens = nb * H * W * reps
        res["cpu_baseline"] = {"value": tokens / dt, "unit": "tokens/s",
                               "cores": max(1, int(round(cpu / dt))), "kind": "oracle",
                               "sample": (f"{wl.name} backward: 1 image x {reps} passes ({tokens} "
                                          f"tokens), fp64 oracle bra_backward in {dt:.1f} s")}
    print(json.dumps(res), flush=True)
    return 0


def run_video(a, wl) -> int:
    """One step = bra_video_forward over one batch of clips (routing over
    each clip's T*S*S regions, attention, per-frame LePE)."""
    import numpy as np
    import torch

    import vision_transformer_dynamic_region_amd as bra
    from vision_transformer_dynamic_region_amd.workloads import bf16_bits, make_video_inputs

    dev = torch.device("cuda:0")
    log(f"workload {wl}")
    x = make_video_inputs(wl)
    if wl.dtype == "bf16":
        up = lambda arr: torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        up = lambda arr: torch.from_numpy(arr).to(dev)
    q0, k0, v0 = up(x["q"]), up(x["k"]), up(x["v"])
    w = torch.from_numpy(x["w"]).to(dev)
    R = wl.T * wl.S * wl.S
    wsb = bra.video_workspace_bytes(wl.B, wl.T, wl.S, wl.C)
    set_bytes = 4 * wl.tensor_bytes
    sets = a.sets or max(1, -(-3 * MALL_BYTES // set_bytes))
    bufs = [dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), out=torch.empty_like(q0),
                 idx=torch.empty((wl.B, R, wl.topk), dtype=torch.int32, device=dev),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=dev)) for _ in range(sets)]
    torch.cuda.synchronize()
    log(f"video: {sets} input sets of {set_bytes / 1e6:.1f} MB rotated per step")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for i in range(a.warmup):
            fn(bufs[i % sets])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(a.steps):
            fn(bufs[i % sets])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    ms = timed(lambda b: bra.video_forward(b["q"], b["k"], b["v"], wl.heads, wl.S, wl.topk, w,
                                           out=b["out"], idx=b["idx"], workspace=b["ws"]))
    t_route = timed(lambda b: bra.video_route(b["q"], b["k"], wl.S, wl.topk, workspace=b["ws"]))
    t_attn = timed(lambda b: bra.video_attend(b["q"], b["k"], b["v"], b["idx"], wl.heads, wl.S,
                                              lepe_w=w, out=b["out"]))
    log(f"video: {ms:.4f} ms/step; pool+route {t_route:.4f}, attend+lepe {t_attn:.4f}")
    attn_bytes = 4 * wl.tensor_bytes
    gbs = attn_bytes / (t_attn * 1e-3) / 1e9
    res = {
        "metric": "BRA video fwd tokens/s (T x S x S regions, clip-wide routing, per-frame "
                  "LePE), 1 GPU",
        "value": wl.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} clips x T={wl.T} frames of {wl.H}x{wl.W}, "
                               f"C={wl.C} heads={wl.heads} S={wl.S} ({R} regions a clip) "
                               f"topk={wl.topk} LePE {wl.lepe_ks}x{wl.lepe_ks}",
                   "tokens_per_step": wl.tokens, "input_sets_rotated": sets},
        "stages_ms": {"pool_route": t_route, "attend_lepe": t_attn},
        "roofline": {"kernel": attend_kernel_name(wl), "bound": "hbm", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": attn_bytes},
    }
    if not a.no_cpu_baseline:
        import oracle as O
        log("timing the fp64 oracle video_forward on the host")
        ru0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < a.cpu_seconds and reps < 50:
            O.video_forward(x["q"][:1], x["k"][:1], x["v"][:1], wl.heads, wl.S, wl.topk, x["w"])
            reps += 1
        dt = time.perf_counter() - t0
        ru1 = resource.getrusage(resource.RUSAGE_SELF)
        cpu = (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)
        tokens = wl.T * wl.H * wl.W * reps
        res["cpu_baseline"] = {"value": tokens / dt, "unit": "tokens/s",
                               "cores": max(1, int(round(cpu / dt))), "kind": "oracle",
                               "sample": (f"{wl.name}: 1 clip x {reps} passes ({tokens} tokens), "
                                          f"fp64 oracle video_forward in {dt:.1f} s")}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    a = parse()
    if a.traffic_from:
        return write_traffic(a)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the BRA forward "
              "pass here is a single-GPU kernel path", file=sys.stderr)
        return 2
    import torch

    import vision_transformer_dynamic_region_amd as bra
    from vision_transformer_dynamic_region_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if a.copy_probe_mb:
        copy_probe(a.copy_probe_mb)
        return 0

    if a.path == "video" or a.workload.startswith("video"):
        from vision_transformer_dynamic_region_amd.workloads import VIDEO_WORKLOADS
        if a.path not in ("bra", "video") or not a.workload.startswith("video"):
            print("--path video takes --workload video or video_tiny", file=sys.stderr)
            return 2
        return run_video(a, VIDEO_WORKLOADS[a.workload])
    wl = WORKLOADS[a.workload]
    if a.path == "module":
        return run_module(a, wl)
    if a.path == "block":
        return run_block(a, wl)
    if a.path == "backward":
        return run_backward(a, wl)
    res = measure_bra(a, wl, bra, headline=True)
    if a.workload == "st1" and not a.no_extra:
        # the other bf16 shapes on the same line (the headline stays st1)
        res["other_workloads"] = {n: measure_bra(a, WORKLOADS[n], bra, headline=False)
                                  for n in OTHER_WORKLOADS}
        # the BRA module and the whole BiFormer block on the same shape, each
        # timed the way --path module / --path block time it (no host baseline)
        res["other_paths"] = {}
        for name, fn in (("module", module_result), ("block", block_result)):
            r = fn(a, wl, cpu=False)
            res["other_paths"][name] = {k: r[k] for k in ("metric", "value", "unit",
                                                           "ms_per_step", "config", "stages_ms")}
            torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(wl, a.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def measure_bra(a, wl, bra, headline: bool) -> dict:
    """The BRA forward pass of one workload: the whole pass over rotating
    input sets (mean over exactly a.steps steps, and the median of per-step
    times), the same steps on one input set left in the MALL (warm), and the
    two stages alone (bra_route: pooling and routing; bra_attend: attention
    with LePE), each between HIP events on the launch stream."""
    import numpy as np
    import torch

    from vision_transformer_dynamic_region_amd.workloads import bf16_bits, make_inputs
    dev = torch.device("cuda:0")
    log(f"workload {wl}")
    x = make_inputs(wl)
    if wl.dtype == "bf16":
        up = lambda arr: torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        up = lambda arr: torch.from_numpy(arr).to(dev)
    q0, k0, v0 = up(x["q"]), up(x["k"]), up(x["v"])
    w = torch.from_numpy(x["w"]).to(dev)
    del x
    set_bytes = 4 * wl.tensor_bytes
    sets = a.sets or max(1, -(-3 * MALL_BYTES // set_bytes))
    wsb = bra.workspace_bytes(wl.B, wl.S, wl.C)
    bufs = []
    for i in range(sets):
        bufs.append(dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), out=torch.empty_like(q0),
                         idx=torch.empty((wl.B, wl.S * wl.S, wl.topk), dtype=torch.int32, device=dev),
                         ws=torch.empty(wsb, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    log(f"{sets} input sets of {set_bytes / 1e6:.1f} MB rotated per step")

    def step(i, rotate=True):
        b = bufs[i % sets] if rotate else bufs[0]
        bra.forward(b["q"], b["k"], b["v"], wl.heads, wl.S, wl.topk, w, out=b["out"],
                    idx=b["idx"], workspace=b["ws"])

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {a.warmup} steps done")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(a.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / a.steps
    log(f"timed {a.steps} steps: {ms:.4f} ms/step (wall {wall * 1e3 / a.steps:.4f} ms/step)")

    # per-step times (an event pair around each step) for the median
    pairs = [(ev(), ev()) for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(pairs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    ms_median = float(np.median([e0.elapsed_time(e1) for e0, e1 in pairs]))

    def loop_ms(fn):
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(a.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    # warm: every step on the same input set, which then stays in the MALL
    ms_warm = loop_ms(lambda i: step(i, rotate=False))
    # per stage, each as its own back-to-back loop over the rotating sets
    t_route = loop_ms(lambda i: bra.route(bufs[i % sets]["q"], bufs[i % sets]["k"], wl.S, wl.topk,
                                          workspace=bufs[i % sets]["ws"]))
    t_attn = loop_ms(lambda i: bra.attend(bufs[i % sets]["q"], bufs[i % sets]["k"],
                                          bufs[i % sets]["v"], bufs[i % sets]["idx"], wl.heads,
                                          wl.S, lepe_w=w, out=bufs[i % sets]["out"]))
    t_attn_warm = loop_ms(lambda i: bra.attend(bufs[0]["q"], bufs[0]["k"], bufs[0]["v"],
                                               bufs[0]["idx"], wl.heads, wl.S, lepe_w=w,
                                               out=bufs[0]["out"]))
    log(f"per stage (ms): pool+route {t_route:.4f}  attend+lepe {t_attn:.4f} "
        f"(warm {t_attn_warm:.4f}); step median {ms_median:.4f}, warm {ms_warm:.4f}")
    del bufs
    torch.cuda.empty_cache()

    tokens = wl.tokens
    attn_bytes = 4 * wl.tensor_bytes           # Q, K, V read once + out written once
    attn_gbs = attn_bytes / (t_attn * 1e-3) / 1e9
    attn_tflops = wl.attn_flops / (t_attn * 1e-3) / 1e12
    route_bytes = 2 * wl.tensor_bytes          # Q and K read once
    config = {"workload": f"{wl.name}: B={wl.B} H=W={wl.H} C={wl.C} heads={wl.heads} "
                          f"d={wl.d} S={wl.S} topk={wl.topk} LePE {wl.lepe_ks}x{wl.lepe_ks}",
              "tokens_per_step": tokens, "input_sets_rotated": sets}
    attention = {"kernel": attend_kernel_name(wl), "ms": t_attn, "ms_warm": t_attn_warm,
                 "tflops": attn_tflops, "frac_bf16_peak": attn_tflops / BF16_PEAK_TFLOPS,
                 "gbs": attn_gbs, "frac_hbm": attn_gbs / HBM_PEAK_GBS}
    stages = {"pool_route": t_route, "attend_lepe": t_attn,
              "pool_route_frac_hbm": route_bytes / (t_route * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not headline:
        return {"config": config, "ms_per_step": ms, "ms_per_step_median": ms_median,
                "ms_per_step_warm": ms_warm, "tokens_per_s": tokens / (ms * 1e-3),
                "attention": attention, "stages_ms": stages}

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_sha") == kernel_sha() and rec.get("workload") == wl.name:
            traffic = rec.get("bytes_per_launch")
    return {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "ms_per_step_warm": ms_warm,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": config,
        "attention": attention,
        "stages_ms": stages,
        "roofline": {"kernel": attend_kernel_name(wl), "bound": "hbm", "achieved": attn_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": attn_bytes},
        "kernel_sha": kernel_sha(),
    }


if __name__ == "__main__":
    sys.exit(main())
