"""Routed-expert FP8 MoE decode benchmark: us per layer and achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3] [--M 4]

One step = one moe_decode_run (routing, activation quant, GEMM1, SwiGLU +
requant, GEMM2, combine) on resident synthetic inputs. Before every step a
1 GiB buffer is overwritten so that the weights come from HBM, not from L2 or
the 256 MB MALL; the flush is outside the per-layer events. Counted bytes =
distinct experts touched x (W13 + W2 FP8 bytes + FP32 scales), plus the shared
expert's weights and scales for a workload that has one. Prints one JSON line
(one per M with --sweep). The default workload is the DeepSeek-V3-shaped decode
at M=4; its line also carries config.sweep, the same metric at M = 1, 2, 4, 8,
16, 32 and 64 (one 64-token handle; the step at M runs its first M tokens).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from fp8_block_scaled_moe_amd import MoeDecode  # noqa: E402

PEAK_HBM_GBS = 8000.0

# HBM bytes per GEMM1 launch from FETCH_SIZE and WRITE_SIZE counter passes
# (each counter scaled by what it read for a plain 256 MiB copy), one entry
# per profiled kernel and workload; the summaries are in profiles/. An entry
# is valid only for its workload and while its kernel's sources hold the
# profiled code (sources_hash: comments and layout do not count); otherwise
# the traffic is null.
GEMM1_TRAFFIC = [
    {"sources": ["fp8_block_scaled_moe_amd/csrc/expert_gemm_wg.hip",
                 "fp8_block_scaled_moe_amd/csrc/gemm_device.h",
                 "fp8_block_scaled_moe_amd/csrc/device_common.h",
                 "fp8_block_scaled_moe_amd/csrc/epilogue_device.h",
                 "fp8_block_scaled_moe_amd/csrc/route_device.h",
                 "fp8_block_scaled_moe_amd/csrc/kernels.h",
                 "fp8_block_scaled_moe_amd/csrc/capi.hip"],  # the plan (K parts, grids)
     "sources_sha256_16": "48844a35fce297ae",
     "workload": "dsv3", "M": 4, "seed": 0, "unique_experts": 27,
     # medians per dispatch (KiB) and the copy kernel's reading of 256 MiB
     "fetch_kib": 387990.5, "write_kib": 512.0, "copy_fetch_kib": 131175.0, "copy_write_kib": 262144.0},
    {"sources": ["fp8_block_scaled_moe_amd/csrc/expert_gemm_fp4.hip",
                 "fp8_block_scaled_moe_amd/csrc/fp4_device.h",
                 "fp8_block_scaled_moe_amd/csrc/gemm_device.h",
                 "fp8_block_scaled_moe_amd/csrc/stream_device.h",
                 "fp8_block_scaled_moe_amd/csrc/device_common.h",
                 "fp8_block_scaled_moe_amd/csrc/kernels.h",
                 "fp8_block_scaled_moe_amd/csrc/capi.hip"],
     "sources_sha256_16": "b6db6df0f6e2c42a",
     "workload": "fp4_share", "M": 16, "seed": 0, "unique_experts": 4,
     "fetch_kib": 49131.38, "write_kib": 342.0, "copy_fetch_kib": 131175.0, "copy_write_kib": 262144.0},
]


def sources_hash(files) -> str:
    """SHA-256 (first 16 hex digits) of the sources' code: comments removed
    and whitespace collapsed, so that edits to comments or layout, which
    leave the compiled kernels unchanged, keep the recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def gemm1_traffic(workload: str, M: int, seed: int, U: int):
    for t in GEMM1_TRAFFIC:
        if (workload, M, seed, U) != (t["workload"], t["M"], t["seed"], t["unique_experts"]):
            continue
        if not t["copy_fetch_kib"] or sources_hash(t["sources"]) != t["sources_sha256_16"]:
            return None
        fetch = t["fetch_kib"] * (262144.0 / t["copy_fetch_kib"])
        write = t["write_kib"] * (262144.0 / t["copy_write_kib"])
        return int(round((fetch + write) * 1024))
    return None


METRIC = "routed-MoE decode µs/layer + achieved HBM GB/s (% peak) at M=1..64 tokens"
KERNELS = ["route_quant", "gemm1", "swiglu_requant", "gemm2", "combine"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3", choices=sorted(synth.CONFIGS))
    p.add_argument("--M", type=int, default=0, help="tokens (default: the workload's)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--path", default="auto", choices=["auto", "valu_splitk", "mfma_splitk", "mfma"])
    p.add_argument("--splits1", type=int, default=0)
    p.add_argument("--splits2", type=int, default=0)
    p.add_argument("--launch-mode", default="auto",
                   choices=["auto", "separate", "combine_in_gemm2", "swiglu_in_gemm1", "route_in_gemm1"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sweep", default="", help="comma-separated M values: one JSON line each")
    p.add_argument("--no-sweep", action="store_true",
                   help="leave out config.sweep (M = 1..64) of the default dsv3 line")
    p.add_argument("--calibrate", action="store_true",
                   help="time a plain 1 GiB device copy and a 4 GiB read-only sum instead")
    p.add_argument("--with-copy", action="store_true",
                   help="after the timed steps, run three 256 MiB device copies (a kernel of "
                        "known traffic to scale hardware byte counters by)")
    return p.parse_args()


def calibrate(args) -> None:
    """Achievable HBM bandwidth on this GPU: a plain device-to-device copy
    of 1 GiB (reads + writes 2 GiB) and a read-only sum over 4 GiB."""
    dev = torch.device("cuda:0")
    src = torch.randint(0, 255, (1 << 30,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    big = torch.ones((1 << 30,), dtype=torch.float32, device=dev)
    out = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: dst.copy_(src), 2 << 30),
                             ("sum_4GiB", lambda: big.sum(), 4 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / args.steps
        out[name] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"calibration": out, "peak_GB/s": PEAK_HBM_GBS}), flush=True)


def workload_name(shape) -> str:
    return (f"{shape.name}: M={shape.M} H={shape.hidden} I={shape.inter} E={shape.experts} "
            f"top_k={shape.top_k}")


def cpu_baseline(inp, counted_bytes: int, min_seconds: float = 10.0, max_runs: int = 8) -> dict:
    """The oracle on the host cores on the same inputs: the whole layer for all
    M tokens (it reads only the touched experts). Every array it reads is
    copied to the host first (an untimed run fills the expert cache); then
    the layer is run until min_seconds have passed (at most max_runs times)
    and the median run is reported."""
    from threadpoolctl import threadpool_info
    import oracle
    from tests.helpers import host

    s = inp.shape
    fp4 = s.weight_format == "fp4"
    x, logits, bias = host(inp.x), host(inp.logits), host(inp.bias)
    cache = {}

    def get(e: int):
        if e not in cache:
            if fp4:
                cache[e] = (inp.w13[e].cpu().numpy(), inp.w13_scale[e].cpu().numpy(),
                            inp.w2[e].cpu().numpy(), inp.w2_scale[e].cpu().numpy())
            else:
                cache[e] = (inp.w13[e].cpu().numpy(), host(inp.w13_scale[e]),
                            inp.w2[e].cpu().numpy(), host(inp.w2_scale[e]))
        return cache[e]

    shared = None
    if s.shared_inter:
        shared = (inp.sw13.cpu().numpy(), host(inp.sw13_scale), inp.sw2.cpu().numpy(), host(inp.sw2_scale))

    def layer():
        if fp4:
            oracle.fp4.moe_decode_fp4(x, logits, bias, get, top_k=s.top_k, routed_scale=s.routed_scale,
                                      limit=s.limit, local_begin=s.local_begin,
                                      local_count=s.local_experts, inter=s.inter)
        else:
            oracle.moe_decode(x, logits, bias, get, top_k=s.top_k, routed_scale=s.routed_scale,
                              limit=s.limit, ue8m0_act=s.ue8m0_act, inter=s.inter)
        if shared:
            oracle.shared_expert(x, *shared, limit=s.shared_limit, ue8m0_act=True)

    layer()  # fills the cache: no device copies inside the timing
    times = []
    while len(times) < max_runs and sum(times) < min_seconds:
        t0 = time.perf_counter()
        layer()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": counted_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds": dt, "runs": len(times), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"the full layer of the same workload ({s.M} tokens, all touched experts), "
                      f"float64 NumPy oracle, median of {len(times)} runs, every input already in "
                      f"host memory"}


def run_one(args, shape, inp, moe, flush, per_kernel=True):
    dev = inp.x.device
    k = shape.top_k
    slots, ids, weights, combined = moe.outputs(shape.M)
    shared_out = None
    if shape.shared_inter:
        shared_out = torch.empty((shape.M, shape.hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.run_into(inp.x, inp.logits, inp.bias, slots, ids, weights, combined,
                     shared_out=shared_out, stream=stream)

    for _ in range(args.warmup):
        flush.zero_()
        step()
    torch.cuda.synchronize()
    local = ids[(ids >= shape.local_begin) & (ids < shape.local_begin + shape.local_experts)]
    U = int(torch.unique(local).numel())  # distinct local experts touched
    counted = U * shape.expert_bytes() + shape.shared_bytes()

    # pass 1: whole layer, events on torch's current stream (the library's stream)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.zero_()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    layer_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    # pass 2: per-kernel times; the library launches each kernel with HIP
    # events that take its dispatch's own start and end (hipExtLaunchKernel)
    per = np.zeros((1, len(KERNELS)))
    if per_kernel:
        moe.set_timing(True)
        per = []
        for i in range(args.steps):
            flush.zero_()
            step()
            per.append(moe.last_timing()[:len(KERNELS)])
        moe.set_timing(False)
        per = np.array(per)
    torch.cuda.synchronize()
    return dict(U=U, counted=counted, layer_ms=layer_ms, per_kernel_ms=per, wall_s=wall, ids=ids)


def boundary_steps_us(dev, reps: int = 200) -> dict:
    """Per-call time of the two boundary steps (include/moe_boundary.h) at
    the expert-parallel page's shape: 5 tokens per rank, latent width 3584,
    partials from 16 ranks. Both are latency-bound (35 KB and 573 KB in);
    HIP events around `reps` back-to-back calls on the current stream."""
    from fp8_block_scaled_moe_amd import mxfp8_quantize, reduce_rmsnorm
    g = torch.Generator(device=dev).manual_seed(5)
    x = torch.randn((5, 3584), generator=g, device=dev).to(torch.bfloat16)
    parts = torch.randn((5, 16, 3584), generator=g, device=dev).to(torch.bfloat16)
    gamma = torch.ones(3584, dtype=torch.bfloat16, device=dev)
    out = {}
    for name, fn in (("mxfp8_quantize", lambda: mxfp8_quantize(x)),
                     ("reduce_rmsnorm", lambda: reduce_rmsnorm(parts, gamma, 1e-5))):
        for _ in range(20):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # a spin kernel keeps the queue ahead of the host, so the calls run
        # back to back on the device and the events time the device work
        torch.cuda._sleep(int(6e7))
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        out[name] = round(a.elapsed_time(b) * 1e3 / reps, 2)
    out["shape"] = "T=5 tokens, D=3584, N=16 partials; calls back to back on the device, inputs L2-resident"
    return out


SWEEP_MS = (1, 2, 4, 8, 16, 32, 64)


def sweep(args, base, dev, flush) -> dict:
    """The metric over M = 1..64: one handle for 64 tokens on the workload's
    seeded inputs at M = 64; the step at M takes the first M tokens. Same
    flush and timing as the headline (HIP events around each layer, median)."""
    shape = base.with_(M=max(SWEEP_MS))
    inp_all = synth.make_inputs(shape, seed=args.seed, device=dev)
    moe = MoeDecode(inp_all.w13, inp_all.w13_scale, inp_all.w2, inp_all.w2_scale,
                    top_k=shape.top_k, limit=shape.limit, routed_scale=shape.routed_scale,
                    max_tokens=shape.M, logits_dtype=inp_all.logits.dtype,
                    ue8m0_act=shape.ue8m0_act)
    points = []
    for M in SWEEP_MS:
        sh = base.with_(M=M)
        inp = synth.MoeInputs(shape=sh, seed=args.seed, x=inp_all.x[:M].contiguous(),
                              logits=inp_all.logits[:M].contiguous(), bias=inp_all.bias,
                              w13=inp_all.w13, w13_scale=inp_all.w13_scale, w2=inp_all.w2,
                              w2_scale=inp_all.w2_scale)
        r = run_one(args, sh, inp, moe, flush, per_kernel=False)
        ms = float(np.median(r["layer_ms"]))
        gbs = r["counted"] / (ms * 1e-3) / 1e9
        points.append({"M": M, "unique_experts": r["U"], "counted_bytes": r["counted"],
                       "us_per_layer": round(ms * 1e3, 2),
                       "us_p10_p90": [round(float(np.quantile(r["layer_ms"], q)) * 1e3, 2)
                                      for q in (0.1, 0.9)],
                       "GB/s": round(gbs, 1), "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2)})
        print(f"# sweep M={M}: {ms * 1e3:.1f} us, {100 * gbs / PEAK_HBM_GBS:.1f}% of peak",
              file=sys.stderr, flush=True)
    moe.close()
    del inp_all
    return {"workload": f"{base.name} at M=64, seed {args.seed}; step M runs its first M tokens "
                        "on one handle",
            "points": points}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the routed-expert path "
                          "has no multi-GPU form in this library (expert-parallel sharding is "
                          "described in DESIGN.md)", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.calibrate:
        calibrate(args)
        return
    dev = torch.device("cuda:0")
    base = synth.CONFIGS[args.workload]
    Ms = [int(m) for m in args.sweep.split(",")] if args.sweep else [args.M or base.M]
    maxM = max(Ms)
    shape = base.with_(M=maxM)
    inp_all = synth.make_inputs(shape, seed=args.seed, device=dev)
    shared = {}
    if shape.shared_inter:
        shared = dict(sw13=inp_all.sw13, sw13_scale=inp_all.sw13_scale, sw2=inp_all.sw2,
                      sw2_scale=inp_all.sw2_scale, shared_limit=shape.shared_limit,
                      shared_ue8m0_act=True)
    fmt = {}
    if shape.weight_format == "fp4":
        fmt = dict(weight_format="nvfp4", experts=shape.experts, local_begin=shape.local_begin)
    moe = MoeDecode(inp_all.w13, inp_all.w13_scale, inp_all.w2, inp_all.w2_scale,
                    top_k=shape.top_k, limit=shape.limit, routed_scale=shape.routed_scale,
                    max_tokens=maxM, logits_dtype=inp_all.logits.dtype, ue8m0_act=shape.ue8m0_act,
                    gemm_path=args.path, splits1=args.splits1, splits2=args.splits2,
                    launch_mode=args.launch_mode, **shared, **fmt)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for M in Ms:
        sh = base.with_(M=M)
        inp = synth.MoeInputs(shape=sh, seed=args.seed, x=inp_all.x[:M].contiguous(),
                              logits=inp_all.logits[:M].contiguous(), bias=inp_all.bias,
                              w13=inp_all.w13, w13_scale=inp_all.w13_scale, w2=inp_all.w2,
                              w2_scale=inp_all.w2_scale, sw13=inp_all.sw13,
                              sw13_scale=inp_all.sw13_scale, sw2=inp_all.sw2,
                              sw2_scale=inp_all.sw2_scale)
        r = run_one(args, sh, inp, moe, flush)
        ms = float(np.median(r["layer_ms"]))
        us = ms * 1e3
        gbs = r["counted"] / (ms * 1e-3) / 1e9
        # dominant kernel: GEMM1 streams W13 (2/3 of the counted bytes), and
        # the shared expert's gate_up weights when there is one
        if sh.weight_format == "fp4":  # packed E2M1 + a UE4M3 byte per 16 values
            g1_bytes = r["U"] * (2 * sh.inter * sh.hidden // 2 + 2 * sh.inter * sh.hidden // 16)
        else:
            g1_bytes = r["U"] * (2 * sh.inter * sh.hidden + (2 * sh.inter // 128) * (sh.hidden // 128) * 4)
        if sh.shared_inter:
            g1_bytes += 2 * sh.shared_inter * sh.hidden + (2 * sh.shared_inter // 128) * (sh.hidden // 128) * 4
        per = np.median(r["per_kernel_ms"], axis=0)
        g1_gbs = g1_bytes / (per[1] * 1e-3) / 1e9
        plan = moe.plan(M)
        line = {
            "metric": METRIC,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp4" if sh.weight_format == "fp4" else "fp8",
            "data": "synthetic",
            "config": {
                "workload": workload_name(sh),
                "M": M, "hidden": sh.hidden, "inter": sh.inter, "experts": sh.experts,
                "top_k": sh.top_k, "unique_experts": r["U"], "counted_bytes": r["counted"],
                "us_per_layer": round(us, 2),
                "us_per_layer_p10_p90": [round(float(np.quantile(r["layer_ms"], q)) * 1e3, 2)
                                         for q in (0.1, 0.9)],
                "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
                "kernel_us": {k: round(float(v) * 1e3, 2) for k, v in zip(KERNELS, per)},
                "wall_ms_per_step_incl_flush": round(r["wall_s"] / args.steps * 1e3, 4),
                "gemm_path": {1: "valu_splitk", 2: "mfma_splitk", 3: "mfma", 4: "fp4"}[plan["path"]],
                "splits": [plan["splits1"], plan["splits2"]],
                "kparts": [plan["kparts1"], plan["kparts2"]],
                "launches": plan["launches"],
                "persistent_wgs": [plan["persist1"], plan["persist2"]],
                "l2_mall_flush": "1 GiB overwrite before every step, outside the timed layer",
            },
            "roofline": {
                "kernel": "gemm1 (W13 up/gate GEMM over the touched experts"
                          + (" and the shared gate_up)" if sh.shared_inter else ")"),
                "bound": "hbm",
                "achieved": round(g1_gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(g1_gbs / PEAK_HBM_GBS, 4),
                "traffic": gemm1_traffic(args.workload, M, args.seed, r["U"]),
                "algorithmic_bytes_per_launch": g1_bytes,
                "avg_launch_us": round(float(per[1]) * 1e3, 2),
            },
        }
        if M == Ms[0]:
            line["config"]["boundary_steps_us"] = boundary_steps_us(dev)
        if not args.no_cpu_baseline and M == Ms[0]:
            line["cpu_baseline"] = cpu_baseline(inp, r["counted"])
        if not args.sweep and not args.no_sweep and args.workload == "dsv3":
            moe.close()
            del inp, inp_all
            torch.cuda.empty_cache()
            line["config"]["sweep"] = sweep(args, base, dev, flush)
        print(json.dumps(line), flush=True)
    moe.close()
    if args.with_copy:
        # uint8 -> int8: an elementwise copy kernel reading and writing 256 MiB,
        # its source flushed out of L2 and the MALL first
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty(256 << 20, dtype=torch.int8, device=dev)
        for _ in range(3):
            flush.zero_()
            dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
