"""Benchmark: DM0-base suffix denoise (28 layers, 10 Euler steps, chunk 50, 816-token prefix KV,
bf16 weights/activations, fp32 accumulation) on one MI355X, through the C ABI.

A "step" is one action chunk: one replay of the captured hipGraph that runs all 10 Euler steps
(time embedding + action_in_proj, 28 merged-attention layers over the cached prefix,
action_out_proj + Euler update) for the batch.  Inputs are resident in HBM before timing.

Prints one JSON line: chunks/s (whole job), p50/p90/p99 chunk latency, the roofline of the
dominant kernel, and the float64 oracle timed on the host cores as a CPU baseline.

  python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config 3|4] [--no-cpu-baseline] [--prefill]
  python bench.py --merged-layer            (one merged layer only, its own JSON line)

The roofline unit is one launch of the captured graph (one chunk): achieved = algorithmic bytes
(batch 1, HBM-bound) or FLOPs (batch 32, MFMA-bound) of the chunk / its mean duration (HIP
events on the stream the graph is launched on); traffic = HBM bytes of the same chunk from
rocprofv3 FETCH_SIZE + WRITE_SIZE counters, scaled against a plain copy
(profiles/*_hbm_traffic.txt, reported only while the kernel sources are unchanged).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl, lens):
    """Bytes and FLOPs of one chunk: every weight byte and every visible prefix K/V byte once per
    Euler step, plus x in and out; GEMM FLOPs 2*params*tokens, attention 4*D*Hq per unmasked
    (query, key) pair."""
    s = wl.shape
    es = 2 if s.dtype == "bf16" else 4
    H, F, D, Hq, Hkv, S, A, L = (s.act_hidden, s.act_ffn, s.head_dim, s.n_q_heads, s.n_kv_heads, s.chunk,
                                 s.action_dim, s.n_layers)
    mat = (s.qkv_rows * H + H * Hq * D + 2 * F * H + H * F) * L
    vec = (2 * H * L + H * A + H + H + A * H + A) * 4          # norms, in/out projections and biases (fp32)
    kv = int(np.sum(lens)) * L * Hkv * D * 2 * es
    x_io = wl.batch * S * A * 4 * 2
    per_step_bytes = mat * es + vec + kv + x_io
    tokens = wl.batch * S
    gemm = 2 * mat * tokens + 2 * (2 * A * H) * tokens
    attn = sum(4 * D * Hq * S * (int(p) + S) for p in lens) * L
    return {"bytes": per_step_bytes * wl.steps, "flops": (gemm + attn) * wl.steps,
            "weight_bytes_per_step": mat * es + vec, "kv_bytes_per_step": kv}


def cpu_baseline(wl, aw, kc, vc, x1, lens):
    """The oracle as it stands (float64 numpy), one full chunk of sample 0."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    P = int(lens[0])
    t0 = time.perf_counter()
    O.suffix_denoise(x1[0], aw, kc[:, 0, :, :P], vc[:, 0, :, :P], wl.shape, wl.steps)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / dt, "unit": "chunks/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"one full chunk of sample 0 ({wl.steps} Euler steps x {wl.shape.n_layers} layers, "
                      f"P={P}) in float64 numpy; {dt:.2f} s on {cores} host cores"}


SOURCES = ["dm_api.cpp", "gemm.hip", "attn.hip", "misc.hip", "common.h", "kernels.h"]


def source_hash():
    """Hash of the kernel sources: HBM traffic measured with counters is only reported while the
    kernels it was measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for name in SOURCES:
        with open(os.path.join(ROOT, "dual_expert_merged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(config):
    return os.path.join(ROOT, "profiles", f"denoise_{'b1_p816' if config == 3 else 'b32_ragged'}_hbm_traffic.txt")


def read_traffic(config):
    """HBM bytes per chunk from the committed counter summary, or None when the kernels changed."""
    path = traffic_file(config)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash():
        return None
    return int(float(vals["hbm_bytes_per_chunk"]))


def _pmc_sum(run_dir, counter, match):
    """Sum of one counter over the dispatches whose kernel name contains `match`, and the number
    of dispatches, from a rocprofv3 --pmc csv run directory."""
    import csv
    import glob
    total, n = 0.0, 0
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
                    total += float(r["Counter_Value"])
                    n += 1
    return total, n


def traffic_summary(args):
    """Writes the HBM-traffic summary of one denoise chunk from four rocprofv3 --pmc runs: the
    bench with FETCH_SIZE, with WRITE_SIZE, and the copy calibration with each.  FETCH_SIZE and
    WRITE_SIZE count KiB per dispatch; both are scaled by bytes-moved / counted for a plain copy
    of known size."""
    lib = lambda name: "dm::" in name or "_ZN2dm" in name
    copy = lambda name: "copybuffer" in name.lower()  # the device-to-device copies, not the fill before them
    cal_bytes = COPY_BYTES * COPY_REPS
    cf, _ = _pmc_sum(args.cal_fetch, "FETCH_SIZE", copy)
    cw, _ = _pmc_sum(args.cal_write, "WRITE_SIZE", copy)
    f_scale, w_scale = cal_bytes / (cf * 1024.0), cal_bytes / (cw * 1024.0)
    fetch, _ = _pmc_sum(args.fetch, "FETCH_SIZE", lib)
    write, _ = _pmc_sum(args.write, "WRITE_SIZE", lib)
    _, n_vel = _pmc_sum(args.fetch, "FETCH_SIZE", lambda n: "velocity_euler" in n)
    from dual_expert_merged_amd.configs import workload
    wl = workload(args.config)
    chunks = n_vel / wl.steps
    per_chunk = (fetch * 1024.0 * f_scale + write * 1024.0 * w_scale) / chunks
    with open(traffic_file(args.config), "w") as f:
        f.write(f"# HBM traffic of one denoise chunk ({wl.name}), rocprofv3 counters\n")
        f.write("# commands (run from the repository root on the MI355X host, each pass its own run):\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -- python3 bench.py "
                f"--config {args.config} --steps 2 --warmup 0 --no-cpu-baseline\n")
        f.write("#   rocprofv3 --pmc WRITE_SIZE ... (same)\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE --output-format csv -d <cal> -- python3 bench.py --copy-calibration\n")
        f.write(f"#   python3 bench.py --traffic-summary --config {args.config} --fetch <fetch> --write <write> "
                "--cal-fetch <cal-fetch> --cal-write <cal-write>\n")
        f.write(f"chunks_profiled: {chunks:g}\n")
        f.write(f"copy_calibration_bytes: {cal_bytes}\n")
        f.write(f"fetch_scale: {f_scale:.4f}\n")
        f.write(f"write_scale: {w_scale:.4f}\n")
        f.write(f"fetch_bytes_per_chunk: {fetch * 1024.0 * f_scale / chunks:.0f}\n")
        f.write(f"write_bytes_per_chunk: {write * 1024.0 * w_scale / chunks:.0f}\n")
        f.write(f"hbm_bytes_per_chunk: {per_chunk:.0f}\n")
        f.write(f"source_hash: {source_hash()}\n")
    print(open(traffic_file(args.config)).read())


COPY_BYTES = 1 << 30
COPY_REPS = 4


def copy_calibration():
    """A plain device copy of known size (COPY_REPS x 1 GiB, hipMemcpy device to device) for scaling
    the traffic counters."""
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_REPS} x {COPY_BYTES} bytes")


def prefill_times(reps=3):
    """Prefix encoding of the prefill workload (B=8, 816 tokens, 28 VLM layers) with the bf16
    MLP and with the FP8 E4M3 MLP: mean ms per call over `reps` calls after one warm-up."""
    import torch
    from dataclasses import replace
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import FP8, workload

    wl = workload(5)
    vlm = inputs.make_vlm_weights(wl)
    emb = torch.from_numpy(inputs.make_prefix_embeds(wl)).cuda()
    lens = torch.from_numpy(inputs.make_prefix_lens(wl)).cuda()
    s = wl.shape
    out = {}
    for name, shape in (("bf16", s), ("fp8_mlp", replace(s, vlm_mlp_dtype=FP8))):
        ctx = bd.Context(shape, 0)
        dv = bd.DeviceExpert(vlm, s.dtype, fp8_mlp=name == "fp8_mlp")
        cshape = (s.n_layers, wl.batch, s.n_kv_heads, wl.prefix_len, s.head_dim)
        k = torch.empty(cshape, dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        ws = ctx.workspace(bd.OP_PREFILL, wl.batch, wl.prefix_len)
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            ctx.prefill_kv(dv, emb, lens, k, v, ws, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                ctx.prefill_kv(dv, emb, lens, k, v, ws, stream=stream)
            e1.record(stream)
            stream.synchronize()
        out[name] = round(e0.elapsed_time(e1) / reps, 3)
        del dv, k, v, ws
        ctx.close()
        torch.cuda.empty_cache()
    flops = 2 * wl.batch * wl.prefix_len * s.n_layers * (s.qkv_rows * s.vlm_hidden + s.vlm_hidden * s.n_q_heads *
                                                         s.head_dim + 3 * s.vlm_ffn * s.vlm_hidden)
    out["workload"] = wl.name
    out["bf16_mfma_frac_of_gemm_flops"] = round(flops / (out["bf16"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    return out


def merged_layer_times(reps=20):
    """One DM0-base merged layer at batch 1 (816 prefix and 50 action tokens through both experts
    with the joint block-masked attention, prefix K/V written out): mean µs per dm_merged_layer
    call (HIP events around each call on its stream; the inputs are restored between calls,
    outside the timed spans) and the fraction of dense bf16 MFMA peak over its algorithmic FLOPs."""
    import torch
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import workload

    wl = workload(2)
    s = wl.shape
    P, S = wl.prefix_len, s.chunk
    ctx = bd.Context(s, 0)
    dv = bd.DeviceExpert(inputs.make_vlm_weights(wl), s.dtype)
    da = bd.DeviceAction(inputs.make_action_weights(wl), s.dtype)
    hp0 = torch.from_numpy(inputs.make_prefix_embeds(wl)).cuda()
    hs0 = torch.from_numpy(inputs.make_suffix_hidden(wl)).cuda()
    hp, hs = hp0.clone(), hs0.clone()
    lens = torch.full((1,), P, dtype=torch.int32, device="cuda")
    ko = torch.empty((1, s.n_kv_heads, P, s.head_dim), dtype=bd.torch_dtype(s.dtype), device="cuda")
    vo = torch.empty_like(ko)
    ws = ctx.workspace(bd.OP_MERGED_LAYER, 1, P)
    stream = torch.cuda.Stream()
    total = 0.0
    with torch.cuda.stream(stream):
        ctx.merged_layer(dv, da.body, 0, hp, hs, lens, ws, ko, vo, stream=stream)  # warm-up
        for _ in range(reps):
            hp.copy_(hp0)
            hs.copy_(hs0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ctx.merged_layer(dv, da.body, 0, hp, hs, lens, ws, ko, vo, stream=stream)
            e1.record(stream)
            stream.synchronize()
            total += e0.elapsed_time(e1)
    ctx.close()
    us = total * 1e3 / reps
    D, Hq = s.head_dim, s.n_q_heads
    params = lambda h, f: s.qkv_rows * h + h * Hq * D + 3 * f * h
    flops = (2 * P * params(s.vlm_hidden, s.vlm_ffn) + 2 * S * params(s.act_hidden, s.act_ffn)
             + 4 * D * Hq * (P * P + S * (P + S)))
    return {"us": round(us, 2), "algorithmic_gflop": round(flops / 1e9, 2),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "workload": "DM0-base merged layer, bf16, B=1, 816 prefix + 50 action tokens"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", action="store_true",
                    help="also time the prefix encoding (B=8, 816 tokens) with the bf16 and the FP8 MLP")
    ap.add_argument("--merged-layer", action="store_true",
                    help="time only one merged layer (both experts, B=1, 816 + 50 tokens) and print it")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the plain copy for counter scaling")
    ap.add_argument("--traffic-summary", action="store_true", help="summarise counter runs (no GPU needed)")
    for name in ("fetch", "write", "cal-fetch", "cal-write"):
        ap.add_argument("--" + name)
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.merged_layer:
        print(json.dumps({"merged_layer": merged_layer_times()}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the suffix denoise path is built for a single MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import workload

    wl = workload(args.config)
    s = wl.shape
    log(f"[bench] generating inputs for: {wl.name}")
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    lens = inputs.make_prefix_lens(wl)

    torch.cuda.set_device(0)
    ctx = bd.Context(s, 0)
    td = bd.torch_dtype(s.dtype)
    da = bd.DeviceAction(aw, s.dtype)
    k = bd.to_device(kc, td)
    v = bd.to_device(vc, td)
    ld = torch.from_numpy(lens).cuda()
    x0 = torch.from_numpy(x1).cuda()
    x = x0.clone()
    ws = ctx.workspace(bd.OP_DENOISE, wl.batch, wl.prefix_len)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        plan = ctx.denoise_plan(da, k, v, ld, x, wl.steps, ws, stream=stream)
        log(f"[bench] plan captured; warmup {args.warmup}")
        for _ in range(args.warmup):
            plan.launch(stream=stream)
        stream.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            plan.launch(stream=stream)
            ends[i].record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    lat = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])  # ms per chunk, GPU clock
    alg = algorithmic(wl, lens)
    ms = wall * 1e3 / args.steps
    value = wl.batch * args.steps / wall
    chunk_s = float(np.mean(lat)) * 1e-3
    gbs = alg["bytes"] / chunk_s / 1e9
    tfs = alg["flops"] / chunk_s / 1e12
    if args.config == 3:  # batch 1: the weights and the cache stream once per step (55 FLOP/B)
        roof = {"bound": "hbm", "kernel": "denoise graph replay (all kernels of one chunk)",
                "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(args.config),
                "algorithmic_bytes_per_launch": alg["bytes"], "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}
    else:  # batch 32: the GEMMs dominate (435 FLOP/B over the chunk)
        roof = {"bound": "mfma", "kernel": "denoise graph replay (all kernels of one chunk)",
                "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfs / BF16_PEAK_TFLOPS, 4), "traffic": read_traffic(args.config),
                "algorithmic_flops_per_launch": alg["flops"], "algorithmic_bytes_per_launch": alg["bytes"],
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    out = {
        "metric": "action chunks/s + p50 chunk latency (DM0-base suffix, 10 steps); % HBM/MFMA peak",
        "value": round(value, 2), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "prefix_len": int(lens.max()),
                   "prefix_len_mean": float(lens.mean()), "chunk": s.chunk, "action_dim": s.action_dim,
                   "euler_steps": wl.steps, "layers": s.n_layers, "parallelism": "single GPU"},
        "latency_ms": {"p50": round(float(np.percentile(lat, 50)), 4), "p90": round(float(np.percentile(lat, 90)), 4),
                       "p99": round(float(np.percentile(lat, 99)), 4), "mean": round(float(np.mean(lat)), 4)},
        "roofline": roof,
    }
    plan.close()
    if args.prefill:
        log("[bench] timing the prefix encoding (bf16 and FP8 MLP)")
        out["prefill_ms"] = prefill_times()
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(wl, aw, kc, vc, x1, lens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
