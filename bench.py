"""Benchmark: DM0-base suffix denoise (28 layers, 10 Euler steps, chunk 50, 816-token prefix KV,
bf16 weights/activations, fp32 accumulation) on one MI355X, through the C ABI.

A "step" is one action chunk: one replay of the captured hipGraph that runs all 10 Euler steps
(time embedding + action_in_proj, 28 merged-attention layers over the cached prefix,
action_out_proj + Euler update) for the batch.  Inputs are resident in HBM before timing.

Prints one JSON line: chunks/s (whole job), p50/p90/p99 chunk latency, the roofline of the
dominant kernel, and the float64 oracle timed on the host cores as a CPU baseline.

  python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config 3|4] [--no-cpu-baseline] [--no-extras]
  python bench.py --merged-layer            (one merged layer only, its own JSON line)

Headline (batch 1, HBM-bound): the whole chunk is one launch of the single-launch denoise
kernel, so its roofline is achieved = algorithmic bytes of the chunk / mean duration of a replay
(HIP events on the stream the graph is launched on); traffic = HBM bytes of the same chunk from
rocprofv3 FETCH_SIZE + WRITE_SIZE counters, scaled against a plain copy
(profiles/*_hbm_traffic.txt, reported only while the kernel sources are unchanged).
Sub-objects of the same line: "batch32" (the batch-32 ragged workload, MFMA-bound: chunks/s,
latency, the chunk's MFMA fraction from live events, each GEMM kernel's MFMA fraction from the
committed kernel statistics), "time_modulated" (the DM0.5-style time-modulated expert, B=4),
"qk_norm" (the per-head QK-norm switch, B=2), "merged_layer" (one joint layer of both experts at
B=1, 816 + 50 tokens: us per call and its MFMA fraction),
"prefill_ms" (the B=8, 816-token prefix encoding with the bf16 and with the FP8 MLP) and
"serving" (the fixed-contract engine on prefill + denoise at B=8: model-core and request
latency percentiles) and "training" (one flow-matching training step on one merged layer:
ms per step and its fp32 matrix-core fraction).
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
    chunk_bytes = per_step_bytes * wl.steps
    chunk_flops = (gemm + attn) * wl.steps
    if getattr(s, "time_mod", False):
        # the modulation tables, once per chunk: time MLP (fp32) and every modulator (weight dtype)
        mod_rows = 6 * H * L + 2 * H
        chunk_bytes += 2 * H * H * 4 + 2 * H * 4 + mod_rows * (H * es + 4)
        chunk_flops += 2 * wl.steps * (2 * H * H + mod_rows * H)
    return {"bytes": chunk_bytes, "flops": chunk_flops,
            "weight_bytes_per_step": mat * es + vec, "kv_bytes_per_step": kv}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, aw, kc, vc, x1, lens):
    """The oracle as it stands (float64 numpy), one full chunk of sample 0."""
    import oracle as O
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max([i.get("num_threads", 1) for i in libs] or [1])
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}, {blas_threads} threads"
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    P = int(lens[0])
    t0 = time.perf_counter()
    O.suffix_denoise(x1[0], aw, kc[:, 0, :, :P], vc[:, 0, :, :P], wl.shape, wl.steps)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / dt, "unit": "chunks/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"one full chunk of sample 0 ({wl.steps} Euler steps x {wl.shape.n_layers} layers, "
                      f"P={P}) in float64 numpy; {dt:.2f} s on {cores} host cores",
            "cpu": cpu_model(), "numpy": np.__version__, "blas": blas}


def environment():
    """The GPU and software the numbers were taken on."""
    import torch
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "memory_gib": round(props.total_memory / 2**30, 1), "rocm": rocm, "hip": torch.version.hip,
            "torch": torch.__version__, "host_cpu": cpu_model()}


SOURCES = ["dm_api.cpp", "gemm.hip", "attn.hip", "misc.hip", "persist.hip", "train.hip", "common.h", "kernels.h", "persist_plan.h",
           "addr_words.h"]


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


def count_chunks(run_dir, counter, wl):
    """Chunks in a counter run: one launch of the single-launch kernel per chunk, else one
    velocity/Euler launch per Euler step."""
    _, n_single = _pmc_sum(run_dir, counter, lambda n: "denoise_b1_kernel" in n)
    if n_single:
        return n_single
    _, n_vel = _pmc_sum(run_dir, counter, lambda n: "velocity_euler" in n)
    return n_vel / wl.steps


def stats_summary(args):
    """Writes profiles/<name>_kernel_stats.txt from a rocprofv3 --kernel-trace --stats run: per
    kernel the calls, calls per unit (chunk or prefill call), mean / min / max duration and share
    of the library's time, plus the source hash of the kernels profiled."""
    import csv
    import glob
    paths = glob.glob(os.path.join(args.stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    assert paths, f"no *kernel_stats.csv under {args.stats_dir}"
    rows = []
    for path in paths:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    units = args.units
    out = os.path.join(ROOT, "profiles", f"{args.name}_kernel_stats.txt")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel statistics: {args.title}\n")
        f.write(f"# command (repository root on the MI355X host): rocprofv3 --kernel-trace --stats --output-format csv "
                f"-d <dir> -o run -- python3 bench.py {args.bench_args}\n")
        f.write(f"# summary: python3 bench.py --stats-summary --stats-dir <dir> --name {args.name} --units {units} "
                f"--title '{args.title}' --bench-args '{args.bench_args}'\n")
        f.write(f"# {units:g} units profiled; kernels total {total / 1e6:.3f} ms = {total / 1e6 / units:.3f} ms per unit\n")
        f.write(f"# source_hash: {source_hash()}\n")
        f.write(f"{'kernel':<96} {'calls':>6} {'per_unit':>9} {'avg_us':>9} {'min_us':>8} {'max_us':>8} {'pct':>6}\n")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"] if len(r["Name"]) <= 95 else r["Name"][:92] + "..."
            calls = int(r["Calls"])
            f.write(f"{name:<96} {calls:>6} {calls / units:>9.4g} {float(r['AverageNs']) / 1e3:>9.2f} "
                    f"{float(r['MinNs']) / 1e3:>8.2f} {float(r['MaxNs']) / 1e3:>8.2f} "
                    f"{100 * float(r['TotalDurationNs']) / total:>6.2f}\n")
    print(open(out).read())


def counter_summary(args):
    """Writes profiles/<name>_mfma_counters.txt from a rocprofv3 --pmc run (derived counters such
    as MfmaUtil and MfmaFlopsBF16 / MfmaFlopsF8, with --kernel-trace for the durations): per
    kernel the dispatches, the mean of every counter per dispatch, the mean duration, and the
    achieved MFMA rate (counted FLOPs / duration) as a fraction of the dense peak of its dtype."""
    import csv
    import glob
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in glob.glob(os.path.join(args.stats_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    durs = collections.defaultdict(list)
    for path in glob.glob(os.path.join(args.stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    assert vals, f"no counter csv under {args.stats_dir}"
    # FLOPs per dispatch: the derived bf16 metric, or raw MFMA operation counts (units of 512 FLOPs)
    flop_counters = {"MfmaFlopsBF16": (1, BF16_PEAK_TFLOPS), "SQ_INSTS_VALU_MFMA_MOPS_BF16": (512, BF16_PEAK_TFLOPS),
                     "SQ_INSTS_VALU_MFMA_MOPS_F8": (512, 2 * BF16_PEAK_TFLOPS)}
    out = os.path.join(ROOT, "profiles", f"{args.name}_mfma_counters.txt")
    names = sorted(vals, key=lambda k: -sum(durs.get(k, [0.0])))
    counters = sorted({c for k in vals for c in vals[k]})
    with open(out, "w") as f:
        f.write(f"# rocprofv3 counters per dispatch: {args.title}\n")
        f.write(f"# command (repository root on the MI355X host): rocprofv3 --kernel-trace --pmc {' '.join(counters)} "
                f"--output-format csv -d <dir> -o run -- python3 bench.py {args.bench_args}\n")
        f.write(f"# summary: python3 bench.py --counter-summary --stats-dir <dir> --name {args.name} "
                f"--title '{args.title}' --bench-args '{args.bench_args}'\n")
        f.write("# MfmaUtil: % of cycles the MFMA units are busy while the GPU is active (SQ_VALU_MFMA_BUSY_CYCLES over\n"
                "# GRBM_GUI_ACTIVE x SIMDs); MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOPs (likewise the raw\n"
                "# F8 operation count); frac_of_peak: those FLOPs over the kernel's mean duration, against the dense\n"
                "# peak of its dtype (bf16 2.5, FP8 5.0 PFLOP/s)\n")
        f.write(f"# source_hash: {source_hash()}\n")
        f.write(f"{'kernel':<70} {'n':>5} {'avg_us':>8} " + " ".join(f"{c:>14}" for c in counters) + f" {'frac_of_peak':>12}\n")
        for k in names:
            n = len(next(iter(vals[k].values())))
            us = float(np.mean(durs[k])) if durs.get(k) else float("nan")
            row = [float(np.mean(vals[k][c])) if vals[k].get(c) else float("nan") for c in counters]
            frac = float("nan")
            for c, (unit, pk) in flop_counters.items():
                if c in counters and vals[k].get(c) and us == us and us > 0:
                    fl = float(np.mean(vals[k][c])) * unit
                    if fl > 0:
                        frac = fl / (us * 1e-6) / 1e12 / pk
            name = k if len(k) <= 69 else k[:66] + "..."
            f.write(f"{name:<70} {n:>5} {us:>8.2f} " + " ".join(f"{v:>14.4g}" for v in row) + f" {frac:>12.4f}\n")
    print(open(out).read())


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
    from dual_expert_merged_amd.configs import workload
    wl = workload(args.config)
    chunks = count_chunks(args.fetch, "FETCH_SIZE", wl)
    per_chunk = (fetch * 1024.0 * f_scale + write * 1024.0 * w_scale) / chunks
    with open(traffic_file(args.config), "w") as f:
        f.write(f"# HBM traffic of one denoise chunk ({wl.name}), rocprofv3 counters\n")
        f.write("# commands (run from the repository root on the MI355X host, each pass its own run):\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -- python3 bench.py "
                f"--config {args.config} --steps 2 --warmup 0 --no-cpu-baseline --no-extras\n")
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


def prefill_times(reps=3, modes=("bf16", "fp8_mlp"), vlm=None):
    """Prefix encoding of the prefill workload (B=8, 816 tokens, 28 VLM layers) with the bf16
    MLP and with the FP8 E4M3 MLP: mean ms per call over `reps` calls after one warm-up."""
    import torch
    from dataclasses import replace
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import FP8, workload

    wl = workload(5)
    if vlm is None:
        vlm = inputs.make_vlm_weights(wl)
    emb = torch.from_numpy(inputs.make_prefix_embeds(wl)).cuda()
    lens = torch.from_numpy(inputs.make_prefix_lens(wl)).cuda()
    s = wl.shape
    out = {}
    for name, shape in (("bf16", s), ("fp8_mlp", replace(s, vlm_mlp_dtype=FP8))):
        if name not in modes:
            continue
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
    if "bf16" in out:
        out["bf16_mfma_frac_of_gemm_flops"] = round(flops / (out["bf16"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    return out


def serving_summary(vlm=None, reps=20, warmup=3):
    """The fixed-contract engine on the prefill + denoise workload (B=8, 816-token prefix, 28 VLM
    and 28 action layers, 10 Euler steps): model-core latency (one replay of the captured prefix
    encoding + denoise over the resident static buffers, HIP events on its stream) and request
    latency (host wall clock around dm_engine_run: copy of the embeddings, lengths and noise
    from pinned host buffers into the static ones, the replay, the chunk copied back)."""
    import torch
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import workload

    wl = workload(5)
    s = wl.shape
    if vlm is None:
        vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)

    def pinned(a):
        t = torch.empty(a.shape, dtype=torch.from_numpy(a).dtype, pin_memory=True)
        t.numpy()[...] = a
        return t

    emb, lens, x1 = (pinned(a) for a in (inputs.make_prefix_embeds(wl), inputs.make_prefix_lens(wl),
                                         inputs.make_noise(wl)))
    actions = torch.empty(x1.shape, dtype=torch.float32, pin_memory=True)
    ctx = bd.Context(s, 0)
    dv, da = bd.DeviceExpert(vlm, s.dtype), bd.DeviceAction(aw, s.dtype)
    stream = torch.cuda.Stream()
    eng = bd.Engine(ctx, dv, da, wl.batch, wl.prefix_len, wl.steps, stream=stream)
    args = (emb.numpy(), lens.numpy(), x1.numpy(), actions.numpy())
    for _ in range(warmup):
        eng.run(*args, stream=stream)
    req = []
    for _ in range(reps):
        t0 = time.perf_counter()
        eng.run(*args, stream=stream)
        req.append((time.perf_counter() - t0) * 1e3)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record(stream)
        eng.replay(stream=stream)
        ends[i].record(stream)
    stream.synchronize()
    core = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    contract = eng.contract()
    eng.close()
    del dv, da
    ctx.close()
    torch.cuda.empty_cache()
    h2d = emb.numel() * 4 + lens.numel() * 4 + x1.numel() * 4
    return {"workload": wl.name, "contract": contract, "model_core_ms": latency(core),
            "request_ms": latency(np.array(req)), "requests_per_s": round(1e3 / float(np.mean(req)), 2),
            "chunks_per_s": round(wl.batch * 1e3 / float(np.mean(req)), 2), "copied_in_bytes": int(h2d),
            "copied_out_bytes": int(x1.numel() * 4), "host_buffers": "pinned"}


FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak, TFLOP/s


def train_flops(s, lens, ki):
    """Algorithmic FLOPs of one training step on one merged layer: every product of the forward
    (prefix K/V projection, action-row Q/K/V, scores and P V over P_b + S keys, O, gate, up, down,
    action_in / out projections) once, and twice again in the backward (input and weight
    gradients; the attention backward's four products); without knowledge insulation the prefix
    K/V projection's two backward products too."""
    S, A, D, Hq, Hkv = s.chunk, s.action_dim, s.head_dim, s.n_q_heads, s.n_kv_heads
    Ha, Hv, F, QKV = s.act_hidden, s.vlm_hidden, s.act_ffn, s.qkv_rows
    total = 0
    for P in (int(p) for p in lens):
        T = P + S
        dense = 2 * S * (Ha * QKV + Hq * D * Ha + 3 * Ha * F + 2 * Ha * A)
        attn = 2 * 2 * S * Hq * T * D
        kv = 2 * P * Hv * 2 * Hkv * D
        total += 3 * dense + attn + 2 * attn + kv + (0 if ki else 2 * kv)
    return total


def train_summary(reps=20, warmup=3, ki=False):
    """One flow-matching training step on the one-layer DM0-base merged layer (B=1, 816-token
    prefix + 50 action tokens, bf16 weights, float32 arithmetic), without knowledge insulation:
    ms per step from HIP events around every call, and the step's fp32 matrix-core fraction."""
    import torch
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import workload

    wl = workload(2)
    s = wl.shape
    vlm, aw, tb = inputs.make_vlm_weights(wl), inputs.make_action_weights(wl), inputs.make_train_batch(wl)
    ctx = bd.Context(s, 0)
    dvlm, daw = bd.DeviceExpert(vlm, s.dtype), bd.DeviceAction(aw, s.dtype)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    args = (dev(tb.h_pre), torch.from_numpy(tb.lens).cuda(), dev(tb.a), dev(tb.eps), dev(tb.t), dev(tb.mask))
    z = lambda shp: torch.empty(tuple(shp), dtype=torch.float32, device="cuda")
    grads = {"attn_norm": z(aw.body.attn_norm.shape[1:]), "w_qkv": z(aw.body.w_qkv.shape[1:]),
             "w_o": z(aw.body.w_o.shape[1:]), "mlp_norm": z(aw.body.mlp_norm.shape[1:]),
             "w_gate": z(aw.body.w_gate.shape[1:]), "w_up": z(aw.body.w_up.shape[1:]),
             "w_down": z(aw.body.w_down.shape[1:]), "w_in": z(aw.w_in.shape), "b_in": z(aw.b_in.shape),
             "final_norm": z(aw.final_norm.shape), "w_out": z(aw.w_out.shape), "b_out": z(aw.b_out.shape),
             "vlm_attn_norm": z(vlm.attn_norm.shape[1:]), "vlm_w_qkv": z(vlm.w_qkv.shape[1:]),
             "h_prefix": z(tb.h_pre.shape)}
    loss = z((1,))
    ws = ctx.workspace(bd.OP_TRAIN, wl.batch, wl.prefix_len)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            ctx.train_merged_layer(dvlm, daw, 0, *args, ki, loss, grads, ws, stream=stream)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            starts[i].record(stream)
            ctx.train_merged_layer(dvlm, daw, 0, *args, ki, loss, grads, ws, stream=stream)
            ends[i].record(stream)
        stream.synchronize()
    lat = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    flops = train_flops(s, tb.lens, ki)
    tfs = flops / (float(np.mean(lat)) * 1e-3) / 1e12
    del dvlm, daw, grads, ws
    ctx.close()
    torch.cuda.empty_cache()
    return {"workload": "flow-matching training step on one DM0-base merged layer, B=1, prefix 816 + 50 action "
                        "tokens, bf16 weights, fp32 arithmetic, no knowledge insulation",
            "ms_per_step": latency(lat), "steps_per_s": round(1e3 / float(np.mean(lat)), 2),
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS, 4), "algorithmic_flops_per_step": int(flops)},
            "dtype": "f32"}


def merged_layer_times(reps=20):
    """One DM0-base merged layer at batch 1 (816 prefix and 50 action tokens through both experts
    with the joint block-masked attention, prefix K/V written out): mean µs per dm_merged_layer
    call (HIP events around each call on its stream; the inputs are restored between calls,
    outside the timed spans) and the fraction of dense bf16 MFMA peak over its algorithmic FLOPs;
    the same for one replay of the call captured into a graph (graph_us)."""
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
    # the same call captured once into a graph (as a deployment captures its fixed-shape work)
    # and replayed: the GPU-side time without the host's per-launch cost
    g = torch.cuda.CUDAGraph()
    hp.copy_(hp0)
    hs.copy_(hs0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ctx.merged_layer(dv, da.body, 0, hp, hs, lens, ws, ko, vo)
    gtotal = 0.0
    cur = torch.cuda.current_stream()
    for r in range(reps + 1):
        hp.copy_(hp0)
        hs.copy_(hs0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        g.replay()
        e1.record(cur)
        cur.synchronize()
        if r > 0:  # the first replay uploads the graph
            gtotal += e0.elapsed_time(e1)
    del g
    ctx.close()
    us = total * 1e3 / reps
    graph_us = gtotal * 1e3 / reps
    D, Hq = s.head_dim, s.n_q_heads
    params = lambda h, f: s.qkv_rows * h + h * Hq * D + 3 * f * h
    flops = (2 * P * params(s.vlm_hidden, s.vlm_ffn) + 2 * S * params(s.act_hidden, s.act_ffn)
             + 4 * D * Hq * (P * P + S * (P + S)))
    return {"us": round(us, 2), "algorithmic_gflop": round(flops / 1e9, 2),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "graph_us": round(graph_us, 2),
            "graph_mfma_frac": round(flops / (graph_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "workload": "DM0-base merged layer, bf16, B=1, 816 prefix + 50 action tokens"}


def kernel_stats(config):
    """Per-kernel rows of the committed rocprofv3 summary for a denoise workload: name, calls per
    chunk, mean duration (us), share of the chunk; and the source hash it was taken at."""
    path = os.path.join(ROOT, "profiles", f"denoise_{'b1_p816' if config == 3 else 'b32_ragged'}_kernel_stats.txt")
    rows, src = [], None
    if not os.path.exists(path):
        return rows, src
    with open(path) as f:
        for line in f:
            if line.startswith("# source_hash"):
                src = line.split(":", 1)[1].strip()
                continue
            if line.startswith("#") or line.startswith("kernel"):
                continue
            parts = line.split()
            if len(parts) >= 7:
                try:
                    rows.append({"kernel": " ".join(parts[:-6]), "per_chunk": float(parts[-5]), "avg_us": float(parts[-4]),
                                 "pct": float(parts[-1])})
                except ValueError:
                    pass
    return rows, src


def b32_kernel_rooflines(wl, lens):
    """MFMA fraction of each GEMM kernel of the batch-32 chunk from the committed kernel
    statistics (mean duration per launch) and the algorithmic FLOPs of one launch; reported
    only while the kernel sources match the summary."""
    rows, src = kernel_stats(4)
    if not rows or src != source_hash():
        return None
    s = wl.shape
    M, H, F, Hq, D = wl.batch * s.chunk, s.act_hidden, s.act_ffn, s.n_q_heads, s.head_dim
    flops = {"EpiQkv": 2 * M * s.qkv_rows * H, "EpiSwiglu": 2 * M * 2 * F * H,
             "EpiResid": (2 * M * H * Hq * D + 2 * M * H * F) / 2}  # O and down alternate: mean per launch
    attn_flops = sum(4 * D * Hq * s.chunk * (int(p) + s.chunk) for p in lens)
    out = []
    for r in rows:
        k = next((e for e in flops if e in r["kernel"]), None)
        if k is None and "attn" not in r["kernel"]:
            continue
        f = flops[k] if k else attn_flops
        out.append({"kernel": r["kernel"][:60], "avg_us": r["avg_us"], "launches_per_chunk": r["per_chunk"],
                    "share_of_chunk": round(r["pct"] / 100, 4), "gflop_per_launch": round(f / 1e9, 3),
                    "mfma_frac": round(f / (r["avg_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)})
    return {"source": "profiles/denoise_b32_ragged_kernel_stats.txt", "kernels": out}


def run_denoise(config, steps, warmup):
    """Replays the captured denoise graph of one workload: HIP events around every replay on
    its stream, wall clock around the timed replays.  Returns (workload, lens, inputs, result)."""
    import torch
    from dual_expert_merged_amd import binding as bd
    from dual_expert_merged_amd import inputs
    from dual_expert_merged_amd.configs import workload

    wl = workload(config)
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
    x = torch.from_numpy(x1).cuda()
    ws = ctx.workspace(bd.OP_DENOISE, wl.batch, wl.prefix_len)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        plan = ctx.denoise_plan(da, k, v, ld, x, wl.steps, ws, stream=stream)
        log(f"[bench] {wl.name}: plan captured; warmup {warmup}, timed {steps}")
        for _ in range(warmup):
            plan.launch(stream=stream)
        stream.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            plan.launch(stream=stream)
            ends[i].record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    lat = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])  # ms per chunk, GPU clock
    plan.close()
    del k, v, ws, da
    ctx.close()
    torch.cuda.empty_cache()
    res = {"value": wl.batch * steps / wall, "ms": wall * 1e3 / steps, "lat": lat,
           "single_launch": config == 3}
    return wl, lens, (aw, kc, vc, x1), res


def latency(lat):
    return {"p50": round(float(np.percentile(lat, 50)), 4), "p90": round(float(np.percentile(lat, 90)), 4),
            "p99": round(float(np.percentile(lat, 99)), 4), "mean": round(float(np.mean(lat)), 4)}


def b1_roofline(wl, lens, lat):
    """Batch 1: one launch of the single-launch denoise kernel is one chunk (all 10 Euler steps,
    28 layers); the graph replay timed around it also holds the small kernel that clears its
    hand-off counters (a few us of the ~10 ms)."""
    alg = algorithmic(wl, lens)
    chunk_s = float(np.mean(lat)) * 1e-3
    gbs = alg["bytes"] / chunk_s / 1e9
    return {"bound": "hbm", "kernel": "dm::pk::denoise_b1_kernel (one launch = one chunk)",
            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(3), "algorithmic_bytes_per_launch": alg["bytes"],
            "launch_us": round(chunk_s * 1e6, 1)}


def b32_summary(steps=20, warmup=3):
    """The batch-32 ragged workload (MFMA-bound): chunks/s, latency, the whole chunk's MFMA and
    HBM fractions from live HIP events, per-kernel MFMA fractions from the committed profile, and
    the HBM traffic of one chunk from the committed counter summary."""
    wl, lens, _, res = run_denoise(4, steps, warmup)
    alg = algorithmic(wl, lens)
    chunk_s = float(np.mean(res["lat"])) * 1e-3
    tfs, gbs = alg["flops"] / chunk_s / 1e12, alg["bytes"] / chunk_s / 1e9
    return {"workload": wl.name, "value": round(res["value"], 2), "unit": "chunks/s", "steps": steps,
            "latency_ms": latency(res["lat"]),
            "roofline": {"bound": "mfma", "kernel": "all kernels of one chunk (graph replay)", "achieved": round(tfs, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                         "traffic": read_traffic(4), "algorithmic_flops_per_launch": alg["flops"],
                         "algorithmic_bytes_per_launch": alg["bytes"], "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
            "per_kernel": b32_kernel_rooflines(wl, lens)}


def tmod_summary(steps=20, warmup=3):
    """The time-modulated action expert (workload 7: DM0-base, B=4, 816-token prefix, 10 steps):
    chunks/s, latency and the chunk's HBM / MFMA fractions from live events."""
    wl, lens, _, res = run_denoise(7, steps, warmup)
    alg = algorithmic(wl, lens)
    chunk_s = float(np.mean(res["lat"])) * 1e-3
    gbs, tfs = alg["bytes"] / chunk_s / 1e9, alg["flops"] / chunk_s / 1e12
    return {"workload": wl.name, "value": round(res["value"], 2), "unit": "chunks/s", "steps": steps,
            "latency_ms": latency(res["lat"]),
            "roofline": {"bound": "hbm", "kernel": "all kernels of one chunk (graph replay)", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": alg["bytes"], "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}}


def qknorm_summary(steps=20, warmup=3):
    """The per-head QK-norm switch in both experts (workload 9: DM0-base, B=2, 816-token prefix,
    10 steps; the kernel sequence): chunks/s, latency and the chunk's HBM / MFMA fractions."""
    wl, lens, _, res = run_denoise(9, steps, warmup)
    alg = algorithmic(wl, lens)
    chunk_s = float(np.mean(res["lat"])) * 1e-3
    gbs, tfs = alg["bytes"] / chunk_s / 1e9, alg["flops"] / chunk_s / 1e12
    return {"workload": wl.name, "value": round(res["value"], 2), "unit": "chunks/s", "steps": steps,
            "latency_ms": latency(res["lat"]),
            "roofline": {"bound": "hbm", "kernel": "all kernels of one chunk (graph replay)", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": alg["bytes"], "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[3, 4],
                    help="the workload of the headline value (3: batch 1, 4: batch 32 ragged)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline workload only: no batch-32 and prefill sub-objects")
    ap.add_argument("--merged-layer", action="store_true",
                    help="time only one merged layer (both experts, B=1, 816 + 50 tokens) and print it")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the plain copy for counter scaling")
    ap.add_argument("--train-only", action="store_true",
                    help="time only the flow-matching training step on one merged layer and print it")
    ap.add_argument("--serving-only", action="store_true",
                    help="time only the fixed-contract engine (prefill + denoise, B=8) and print it")
    ap.add_argument("--prefill-only", choices=["both", "bf16", "fp8_mlp"],
                    help="time only the prefix encoding (B=8, 816 tokens) with the bf16 MLP, the FP8 MLP or both")
    ap.add_argument("--traffic-summary", action="store_true", help="summarise counter runs (no GPU needed)")
    ap.add_argument("--stats-summary", action="store_true", help="summarise a --kernel-trace --stats run (no GPU)")
    ap.add_argument("--counter-summary", action="store_true", help="summarise a --pmc (+ --kernel-trace) run (no GPU)")
    for name in ("fetch", "write", "cal-fetch", "cal-write", "stats-dir", "name", "title", "bench-args"):
        ap.add_argument("--" + name)
    ap.add_argument("--units", type=float, default=1.0)
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.stats_summary:
        stats_summary(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.prefill_only:
        modes = ("bf16", "fp8_mlp") if args.prefill_only == "both" else (args.prefill_only,)
        print(json.dumps({"prefill_ms": prefill_times(modes=modes)}), flush=True)
        return
    if args.merged_layer:
        print(json.dumps({"merged_layer": merged_layer_times()}), flush=True)
        return
    if args.serving_only:
        print(json.dumps({"serving": serving_summary()}), flush=True)
        return
    if args.train_only:
        print(json.dumps({"training": train_summary()}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the suffix denoise path is built for a single MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    wl, lens, (aw, kc, vc, x1), res = run_denoise(args.config, args.steps, args.warmup)
    s = wl.shape
    if args.config == 3:
        roof = b1_roofline(wl, lens, res["lat"])
    else:
        alg = algorithmic(wl, lens)
        tfs = alg["flops"] / (float(np.mean(res["lat"])) * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "all kernels of one chunk (graph replay)", "achieved": round(tfs, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                "traffic": read_traffic(4), "algorithmic_flops_per_launch": alg["flops"]}
    out = {
        "metric": "action chunks/s + p50 chunk latency (DM0-base suffix, 10 steps); % HBM/MFMA peak",
        "value": round(res["value"], 2), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "prefix_len": int(lens.max()),
                   "prefix_len_mean": float(lens.mean()), "chunk": s.chunk, "action_dim": s.action_dim,
                   "euler_steps": wl.steps, "layers": s.n_layers, "parallelism": "single GPU"},
        "latency_ms": latency(res["lat"]),
        "roofline": roof,
        "env": environment(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(wl, aw, kc, vc, x1, lens)
    del kc, vc
    if not args.no_extras:
        if args.config == 3:
            out["batch32"] = b32_summary()
        log("[bench] timing the time-modulated expert")
        out["time_modulated"] = tmod_summary()
        log("[bench] timing the QK-norm switch")
        out["qk_norm"] = qknorm_summary()
        log("[bench] timing one merged layer (both experts, B=1)")
        out["merged_layer"] = merged_layer_times()
        from dual_expert_merged_amd import inputs
        from dual_expert_merged_amd.configs import workload
        log("[bench] generating the VLM expert of the prefill workload")
        vlm = inputs.make_vlm_weights(workload(5))
        log("[bench] timing the prefix encoding (bf16 and FP8 MLP)")
        out["prefill_ms"] = prefill_times(vlm=vlm)
        log("[bench] timing the fixed-contract engine (prefill + denoise, B=8)")
        out["serving"] = serving_summary(vlm=vlm)
        del vlm
        log("[bench] timing the training step (one merged layer)")
        out["training"] = train_summary()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
