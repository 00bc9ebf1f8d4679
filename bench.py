#!/usr/bin/env python3
"""Decode benchmark of the W4A16 batch-1 decode step on one MI355X.

Workload: the Qwen2.5-7B-shaped decoder (28 layers, hidden 3584, MLP 18944,
28 q / 4 kv heads of 128, vocab 152064), random-init int4 group-128
projections with fp16 scales, fp16 embeddings / norms / lm_head.  A 512-token
seeded prompt is fed through the decode step (teacher-forced, untimed; its
last W steps are the warmup), then K greedy steps are timed, each one graph
replay of the whole step: one launch of the persistent decode kernel (plus a
one-thread page-append kernel on the steps that open a KV page).  Prints one
JSON line.

Also reported: the roofline of the persistent decode kernel (algorithmic
bytes of a step over its average duration, from HIP events recorded around
every timed step on the launch stream), its HBM traffic from the committed
rocprofv3 counter summary when that summary was taken on the current
kernel sources, eager-launch ms/token, per-kernel times of the kernel-per-op
variant, the standalone C-ABI calls on the single-GEMV, MLP and attention
shapes (w4a16_gemv, w4a16_mlp, paged_attn_decode; operands rotated over
>= 1 GiB of copies so the Infinity Cache cannot serve them), and the CPU
oracle timed on a bounded sample on the host cores.

Measurement modes (run by hand, results committed under profiles/):
  --measure-traffic   runs this file twice under `rocprofv3 --pmc` (FETCH_SIZE,
                      then WRITE_SIZE) with --traffic-probe, calibrates both
                      counters on a device-to-device copy of known size, and
                      writes profiles/decode_step_qwen7b_traffic.md
  --launch-study      eager launches vs graph replay of the persistent and the
                      kernel-per-op step at the same positions; writes
                      profiles/decode_step_qwen7b_launch_study.md
  --summarize-trace D writes the kernel statistics of a
                      `rocprofv3 --kernel-trace --stats -d D -o run` run of
                      this file to profiles/decode_step_qwen7b_persistent_kernel_stats.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, TFLOP/s
PAGES_PUBLISHED_TTFT_MS = 128.0  # the pages' runtime, 512-token prompt, H100 (context)
PAGES_PUBLISHED_TOKS = 60.0    # the pages' runtime on an H100 for this workload (context)
TRAFFIC_MD = os.path.join(HERE, "profiles", "decode_step_qwen7b_traffic.md")
STATS_MD = os.path.join(HERE, "profiles", "decode_step_qwen7b_persistent_kernel_stats.md")
PREFILL_MD = os.path.join(HERE, "profiles", "prefill_qwen7b_512_kernel_stats.md")
KERNEL = "decode_persistent_kernel"


def _a8_kernel(name: str) -> bool:
    """The int8-activation instantiation of the persistent kernel (kA8 = true)."""
    return KERNEL in name and ("<true>" in name or "ILb1E" in name)


def _f16_kernel(name: str) -> bool:
    return KERNEL in name and not _a8_kernel(name)
CALIB_BYTES = 256 << 20        # device-to-device copy used to calibrate the byte counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _profile_open(path: str):
    """Open a profiles/ summary for writing; a copy also lands in
    gpurun_out/profiles/ when that folder exists (results written on a remote
    machine come back only from there)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)

    class _Both:
        def __init__(self):
            self.fh = open(path, "w")
            out = os.path.join(HERE, "gpurun_out")
            self.copy = None
            if os.path.isdir(out):
                os.makedirs(os.path.join(out, "profiles"), exist_ok=True)
                self.copy = open(os.path.join(out, "profiles", os.path.basename(path)), "w")

        def write(self, text):
            self.fh.write(text)
            if self.copy:
                self.copy.write(text)

        def __enter__(self):
            return self

        def __exit__(self, *exc):
            self.fh.close()
            if self.copy:
                self.copy.close()
    return _Both()


def source_hash() -> str:
    """Hash of the HIP sources the library is built from (a traffic figure
    is only reported for the sources it was measured on)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(HERE, "int4_weight_only_dequant_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def step_bytes(dims, ctx_lo: int, ctx_hi: int) -> float:
    """Algorithmic HBM bytes of one decode step, averaged over ctx in [ctx_lo, ctx_hi]:
    every weight byte once (int4 codes + fp16 scales, fp16 bias / norms / lm_head),
    the embedding row, the KV cache read over the context and the new K/V written."""
    d, f, L = dims.d_model, dims.d_ff, dims.n_layers
    qkv_rows = dims.qkv_dim

    def w4(n, k):
        return n * k // 2 + n * (k // 128) * 2

    layer = w4(qkv_rows, d) + w4(d, dims.q_dim) + w4(2 * f, d) + w4(d, f)
    small = L * (2 * d * 2 + qkv_rows * 2) + d * 2 + d * 2            # norms, bias, final norm, embed row
    lm = dims.vocab * d * 2
    kv_per_tok = L * 2 * dims.n_kv_heads * dims.head_dim * 2
    mean_ctx = (ctx_lo + ctx_hi) / 2.0
    return L * layer + small + lm + kv_per_tok * mean_ctx + kv_per_tok


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_time(fn, reps: int) -> float:
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline(dims, glob_w, n_prompt: int = 512, pos: int = 576, sample_layers: int = 2):
    """The float64 numpy oracle on the host cores, on bounded samples of every
    workload (about 30 s of CPU work in all):

    * configs 0 and 1: oracle.gemv on the 3584 x 3584 GEMV and oracle.mlp on the
      MLP shapes, ms per call (the oracle dequantises inside each call);
    * config 2: oracle.paged_attention at context 640 (40 shuffled pages), ms per call;
    * config 3: the sequential decode step with the weights dequantised to fp64
      once before timing (the lm_head converted once): `sample_layers` decoder
      layers timed over 3 steps at position `pos`, extrapolated to every layer,
      plus the final norm, lm_head and argmax -> ms/token and tok/s (the headline
      `value`);
    * config 4: CPU "time to first token": the batched teacher-forced pass over
      the 512-token prompt, one decoder layer timed (dequantising as the oracle
      does) and extrapolated to every layer, plus the last row's lm_head.
    """
    import oracle
    import oracle.ref as oref
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    t_all = time.time()
    res = {}
    # config 0
    q, s_, x = synth.gemv_cfg0()
    res["cfg0_gemv_ms"] = round(_median_time(lambda: oracle.gemv(q, s_, x), 3) * 1e3, 2)
    # config 1
    m = synth.mlp_cfg1()
    res["cfg1_mlp_ms"] = round(_median_time(lambda: oracle.mlp(m["x"], m["gate"], m["up"], m["down"]), 2) * 1e3, 1)
    del m
    # config 2
    qa, kp, vp, table = synth.attn_cfg2()
    res["cfg2_attention_ms"] = round(_median_time(
        lambda: oracle.paged_attention(qa, kp, vp, table, 640, 1 / np.sqrt(128)), 3) * 1e3, 2)
    # config 3: weights dequantised once (fp64) before timing
    layers = [synth.layer_weights(dims, l) for l in range(sample_layers)]
    deq_cache = {}
    orig_deq = oref.deq

    def cached_deq(q_, s2, group=128):
        key = (id(q_), id(s2))
        if key not in deq_cache:
            deq_cache[key] = orig_deq(q_, s2, group)
        return deq_cache[key]

    n_pages = pos // 16 + 1
    rng = np.random.default_rng(7)
    cache = oracle.KVCache(dims, n_pages, np.arange(n_pages, dtype=np.int32))
    kv = rng.standard_normal(cache.k[0].shape, dtype=np.float32).astype(np.float16)
    for l in range(dims.n_layers):       # seeded filler; the oracle's cost does not depend on it
        cache.k[l] = kv
        cache.v[l] = kv
    lm64 = glob_w.lm_head.astype(np.float64)
    oref.deq = cached_deq
    try:
        x0 = glob_w.embed[123].astype(np.float64)
        for lw in layers:                # dequantise (untimed)
            x0 = oracle.layer_step(dims, lw, x0, pos, cache, 0)
        t_layer = []
        for _ in range(3):
            xx = glob_w.embed[123].astype(np.float64)
            for l, lw in enumerate(layers):
                t0 = time.perf_counter()
                xx = oracle.layer_step(dims, lw, xx, pos, cache, l)
                t_layer.append(time.perf_counter() - t0)
    finally:
        oref.deq = orig_deq
    deq_cache.clear()

    def head():
        xf = oracle.f16(oracle.rmsnorm(xx, glob_w.lnf, dims.eps))
        return oracle.argmax_first(lm64 @ xf.astype(np.float64))
    t_head = _median_time(head, 2)
    del lm64
    per_tok = dims.n_layers * float(np.mean(t_layer)) + t_head
    res["cfg3_ms_per_token"] = round(per_tok * 1e3, 1)
    # config 4: batched 512-token pass, one layer timed as the oracle runs it
    prompt = synth.prompt_ids(dims, n_prompt)
    one = synth.ModelDims(**{**dims.__dict__, "n_layers": 1, "vocab": 1})
    glob_small = synth.GlobalWeights(embed=glob_w.embed, lnf=glob_w.lnf, lm_head=glob_w.lm_head[:1])
    t0 = time.perf_counter()
    oracle.forward_teacher_forced(one, [layers[0]], glob_small, prompt, [n_prompt - 1])
    t_pass_layer = time.perf_counter() - t0
    ttft = dims.n_layers * t_pass_layer + t_head
    res["cfg4_ttft_s"] = round(ttft, 2)
    return {
        "value": round(1.0 / per_tok, 4), "unit": "tok/s", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"config 3: {sample_layers} of {dims.n_layers} decoder layers, weights dequantised to fp64 "
                   f"once before timing, 3 steps at position {pos}, extrapolated to {dims.n_layers} layers "
                   f"({np.mean(t_layer) * 1e3:.0f} ms per layer) + final norm, fp64 lm_head and argmax "
                   f"({t_head * 1e3:.0f} ms); config 4: 1 layer of the batched {n_prompt}-token pass "
                   f"({t_pass_layer:.2f} s, dequantising inside) x {dims.n_layers} + the lm_head"),
        "ms_per_token": round(per_tok * 1e3, 1),
        "configs": res,
        "cpu_model": _cpu_model(),
        "blas_threads": int(threads),
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "wall_s": round(time.time() - t_all, 1),
    }


def read_traffic():
    """Per-launch HBM bytes of the persistent kernel from the committed
    counter summary, or None if it was taken on other kernel sources."""
    try:
        with open(TRAFFIC_MD) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("source_hash") == source_hash():
                        return rec
    except OSError:
        pass
    return None


def build_model(dims, n_prompt, n_steps):
    import synth
    import int4_weight_only_dequant_amd as w4
    total_pos = n_prompt + n_steps
    max_pages = -(-total_pos // 16)
    t0 = time.time()
    log(f"[bench] generating + packing the model ({max_pages} KV pages)")
    glob_w = synth.global_weights(dims)
    free = synth.page_free_list(max_pages)
    model = w4.DecodeModel(dims, lambda l: synth.layer_weights(dims, l), glob_w, free, max_pages,
                           progress=lambda l: log(f"[bench] layer {l} uploaded ({time.time() - t0:.0f}s)")
                           if l % 7 == 6 else None)
    return model, glob_w, max_pages


def traffic_probe():
    """Child of --measure-traffic (runs under rocprofv3 --pmc): the prompt, 16
    persistent steps, then a device-to-device copy of CALIB_BYTES."""
    import torch
    import synth
    dims = synth.QWEN7B
    model, _, _ = build_model(dims, 512, 16)
    model.reset(synth.prompt_ids(dims, 512))
    for _ in range(512 + 16):
        model.step()
    torch.cuda.synchronize()
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    print("traffic probe done", flush=True)


def _pmc_rows(path):
    rows = list(csv.DictReader(open(path)))
    return rows


def _traffic_cmd(out_dir: str, ctr: str):
    d = os.path.join(out_dir, f"pmc_{ctr.lower()}")
    return d, ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", d, "-o", "pmc", "--",
               sys.executable, "-u", os.path.join(HERE, "bench.py"), "--traffic-probe"]


def measure_traffic(out_dir: str):
    """Two rocprofv3 --pmc runs of the traffic probe, then summarize_traffic."""
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        _, cmd = _traffic_cmd(out_dir, ctr)
        log("[bench] " + " ".join(cmd))
        env = dict(os.environ, TMPDIR="/tmp")
        r = subprocess.run(cmd, env=env, timeout=600)
        if r.returncode != 0:
            sys.exit(f"rocprofv3 {ctr} run failed ({r.returncode})")
    summarize_traffic(out_dir)


def summarize_traffic(out_dir: str):
    """Counter files of measure_traffic's two runs -> TRAFFIC_MD."""
    res = {}
    cmds = []
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d, cmd = _traffic_cmd(out_dir, ctr)
        cmds.append(" ".join(cmd[:-4] + ["python3", "-u", "bench.py", "--traffic-probe"]))
        files = glob.glob(os.path.join(d, "**", "pmc_counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no counter file under {d}")
        rows = _pmc_rows(files[0])
        kern = [float(r["Counter_Value"]) for r in rows if _f16_kernel(r["Kernel_Name"]) and r["Counter_Name"] == ctr]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == ctr]
        if len(kern) < 16 or not copy:
            sys.exit(f"{ctr}: {len(kern)} kernel dispatches, {len(copy)} copy dispatches")
        res[ctr] = {"kernel_kib": float(np.mean(kern[-16:])), "copy_kib": max(copy), "dispatches": len(kern)}
    f_scale = CALIB_BYTES / (res["FETCH_SIZE"]["copy_kib"] * 1024.0)
    w_scale = CALIB_BYTES / (res["WRITE_SIZE"]["copy_kib"] * 1024.0)
    fetch = res["FETCH_SIZE"]["kernel_kib"] * 1024.0 * f_scale
    write = res["WRITE_SIZE"]["kernel_kib"] * 1024.0 * w_scale
    import synth
    algo = step_bytes(synth.QWEN7B, 513, 528)
    rec = {"source_hash": source_hash(), "fetch_bytes": fetch, "write_bytes": write,
           "traffic_bytes": fetch + write, "algorithmic_bytes": algo,
           "fetch_kib_raw": res["FETCH_SIZE"]["kernel_kib"], "write_kib_raw": res["WRITE_SIZE"]["kernel_kib"],
           "copy_fetch_kib": res["FETCH_SIZE"]["copy_kib"], "copy_write_kib": res["WRITE_SIZE"]["copy_kib"],
           "fetch_scale": f_scale, "write_scale": w_scale}
    lines = [
        "# HBM traffic of the persistent decode kernel (rocprofv3 counters)", "",
        "Commands (from the repository root on one MI355X; each counter in a run of its own):", "",
        "```", "export TMPDIR=/tmp", *cmds, "```", "",
        "Both runs execute `bench.py --traffic-probe`: the Qwen2.5-7B-shaped model, the 512-token prompt",
        "through the decode step, 16 more steps (context 513-528), then one device-to-device copy of",
        f"{CALIB_BYTES} bytes (`__amd_rocclr_copyBuffer`) that calibrates the counters: it reads and writes",
        "exactly that many bytes, so each counter is scaled by copy bytes / counted bytes.", "",
        "| | FETCH_SIZE | WRITE_SIZE |", "|---|---:|---:|",
        f"| copy kernel, KiB counted | {res['FETCH_SIZE']['copy_kib']:.0f} | {res['WRITE_SIZE']['copy_kib']:.0f} |",
        f"| scale (copy bytes / counted bytes) | {f_scale:.4f} | {w_scale:.4f} |",
        f"| `{KERNEL}`, KiB per launch (mean of the last 16) | {res['FETCH_SIZE']['kernel_kib']:.0f} | "
        f"{res['WRITE_SIZE']['kernel_kib']:.0f} |",
        f"| `{KERNEL}`, scaled bytes per launch | {fetch:.4g} | {write:.4g} |", "",
        f"Traffic per launch {fetch + write:.4g} bytes against {algo:.4g} algorithmic bytes "
        f"({(fetch + write) / algo:.3f}x).", "",
        "The line below is read by bench.py, which reports the traffic only while the kernel sources",
        "still hash to `source_hash`.", "",
        "traffic-json: " + json.dumps(rec), ""]
    os.makedirs(os.path.dirname(TRAFFIC_MD), exist_ok=True)
    with _profile_open(TRAFFIC_MD) as fh:
        fh.write("\n".join(lines))
    print(json.dumps(rec), flush=True)


def summarize_trace(d: str, steps: int, cmd: str):
    """Kernel statistics of a --kernel-trace --stats run of this file; the
    persistent kernel's mean over its last `steps` dispatches (the timed
    steps) is listed beside its mean over all dispatches."""
    stats = glob.glob(os.path.join(d, "**", "run_kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "run_kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        sys.exit(f"no rocprofv3 csv files under {d}")
    rows = list(csv.DictReader(open(stats[0])))
    all_tr = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    tr = [r for r in all_tr if _f16_kernel(r["Kernel_Name"])]
    tr8 = [r for r in all_tr if _a8_kernel(r["Kernel_Name"])]
    dur = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr], dtype=np.float64) / 1e3
    dur8 = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr8], dtype=np.float64) / 1e3
    lines = ["# rocprofv3 kernel statistics: persistent decode step", "",
             "Command (run from the repository root on one MI355X):", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        if float(r["Percentage"]) < 0.01:
            continue
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"`{KERNEL}`: {len(dur)} dispatches; mean over all {dur.mean():.1f} us; "
              f"mean over the last {steps} (the timed steps, context 513-{512 + steps}) "
              f"{dur[-steps:].mean():.1f} us (min {dur[-steps:].min():.1f}, max {dur[-steps:].max():.1f}).", "",
              "The earlier dispatches are the teacher-forced prompt (contexts 1-512, 16 of them eager",
              "launches) and the warmup; the kernel-per-op rows are the timing-hook replays of that variant.", ""]
    if len(dur8):
        lines += [f"The int8-activation instantiation (`W4_A8`, timed after the fp16 steps): {len(dur8)} dispatches, "
                  f"mean {dur8.mean():.1f} us (min {dur8.min():.1f}, max {dur8.max():.1f}).", ""]
    os.makedirs(os.path.dirname(STATS_MD), exist_ok=True)
    with _profile_open(STATS_MD) as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_prefill_trace(d: str, cmd: str):
    """Per-kernel times of the last 512-token prefill in a kernel trace of this
    file (the bench runs the prefill 4 times before the decode steps)."""
    import collections
    path = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if "pf_embed_kernel" in r["Kernel_Name"]]
    s = starts[-1]
    e = next(i for i in range(s, len(rows)) if "finalize_kernel" in rows[i]["Kernel_Name"]) + 1
    agg, cnt = collections.defaultdict(float), collections.Counter()
    per_layer = collections.defaultdict(list)
    gemm_kind = ["QKV (N=4608, K=3584)", "O (N=3584, K=3584)", "gate+up + SwiGLU (N=37888, K=3584)",
                 "down (N=3584, K=18944)"]
    gi = 0
    for r in rows[s:e]:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        k = r["Kernel_Name"].split("(")[0].replace("w4::", "").replace("void ", "")
        agg[k] += us
        cnt[k] += 1
        if "w4_gemm_kernel" in k:
            per_layer[gemm_kind[gi % 4]].append(us)
            gi += 1
    span = (int(rows[e - 1]["End_Timestamp"]) - int(rows[s]["Start_Timestamp"])) / 1e3
    flops = {"QKV (N=4608, K=3584)": 2 * 512 * 4608 * 3584, "O (N=3584, K=3584)": 2 * 512 * 3584 * 3584,
             "gate+up + SwiGLU (N=37888, K=3584)": 2 * 512 * 37888 * 3584,
             "down (N=3584, K=18944)": 2 * 512 * 3584 * 18944}
    out = ["# Prefill of a 512-token prompt, Qwen2.5-7B shape: kernel times", "",
           "Command (from the repository root on one MI355X):", "", "```", cmd, "```", "",
           f"Last of the bench's 4 prefill calls: {e - s} dispatches, first-to-last span {span:.1f} us "
           f"(kernel time {sum(agg.values()):.1f} us).", "",
           "| kernel | calls | total us | us/call |", "|---|---|---|---|"]
    for k, v in sorted(agg.items(), key=lambda x: -x[1]):
        out.append(f"| `{k}` | {cnt[k]} | {v:.1f} | {v / cnt[k]:.2f} |")
    out += ["", "W4A16 GEMM per projection (mean over the 28 layers; fp16 MFMA peak 2500 TFLOP/s):", "",
            "| projection | us | TFLOP/s | fraction of peak |", "|---|---|---|---|"]
    for k, v in per_layer.items():
        m = sum(v) / len(v)
        tf = flops[k] / (m * 1e-6) / 1e12
        out.append(f"| {k} | {m:.1f} | {tf:.0f} | {tf / MFMA_F16_PEAK_TFLOPS:.3f} |")
    os.makedirs(os.path.dirname(PREFILL_MD), exist_ok=True)
    with _profile_open(PREFILL_MD) as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def long_context(args):
    """The long-context workload: TTFT of a 512-token prompt (one prefill from
    an empty cache), then a ctx-token prompt filled by 512-token prefill chunks
    over a shuffled page table, and args.steps greedy graph steps timed at
    positions ctx .. ctx + steps - 1.  Prints one JSON line."""
    import torch
    import synth
    from int4_weight_only_dequant_amd import _lib as L

    dims = synth.QWEN7B
    ctx = args.context
    t0 = time.time()
    model, _, max_pages = build_model(dims, ctx, args.steps)
    prompt = synth.prompt_ids(dims, ctx)
    stream = torch.cuda.current_stream()
    ttft = []
    for r in range(4):
        model.reset(prompt[:512])
        torch.cuda.synchronize()
        tp = time.perf_counter()
        model.prefill(512)
        torch.cuda.synchronize()
        if r:
            ttft.append((time.perf_counter() - tp) * 1e3)
    model.reset(prompt)
    fill_to = ctx - args.warmup
    torch.cuda.synchronize()
    tf = time.perf_counter()
    while model.pos < fill_to:
        model.prefill(min(512, fill_to - model.pos))
    torch.cuda.synchronize()
    fill_ms = (time.perf_counter() - tf) * 1e3
    for _ in range(args.warmup):
        model.step(L.W4_GRAPH)
    torch.cuda.synchronize()
    log(f"[bench] {ctx}-token context filled by prefill chunks in {fill_ms:.1f} ms; warmup {args.warmup} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    tstart = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        model.step(L.W4_GRAPH)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - tstart
    assert model.device_error() == 0, "device error during the timed steps"
    step_us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)])
    boundary = np.array([(ctx + i) % 16 == 0 for i in range(args.steps)])
    kern_us = float(step_us[~boundary].mean())
    gen = model.tokens[ctx: ctx + 8].cpu().numpy()
    model.close()
    sb = step_bytes(dims, ctx + 1, ctx + args.steps)
    achieved = sb / (kern_us * 1e-6) / 1e9
    line = {
        "metric": f"decode ms/token & tok/s at {ctx}-token context (batch 1); TTFT of a 512-token prompt",
        "value": round(args.steps / elapsed, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded random-init weights of the Qwen2.5-7B shapes, uniform random prompt ids)",
        "config": {"workload": f"Qwen2.5-7B-shaped W4A16 decode step, batch 1, {ctx}-token prompt filled by "
                               f"512-token prefill chunks, {args.steps} greedy graph-captured steps",
                   "context": f"{ctx + 1}-{ctx + args.steps}", "kv_pages": max_pages, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": f"{KERNEL} (the whole decode step, one launch per token)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(sb), "avg_launch_us": round(kern_us, 2)},
        "ttft_ms": round(float(np.median(ttft)), 3), "fill_ms": round(fill_ms, 2),
        "tokens_head": [int(t) for t in gen],
    }
    log(f"[bench] done in {time.time() - t0:.0f}s")
    print(json.dumps(line), flush=True)



# ------------------------------------------------------------------------------------------
# Phase timestamps of the persistent decode kernel (trace build: libw4a16_trace.so, built by
# `python -m int4_weight_only_dequant_amd.build --trace`).  Runs the 512-token prompt through
# the step and 8 more steps, then reads the last step's timestamps and summarises, per phase
# kind and averaged over layers 1-27, where the time goes.

TRACE_MD = os.path.join(HERE, "profiles", "decode_step_qwen7b_phase_trace.md")


def phase_trace(write_md: bool = True, context: int = 512):
    import ctypes
    import torch
    import synth
    from int4_weight_only_dequant_amd import _lib, build as w4build
    if not os.path.exists(w4build.TRACE_LIB):
        sys.exit(f"{w4build.TRACE_LIB} is not built: run `python -m int4_weight_only_dequant_amd.build --trace`")
    _lib.LIB_PATH = w4build.TRACE_LIB
    L = _lib
    lib = L.lib()
    lib.w4_model_trace_copy.restype = ctypes.c_int
    lib.w4_model_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    dims = synth.QWEN7B
    n_prompt, n_extra = context, 8
    model, _, _ = build_model(dims, n_prompt, n_extra)
    model.reset(synth.prompt_ids(dims, n_prompt))
    if context == 512:
        for _ in range(n_prompt + n_extra):
            model.step(L.W4_GRAPH)
    else:   # a long prompt goes through the prefill, as in the long-context workload
        while model.pos < n_prompt - 1:
            model.prefill(min(512, n_prompt - 1 - model.pos))
        for _ in range(1 + n_extra):
            model.step(L.W4_GRAPH)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    P, n_ph = model.grid(), 4 * dims.n_layers + 1
    tr = np.zeros((P, n_ph, 8), dtype=np.uint64)
    L.check(lib.w4_model_trace_copy(model._m, tr.ctypes.data, tr.nbytes))
    pos = model.pos - 1
    model.close()
    raw_dir = os.path.join(HERE, "gpurun_out")
    if os.path.isdir(raw_dir):
        np.save(os.path.join(raw_dir, "pk_trace.npy"), tr)
    t = tr.astype(np.float64)
    t0 = t[:, 0, 0].min()
    t_end = t[:, :, :].max()
    valid = t >= t0                                  # stale slots (earlier steps / not reached) are older
    us = np.where(valid, (t - t0) / 100.0, np.nan)   # 100 MHz ticks -> us since the kernel's first stamp
    kinds = ["QKV", "O", "gate+up", "down"]

    def med(a):
        a = a[~np.isnan(a)]
        return float(np.median(a)) if a.size else float("nan")

    def mx(a):
        a = a[~np.isnan(a)]
        return float(a.max()) if a.size else float("nan")

    sig_last = np.array([mx(us[:, ph, 4]) for ph in range(n_ph)])
    rows = {k: [] for k in kinds}
    att = []
    for l in range(1, dims.n_layers):
        for kind in range(4):
            ph = 4 * l + kind
            prev = sig_last[ph - 1]
            # dependency: QKV and gate+up wait for every work-group of the phase before
            # (down, O); O waits for attention heads; down for gate+up
            waited, staged, tiles, sig = us[:, ph, 1], us[:, ph, 2], us[:, ph, 3], us[:, ph, 4]
            dep_ref = prev if kind != 1 else mx(us[:, ph, 6])
            rows[kinds[kind]].append([
                med(waited) - dep_ref,              # last producer signal -> median wait passed
                med(staged - waited),               # staging
                med(tiles - staged),                # wave 0's tiles
                med(sig - tiles),                   # reduce + atomics + signal
                mx(sig) - med(sig),                 # tail: median -> last signal
                sig_last[ph] - prev,                # phase span (last signal to last signal)
            ])
            if kind == 1:
                a0, a1 = us[:, ph, 5], us[:, ph, 6]
                att.append([med(a1 - a0), mx(a1) - sig_last[ph - 1], mx(a1) - med(a1)])
    hdr = ("| phase | producer's last signal -> median wait passed (us) | staging (us) | wave 0 tiles (us) | "
           "reduce + signal (us) | median -> last signal (us) | span, last signal to last signal (us) |")
    lines = [hdr, "|---|---:|---:|---:|---:|---:|---:|"]
    for k in kinds:
        a = np.nanmean(np.array(rows[k]), axis=0)
        lines.append(f"| {k} | " + " | ".join(f"{v:.2f}" for v in a) + " |")
    a = np.nanmean(np.array(att), axis=0)
    per_layer = (sig_last[4 * dims.n_layers - 1] - sig_last[3]) / (dims.n_layers - 1)
    lm = sig_last[n_ph - 1] - sig_last[n_ph - 2]
    first = sig_last[3]
    summary = {"position": pos, "grid": P, "kernel_us": round((t_end - t0) / 100.0, 1),
               "layer0_us": round(first, 2), "per_layer_us": round(per_layer, 2), "lm_head_us": round(lm, 2),
               "attention_unit_us": round(float(a[0]), 2),
               "attention_last_publish_after_qkv_us": round(float(a[1]), 2)}
    log(f"[trace] {json.dumps(summary)}")
    for ln in lines:
        log(ln)
    if write_md:
        md = TRACE_MD if context == 512 else TRACE_MD.replace(".md", f"_{context}.md")
        with _profile_open(md) as fh:
            fh.write(f"# Phase timeline of the persistent decode kernel (Qwen2.5-7B shape, context {pos + 1})\n\n")
            fh.write("Command (from the repository root on one MI355X, after `python -m "
                     "int4_weight_only_dequant_amd.build --trace` on the build host):\n\n")
            fh.write("```\npython3 -u bench.py --phase-trace" + ("" if context == 512 else f" --context {context}")
                     + "\n```\n\n")
            fh.write("The trace build records, in wave 0 of every work-group, the 100 MHz real-time counter "
                     "at the top of each phase, when its dependency wait passes, when its input is staged, "
                     "when wave 0's tiles are done and when the work-group's completion is signalled "
                     "(attention work-groups also around the attention).  One step at position "
                     f"{pos}; phases of layers 1-27 averaged per kind; medians and maxima over the work-groups.\n\n")
            fh.write(f"Kernel {summary['kernel_us']} us (trace build); layer 0 done at {summary['layer0_us']} us; "
                     f"{summary['per_layer_us']} us per layer; lm_head phase {summary['lm_head_us']} us.\n"
                     f"Attention: a (head, chunk) unit takes {summary['attention_unit_us']} us from its start "
                     f"(before its QKV wait) to publishing; the last unit publishes "
                     f"{summary['attention_last_publish_after_qkv_us']} us after the last QKV signal.\n\n")
            fh.write("\n".join(lines) + "\n")
    return summary


LAUNCH_MD = os.path.join(HERE, "profiles", "decode_step_qwen7b_launch_study.md")
PAGES_EAGER_MS, PAGES_GRAPH_MS = 119.0, 17.0   # the pages' eager and graph ms/token on an H100 (context)


def launch_study(args):
    """Eager launches vs graph replay, for the persistent and the kernel-per-op step.

    Each variant starts from the same state (the 512-token prompt prefilled by
    one prefill call), runs 8 untimed steps and then times args.steps greedy
    steps from position 520, so all four see the same positions and contexts.
    Wall clock with device synchronisation at both ends; the graph variants also
    get HIP events per step on the launch stream."""
    import torch
    import synth
    from int4_weight_only_dequant_amd import _lib as L
    dims = synth.QWEN7B
    n_prompt, n_warm = 512, 8
    model, _, _ = build_model(dims, n_prompt, n_warm + args.steps)
    prompt = synth.prompt_ids(dims, n_prompt)
    stream = torch.cuda.current_stream()
    variants = (("persistent, graph replay", L.W4_GRAPH), ("persistent, eager launch", L.W4_EAGER),
                ("kernel-per-op, graph replay", L.W4_MULTI | L.W4_GRAPH),
                ("kernel-per-op, eager launch", L.W4_MULTI | L.W4_EAGER))
    rows, toks = [], {}
    p0 = n_prompt + n_warm
    for name, flags in variants:
        # pass 1: steps enqueued back to back; pass 2: the host waits for every
        # step's token before enqueuing the next (a serving loop that inspects it)
        res = {}
        for synced in (False, True):
            model.reset(prompt)
            model.prefill(n_prompt)
            for _ in range(n_warm):
                model.step(flags)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            enq = 0.0
            t0 = time.perf_counter()
            for i in range(args.steps):
                ev[i].record(stream)
                te = time.perf_counter()
                model.step(flags)
                enq += time.perf_counter() - te
                if synced:
                    torch.cuda.synchronize()
            ev[-1].record(stream)
            torch.cuda.synchronize()
            res[synced] = ((time.perf_counter() - t0) * 1e3 / args.steps,
                           ev[0].elapsed_time(ev[-1]) / args.steps, enq * 1e6 / args.steps)
            assert model.device_error() == 0, f"device error in {name}"
            if not synced:
                toks[name] = model.tokens[p0 + 1: p0 + args.steps + 1].cpu().numpy()
        ms, dev_ms, enq_us = res[False]
        launches = model.launches_per_step(flags & L.W4_MULTI)
        rows.append({"variant": name, "launches_per_step": launches, "ms_per_token": round(ms, 4),
                     "tok_s": round(1e3 / ms, 1), "device_ms_per_token": round(dev_ms, 4),
                     "host_enqueue_us_per_step": round(enq_us, 1),
                     "host_enqueue_us_per_step_host_sync": round(res[True][2], 1),
                     "ms_per_token_host_sync_each_step": round(res[True][0], 4)})
        log(f"[launch] {name}: {launches} launches, {ms:.3f} ms/token (events {dev_ms:.3f}), host enqueue "
            f"{enq_us:.1f} us/step; {res[True][0]:.3f} ms/token with a host sync per step (host enqueue "
            f"{res[True][2]:.1f} us/step)")
    model.close()
    ref = toks[variants[0][0]]
    for r in rows:
        r["tokens_equal_persistent_graph"] = bool(np.array_equal(toks[r["variant"]], ref))
    by = {r["variant"]: r for r in rows}
    ratio_multi = by["kernel-per-op, eager launch"]["ms_per_token"] / by["kernel-per-op, graph replay"]["ms_per_token"]
    ratio_sync = (by["kernel-per-op, eager launch"]["ms_per_token_host_sync_each_step"] /
                  by["kernel-per-op, graph replay"]["ms_per_token_host_sync_each_step"])
    fused = by["kernel-per-op, graph replay"]["ms_per_token"] / by["persistent, graph replay"]["ms_per_token"]
    summary = {"positions": f"{n_prompt + n_warm}-{n_prompt + n_warm + args.steps - 1}", "variants": rows,
               "eager_over_graph_kernel_per_op": round(ratio_multi, 2),
               "eager_over_graph_kernel_per_op_host_sync": round(ratio_sync, 2),
               "kernel_per_op_graph_over_persistent_graph": round(fused, 2),
               "pages_eager_over_graph": round(PAGES_EAGER_MS / PAGES_GRAPH_MS, 2)}
    print(json.dumps({"launch_study": summary}), flush=True)
    with _profile_open(LAUNCH_MD) as fh:
        fh.write("# Eager launches vs graph replay of the decode step (Qwen2.5-7B shape)\n\n")
        fh.write("Command (from the repository root on one MI355X):\n\n")
        fh.write(f"```\npython3 -u bench.py --launch-study --steps {args.steps}\n```\n\n")
        fh.write("Every variant starts from the same 512-token prompt (one prefill call), runs 8 untimed "
                 f"greedy steps and times {args.steps} more at positions {summary['positions']}; ms/token is "
                 "wall clock with device synchronisation at both ends, `events` the HIP events on the "
                 "launch stream, `host enqueue` the host time inside the decode_step calls (back to back it "
                 "includes waiting for room in the launch queue while the device is behind).  A second pass "
                 "over the same positions waits on the host for every step before enqueuing the next, so its "
                 "enqueue time is the host's own cost per step.  "
                 "Launches per step exclude the page append of steps that open a KV page.\n\n")
        fh.write("| variant | launches per step | ms/token | tok/s | events ms/token | host enqueue us/step | "
                 "ms/token, host sync per step | host enqueue us/step, host sync per step | "
                 "tokens equal to the persistent graph |\n")
        fh.write("|---|---:|---:|---:|---:|---:|---:|---:|---|\n")
        for r in rows:
            fh.write(f"| {r['variant']} | {r['launches_per_step']} | {r['ms_per_token']} | {r['tok_s']} | "
                     f"{r['device_ms_per_token']} | {r['host_enqueue_us_per_step']} | "
                     f"{r['ms_per_token_host_sync_each_step']} | {r['host_enqueue_us_per_step_host_sync']} | "
                     f"{r['tokens_equal_persistent_graph']} |\n")
        fh.write(f"\nKernel-per-op step, eager over graph: {summary['eager_over_graph_kernel_per_op']}x "
                 f"({summary['eager_over_graph_kernel_per_op_host_sync']}x with a host sync per step) "
                 f"(the pages: {PAGES_EAGER_MS:.0f} vs {PAGES_GRAPH_MS:.0f} ms/token on an H100, "
                 f"{summary['pages_eager_over_graph']}x).  Kernel-per-op graph over the persistent graph: "
                 f"{summary['kernel_per_op_graph_over_persistent_graph']}x.\n")
    return summary


SA_MD = os.path.join(HERE, "profiles", "standalone_calls_kernel_stats.md")


def summarize_standalone_trace(d: str, cmd: str):
    """Per-call kernel durations of a --kernel-trace run of `bench.py --standalone-only`
    (the calls run in a fixed order, so dispatches of equal grids are told apart by it)."""
    trace = glob.glob(os.path.join(d, "**", "run_kernel_trace.csv"), recursive=True)
    if not trace:
        sys.exit(f"no rocprofv3 kernel trace under {d}")
    rows = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    seq = [(r["Kernel_Name"], r["Grid_Size_X"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
           for r in rows if any(k in r["Kernel_Name"] for k in ("sg_gemv", "attn_decode", "a8_quantize"))]
    B = {"w4a16_gemv 3584x3584 (config 0)": 6637568, "w4a16_gemv 37888x3584": 70099968,
         "w4a16_gemv 3584x18944": 35053568, "w4a16_mlp: gate+up with SwiGLU": 70062080,
         "w4a16_mlp: down": 35053568, "w4a8_gemv 3584x3584": None, "w4a8_gemv 37888x3584": None,
         "w4a8_gemv 3584x18944": None, "w4a8_quantize_act": None,
         "paged_attn_decode ctx 640 (config 2)": 1325216, "paged_attn_decode ctx 8192": 16793600}
    groups = {k: [] for k in B}

    def n_disp(n, k):
        # dispatches of one shape in standalone_kernels: 2 eager calls, 1 + 3 replays of
        # R captured calls, and the check call
        r = max(2, -(-ROTATE_BYTES // (n * k // 2 + n * (k // 128) * 2)))
        return 2 + 4 * r + 1

    full = str(512 * 256)              # the large shapes run the full 512-work-group grid
    att_grids = sorted({int(g) for n_, g, _ in seq if "attn_decode" in n_})
    n_gu, n_dn = n_disp(37888, 3584), n_disp(3584, 18944)
    n16 = 0
    a8_grids = []
    for name, grid, t in seq:
        if "attn_decode" in name:
            # context 640 launches fewer splits than context 8192
            groups["paged_attn_decode ctx 640 (config 2)" if int(grid) < att_grids[-1]
                   else "paged_attn_decode ctx 8192"].append(t)
        elif "a8_quantize" in name:
            groups["w4a8_quantize_act"].append(t)
        elif "EpiStoreF16, true" in name:   # the int8-activation GEMV
            a8_grids.append((grid, t))
        elif "SwiGLU" in name:
            groups["w4a16_mlp: gate+up with SwiGLU"].append(t)
        elif grid != full:
            groups["w4a16_gemv 3584x3584 (config 0)"].append(t)
        else:
            n16 += 1
            k = ("w4a16_gemv 37888x3584" if n16 <= n_gu else "w4a16_gemv 3584x18944" if n16 <= n_gu + n_dn
                 else "w4a16_mlp: down")
            groups[k].append(t)
    # int8-activation GEMVs in call order: 3584x3584 (the smaller grid), then 37888x3584, then 3584x18944
    n_big = 0
    for grid, t in a8_grids:
        if grid != full:
            groups["w4a8_gemv 3584x3584"].append(t)
        else:
            n_big += 1
            groups["w4a8_gemv 37888x3584" if n_big <= n_gu else "w4a8_gemv 3584x18944"].append(t)
    for k, n, kk in (("w4a8_gemv 3584x3584", 3584, 3584), ("w4a8_gemv 37888x3584", 37888, 3584),
                     ("w4a8_gemv 3584x18944", 3584, 18944)):
        act = (kk + 255) // 256 * 256 + (kk // 32 + 255) // 256 * 256 + kk // 32   # w4a8_act_bytes(K)
        B[k] = n * kk // 2 + n * (kk // 128) * 2 + act + n * 2
    lines = ["# Standalone C-ABI calls: kernel durations (GEMV, MLP, int8-activation GEMV, paged attention)", "",
             "Command (from the repository root on one MI355X):", "", "```", cmd, "```", "",
             "`bench.py --standalone-only` calls `w4a16_gemv` on the single-GEMV shape (3584 x 3584) and on the",
             "two MLP shapes, `w4a16_mlp` (gate+up with the SwiGLU epilogue, then down: two launches of",
             "`sg_gemv_kernel`), `w4a8_quantize_act` + `w4a8_gemv` on the same three shapes, and",
             "`paged_attn_decode` at contexts 640 and 8192.  Each call reads its own copy of the weights (or its",
             "own pages of one large pool): the copies total at least 1 GiB, so no call finds its operands in the",
             "256 MB Infinity Cache.  The calls are captured into one graph per shape and replayed (2 eager calls",
             "first, then 1 + 3 replays, then one check call).  Durations are rocprofv3's kernel begin/end per",
             "dispatch; algorithmic",
             "bytes are int4 codes + fp16 scales + activations in (int8 codes, scales and sums for the int8 path)",
             "+ fp16 outputs; attention: the K and V pages of the context, q, o and the page table.", "",
             "| call | dispatches | mean us | median us | min us | algorithmic bytes | GB/s (mean) | fraction of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for k, v in groups.items():
        if not v:
            continue
        srt = sorted(v)
        m = sum(v) / len(v)
        if B[k]:
            lines.append(f"| {k} | {len(v)} | {m:.2f} | {srt[len(srt) // 2]:.2f} | {srt[0]:.2f} | {B[k]:,} | "
                         f"{B[k] / m / 1e3:.0f} | {B[k] / m / 1e3 / HBM_PEAK_GBS:.3f} |")
        else:
            lines.append(f"| {k} | {len(v)} | {m:.2f} | {srt[len(srt) // 2]:.2f} | {srt[0]:.2f} | - | - | - |")
    with _profile_open(SA_MD) as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------------------------------
# Standalone calls of configs 0-2 through the C ABI, rotating over distinct copies of the
# operands (>= 1 GiB in total) so that no call finds its weights or pages in the 256 MB
# Infinity Cache; R calls are captured in one graph and the graph replayed.

ROTATE_BYTES = 1 << 30


def _w4_bytes(n, k):
    """Algorithmic bytes of one W4A16 GEMV: codes, scales, x and the fp16 output."""
    return n * k // 2 + n * (k // 128) * 2 + k * 2 + n * 2


def _graph_time_us(torch, calls, reps=3):
    """Mean time per call of a list of launch closures, captured once into a
    graph and replayed `reps` times (after one warmup replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls[:2]:
            c()          # eager warmup outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(calls))
    del g
    return us


def standalone_kernels(attention: bool = True):
    """Configs 0-2 through w4a16_gemv, w4a16_mlp and paged_attn_decode."""
    import torch
    import synth
    import int4_weight_only_dequant_amd as w4
    from int4_weight_only_dequant_amd import _lib as L

    lib = L.lib()
    dev = torch.device("cuda")
    out = {}

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def rotated(arr_u8, copies):
        """[copies, nbytes] device buffer, every row a copy of arr_u8."""
        t = torch.from_numpy(np.ascontiguousarray(arr_u8).view(np.uint8).reshape(-1)).to(dev)
        buf = torch.empty((copies, t.numel()), dtype=torch.uint8, device=dev)
        buf.copy_(t.unsqueeze(0).expand(copies, -1))
        return buf

    def gemv_entry(name, n, k, pq, ps):
        nb = pq.nbytes + ps.nbytes
        R = max(2, -(-ROTATE_BYTES // nb))
        bq, bs = rotated(pq, R), rotated(ps, R)
        x = torch.from_numpy(synth.normal_f16(synth.rng(0, synth.GLOBAL_LAYER, synth.T_X), (k,))).to(dev)
        y = torch.empty(n, dtype=torch.float16, device=dev)
        ws = torch.zeros(max(lib.w4_gemv_ws_bytes(n, k), 256), dtype=torch.uint8, device=dev)

        def mk(r):
            def c():
                L.check(lib.w4a16_gemv(bq[r].data_ptr(), bs[r].data_ptr(), x.data_ptr(), y.data_ptr(), n, k,
                                       ws.data_ptr(), ws.numel(), cur()))
            return c
        us = _graph_time_us(torch, [mk(r) for r in range(R)])
        # the replays did the whole call: the last one's output equals a call
        # on a fresh workspace
        want = w4.w4a16_gemv(bq[R - 1], bs[R - 1], x, n, k)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"{name}: replayed output differs"
        b = _w4_bytes(n, k)
        out[name] = {"N": n, "K": k, "us_per_call": round(us, 2), "bytes": b,
                     "GBps": round(b / (us * 1e-6) / 1e9, 1), "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "copies": R}
        del bq, bs

    # config 0: one 3584 x 3584 GEMV
    q, s, _ = synth.gemv_cfg0()
    pq, ps = w4.pack_int4_weights(q, s)
    gemv_entry("gemv_3584x3584", 3584, 3584, pq, ps)
    # config 1 shapes as single GEMVs (fp16 output), then the MLP call
    m = synth.mlp_cfg1()
    d, f = 3584, 18944
    cfg = L.ModelConfig(d_model=d, d_ff=f, n_layers=1, n_q_heads=28, n_kv_heads=4, head_dim=128,
                        vocab=1, max_pages=1, eps=1e-6, theta=1e6)
    perm = w4.model_row_perm(L.W4_PERM_GATE_UP, cfg)
    pgq, pgs = w4.pack_int4_weights(np.concatenate([m["gate"][0], m["up"][0]]),
                                    np.concatenate([m["gate"][1], m["up"][1]]), row_perm=perm)
    pdq, pds = w4.pack_int4_weights(*m["down"])
    gemv_entry("gemv_gate_up_37888x3584", 2 * f, d, pgq, pgs)
    gemv_entry("gemv_down_3584x18944", d, f, pdq, pds)
    nb = pgq.nbytes + pgs.nbytes + pdq.nbytes + pds.nbytes
    R = max(2, -(-ROTATE_BYTES // nb))
    bgq, bgs, bdq, bds = rotated(pgq, R), rotated(pgs, R), rotated(pdq, R), rotated(pds, R)
    x = torch.from_numpy(m["x"]).to(dev)
    h = torch.empty(f, dtype=torch.float16, device=dev)
    y = torch.empty(d, dtype=torch.float16, device=dev)
    ws = torch.zeros(max(lib.w4_mlp_ws_bytes(d, f), 256), dtype=torch.uint8, device=dev)

    def mk_mlp(r):
        def c():
            L.check(lib.w4a16_mlp(bgq[r].data_ptr(), bgs[r].data_ptr(), bdq[r].data_ptr(), bds[r].data_ptr(),
                                  x.data_ptr(), h.data_ptr(), y.data_ptr(), d, f, ws.data_ptr(), ws.numel(), cur()))
        return c
    us = _graph_time_us(torch, [mk_mlp(r) for r in range(R)])
    _, want = w4.w4a16_mlp(bgq[R - 1], bgs[R - 1], bdq[R - 1], bds[R - 1], x, d, f)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), want.view(torch.int16)), "mlp: replayed output differs"
    # weights and scales of both matrices, x, h written and read back, y
    b = 2 * f * d // 2 + 2 * f * (d // 128) * 2 + d * f // 2 + d * (f // 128) * 2 + 2 * d + 2 * (2 * f) + 2 * d
    out["mlp_cfg1"] = {"D": d, "F": f, "us_per_call": round(us, 2), "bytes": b,
                       "GBps": round(b / (us * 1e-6) / 1e9, 1), "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "launches": 3, "copies": R}
    del bgq, bgs, bdq, bds

    # int8 activations (the pages' integer path) on the config 0 and config 1 shapes: the
    # quantisation launch and the GEMV, each timed alone
    for name, (n, k, pq_, ps_) in (("w4a8_gemv_3584x3584", (3584, 3584, pq, ps)),
                                   ("w4a8_gemv_37888x3584", (2 * f, d, pgq, pgs)),
                                   ("w4a8_gemv_3584x18944", (d, f, pdq, pds))):
        nb = pq_.nbytes + ps_.nbytes
        R = max(2, -(-ROTATE_BYTES // nb))
        bq, bs = rotated(pq_, R), rotated(ps_, R)
        xk = torch.from_numpy(synth.normal_f16(synth.rng(0, synth.GLOBAL_LAYER, synth.T_X), (k,))).to(dev)
        act = torch.empty(lib.w4a8_act_bytes(k), dtype=torch.uint8, device=dev)
        L.check(lib.w4a8_quantize_act(xk.data_ptr(), k, act.data_ptr(), cur()))
        yk = torch.empty(n, dtype=torch.float16, device=dev)
        wsk = torch.zeros(max(lib.w4_gemv_ws_bytes(n, k), 256), dtype=torch.uint8, device=dev)

        def mk8(r, bq=bq, bs=bs, act=act, yk=yk, wsk=wsk, n=n, k=k):
            def c():
                L.check(lib.w4a8_gemv(bq[r].data_ptr(), bs[r].data_ptr(), act.data_ptr(), yk.data_ptr(), n, k,
                                      wsk.data_ptr(), wsk.numel(), cur()))
            return c

        def mkq(xk=xk, act=act, k=k):
            def c():
                L.check(lib.w4a8_quantize_act(xk.data_ptr(), k, act.data_ptr(), cur()))
            return c
        us = _graph_time_us(torch, [mk8(r) for r in range(R)])
        want = w4.w4a8_gemv(bq[R - 1], bs[R - 1], act, n, k)
        torch.cuda.synchronize()
        assert torch.equal(yk.view(torch.int16), want.view(torch.int16)), f"{name}: replayed output differs"
        qus = _graph_time_us(torch, [mkq() for _ in range(64)])
        b = n * k // 2 + n * (k // 128) * 2 + lib.w4a8_act_bytes(k) + n * 2
        out[name] = {"N": n, "K": k, "us_per_call": round(us, 2), "bytes": b,
                     "GBps": round(b / (us * 1e-6) / 1e9, 1), "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "quantize_us_per_call": round(qus, 2), "copies": R}
        del bq, bs

    # config 2: paged decode attention; every call reads its own 40 pages of one large pool
    for ctx in ((640, 8192) if attention else ()):
        n_pg = ctx // 16
        q, kp, vp, table = synth.attn_case(ctx)
        page_bytes = kp[0].nbytes
        R = max(2, -(-ROTATE_BYTES // (2 * n_pg * page_bytes)))
        kt = torch.from_numpy(kp).to(dev)
        vt = torch.from_numpy(vp).to(dev)
        kpool = kt.repeat(R, 1, 1, 1)
        vpool = vt.repeat(R, 1, 1, 1)
        tables = torch.from_numpy(np.stack([table + r * n_pg for r in range(R)]).astype(np.int32)).to(dev)
        qt = torch.from_numpy(q).to(dev)
        o = torch.empty_like(qt)
        ws = torch.zeros(max(lib.w4_attn_ws_bytes(28, 4, n_pg), 256), dtype=torch.uint8, device=dev)

        def mk_att(r):
            def c():
                L.check(lib.paged_attn_decode(qt.data_ptr(), kpool.data_ptr(), vpool.data_ptr(), tables[r].data_ptr(),
                                              ctx, 28, 4, 128, n_pg, float(1 / np.sqrt(128)), o.data_ptr(),
                                              ws.data_ptr(), ws.numel(), cur()))
            return c
        us = _graph_time_us(torch, [mk_att(r) for r in range(R)])
        want = w4.paged_attn_decode(qt, kpool, vpool, tables[R - 1], ctx, float(1 / np.sqrt(128)))
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), want.view(torch.int16)), f"attention {ctx}: replayed output differs"
        b = 2 * n_pg * page_bytes + 2 * q.nbytes + n_pg * 4
        out[f"attn_ctx{ctx}"] = {"ctx": ctx, "pages": n_pg, "us_per_call": round(us, 2), "bytes": b,
                                 "GBps": round(b / (us * 1e-6) / 1e9, 1),
                                 "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "copies": R}
        del kpool, vpool
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=112)
    ap.add_argument("--no-standalone", action="store_true",
                    help="skip the standalone GEMV / MLP / attention calls of configs 0-2")
    ap.add_argument("--standalone-only", action="store_true",
                    help="run only the standalone calls of configs 0-2 (for kernel profiles)")
    ap.add_argument("--summarize-standalone-trace", metavar="DIR")
    ap.add_argument("--launch-study", action="store_true",
                    help="eager vs graph, persistent vs kernel-per-op step (writes a profiles/ summary)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="phase timestamps of the persistent kernel (needs the trace build)")
    ap.add_argument("--traffic-probe", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--measure-traffic", metavar="OUT_DIR")
    ap.add_argument("--summarize-traffic", metavar="OUT_DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--trace-command", default="")
    ap.add_argument("--summarize-prefill-trace", metavar="DIR")
    ap.add_argument("--context", type=int, default=512,
                    help="prompt length; above 512 runs the long-context workload (prefill-filled cache)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is described in DESIGN.md but not built", file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        return traffic_probe()
    if args.measure_traffic:
        return measure_traffic(args.measure_traffic)
    if args.summarize_traffic:
        return summarize_traffic(args.summarize_traffic)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.steps, args.trace_command)
    if args.summarize_prefill_trace:
        return summarize_prefill_trace(args.summarize_prefill_trace, args.trace_command)

    if args.summarize_standalone_trace:
        return summarize_standalone_trace(args.summarize_standalone_trace, args.trace_command)
    if args.launch_study:
        launch_study(args)
        return None
    if args.phase_trace:
        phase_trace(context=args.context)
        return None
    if args.standalone_only:
        res = standalone_kernels()
        for k_, v_ in res.items():
            log(f"[bench]   {k_}: {v_['us_per_call']} us/call, {v_['GBps']} GB/s ({v_['frac']:.3f} of peak)")
        print(json.dumps({"standalone_calls": res}), flush=True)
        return None
    if args.context != 512:
        if args.context < 512 or args.context % 16:
            sys.exit("--context must be 512 or a larger multiple of 16")
        return long_context(args)

    import torch
    import synth
    from int4_weight_only_dequant_amd import _lib as L

    dims = synth.QWEN7B
    n_prompt = 512
    if args.warmup > n_prompt - 1:
        sys.exit("warmup must be below the prompt length")
    t0 = time.time()
    model, glob_w, max_pages = build_model(dims, n_prompt, args.steps)
    prompt = synth.prompt_ids(dims, n_prompt)
    stream = torch.cuda.current_stream()
    launches = model.launches_per_step()
    log(f"[bench] model ready in {time.time() - t0:.0f}s; grid {model.grid()} work-groups, "
        f"{launches} launch per step (+ page append at page boundaries)")

    # time to first token: one prefill call over the 512-token prompt (first run warms up)
    ttft = []
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(4):
        model.reset(prompt)
        torch.cuda.synchronize()
        tp = time.perf_counter()
        pe0.record(stream)
        model.prefill(n_prompt)
        pe1.record(stream)
        torch.cuda.synchronize()
        if r:
            ttft.append(((time.perf_counter() - tp) * 1e3, pe0.elapsed_time(pe1)))
    assert model.device_error() == 0, "device error during the prefill"
    prefill_tok = int(model.tokens[n_prompt].item())
    ttft_ms = float(np.median([t[0] for t in ttft]))
    ttft_dev_ms = float(np.median([t[1] for t in ttft]))
    log(f"[bench] prefill of {n_prompt} tokens: TTFT {ttft_ms:.2f} ms (device {ttft_dev_ms:.2f} ms), token {prefill_tok}")

    # prompt through the decode step (teacher-forced); the last W steps are the warmup
    model.reset(prompt)
    for p in range(n_prompt):
        model.step(L.W4_GRAPH)
        if p == n_prompt - args.warmup - 1:
            torch.cuda.synchronize()
            log(f"[bench] prompt prefilled through decode steps; warmup {args.warmup} steps")
    torch.cuda.synchronize()

    # timed region: K graph replays, positions 512 .. 512+K-1, a HIP event on
    # the launch stream before every step
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    tstart = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        model.step(L.W4_GRAPH)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - tstart
    ms = elapsed * 1e3 / args.steps
    tok_s = args.steps / elapsed
    step_us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)])
    boundary = np.array([(n_prompt + i) % 16 == 0 for i in range(args.steps)])
    kern_us = float(step_us[~boundary].mean())      # steps without the page append: the kernel alone
    assert model.device_error() == 0, "device error during the timed steps"
    gen = model.tokens[n_prompt: n_prompt + args.steps + 1].cpu().numpy()
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/token, {tok_s:.1f} tok/s; persistent kernel "
        f"{kern_us:.1f} us per launch (events); first tokens {gen[:8]}")

    # eager launches at the positions the graph steps were timed at (the
    # prompt refilled by one prefill call): the same steps enqueued back to back
    eager_n = min(16, args.steps)
    model.reset(prompt)
    model.prefill(n_prompt)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for _ in range(eager_n):
        model.step(L.W4_EAGER)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / eager_n
    graph_same_ms = float(step_us[:eager_n].mean()) / 1e3
    assert model.device_error() == 0, "device error during the eager steps"

    # the int8-activation variant (W4_A8: the pages' Path A), graph replays
    # after the same prefill; 4 warmup steps (the first captures its graphs)
    a8_n = max(1, min(60, args.steps - 4))   # the pool holds n_prompt + steps positions
    model.reset(prompt)
    model.prefill(n_prompt)
    for _ in range(4):
        model.step(L.W4_GRAPH | L.W4_A8)
    torch.cuda.synchronize()
    ev8 = [torch.cuda.Event(enable_timing=True) for _ in range(a8_n + 1)]
    t8 = time.perf_counter()
    for i in range(a8_n):
        ev8[i].record(stream)
        model.step(L.W4_GRAPH | L.W4_A8)
    ev8[-1].record(stream)
    torch.cuda.synchronize()
    a8_ms = (time.perf_counter() - t8) * 1e3 / a8_n
    a8_us = np.array([ev8[i].elapsed_time(ev8[i + 1]) * 1e3 for i in range(a8_n)])
    a8_bnd = np.array([(n_prompt + 4 + i) % 16 == 0 for i in range(a8_n)])
    a8_kern_us = float(a8_us[~a8_bnd].mean())
    assert model.device_error() == 0, "device error during the int8-activation steps"
    log(f"[bench] int8-activation step: {a8_ms:.3f} ms/token, kernel {a8_kern_us:.1f} us "
        f"(fp16 path {kern_us:.1f} us)")

    # kernel-per-op variant, per-kernel times (timing hook; clobbers the activation scratch)
    kern = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, kind, r in (("gate_up", L.W4_KERNEL_GATE_UP, args.kernel_reps), ("down", L.W4_KERNEL_DOWN, 28),
                          ("o_proj", L.W4_KERNEL_O, 28), ("lm_head", L.W4_KERNEL_LM_HEAD, 8)):
        model.kernel_replay(kind, 4)
        e0.record(stream)
        model.kernel_replay(kind, r)
        e1.record(stream)
        torch.cuda.synchronize()
        kern[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / r, 2)
    multi_launches = model.launches_per_step(L.W4_MULTI)
    model.close()
    d_, f_, qd_ = dims.d_model, dims.d_ff, dims.n_q_heads * dims.head_dim
    for name, (n_, k_) in (("gate_up", (2 * f_, d_)), ("down", (d_, f_)), ("o_proj", (d_, qd_))):
        kern[name + "_GBps"] = round(_w4_bytes(n_, k_) / (kern[name + "_us"] * 1e-6) / 1e9, 1)
    kern["lm_head_GBps"] = round((dims.vocab * d_ * 2 + d_ * 2 + dims.vocab * 4) / (kern["lm_head_us"] * 1e-6) / 1e9, 1)
    standalone = None
    if not args.no_standalone:
        log("[bench] standalone calls of configs 0-2 (rotated operands, graph-replayed)")
        torch.cuda.empty_cache()
        standalone = standalone_kernels()
        for k_, v_ in standalone.items():
            log(f"[bench]   {k_}: {v_['us_per_call']} us/call, {v_['GBps']} GB/s ({v_['frac']:.3f} of peak)")

    ctx_lo, ctx_hi = n_prompt + 1, n_prompt + args.steps
    sb = step_bytes(dims, ctx_lo, ctx_hi)
    achieved = sb / (kern_us * 1e-6) / 1e9
    tr = read_traffic()
    qkv_rows = (dims.n_q_heads + 2 * dims.n_kv_heads) * dims.head_dim
    qd = dims.n_q_heads * dims.head_dim
    lin_flop = 2.0 * n_prompt * dims.n_layers * (qkv_rows * dims.d_model + dims.d_model * qd +
                                                 2 * dims.d_ff * dims.d_model + dims.d_model * dims.d_ff)
    line = {
        "metric": "decode ms/token & tok/s (batch 1, 512+128); W4A16 GEMV achieved HBM TB/s",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tok_s / PAGES_PUBLISHED_TOKS, 3),
        "dtype": "fp16",
        "data": "synthetic (seeded random-init weights of the Qwen2.5-7B shapes, uniform random prompt ids)",
        "config": {"workload": f"Qwen2.5-7B-shaped W4A16 decode step, batch 1, {n_prompt}-token prompt + "
                               f"{args.steps} greedy graph-captured steps, int4 group-128 projections with fp16 "
                               "scales",
                   "layers": dims.n_layers, "hidden": dims.d_model, "mlp": dims.d_ff,
                   "heads": f"{dims.n_q_heads}q/{dims.n_kv_heads}kv x {dims.head_dim}",
                   "vocab": dims.vocab, "context": f"{ctx_lo}-{ctx_hi}",
                   "kv_pages": max_pages, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": f"{KERNEL} (the whole decode step, one launch per token)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": round(tr["traffic_bytes"]) if tr else None,
                     "bytes_per_launch": int(sb), "avg_launch_us": round(kern_us, 2),
                     "traffic_source": os.path.relpath(TRAFFIC_MD, HERE) if tr else None},
        "vs_baseline_note": f"ratio to the pages' {PAGES_PUBLISHED_TOKS:.0f} tok/s on an H100-class GPU (context)",
        "eager_ms_per_step": round(eager_ms, 3),
        "eager_vs_graph": {"positions": f"{n_prompt}-{n_prompt + eager_n - 1}", "eager_ms_per_step": round(eager_ms, 3),
                           "graph_ms_per_step_same_positions": round(graph_same_ms, 3)},
        "launches_per_step": launches,
        "int8_activation_step": {"flag": "W4_A8", "positions": f"{n_prompt + 4}-{n_prompt + 3 + a8_n}",
                                 "ms_per_step": round(a8_ms, 4), "kernel_us": round(a8_kern_us, 2),
                                 "fp16_kernel_us": round(kern_us, 2),
                                 "note": "every int4 GEMV input quantised per group of 128 to int8 inside "
                                         "the persistent kernel's staging; integer dot products; lm_head fp16"},
        "kernel_per_op_variant": {"launches_per_step": multi_launches, **kern},
        "standalone_calls": standalone,
        "tokens_head": [int(t) for t in gen[:16]],
        "prefill": {"ttft_ms": round(ttft_ms, 3), "device_ms": round(ttft_dev_ms, 3), "prompt_tokens": n_prompt,
                    "linear_tflop": round(lin_flop / 1e12, 3),
                    "linear_tflops_over_ttft": round(lin_flop / (ttft_dev_ms * 1e-3) / 1e12, 1),
                    "mfma_fp16_peak_tflops": MFMA_F16_PEAK_TFLOPS,
                    "frac_of_peak": round(lin_flop / (ttft_dev_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                    "first_token_matches_decode_path": prefill_tok == int(gen[0]),
                    "pages_ttft_ms": PAGES_PUBLISHED_TTFT_MS},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(dims, glob_w)
    log(f"[bench] done in {time.time() - t0:.0f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
