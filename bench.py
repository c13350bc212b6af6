"""Benchmark: one batched codec-LM decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]
                    [--no-cpu-baseline] [--copy-calibration]

A step is the whole hot path over one batch: kv_cache_append ->
decode_attention -> codebook_head -> sample_or_argmax (spec_verify for the
speculative workload), all through the C ABI, inputs resident in HBM.  The
timed steps are eager calls; --graph on times launches of the native decode
loop instead (--graph-steps steps captured as one HIP graph by
clm_decode_loop_create, lengths advancing on the device, reset between
launches by two small device copies).  Per-call durations always come from
HIP events around eager calls.  The
default workload is 256 streams with log-uniform KV lengths in [64, 8192],
16 query / 8 KV heads of width 128, bf16 cache, a 2048 -> 16384 head and
greedy decoding: the one that fills the GPU and exposes the attention
roofline.

Prints ONE JSON line: value = stream-steps/s (streams x query tokens per
second), the attention kernel's roofline (algorithmic K/V/q/o bytes per
launch over its HIP-event-timed duration, against 8 TB/s), and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "codec decode steps/s (streams×tokens) and % HBM roofline of KV attention"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (the fp32 workload's GEMV)
DEFAULT_WORKLOAD = "c5"          # 256 streams, log-uniform 64..8192 keys (the metric's workload)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_c5_traffic.txt")
ATTN_SRCS = [os.path.join(ROOT, "codec_language_model_amd", "csrc", f) for f in ("attention.hip", "clm_device.h")]
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs (1 only: the step runs on one GPU; more exits with a message)")
    ap.add_argument("--steps", type=int, default=100, help="timed steps")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before them")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="c1 (1 stream, fp32), c2 (16 streams, sampling), c3 (64 streams, 3 stage heads), "
                         "c4 (32 x 6-query speculative verification) or c5 (256 streams, the default)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (cpu_baseline is then null)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the chosen workload (by default the 256-stream step is followed by "
                         "short eager runs of the four smaller workloads, reported under other_workloads, "
                         "and by the one- and 16-stream steps as graph loops, under graph_loop; profiler "
                         "runs of one workload pass this flag)")
    ap.add_argument("--cpu-streams", type=int, default=0,
                    help="streams in the oracle's timed sample (0 = the whole batch)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle is repeated over its sample until this much CPU time has passed")
    ap.add_argument("--head", choices=("linear", "mlp"), default="linear",
                    help="codebook head: one linear map per stage (the workloads' head) or TontaubeV1's "
                         "two-layer d -> 4096 -> Mish -> V head (random N(0, 0.02) weights)")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="KV cache element: the workloads' bf16, or E4M3 bytes with per-row scales "
                         "(random codes and scales of the same shapes)")
    ap.add_argument("--append", choices=("plain", "rope"), default="plain",
                    help="plain KV append, or the append with rotary embedding at logical positions "
                         "(len_before + 1000 + t, base 1e6) applied to the new keys and the queries")
    ap.add_argument("--graph", choices=("on", "off"), default="off",
                    help="time the steps as launches of the native decode loop - --graph-steps steps "
                         "captured as one HIP graph, lengths advancing on the device (on) - or as eager "
                         "calls (off)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="KV pages of this many slots instead of the workload's 16 (a multiple of 16, <= 128)")
    ap.add_argument("--graph-steps", type=int, default=16,
                    help="steps per captured decode loop with --graph on")
    ap.add_argument("--no-copy-check", action="store_true",
                    help="skip timing a plain 1 GiB device copy after the main measurement (reported as "
                         "hbm_copy: the box's practical copy bandwidth and attention's share of it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling PMC byte counters)")
    ap.add_argument("--measuring-stick", action="store_true",
                    help="no decode step: time hipBLASLt (torch.mm, bf16) on a large square GEMM and on the "
                         "codebook head's shapes, weights rotated over replicas, as the box's practical "
                         "matrix-core ceiling")
    ap.add_argument("--cpu-table", action="store_true",
                    help="no GPU work: the CPU oracle's time per call (append, attention, head, token choice "
                         "or verification) and for the chained step, on all five workloads, with every host "
                         "thread and with one (the CPU baseline protocol); prints a markdown table")
    ap.add_argument("--pmc-table", metavar="COUNTER_CSV",
                    help="no GPU work: per-kernel averages of every counter in a rocprofv3 "
                         "counter_collection.csv")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-calibration run into the attention traffic record")
    return ap.parse_args()


def copy_bandwidth(dev, reps=5):
    """GB/s (read + write bytes) of a plain 1 GiB device-to-device copy
    (torch's copy kernel), timed with HIP events on the current stream: the
    box's practical HBM rate for a streaming copy."""
    import torch
    src = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def attention_bytes(cfg, kv_len, fp8=False):
    """Algorithmic bytes of one decode_attention launch: every visible K and V
    row once (2 * H_kv * D * elem bytes per token, plus its fp32 scale with an
    FP8 cache), q read once, o written once."""
    e = 2 if cfg.dtype == "bf16" else 4
    row = cfg.D + 4 if fp8 else cfg.D * e
    kv = int(kv_len.astype("int64").sum()) * 2 * cfg.H_kv * row
    qo = 2 * cfg.B * cfg.Kq * cfg.H_q * cfg.D * e
    return kv + qo


def attention_source_hash():
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _synth():
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    return synth


def pmc_summary(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """HBM bytes per decode_attention launch from two PMC runs.  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are averaged per kernel over its dispatches,
    summed over the call's kernels (split pass and merge pass), and each scaled
    by what the same counter reads for a plain 1 GiB device copy."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        copies = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            m = re.search(r"attn_\w+", name)
            if m:
                vals[m.group(0)].append(v)
            elif "copyBuffer" in name and int(r["Grid_Size"]) >= 65536:
                copies.append(v)
        if not vals or not copies:
            raise SystemExit(f"{path}: no attention dispatches or no 1 GiB copy for {counter}")
        avg = {k: sum(v) / len(v) for k, v in vals.items()}
        return avg, sum(copies) / len(copies)

    f_avg, f_copy = per_kernel(fetch_csv, "FETCH_SIZE")
    w_avg, w_copy = per_kernel(write_csv, "WRITE_SIZE")
    # a 1 GiB copy reads and writes 1 GiB = 1048576 KiB
    f_scale = (COPY_BYTES / 1024) / f_copy
    w_scale = (COPY_BYTES / 1024) / w_copy
    fetch = sum(f_avg.values()) * f_scale * 1024
    write = sum(w_avg.values()) * w_scale * 1024
    lines = [
        "# HBM traffic of one decode_attention call (its split pass and merge pass),",
        "# 256 streams, 16/8 heads, head_dim 128, bf16, log-uniform KV lengths in [64, 8192].",
        "# Counters from two runs of",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o f -- python3 bench.py --steps 3 --warmup 1 "
        "--no-cpu-baseline --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o w -- python3 bench.py --steps 3 --warmup 1 "
        "--no-cpu-baseline --copy-calibration",
        "# reduced by: python3 bench.py --pmc-summary <dir>/f_counter_collection.csv "
        "<dir>/w_counter_collection.csv",
        "# Each counter is scaled by its reading for a plain 1 GiB device-to-device copy.",
    ]
    for k in sorted(f_avg):
        lines.append(f"# {k}: FETCH_SIZE {f_avg[k]:.1f} KiB, WRITE_SIZE {w_avg.get(k, 0.0):.1f} KiB per dispatch")
    lines += [
        f"# 1 GiB copy: FETCH_SIZE {f_copy:.1f} KiB, WRITE_SIZE {w_copy:.1f} KiB per dispatch",
        f"attention_source_sha256_16 = {attention_source_hash()}",
        f"workload = {_synth().get_config(DEFAULT_WORKLOAD).workload}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        f"hbm_fetch_bytes_per_launch = {fetch:.0f}",
        f"hbm_write_bytes_per_launch = {write:.0f}",
        f"hbm_bytes_per_launch = {fetch + write:.0f}",
    ]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_table(path):
    """Per-kernel averages of each counter of a rocprofv3 counter CSV, plus the
    matrix-core figures derived from them where the counters are present:
    bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, rocprofv3's own
    MfmaFlopsBF16 expression) and the MFMA busy share per SIMD: the busy
    cycles, summed over the 1024 SIMDs, per SIMD, over the kernel's elapsed
    cycles.  GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs (divided by 8 it
    matches each kernel's traced duration at the shader clock), so the
    elapsed cycles are GRBM_GUI_ACTIVE / 8."""
    import csv
    from collections import defaultdict
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        vals[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in vals})
    for k in kernels:
        row = {c: sum(v) / len(v) for (kk, c), v in vals.items() if kk == k}
        n = max(len(v) for (kk, _), v in vals.items() if kk == k)
        short = re.sub(r"\(.*", "", k.replace("clm::(anonymous namespace)::", ""))[:80]
        parts = [f"{c} {row[c]:.6g}" for c in sorted(row)]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in row:
            parts.append(f"bf16 MFMA GFLOP {row['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.4g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in row and row.get("GRBM_GUI_ACTIVE"):
            busy = row["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
            elapsed = row["GRBM_GUI_ACTIVE"] / 8
            parts.append(f"MFMA busy per SIMD {busy:.0f} of {elapsed:.0f} cycles = {100 * busy / elapsed:.1f}%")
        print(f"{short} [{n} dispatches]: " + "; ".join(parts))


def measuring_stick():
    """hipBLASLt through torch.mm in bf16: one large square GEMM and the codebook
    head's own shapes (fp32 accumulate, bf16 out), weights rotated over
    replicas so they come from HBM.  The box's practical matrix-core figure."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    out = []
    for name, M, K, N, reps in (("square 8192^3", 8192, 8192, 8192, 2),
                                ("head 256 x 2048 -> 16384", 256, 2048, 16384, 5),
                                ("head 192 x 2048 -> 4096", 192, 2048, 4096, 5),
                                ("head 16 x 2048 -> 16384", 16, 2048, 16384, 5)):
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        ws = [torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16) for _ in range(reps)]
        for i in range(3):
            torch.mm(a, ws[i % reps].t())
        torch.cuda.synchronize()
        iters = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            torch.mm(a, ws[i % reps].t())
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        tf = 2.0 * M * K * N / (us * 1e-6) / 1e12
        line = {"gemm": name, "us": round(us, 2), "tflops": round(tf, 1), "frac_of_2500": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        print(json.dumps(line), flush=True)
        out.append(line)
        del a, ws
    return out


def traffic_for_current_kernel(workload):
    """HBM bytes per attention launch measured by rocprofv3 PMC counters, if
    the record was taken on the current attention source and on this workload;
    else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src_hash = attention_source_hash()
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("attention_source_sha256_16") != src_hash or vals.get("workload") != workload:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info():
    """The host the oracle ran on: model, logical CPUs, this process's
    affinity and RAM (from /proc on Linux)."""
    info = {"cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                info["ram_gb"] = round(int(line.split()[1]) / 2**20, 1)
                break
    except OSError:
        pass
    return info


def cpu_baseline(x, n_streams, min_seconds, threads=None, keep_ref=False):
    """The oracle, as it stands, on n_streams streams spread over the length
    distribution (all of them when n_streams is 0 or >= B): attention, head
    and token choice per stream, repeated until min_seconds have passed.
    threads: BLAS/OpenMP thread limit for the run (None: the library default,
    all cores).  keep_ref: also return the last repetition's outputs and the
    streams they cover, under "_ref"."""
    import contextlib

    import numpy as np

    import oracle
    c = x.cfg
    if n_streams <= 0 or n_streams > c.B:
        n_streams = c.B
    order = np.argsort(x.kv_len)
    streams = sorted(set(int(order[i]) for i in np.linspace(0, c.B - 1, n_streams).astype(int)))
    keys = {b: x.logical_k(b) for b in streams}
    vals = {b: x.logical_v(b) for b in streams}
    q = x.f32(x.q)
    W = x.f32(x.W)
    scale = 1.0 / math.sqrt(c.D)
    try:
        import threadpoolctl
    except ImportError:
        threadpoolctl = None
    limit = (threadpoolctl.threadpool_limits(limits=threads) if threadpoolctl is not None and threads
             else contextlib.nullcontext())
    with limit:
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t0 < min_seconds:
            ref = oracle.decode_step(q, keys, vals, x.kv_len, scale, c.H_kv, W, x.head_id if c.G > 1 else None,
                                     c.dtype == "bf16", streams=streams)
            reps += 1
        dt = time.perf_counter() - t0
        used = os.cpu_count()
        if threadpoolctl is not None:
            blas = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
            if blas:
                used = max(blas)
    rows = len(streams) * c.Kq * reps
    what = "the whole batch" if len(streams) == c.B else \
        f"{len(streams)} of {c.B} streams (spread over the KV-length order)"
    out = {"value": round(rows / dt, 3), "unit": "stream-steps/s", "cores": used, "kind": "oracle",
           "sample": f"{what}, {int(sum(x.kv_len[b] for b in streams))} cached tokens, full head, "
                     f"{reps} repetitions: {dt:.1f} s"}
    if keep_ref:
        out["_ref"] = (streams, ref)
    return out


def parity_of_step(c, streams, ref, o, logits, tokens):
    """The timed step's own outputs against the oracle's for the same inputs
    (the CPU baseline's last repetition): attention outputs and logits by the
    |gpu - oracle| <= 2e-2 + 2e-2 |oracle| bar, greedy tokens equal except
    where the oracle's top-2 logit gap is under 1e-3 (then the GPU's token
    must be within 1e-3 of the oracle's max)."""
    import numpy as np
    rows = np.array([b * c.Kq + j for b in streams for j in range(c.Kq)])
    o_g = o.float().cpu().numpy()[streams].astype(np.float64)
    l_g = logits.cpu().numpy()[rows].astype(np.float64)
    t_g = tokens.cpu().numpy()[rows]
    o_r = np.asarray(ref["o"])[streams]
    l_r = np.asarray(ref["logits"], np.float64)[rows]

    def bar(g, r):
        err = np.abs(g - r)
        return float(err.max()), float((err / (2e-2 + 2e-2 * np.abs(r))).max())
    eo, so = bar(o_g, o_r)
    el, sl = bar(l_g, l_r)
    top2 = np.sort(l_r, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    want = np.argmax(l_r, axis=1)
    equal = t_g == want
    near = l_r[np.arange(len(rows)), t_g] >= top2[:, 1] - 1e-3
    exempt = (~equal) & (gap < 1e-3) & near
    return {"streams": len(streams), "rows": int(len(rows)),
            "attention_max_abs_err": round(eo, 6), "attention_bar_share": round(so, 4),
            "logits_max_abs_err": round(el, 6), "logits_bar_share": round(sl, 4),
            "tokens_equal": int(equal.sum()), "tokens_exempt": int(exempt.sum()),
            "pass": bool(so <= 1.0 and sl <= 1.0 and (equal | exempt).all())}


def cpu_baseline_table(reps=3):
    """The CPU baseline protocol over every workload: the oracle as it stands,
    one call at a time and chained, one warm-up then `reps` timed runs (the
    median), with all host threads and with one.  Prints a markdown table."""
    import contextlib

    import numpy as np

    import oracle
    synth = _synth()
    try:
        import threadpoolctl
    except ImportError:
        threadpoolctl = None

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)) * 1e3

    print(f"host: {host_info()}; {reps} timed runs after one warm-up, median ms", flush=True)
    print("| workload | threads | append | attention | head | token / verify | chained step | stream-steps/s |")
    print("|---|---|---|---|---|---|---|---|")
    for i in range(1, 6):
        x = synth.make_inputs(i)
        c = x.cfg
        kp, vp = x.build_pool(include_new=False)
        keys = [x.logical_k(b) for b in range(c.B)]
        vals = [x.logical_v(b) for b in range(c.B)]
        q, W = x.f32(x.q), x.f32(x.W)
        hid = x.head_id if c.G > 1 else None
        scale = 1.0 / math.sqrt(c.D)
        bf = c.dtype == "bf16"
        temp = np.full(c.M, c.temperature, np.float32) if c.mode == "sample" else None
        uni = x.uniforms() if c.mode == "sample" else None
        spec = x.spec_inputs() if c.mode == "spec" else None
        o = oracle.decode_attention(q, keys, vals, x.kv_len, scale, c.H_kv)
        h = (oracle.round_to_bf16(o) if bf else o.astype(np.float32)).reshape(c.M, c.H_q * c.D)
        logits = oracle.codebook_head(h, W, hid).astype(np.float32)

        def token():
            if spec is not None:
                oracle.spec_verify(logits.reshape(c.B, c.Kq, c.V), spec["draft_probs"], spec["draft_tokens"],
                                   spec["u_accept"], spec["u_resample"], c.temperature)
            else:
                oracle.sample_or_argmax(logits, temp, uni)

        def chained():
            t = temp if c.mode == "sample" else (c.temperature if c.mode == "spec" else None)
            oracle.decode_step(q, keys, vals, x.kv_len, scale, c.H_kv, W, hid, bf, mode=c.mode,
                               temperature=t, uniforms=uni, spec=spec)

        for threads in (None, 1):
            limit = (threadpoolctl.threadpool_limits(limits=threads) if threadpoolctl is not None and threads
                     else contextlib.nullcontext())
            with limit:
                t_app = timed(lambda: oracle.kv_cache_append(kp, vp, x.block_table, x.len_before, x.k_new, x.v_new,
                                                             c.block_size))
                t_att = timed(lambda: oracle.decode_attention(q, keys, vals, x.kv_len, scale, c.H_kv))
                t_head = timed(lambda: oracle.codebook_head(h, W, hid))
                t_tok = timed(token)
                t_step = timed(chained)
            print(f"| {c.workload} | {'all' if threads is None else threads} | {t_app:.1f} | {t_att:.1f} | "
                  f"{t_head:.1f} | {t_tok:.1f} | {t_step:.1f} | {c.B * c.Kq / (t_step * 1e-3):.1f} |", flush=True)


def main():
    args = parse()
    if args.cpu_table:
        cpu_baseline_table()
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.measuring_stick:
        measuring_stick()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode step shards by stream with no exchange "
              f"between GPUs, so a multi-GPU figure is N independent copies of this one "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import codec_language_model_amd as clm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    clm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def run_one(args):
        """One workload: draw inputs, time the steps, return the JSON object."""
        cfg = synth.get_config(args.workload)
        if args.block_size:
            import dataclasses
            cfg = dataclasses.replace(cfg, block_size=args.block_size)
        graph = args.graph == "on"
        t_gen = time.perf_counter()
        x = synth.make_inputs(cfg)
        c = x.cfg
        bf = c.dtype == "bf16"
        n_loop = max(1, args.graph_steps) if graph else 1
        # pages for the loop's later steps (the same pages as the step's own for
        # every position the eager step touches)
        kp, vp, bt_np, _ = x.pool_with_room((n_loop - 1) * c.Kq)
        log(f"[bench] {c.workload}: inputs drawn in {time.perf_counter() - t_gen:.1f} s "
            f"(sum kv_len {int(x.kv_len.sum())}, pool {kp.nbytes * 2 / 2**30:.2f} GiB)")

        def dev_t(a, bf16):
            a = np.ascontiguousarray(a)
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
            return t.to(dev)

        k_cache, v_cache = dev_t(kp, bf), dev_t(vp, bf)
        f8 = None
        if args.kv == "fp8":
            if not bf:
                print("--kv fp8 needs a bf16 workload", file=sys.stderr)
                sys.exit(2)
            # synthetic E4M3 cache of the pool's shapes: uniform codes without the
            # two NaN codes, row scales uniform in [0.002, 0.01] (max|x|/448 for
            # rows of N(0,1) values is ~0.007)
            g = torch.Generator(device=dev).manual_seed(4321)
            def codes(shape):
                cde = torch.randint(0, 254, shape, generator=g, device=dev, dtype=torch.int32)
                cde = cde + (cde >= 0x7F).to(torch.int32)
                return cde.to(torch.uint8)
            nb_, hk_, bs_ = kp.shape[0], kp.shape[1], kp.shape[2]
            f8 = (codes((nb_, hk_, c.D // 8, bs_, 8)), codes(tuple(vp.shape)),
                  torch.empty((nb_, hk_, bs_), device=dev).uniform_(0.002, 0.01, generator=g),
                  torch.empty((nb_, hk_, bs_), device=dev).uniform_(0.002, 0.01, generator=g))
            del k_cache, v_cache
            k_cache = v_cache = None
        del kp, vp
        bt, kv_len, len_before = dev_t(bt_np, False), dev_t(x.kv_len, False), dev_t(x.len_before, False)
        k_new, v_new, q = dev_t(x.k_new, bf), dev_t(x.v_new, bf), dev_t(x.q, bf)
        W = dev_t(x.W, bf)
        head_id = dev_t(x.head_id, False) if c.G > 1 else None
        mlp = None
        if args.head == "mlp":
            if not bf:
                print("--head mlp needs a bf16 workload", file=sys.stderr)
                sys.exit(2)
            F = 4096
            gen = torch.Generator(device=dev).manual_seed(1234)
            W1 = (torch.randn((c.G, F, c.d_model), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            W2 = (torch.randn((c.G, c.V, F), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            act = torch.empty((c.M, F), dtype=torch.bfloat16, device=dev)
            mlp = (W1, W2, act, F)
        max_kv = int(x.kv_len.max()) + (n_loop - 1) * c.Kq
        rope_pos = None
        if args.append == "rope":
            rope_pos = dev_t((x.len_before[:, None] + 1000 + np.arange(c.Kq)[None, :]).astype(np.int32), False)
        scale = 1.0 / math.sqrt(c.D)
        o = torch.empty_like(q)
        logits = torch.empty((c.M, c.V), dtype=torch.float32, device=dev)
        tokens = torch.empty(c.M, dtype=torch.int32, device=dev)
        ws = clm.Workspace.get(clm.decode_attention_workspace_size(c.B, c.Kq, c.H_q, c.H_kv, c.D, max_kv), dev)
        temp = uni = None
        if c.mode == "sample":
            temp = torch.full((c.M,), c.temperature, dtype=torch.float32, device=dev)
            uni = dev_t(x.uniforms(), False)
        spec = None
        if c.mode == "spec":
            s = x.spec_inputs()
            spec = tuple(dev_t(s[k], False) for k in ("draft_probs", "draft_tokens", "u_accept", "u_resample"))
            out_tok = torch.empty((c.B, c.Kq), dtype=torch.int32, device=dev)
            num_em = torch.empty(c.B, dtype=torch.int32, device=dev)
        # Input replicas: eager steps rotate over R copies of the KV pool, the
        # head weights and the logits, so that the bytes a step touches are
        # at least 512 MiB, twice the 256 MiB Infinity Cache, and every step
        # reads from HBM as a serving step would.  The 256-stream pool alone
        # is 1.6 GB (R = 1).  The decode loop captures one set (R = 1).
        def nbytes(t):
            return 0 if t is None else t.numel() * t.element_size()
        kv_set = (k_cache, v_cache) if f8 is None else f8
        per_set = sum(nbytes(t) for t in kv_set) + nbytes(W) + nbytes(logits) + \
            (0 if mlp is None else nbytes(mlp[0]) + nbytes(mlp[1]))
        n_rep = 1 if graph else int(min(8, max(1, -(-(512 << 20) // per_set))))
        reps = [(kv_set, W, logits, mlp)]
        for _ in range(n_rep - 1):
            reps.append((tuple(t.clone() for t in kv_set), W.clone(), torch.empty_like(logits),
                         None if mlp is None else (mlp[0].clone(), mlp[1].clone(), mlp[2], mlp[3])))
        rep_i = [0]
        torch.cuda.synchronize()

        def step(ev=None):
            kvs, W_, logits_, mlp_ = reps[rep_i[0] % n_rep]
            rep_i[0] += 1
            if ev is not None:
                ev[0].record()
            if f8 is not None and rope_pos is not None:
                clm.rope_kv_cache_append_fp8(q, k_new, v_new, *kvs, bt, len_before, rope_pos, 1.0e6,
                                             block_size=c.block_size)
            elif f8 is not None:
                clm.kv_cache_append_fp8(k_new, v_new, *kvs, bt, len_before, block_size=c.block_size)
            elif rope_pos is None:
                clm.kv_cache_append(k_new, v_new, kvs[0], kvs[1], bt, len_before, block_size=c.block_size)
            else:
                clm.rope_kv_cache_append(q, k_new, v_new, kvs[0], kvs[1], bt, len_before, rope_pos, 1.0e6,
                                         block_size=c.block_size)
            if ev is not None:
                ev[1].record()
            if f8 is None:
                clm.decode_attention(q, kvs[0], kvs[1], bt, kv_len, max_kv, scale=scale, out=o, workspace=ws,
                                     block_size=c.block_size)
            else:
                clm.decode_attention_fp8(q, *kvs, bt, kv_len, max_kv, scale=scale, out=o, workspace=ws)
            if ev is not None:
                ev[2].record()
            if mlp_ is None:
                clm.codebook_head(o.view(c.M, c.d_model), W_, head_id, out=logits_)
            else:
                clm.codebook_head_mlp(o.view(c.M, c.d_model), mlp_[0], mlp_[1], head_id, act=mlp_[2], out=logits_)
            if ev is not None:
                ev[3].record()
            if spec is not None:
                clm.spec_verify(logits_.view(c.B, c.Kq, c.V), *spec, c.temperature, out_tokens=out_tok,
                                num_emitted=num_em)
            else:
                clm.sample_or_argmax(logits_, temp, uni, out=tokens)
            if ev is not None:
                ev[4].record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

        # The decode loop: n_loop steps captured natively as one HIP graph
        # (clm_decode_loop_*), the lengths (and positions) advancing on the
        # device between steps.  Each launch runs n_loop steps; the lengths are
        # then reset by two small device copies so every launch sees the same
        # workload.
        run = step
        steps_per_run = 1
        if graph:
            rep = lambda t: t.unsqueeze(0).expand((n_loop,) + tuple(t.shape)).contiguous()
            lg_all = torch.empty((n_loop, c.M, c.V), dtype=torch.float32, device=dev)
            kv_args = dict(k_cache=k_cache, v_cache=v_cache) if f8 is None else \
                dict(k_cache=f8[0], v_cache=f8[1], k_scale=f8[2], v_scale=f8[3])
            lp = dict(**kv_args, block_table=bt, len_before=len_before, kv_len=kv_len,
                      max_kv_len=max_kv, k_new=rep(k_new), v_new=rep(v_new), q=rep(q), W=W, head_id=head_id,
                      o=torch.empty_like(rep(q)), logits=lg_all, mode=c.mode, attn_workspace=ws,
                      block_size=c.block_size)
            if mlp is not None:
                lp.update(W=mlp[0], W2=mlp[1], act=mlp[2])
            if rope_pos is not None:
                lp.update(positions=rope_pos, rope_base=1.0e6)
            if c.mode == "spec":
                lp.update(spec_temperature=c.temperature, draft_probs=rep(spec[0].view(c.B, c.Kq, c.V)),
                          draft_tokens=rep(spec[1]), u_accept=rep(spec[2]), u_resample=rep(spec[3]),
                          out_tokens=torch.empty((n_loop, c.B, c.Kq), dtype=torch.int32, device=dev),
                          num_emitted=torch.empty((n_loop, c.B), dtype=torch.int32, device=dev))
            else:
                lp.update(tokens=torch.empty((n_loop, c.M), dtype=torch.int32, device=dev))
                if c.mode == "sample":
                    lp.update(temperature=rep(temp), uniforms=rep(uni))
            state0 = [t.clone() for t in (len_before, kv_len) + ((rope_pos,) if rope_pos is not None else ())]
            loop = clm.DecodeLoop(**lp)

            def run():
                loop.launch()
                for t, t0 in zip((len_before, kv_len, rope_pos), state0):
                    t.copy_(t0)
            steps_per_run = n_loop
            for _ in range(max(1, args.warmup // n_loop)):
                run()
            torch.cuda.synchronize()

        # whole-step throughput: K steps back to back, no events inside
        n_runs = max(1, -(-args.steps // steps_per_run))
        t0 = time.perf_counter()
        for _ in range(n_runs):
            run()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        timed_steps = n_runs * steps_per_run

        # per-call durations: the same K steps again with HIP events between the
        # calls, recorded on the stream the kernels run on (torch's current stream)
        # and read after one synchronisation at the end, so the host stays ahead of
        # the GPU and no launch gap is timed
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        dur = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs]) * 1e3   # [steps, 4] us
        per_us = dur.mean(axis=0)
        pct = np.percentile(dur, [10, 50, 90], axis=0)                                          # [3, 4]
        step_pct = np.percentile(dur.sum(axis=1), [10, 50, 90])

        ms_per_step = wall / timed_steps * 1e3
        value = c.B * c.Kq / (wall / timed_steps)
        attn_s = per_us[1] * 1e-6
        attn_bytes = attention_bytes(c, x.kv_len, fp8=f8 is not None)
        achieved = attn_bytes / attn_s / 1e9
        traffic = traffic_for_current_kernel(c.workload) if f8 is None else None
        log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step; per call (us): append {per_us[0]:.1f}, "
            f"attention {per_us[1]:.1f}, head {per_us[2]:.1f}, token {per_us[3]:.1f}; attention "
            f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")

        if args.copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
            torch.cuda.synchronize()
            log("[bench] copy calibration: 5 x 1 GiB device-to-device copies done")
            del src, dst

        cpu = None
        parity = None
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle on all cores, then on one ...")
            cpu = cpu_baseline(x, args.cpu_streams, args.cpu_seconds, keep_ref=True)
            streams_ref, ref = cpu.pop("_ref")
            one = cpu_baseline(x, args.cpu_streams, args.cpu_seconds, threads=1)
            cpu["single_core"] = {"value": one["value"], "cores": one["cores"], "sample": one["sample"]}
            cpu["host"] = host_info()
            log(f"[bench] cpu oracle: {cpu['value']:.2f} {cpu['unit']} on {cpu['cores']} threads, "
                f"{one['value']:.2f} on {one['cores']} ({cpu['host']})")
            # the timed step's outputs against the oracle's on the same inputs (the
            # plain greedy step only: the other modes change what the step computes)
            if f8 is None and rope_pos is None and mlp is None and not graph and c.mode == "greedy":
                parity = parity_of_step(c, streams_ref, ref, o, reps[0][2], tokens)
                log(f"[bench] parity against the oracle: {parity}")

        head_flops = 2.0 * c.M * c.d_model * c.V if mlp is None else 2.0 * c.M * mlp[3] * (c.d_model + c.V)
        head_roof = None
        if mlp is None:
            # the head's own roofline: min(matrix-core peak, arithmetic intensity x HBM peak),
            # with W, h and the fp32 logits each moved once
            e = 2 if bf else 4
            hb = c.G * c.V * c.d_model * e + c.M * c.d_model * e + c.M * c.V * 4
            peak = MFMA_BF16_PEAK_TFLOPS if bf else FP32_VECTOR_PEAK_TFLOPS
            roof = min(peak, head_flops / hb * HBM_PEAK_GBS / 1e3)
            got = head_flops / (per_us[2] * 1e-6) / 1e12
            head_roof = {"roofline_tflops": round(roof, 1), "bound": "mfma" if roof == peak else "hbm",
                         "frac": round(got / roof, 4), "bytes": hb}
        copy = None
        if args.copy_check:
            copy = copy_bandwidth(dev)
            log(f"[bench] device copy: {copy:.0f} GB/s (read + write bytes); attention at {achieved / copy:.1%} of it")
        out = {
            "metric": METRIC,
            "value": round(value, 1),
            "unit": "stream-steps/s",
            "n_gpus": 1,
            "steps": timed_steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": ("bf16" if bf else "f32") if f8 is None else "bf16 q/o, e4m3 kv",
            "data": "synthetic (seeded N(0,1) q/K/V, N(0,0.02) head weights; no dataset or checkpoint)",
            "config": {
                "workload": c.workload,
                "streams": c.B, "queries_per_stream": c.Kq, "q_heads": c.H_q, "kv_heads": c.H_kv,
                "head_dim": c.D, "kv_len": "x".join(str(a) for a in c.kv_len_dist), "block_size": c.block_size,
                "d_model": c.d_model, "codebook": c.V, "heads": c.G, "decoding": c.mode,
                "launch": f"decode loop: {n_loop} steps per HIP graph" if graph else "eager",
                "head": "linear" if mlp is None else "two-layer d->4096->Mish->V",
                "append": "plain" if rope_pos is None else "rope at logical positions",
                "kv_cache": "bf16" if f8 is None else "e4m3 + fp32 row scales",
            },
            "roofline": {
                "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "decode_attention",
                "algorithmic_bytes_per_launch": attn_bytes,
            },
            "per_call_us": {("kv_cache_append" if rope_pos is None else "rope_kv_cache_append"): round(per_us[0], 2), "decode_attention": round(per_us[1], 2),
                            ("codebook_head" if mlp is None else "codebook_head_mlp"): round(per_us[2], 2),
                            ("spec_verify" if spec is not None else "sample_or_argmax"): round(per_us[3], 2)},
            "per_call_us_p10_median_p90": {k: [round(float(v), 2) for v in pct[:, i]] for i, k in enumerate(
                ("append", "decode_attention", "head", "verify" if spec is not None else "token"))},
            "step_us_p10_median_p90_events": [round(float(v), 2) for v in step_pct],
            "input_replicas": n_rep,
            "codebook_head_tflops": round(head_flops / (per_us[2] * 1e-6) / 1e12, 2),
            "codebook_head_roofline": head_roof,
            "hbm_copy": None if copy is None else {"copy_GBs": round(copy, 1),
                                                   "attention_frac_of_copy": round(achieved / copy, 4)},
            "cpu_baseline": cpu,
            "parity": parity,
        }
        if bf:
            out["codebook_head_mfma_frac"] = round(head_flops / (per_us[2] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        if spec is not None:
            # verified positions are B*Kq per step; the tokens kept are what the
            # verification emitted (the same every step: the inputs do not change)
            emitted = int(num_em.sum().item())
            out["emitted_tokens_per_s"] = round(emitted / (wall / timed_steps), 1)
            out["emitted_per_stream"] = round(emitted / c.B, 3)
        return out

    args.copy_check = not args.no_copy_check
    out = run_one(args)
    default_step = (args.workload == DEFAULT_WORKLOAD and args.kv == "bf16" and args.head == "linear"
                    and args.append == "plain" and args.graph == "off" and not args.copy_calibration)
    if default_step and not args.no_other_workloads:
        # the four smaller workloads, eager, after the main measurement: each
        # one's own step time and attention rate (not part of `value`)
        import copy
        others = {}
        for w in ("c1", "c2", "c3", "c4"):
            a = copy.copy(args)
            a.workload, a.no_cpu_baseline, a.copy_check = w, True, False
            a.steps, a.warmup = min(args.steps, 50), min(args.warmup, 10)
            torch.cuda.empty_cache()
            o = run_one(a)
            keep = {k: o[k] for k in ("value", "unit", "ms_per_step", "steps", "dtype", "per_call_us",
                                     "per_call_us_p10_median_p90", "input_replicas",
                                     "codebook_head_tflops", "codebook_head_mfma_frac", "codebook_head_roofline",
                                     "emitted_tokens_per_s", "emitted_per_stream") if k in o}
            keep["attention_hbm_frac"] = o["roofline"]["frac"]
            others[o["config"]["workload"]] = keep
        out["other_workloads"] = others
        # the launch-bound steps (one and 16 streams) again as the native decode
        # loop: 16 steps per HIP graph, lengths advancing on the device
        loops = {}
        for w in ("c1", "c2"):
            a = copy.copy(args)
            a.workload, a.no_cpu_baseline, a.copy_check, a.graph = w, True, False, "on"
            a.steps, a.warmup = 48, 16
            torch.cuda.empty_cache()
            o = run_one(a)
            loops[o["config"]["workload"]] = {k: o[k] for k in ("value", "unit", "ms_per_step", "steps")}
        out["graph_loop"] = loops
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
