#!/usr/bin/env python3
"""Benchmark of the MI355X MLA Prolog (one GPU).

One step = one whole prolog (every kernel of mlap_run) over one batch of
synthetic tokens already resident in HBM. The headline workload is the
DeepSeek-V3-shape prolog in prefill (T=8192 tokens, hidden 7168, q_lora 1536,
kv_lora 512, rope 64, nope 128, 128 heads, bf16, 1% outlier channels x20); the
same line carries the V3 decode batch (T=256) as a second measurement, timed
with four rotating weight/input sets (423 MB) so the 256 MB last-level cache
cannot hold the weights between steps.

Each workload is timed twice: eager launches (one prepared mlap_run call per
step) and a replay of the same steps from a HIP graph captured once. Both run the
whole step; the faster is the headline (``launch`` says which) and both are
reported (at decode the graph removes host launch gaps; at prefill, where the
host is far ahead, eager launches have measured slightly faster).

Prints ONE JSON line. ``roofline`` is for the dominant kernel (the q up
projection, gemm_up_q): its algorithmic FLOPs (or bytes) per step divided by its
time per step, measured with HIP events recorded around each of its launches on
the stream it runs on (large batches launch it once per token block). ``cpu_baseline`` times the CPU oracle on a
bounded sample of token rows of the same workload.

The default warmup is long (2000 steps, about 2 s at prefill) because the board's power
controller raises the shader clock gradually over the first seconds of sustained load
after idle: with 5 warmup steps the prefill step measured 0.98 ms at 1.6 GHz inside the q
projection, with 2000 0.94 ms at 1.8 GHz; the timed steps then see the steady state that a
continuously loaded GPU runs at.

    python bench.py [--gpus 1] [--steps 200] [--warmup 2000]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DOMINANT = "gemm_up_q"
PROFILE_INPUTS = os.path.join(ROOT, "profiles", "roofline_inputs.json")


def up_q_work(cfg, T):
    """Algorithmic FLOPs and bytes of one gemm_up_q launch over T tokens.

    FLOPs: 2*T*N*K with N = H*(nope+rope), K = q_lora. Bytes: the q_b weight once,
    q_norm in, q_nope and q_pe out (bf16), and each token's cos/sin row."""
    N = cfg.n_heads * cfg.q_head
    mfma8 = getattr(cfg, "mxfp8_mfma", False)  # E4M3 weights read directly, one scale per 32
    wbytes = N * cfg.q_lora * (1 if cfg.w8a8 else 1 + 1 / 32 if mfma8 else 2)
    flops = 2.0 * T * N * cfg.q_lora
    byts = wbytes + T * cfg.q_lora * 2 + T * N * 2 + T * cfg.rope_dim * 8
    return flops, byts


def up_kv_work(cfg, T):
    """Algorithmic FLOPs and bytes of one gemm_up_kv launch (KV-Prolog mode): the kv_b weight
    once, kv_norm in, k_nope and value out (bf16)."""
    N = cfg.n_heads * (cfg.nope_dim + cfg.v_dim)
    flops = 2.0 * T * N * cfg.kv_lora
    byts = N * cfg.kv_lora * 2 + T * cfg.kv_lora * 2 + T * N * 2
    return flops, byts


def path_work(cfg, T):
    """Algorithmic FLOPs and HBM bytes of the whole prolog (weights, x and outputs once)."""
    H, Dn, R, Lq, Lkv, Hd = cfg.n_heads, cfg.nope_dim, cfg.rope_dim, cfg.q_lora, cfg.kv_lora, cfg.hidden
    wb = 1 if cfg.w8a8 else 2
    N1 = Lq + Lkv + R
    flops = 2.0 * T * (N1 * Hd + H * (Dn + R) * Lq)
    weights = (N1 * Hd + H * (Dn + R) * Lq) * wb + (Lq + Lkv) * 2
    per_tok = (Hd * 2 + 4 + R * 8 + H * Dn * 2 + H * R * 2 + Lkv * 2 + R * 2 +
               H * (Dn + R) + 4 + Lkv + 4)
    return flops, weights + T * per_tok


def code_only(text):
    """C++ source without its comments and blank lines (the code a profile measured)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_hash():
    """Hash of the code that defines and launches the dominant kernel (the GEMM kernels,
    their tile choice and the host code that plans and launches them; sorted by name),
    comments left out so that a documentation edit does not void the profiles. The row
    kernels (row_kernels.hip) are left out: the up projections read nothing from them but
    their outputs."""
    d = os.path.join(ROOT, "mla_prolog_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")) and f != "row_kernels.hip":
            with open(os.path.join(d, f), encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def profiled(workload):
    """The committed rocprofv3 figures of the workload's dominant kernel (profiles/
    roofline_inputs.json, written by --summarize): HBM bytes per launch and the trace's
    average / median duration; None when missing or the kernel sources changed since."""
    try:
        with open(PROFILE_INPUTS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent


VARIANTS = dict(norm_rsqrt=True, rope_interleaved=True, q_quant_per_head=True)


def bench_workload(name, steps, warmup, rotate, dominant=DOMINANT, graph=True, kv_cache=False,
                   variants=False, mfma=False):
    """Times `steps` whole prolog runs of workload `name`, cycling through `rotate` input and
    weight sets. Two timed passes: eager (one mlap_run per step from a prepared call, with
    HIP events around every launch of the dominant kernel) and, when `graph`, the same
    steps replayed from a HIP graph that captured `rotate` consecutive runs (no host
    launch cost between kernels). With `kv_cache`, every step also writes the kv rows of its
    tokens into KV caches of 4 T slots (all four caches, every token cached); with
    `variants`, the run uses RMSNorm variant A, the de-interleaved RoPE and per-head q
    quant (VARIANTS); with `mfma`, MXFP8 runs on the block-scaled MFMA. Returns (cfg,
    eager ms/step, dominant kernel ms, eager percentiles, graph ms/step or None, graph
    percentiles or None). The dominant kernel entry is (ms per step by HIP events, shader clock in
    MHz averaged over its workgroups during the timed pass, or None where it did not run on
    the LDS-DMA GEMM)."""
    import torch

    import mla_prolog_amd as mlap
    import synth

    cfg = synth.get_config(name, **(VARIANTS if variants else {}), **({"mxfp8_mfma": True} if mfma else {}))
    T = cfg.T
    sets = []
    for r in range(rotate):
        seed = None if r == 0 else synth.seed_for(cfg) + 100 * r
        inp = synth.make_inputs(cfg, seed=seed)
        sets.append({k: v.cuda() for k, v in inp.items()})
        del inp
    p = mlap.Prolog.from_config(cfg)
    outs = p.alloc_outputs(T)
    if kv_cache:
        n_slots = 4 * T
        slots = synth.slot_mapping(T, n_slots, seed=1, pad_frac=0.0, out_of_range=0).cuda()
        for st in sets:
            st["slot_mapping"] = slots
        outs.update(kv_cache=torch.zeros(n_slots, cfg.kv_lora, dtype=torch.bfloat16, device="cuda"),
                    kv_cache_i8=torch.zeros(n_slots, cfg.kv_lora, dtype=torch.int8, device="cuda"),
                    kv_cache_scale=torch.zeros(n_slots, dtype=torch.float32, device="cuda"),
                    kr_cache=torch.zeros(n_slots, cfg.rope_dim, dtype=torch.bfloat16, device="cuda"))
    ws = p.workspace(T)
    runs = [p.bind(sets[r], outputs=outs, workspace=ws) for r in range(rotate)]
    for i in range(warmup):
        runs[i % rotate]()
    torch.cuda.synchronize()

    def timed(step_fn, n):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        marks[0].record()
        for i in range(n):
            step_fn(i)
            marks[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(n))
        pct = {"p10": round(per[int(0.1 * (n - 1))], 5), "p50": round(per[int(0.5 * (n - 1))], 5),
               "p90": round(per[int(0.9 * (n - 1))], 5)}
        return marks[0].elapsed_time(marks[-1]), pct

    # the dominant kernel may run as several launches per step (token blocks at large
    # batches): its time per step is the sum of its launches over the step
    p.timing_begin(dominant, steps * 8)
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    p.timing_clock(clk)  # shader clock of the dominant kernel's workgroups, over the timed pass
    total, pct = timed(lambda i: runs[i % rotate](), steps)
    ms_step = total / steps
    kms = p.timing_end()
    p.timing_clock(None)
    c = clk.cpu().tolist()
    sclk = round(c[0] / c[1] * 100.0) if c[1] > 0 else None
    k_avg = sum(kms) / steps

    g_ms = g_pct = None
    if graph:
        assert steps % rotate == 0, "graph replay covers whole rotations"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(rotate):
                p.bind(sets[r], outputs=outs, workspace=ws)()  # bound to the capture stream
        g.replay()
        torch.cuda.synchronize()
        gtotal, g_pct = timed(lambda i: g.replay(), steps // rotate)
        g_ms = gtotal / steps
        g_pct = {k: round(v / rotate, 5) for k, v in g_pct.items()}
        del g
    del sets
    return cfg, ms_step, (k_avg, sclk), pct, g_ms, g_pct


def power_sample(name, seconds, rotate=1):
    """Board power and shader clocks while workload `name` runs back to back for `seconds`
    (eager launches, `rotate` input sets): `amd-smi metric -p -c` is sampled from a second
    thread, a read-only sensor query. Returns one JSON-able dict: steps run, ms per step,
    socket power in W and the mean gfx clock over the XCDs in MHz (median, min, max over the
    samples taken in the middle half of the run)."""
    import subprocess
    import threading

    import torch

    import mla_prolog_amd as mlap
    import synth

    cfg = synth.get_config(name)
    sets = [{k: v.cuda() for k, v in synth.make_inputs(cfg, seed=None if r == 0 else synth.seed_for(cfg) + 100 * r).items()}
            for r in range(rotate)]
    p = mlap.Prolog.from_config(cfg)
    outs = p.alloc_outputs(cfg.T)
    ws = p.workspace(cfg.T)
    runs = [p.bind(sets[r], outputs=outs, workspace=ws) for r in range(rotate)]
    for i in range(10):
        runs[i % rotate]()
    torch.cuda.synchronize()
    samples, stop, errors = [], [], []

    def sampler():
        while not stop:
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True,
                                   text=True, timeout=30)
            except (OSError, subprocess.SubprocessError) as e:  # no amd-smi, or it hung
                errors.append(repr(e))
                return
            try:
                g = json.loads(r.stdout)
                g = g["gpu_data"][0] if isinstance(g, dict) and "gpu_data" in g else g[0]
                w = float(g["power"]["socket_power"]["value"])
                clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                samples.append((time.time(), w, sum(clks) / len(clks) if clks else None))
            except (ValueError, KeyError, TypeError, IndexError):
                pass
            time.sleep(0.25)

    th = threading.Thread(target=sampler)
    t0 = time.time()
    n = 0
    th.start()
    while time.time() - t0 < seconds:
        for i in range(20):
            runs[n % rotate]()
            n += 1
        torch.cuda.synchronize()
    dt = time.time() - t0
    stop.append(True)
    th.join()
    mid = [s for s in samples if t0 + 0.25 * dt <= s[0] <= t0 + 0.75 * dt]

    def stats(v):
        v = sorted(x for x in v if x is not None)
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1]} if v else None

    return {"workload": name, "T": cfg.T, "seconds": round(dt, 2), "steps": n, "ms_per_step": round(dt / n * 1e3, 5),
            "samples": len(mid), "socket_power_w": stats([s[1] for s in mid]),
            "gfx_clock_mhz": stats([s[2] for s in mid]),
            "source": "amd-smi metric -g 0 -p -c --json, sampled every ~0.25 s",
            "error": errors[0] if errors else (None if mid else "no readable amd-smi samples")}


def roofline_for(cfg, T, k, workload):
    """Roofline of the dominant kernel: its algorithmic FLOPs (MFMA-bound) or bytes (HBM-bound)
    per launch over its duration by HIP events in this run (``kernel_ms``); beside it the
    duration in the committed rocprofv3 trace of the same workload (``kernel_ms_trace``,
    average and median) with the ``frac`` that gives, the HBM bytes per launch from the
    committed counters (``traffic``), and the shader clock measured in the kernel (``sclk_mhz``)."""
    k_ms, sclk = k
    kv_mode = cfg.q_lora == 0
    flops, byts = (up_kv_work if kv_mode else up_q_work)(cfg, T)
    kernel = "gemm_up_kv" if kv_mode else DOMINANT
    intensity = flops / byts
    mfma8 = getattr(cfg, "mxfp8_mfma", False)
    peak_c = PEAK_I8_TOPS if cfg.w8a8 else PEAK_FP8_TFLOPS if mfma8 else PEAK_BF16_TFLOPS
    ridge = peak_c * 1e12 / (PEAK_HBM_GBS * 1e9)
    prof = profiled(workload)
    mfma = intensity >= ridge
    rate = (lambda ms: flops / (ms * 1e-3) / 1e12) if mfma else (lambda ms: byts / (ms * 1e-3) / 1e9)
    peak = peak_c if mfma else PEAK_HBM_GBS
    ach = rate(k_ms)
    out = {"bound": "mfma" if mfma else "hbm", "achieved": round(ach, 2 if mfma else 1), "peak": peak,
           "unit": ("TOP/s" if cfg.w8a8 else "TFLOP/s") if mfma else "GB/s", "frac": round(ach / peak, 4),
           "traffic": None, "kernel": kernel,
           "kernel_ms": round(k_ms, 5), "kernel_ms_trace": None, "frac_trace": None, "sclk_mhz": sclk,
           "algorithmic_flops": flops, "algorithmic_bytes": byts}
    if prof and prof.get("trace_us_avg"):
        # FLOPs, bytes and times are per step; a kernel launched once per token block
        # (launches_per_step > 1) adds its launches up
        n = prof.get("launches_per_step", 1)
        t_ms = n * prof["trace_us_avg"] / 1e3
        out["launches_per_step"] = n
        out["kernel_ms_trace"] = {"avg": round(t_ms, 5), "median": round(n * prof["trace_us_median"] / 1e3, 5),
                                  "sclk_mhz_traced": prof.get("sclk_mhz_traced"), "summary": prof.get("summary")}
        out["frac_trace"] = round(rate(t_ms) / peak, 4)
        if prof.get("hbm_bytes_per_launch"):
            out["traffic"] = n * prof["hbm_bytes_per_launch"]
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, seconds=20.0):
    """The CPU oracle, as it stands, on the first token rows of the same workload: on every
    host core this process may use and on one core, each the median of three timed runs on a
    fixed sample of rows sized from a probe so the whole measurement takes about `seconds`."""
    import statistics

    import numpy as np

    import oracle
    import synth

    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    ncores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def rate(threads, share):
        oracle.set_num_threads(threads)
        n = 2 * threads
        t0 = time.time()
        oracle.prolog(cfg, inp, rows=np.arange(n, dtype=np.int32))   # probe (also warms up)
        per_row = (time.time() - t0) / n
        n = int(min(cfg.T, max(threads, share / 3 / per_row)))
        rows = np.arange(n, dtype=np.int32)
        times = []
        for _ in range(3):
            t0 = time.time()
            oracle.prolog(cfg, inp, rows=rows)
            times.append(time.time() - t0)
        med = statistics.median(times)
        return n / med, n, med

    all_rate, n_all, t_all = rate(ncores, 0.75 * seconds)
    one_rate, n_one, t_one = rate(1, 0.25 * seconds)
    oracle.set_num_threads(ncores)
    return {"value": round(all_rate, 2), "unit": "tokens/s", "cores": ncores, "kind": "oracle",
            "one_core": {"value": round(one_rate, 3), "unit": "tokens/s", "cores": 1},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": "first %d (all cores) and %d (one core) of the %d token rows of %s, whole prolog "
                      "per row (fp64 sums, OpenMP over rows); median of 3 runs each: %.2f s and %.2f s"
                      % (n_all, n_one, cfg.T, name, t_all, t_one)}


def short_kernel(name):
    """Readable kernel name: drop the namespace, the argument list and spell bf16."""
    n = name.replace("void ", "").replace("mlap::", "").replace("unsigned short", "bf16")
    n = n.replace("signed char", "int8").replace("(Epi)", "Epi")
    return n.split("(")[0].strip()  # the argument list goes


def summarize(a):
    """rocprofv3 CSVs -> a markdown summary and the workload's entry in
    profiles/roofline_inputs.json (for the dominant kernel, matched by ``--dominant``).

    The summary gives, per kernel: the trace statistics; HBM bytes per dispatch from
    FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter read for the largest
    calibration dispatch of its run (a device copy of --calibrate-mib MiB for FETCH_SIZE, a
    fill of as many bytes for WRITE_SIZE); the MFMA pipe's busy share, SQ_VALU_MFMA_BUSY_CYCLES
    (summed over the 1024 SIMDs) over the trace median at the shader clock measured in the
    traced run (--sclk-mhz); the L2 hit rate; LDS bank-conflict cycles per LDS instruction;
    and the raw per-dispatch averages of every counter."""
    import csv
    import statistics
    from collections import defaultdict

    lines = ["# %s" % a.title, "", "Commands (from the repository root on the MI355X box):", ""]
    lines += ["    " + c for c in a.command]
    dur = defaultdict(list)
    with open(a.trace) as fh:
        for r in csv.DictReader(fh):
            dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in dur.values())
    cnt = defaultdict(lambda: defaultdict(list))
    for path in a.pmc:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                cnt[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    avg = {k: {c: sum(x) / len(x) for c, x in d.items()} for k, d in cnt.items()}
    calib = a.calibrate_mib * 1024.0  # KiB the calibration copy reads and the fill writes

    def largest(tag, counter):
        vals = [x for k in cnt if tag in k for x in cnt[k].get(counter, [])]
        return max(vals) if vals else 0.0

    f_ref, w_ref = largest("copyBuffer", "FETCH_SIZE"), largest("FillFunctor", "WRITE_SIZE")
    fscale = calib / f_ref if f_ref > 0 else None
    wscale = calib / w_ref if w_ref > 0 else None
    ours = [k for k in dur if "mlap::" in k]
    steps = min(len(dur[k]) for k in ours) if ours else 1

    def hbm(d):
        if fscale and wscale and "FETCH_SIZE" in d and "WRITE_SIZE" in d:
            return (d["FETCH_SIZE"] * fscale + d["WRITE_SIZE"] * wscale) * 1024
        return None

    lines += ["", "Per kernel. Durations in us from the kernel trace (averages include the first, cold "
              "launches). HBM bytes per dispatch are FETCH_SIZE and WRITE_SIZE scaled by the calibration "
              "below; MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over the trace median at %s; L2 hit "
              "is TCC_HIT / (TCC_HIT + TCC_MISS); LDS conflict is SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS; L2 read "
              "latency is TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ in cycles (where that pass ran)."
              % ("%d MHz" % a.sclk_mhz if a.sclk_mhz else "(no clock given)"), "",
              "| kernel | calls | avg | median | % of GPU time | HBM MB / dispatch | MFMA busy | L2 hit | LDS conflict | L2 read latency |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        d = avg.get(k, {})
        med = statistics.median(v)
        b = hbm(d)
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES")
        mf = "%.1f%%" % (100 * busy / 1024.0 / (med * a.sclk_mhz)) if busy and a.sclk_mhz else ""
        hit = ("%.1f%%" % (100 * d["TCC_HIT_sum"] / max(1.0, d["TCC_HIT_sum"] + d["TCC_MISS_sum"]))
               if "TCC_HIT_sum" in d and "TCC_MISS_sum" in d else "")
        lds = "%.3f" % (d.get("SQ_LDS_BANK_CONFLICT", 0) / d["SQ_INSTS_LDS"]) if d.get("SQ_INSTS_LDS") else ""
        lat = ("%.0f" % (d["TCP_TCC_READ_REQ_LATENCY_sum"] / d["TCP_TCC_READ_REQ_sum"])
               if d.get("TCP_TCC_READ_REQ_sum") and "TCP_TCC_READ_REQ_LATENCY_sum" in d else "")
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %s | %s | %s | %s | %s |" % (
            short_kernel(k), len(v), sum(v) / len(v), med, 100 * sum(v) / total,
            "%.1f" % (b / 1e6) if b is not None else "", mf, hit, lds, lat))
    names = sorted({c for d in avg.values() for c in d})
    lines += ["", "Raw counters, average per dispatch (one rocprofv3 --pmc pass per group of counters; "
              "FETCH_SIZE and WRITE_SIZE in KiB):", "",
              "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k in sorted(avg, key=lambda k: -sum(dur.get(k, [0]))):
        lines.append("| `%s` | " % short_kernel(k) + " | ".join(
            ("%.4g" % avg[k][c]) if c in avg[k] else "" for c in names) + " |")
    lines += ["", "Calibration and derived figures:", ""]
    if fscale:
        lines.append("- FETCH_SIZE read %.0f KiB for the %d MiB device copy (scale %.3f); WRITE_SIZE read %s "
                     "KiB for the %d MiB fill (scale %s)." % (
                         f_ref, a.calibrate_mib, fscale, "%.0f" % w_ref if w_ref else "n/a",
                         a.calibrate_mib, "%.3f" % wscale if wscale else "n/a"))
    entry = None
    dom = [k for k in dur if a.dominant and a.dominant in k]
    if dom:
        k = dom[0]
        v = dur[k]
        per_step = len(v) / steps
        entry = {"kernel_source_hash": kernel_source_hash(), "kernel_name": short_kernel(k),
                 "launches_per_step": round(per_step),
                 "trace_us_avg": round(sum(v) / len(v), 3), "trace_us_median": round(statistics.median(v), 3),
                 "summary": os.path.relpath(a.out, ROOT), "sclk_mhz_traced": a.sclk_mhz}
        b = hbm(avg.get(k, {}))
        if b is not None:
            entry["hbm_bytes_per_launch"] = int(b)
            lines.append("- Dominant kernel `%s`: %d launch(es) per step, trace average %.2f us, median %.2f us; "
                         "HBM %.1f MB per launch (FETCH %.1f MB + WRITE %.1f MB, scaled)." % (
                             entry["kernel_name"], entry["launches_per_step"], entry["trace_us_avg"],
                             entry["trace_us_median"], b / 1e6, avg[k]["FETCH_SIZE"] * fscale * 1.024e-3,
                             avg[k]["WRITE_SIZE"] * wscale * 1.024e-3))
    if a.sclk_mhz:
        lines.append("- Shader clock %d MHz: measured inside the dominant kernel (clock64 over "
                     "wall_clock64, summed over its workgroups) by bench.py in the traced run." % a.sclk_mhz)
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if entry:
        try:
            with open(PROFILE_INPUTS) as fh:
                rec = json.load(fh)
        except (OSError, ValueError):
            rec = {}
        rec[a.workload] = entry
        with open(PROFILE_INPUTS, "w") as fh:
            json.dump(rec, fh, indent=1, sort_keys=True)
            fh.write("\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--decode-workload", default="v3_decode")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--extra-workloads", default="v3_w8a8,v2lite_kv_decode,v3_decode+kvcache,v3_decode+variants,v4_decode,"
                            "v3_mxfp8,v3_mxfp8+mfma,v3_mxfp8_decode,v3_mxfp8_decode+mfma",
                    help="comma-separated workloads reported as extra objects (empty: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay pass)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--rotate", type=int, default=1,
                    help="weight/input sets the headline workload cycles through")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (the reference "
                         "kernel whose HBM counters scale the profiled traffic)")
    ap.add_argument("--summarize", action="store_true",
                    help="no GPU: turn rocprofv3 CSVs (--trace, --pmc) into --out and the workload's "
                         "entry of profiles/roofline_inputs.json")
    ap.add_argument("--trace", help="rocprofv3 kernel_trace.csv (with --summarize)")
    ap.add_argument("--pmc", nargs="*", action="extend", default=[], help="rocprofv3 counter_collection.csv files")
    ap.add_argument("--out", help="summary to write (with --summarize)")
    ap.add_argument("--title", default="rocprofv3 summary")
    ap.add_argument("--command", action="append", default=[], help="a command that produced the CSVs")
    ap.add_argument("--dominant", help="substring of the dominant kernel's name (with --summarize)")
    ap.add_argument("--calibrate-mib", type=int, default=512)
    ap.add_argument("--sclk-mhz", type=int, default=None)
    ap.add_argument("--board-seconds", type=float, default=3.0, metavar="SECONDS",
                    help="after timing the headline workload, run it back to back this long and "
                         "record the board power and clocks in the line (0: skip)")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="instead of the benchmark: run --workload back to back for SECONDS and print "
                         "the board power and shader clocks sampled meanwhile (amd-smi)")
    a = ap.parse_args()
    if a.summarize:
        summarize(a)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.power > 0:
        print(json.dumps(power_sample(a.workload, a.power, rotate=a.rotate)), flush=True)
        return

    if a.copy_calibrate:
        n = a.copy_calibrate * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    import synth

    def dominant_of(name):  # the up projection that dominates: q_b, or kv_b in KV-Prolog mode
        return "gemm_up_kv" if synth.get_config(name).q_lora == 0 else DOMINANT

    cfg, e_ms, k_ms, e_pct, g_ms, g_pct = bench_workload(a.workload, a.steps, a.warmup, rotate=a.rotate,
                                                         dominant=dominant_of(a.workload),
                                                         graph=not a.no_graph)
    # headline: the faster of the two launch modes (both run the whole step); both reported
    use_g = g_ms is not None and g_ms < e_ms
    ms, pct = (g_ms, g_pct) if use_g else (e_ms, e_pct)
    T = cfg.T
    pf, pb = path_work(cfg, T)
    line = {
        "metric": "MLA Prolog tokens/s at V3 dims (T=256, T=8192); % MFMA / HBM roofline",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_percentiles": pct,
        "launch": "hip_graph" if use_g else "eager",
        "eager_ms_per_step": round(e_ms, 5),
        "graph_ms_per_step": round(g_ms, 5) if g_ms else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if cfg.w8a8 else "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: DeepSeek-V3 MLA Prolog, T=%d, hidden %d, q_lora %d, kv_lora %d, "
                               "rope %d, nope %d, heads %d" % (cfg.name, T, cfg.hidden, cfg.q_lora,
                                                               cfg.kv_lora, cfg.rope_dim,
                                                               cfg.nope_dim, cfg.n_heads),
                   "tokens": T, "parallelism": "none (1 GPU)"},
        "roofline": roofline_for(cfg, T, k_ms, cfg.name),
        "path": {"tflops": round(pf / (ms * 1e-3) / 1e12, 2),
                 "frac_bf16_peak": round(pf / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    if a.board_seconds > 0:
        # the board's socket power and shader clocks under sustained load of the headline
        # workload (the prefill step runs at the power limit, which sets its clock)
        b = power_sample(a.workload, a.board_seconds, rotate=a.rotate)
        line["board"] = {k: b[k] for k in ("seconds", "ms_per_step", "samples", "socket_power_w",
                                           "gfx_clock_mhz", "source", "error")}
    if a.decode_workload:
        dcfg, de_ms, dk_ms, de_pct, dg_ms, dg_pct = bench_workload(a.decode_workload, a.decode_steps,
                                                                   a.warmup, rotate=4,
                                                                   dominant=dominant_of(a.decode_workload),
                                                                   graph=not a.no_graph)
        d_use_g = dg_ms is not None and dg_ms < de_ms
        dms, dpct = (dg_ms, dg_pct) if d_use_g else (de_ms, de_pct)
        dpf, dpb = path_work(dcfg, dcfg.T)
        line["decode"] = {
            "workload": "%s: DeepSeek-V3 MLA Prolog decode batch, T=%d, 4 rotating weight sets"
                        % (dcfg.name, dcfg.T),
            "value": round(dcfg.T / (dms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(dms, 5), "step_ms_percentiles": dpct, "steps": a.decode_steps,
            "launch": "hip_graph" if d_use_g else "eager", "eager_ms_per_step": round(de_ms, 5),
            "graph_ms_per_step": round(dg_ms, 5) if dg_ms else None,
            "roofline": roofline_for(dcfg, dcfg.T, dk_ms, dcfg.name),
            "path": {"hbm_gbs": round(dpb / (dms * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(dpb / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": dpb},
        }
        # the same batch with one weight set, which stays in the 256 MB last-level cache
        # between steps (a serving loop that runs nothing else): the warm figure
        _, we_ms, wk_ms, _, wg_ms, _ = bench_workload(a.decode_workload, a.decode_steps, a.warmup,
                                                      rotate=1, graph=not a.no_graph)
        wms = min(wg_ms, we_ms) if wg_ms else we_ms
        line["decode"]["warm"] = {"value": round(dcfg.T / (wms * 1e-3), 1), "unit": "tokens/s",
                                  "ms_per_step": round(wms, 5), "eager_ms_per_step": round(we_ms, 5),
                                  "gemm_up_q_ms": round(wk_ms[0], 5)}
    extra = {}
    for name in [w for w in a.extra_workloads.split(",") if w]:
        import synth
        base, _, opt = name.partition("+")
        ecfg0 = synth.get_config(base)
        dom = "gemm_up_kv" if ecfg0.q_lora == 0 else DOMINANT
        # decode-sized batches rotate weight sets so the last-level cache cannot hold them
        rot = 4 if ecfg0.T <= 512 else 1
        ecfg, ee_ms, ek_ms, ee_pct, eg_ms, eg_pct = bench_workload(base, a.steps, a.warmup, rotate=rot,
                                                                   dominant=dom, graph=not a.no_graph,
                                                                   kv_cache=opt == "kvcache",
                                                                   variants=opt == "variants",
                                                                   mfma=opt == "mfma")
        e_use_g = eg_ms is not None and eg_ms < ee_ms
        ems, epct = (eg_ms, eg_pct) if e_use_g else (ee_ms, ee_pct)
        epf, epb = path_work(ecfg, ecfg.T) if ecfg.q_lora else (None, None)
        ent = {"value": round(ecfg.T / (ems * 1e-3), 1), "unit": "tokens/s", "tokens": ecfg.T,
               "dtype": "int8" if ecfg.w8a8 else "fp8" if ecfg.mxfp8_mfma else "bf16",
               "ms_per_step": round(ems, 5),
               "step_ms_percentiles": epct, "steps": a.steps, "rotating_sets": rot,
               "launch": "hip_graph" if e_use_g else "eager", "eager_ms_per_step": round(ee_ms, 5),
               "graph_ms_per_step": round(eg_ms, 5) if eg_ms else None,
               "roofline": roofline_for(ecfg, ecfg.T, ek_ms, name)}
        if ecfg.mxfp8 and ecfg.mxfp8_mfma:
            ent["mxfp8"] = ("E4M3 weights with E8M0 scales per 32 of K on the block-scaled MFMA "
                            "(v_mfma_scale_f32_32x32x64_f8f6f4); activations converted to E4M3 codes "
                            "(mx_convert); roofline against the dense fp8 peak")
            ent["parity"] = ("opt-in route below the 99.9% INT8 code bar: the instruction's own sum "
                             "of 64 products is not exact, codes 99.86-99.94% exact against the "
                             "oracle at V3 sizes (bf16 outputs within the bound)")
        elif ecfg.mxfp8:
            ent["mxfp8"] = ("E4M3 weights with E8M0 scales per 32 of K, decoded to bf16 every step "
                            "(mx_convert) with the activations' MX conversion; bf16 MFMA GEMMs")
        if opt == "variants":
            ent["variants"] = "RMSNorm variant A (rsqrt), de-interleaved RoPE, per-(token, head) q quant"
        if opt == "kvcache":
            ent["kv_cache"] = {"slots": 4 * ecfg.T, "caches": "kv_norm bf16, kv codes, kv scale, k_pe",
                               "bytes_per_token": ecfg.kv_lora * 3 + 4 + ecfg.rope_dim * 2}
        if epf:
            peak = PEAK_I8_TOPS if ecfg.w8a8 else PEAK_FP8_TFLOPS if ecfg.mxfp8_mfma else PEAK_BF16_TFLOPS
            ent["path"] = {"tops": round(epf / (ems * 1e-3) / 1e12, 2),
                           "frac_peak": round(epf / (ems * 1e-3) / 1e12 / peak, 4)}
        extra[name] = ent
    if extra:
        line["extra_workloads"] = extra
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a.workload, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
