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

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DOMINANT = "gemm_up_q"
KERNEL_SOURCES = ["common.hpp", "gemm.hpp", "gemm_big.hpp", "gemm_kernels.hip", "launch.hpp", "mlap_host.hip"]


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


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_prolog_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "gemm_up_q_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


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
    percentiles or None)."""
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
    total, pct = timed(lambda i: runs[i % rotate](), steps)
    ms_step = total / steps
    kms = p.timing_end()
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
    return cfg, ms_step, k_avg, pct, g_ms, g_pct


def roofline_for(cfg, T, k_ms, workload):
    kv_mode = cfg.q_lora == 0
    flops, byts = (up_kv_work if kv_mode else up_q_work)(cfg, T)
    kernel = "gemm_up_kv" if kv_mode else DOMINANT
    intensity = flops / byts
    mfma8 = getattr(cfg, "mxfp8_mfma", False)
    peak_c = PEAK_I8_TOPS if cfg.w8a8 else PEAK_FP8_TFLOPS if mfma8 else PEAK_BF16_TFLOPS
    ridge = peak_c * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(workload)
    if intensity >= ridge:
        ach = flops / (k_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_c,
                "unit": "TOP/s" if cfg.w8a8 else "TFLOP/s", "frac": round(ach / peak_c, 4),
                "traffic": traffic, "kernel": kernel, "kernel_ms": round(k_ms, 5),
                "algorithmic_flops": flops, "algorithmic_bytes": byts}
    ach = byts / (k_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kernel,
            "kernel_ms": round(k_ms, 5), "algorithmic_flops": flops, "algorithmic_bytes": byts}


def cpu_baseline(name, seconds=12.0):
    """The CPU oracle, as it stands, on the first token rows of the same workload."""
    import numpy as np

    import oracle
    import synth

    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    n = 8
    for _ in range(2):  # size the sample from a timed probe (the second one warm and larger)
        t0 = time.time()
        oracle.prolog(cfg, inp, rows=np.arange(n, dtype=np.int32))
        dt = time.time() - t0
        n = int(min(cfg.T, max(n, seconds / max(dt / n, 1e-6) / (4 if _ == 0 else 1))))
    t0 = time.time()
    oracle.prolog(cfg, inp, rows=np.arange(n, dtype=np.int32))
    dt = time.time() - t0
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "first %d of the %d token rows of %s (whole prolog per row, fp64 sums, "
                      "OpenMP over rows), %.1f s" % (n, cfg.T, name, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
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
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

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
                                  "gemm_up_q_ms": round(wk_ms, 5)}
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
               "roofline": roofline_for(ecfg, ecfg.T, ek_ms, ecfg.name)}
        if ecfg.mxfp8 and ecfg.mxfp8_mfma:
            ent["mxfp8"] = ("E4M3 weights with E8M0 scales per 32 of K on the block-scaled MFMA "
                            "(v_mfma_scale_f32_32x32x64_f8f6f4); activations converted to E4M3 codes "
                            "(mx_convert); roofline against the dense fp8 peak")
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
