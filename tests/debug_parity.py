#!/usr/bin/env python3
"""Parity under the debug build (not a test module; tests/test_gpu_debug_build.py runs it).

Loads the bounds-checked library (mla_prolog_amd/libmlap_debug.so, compiled with MLAP_DEBUG,
named by MLAP_LIBRARY) and runs the staged parity check (tests/parity.py) at batch sizes that
leave ragged tiles on every tile shape: the 32-, 64- and 256-row weight-streaming tiles, the
256 x 256 tiles with their extra k_pe columns and the W8A8 token blocks, the V4 head norm, both
MXFP8 routes and the KV-cache scatter. After every case the kernels' failed bounds checks must
be none (mlap_debug_flags == 0). A last run with two positions outside the cos/sin table (which
the kernels clamp) must raise the position bit and nothing else, which shows the checks are
live. Prints one line per case.

    MLAP_LIBRARY=mla_prolog_amd/libmlap_debug.so python tests/debug_parity.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import torch  # noqa: E402

import mla_prolog_amd as mlap  # noqa: E402
import synth  # noqa: E402
from parity import check_prolog, run_staged  # noqa: E402

CASES = [
    ("tiny_kv", None, {}),
    ("v2lite_kv_decode", 1, {}),
    ("v2lite_kv_decode", 33, {}),
    ("v2lite_kv_decode", 301, {}),
    ("v3_decode", 1, {}),
    ("v3_decode", 33, {}),
    ("v3_decode", 65, {}),
    ("v3_decode", 257, {}),
    ("v3_decode", 511, dict(norm_rsqrt=True, rope_interleaved=True, q_quant_per_head=True)),
    ("v3_prefill", 513, {}),
    ("v3_prefill", 1001, dict(rope_interleaved=True)),
    ("v3_w8a8", 37, {}),
    ("v3_w8a8", 701, {}),
    ("v3_w8a8", 2049, dict(rope_interleaved=True)),
    ("v4_decode", 17, {}),
    ("v4_decode", 1001, {}),
    ("v3_mxfp8", 513, {}),
    ("v3_mxfp8", 513, dict(mxfp8_mfma=True)),
]


def main():
    lib = mlap.lib_path()
    assert lib.endswith("libmlap_debug.so"), "run with MLAP_LIBRARY naming the debug build, not " + lib
    assert mlap.debug_flags() is not None, "the library has no bounds checks"
    dev = torch.device("cuda:0")
    for name, T, var in CASES:
        cfg = synth.get_config(name, T=T, **var)
        print("case", name, "T=%d" % cfg.T, var or "", flush=True)
        inp = synth.make_inputs(cfg)
        p = mlap.Prolog.from_config(cfg)
        out, out0 = run_staged(p, cfg, {k: v.to(dev) for k, v in inp.items()})
        check_prolog(cfg, inp, out, out0)
        flags = mlap.debug_flags(reset=True)
        print("  parity ok, bounds-check flags 0x%x" % flags, flush=True)
        assert flags == 0, "%s T=%d: failed bounds checks 0x%x" % (name, cfg.T, flags)
    # the KV-cache scatter: padding (-1) and out-of-range slots are skipped, not violations
    cfg = synth.get_config("v3_decode", T=37)
    inp = {k: v.to(dev) for k, v in synth.make_inputs(cfg).items()}
    slots = synth.slot_mapping(cfg.T, 64, seed=3, pad_frac=0.2, out_of_range=2).to(dev)
    p = mlap.Prolog.from_config(cfg)
    outs = p.alloc_outputs(cfg.T)
    outs.update(kv_cache=torch.zeros(64, cfg.kv_lora, dtype=torch.bfloat16, device=dev),
                kr_cache=torch.zeros(64, cfg.rope_dim, dtype=torch.bfloat16, device=dev))
    p.run(dict(inp, slot_mapping=slots), outputs=outs)
    flags = mlap.debug_flags(reset=True)
    print("case kv cache scatter T=37, 64 slots: bounds-check flags 0x%x" % flags, flush=True)
    assert flags == 0
    # positive control: positions outside [0, max_pos) are clamped by the kernels (outside the
    # contract of mlap_run) and must raise exactly the position bit, so the checks are live
    cfg = synth.get_config("v3_decode", T=37)
    inp = {k: v.to(dev) for k, v in synth.make_inputs(cfg).items()}
    pos = inp["positions"].clone()
    pos[3] = cfg.max_pos + 5
    pos[20] = -3
    p = mlap.Prolog.from_config(cfg)
    p.run(dict(inp, positions=pos))
    flags = mlap.debug_flags(reset=True)
    print("case positions outside the table (control): bounds-check flags 0x%x" % flags, flush=True)
    assert flags == 64, "the position check did not fire alone: 0x%x" % flags
    print("debug build: every bounds check held", flush=True)


if __name__ == "__main__":
    main()
