"""The allocation-free entry point mlap_run_static against mlap_run, through the C ABI.

mlap_run_static runs the same kernels as mlap_run with the library's own device scratch (one
64 MiB array per GPU) in place of the caller's workspace, for callers that cannot allocate. Its
outputs must equal mlap_run's bit for bit (the same kernels on the same inputs; mlap_run itself
is held to the oracle by the parity tests), over two calls in a row on one handle, the second
with fewer tokens (so it runs over the larger first call's leftovers in the shared scratch),
and across configurations and batch-size buckets: the decode tiles, the large-batch tiles, the
KV-Prolog mode and W8A8 on its large-batch int8 tiles.
"""
import sys

import pytest
import torch

import mla_prolog_amd as mlap
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _all_outputs(p, cfg, T):
    want = list(p.alloc_outputs(0).keys()) + (["q_norm"] if cfg.q_lora > 0 else [])
    return p.alloc_outputs(T, want=want)


@pytest.mark.parametrize("name,T1,T2", [("v3_decode", 256, 37), ("v3_prefill", 1000, 513),
                                         ("v2lite_kv_decode", 64, 5), ("v3_w8a8", 2048, 130),
                                         ("v4_decode", 16, 3)])
def test_run_static_matches_run(name, T1, T2):
    cfg1 = synth.get_config(name, T=T1)
    p = mlap.Prolog.from_config(cfg1, t_max=T1)
    assert p.workspace_size(T1) <= mlap.MLAP_STATIC_SCRATCH_BYTES
    for T in (T1, T2):
        say("run_static vs run", name, "T=%d" % T)
        cfg = synth.get_config(name, T=T)
        inp = {k: v.to(DEV) for k, v in synth.make_inputs(cfg).items()}
        ref = p.run(inp, outputs=_all_outputs(p, cfg, T))
        got = _all_outputs(p, cfg, T)
        for v in got.values():
            v.fill_(3)
        p.run_static(inp, outputs=got)
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(got[k], v), "%s T=%d: %s differs from mlap_run" % (name, T, k)
    say("  both calls bit-identical to mlap_run")


def test_run_static_rejects_runs_beyond_its_scratch():
    cfg = synth.get_config("v3_w8a8")     # T = 16384: ~190 MB of workspace
    p = mlap.Prolog.from_config(cfg)
    assert p.workspace_size(cfg.T) > mlap.MLAP_STATIC_SCRATCH_BYTES
    inp = {k: v.to(DEV) for k, v in synth.make_inputs(synth.get_config("v3_w8a8", T=8)).items()}
    x = torch.zeros(cfg.T, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    big = dict(inp, x=x, positions=torch.zeros(cfg.T, dtype=torch.int32, device=DEV))
    with pytest.raises(mlap.MlapError) as e:
        p.run_static(big, outputs=p.alloc_outputs(cfg.T, want=["kv_norm"]))
    assert e.value.status == mlap.MLAP_ERR_WORKSPACE
