"""KV cache write on the GPU (the ScatterUpdate of the prolog's kv results into the cache:
[V32] page, section 2.4; [BLOG] page, step 2), through the C ABI.

Each case runs the prolog with caches pre-filled with values the path never produces
(bf16 NaN bits, code -128, scale -1) and a seeded slot mapping with padding (-1) and
out-of-range slots. Checks:

* every cache row a token maps to holds exactly that token's per-token output (bit for
  bit: the kernels store the same values twice), every other row keeps its fill;
* a run that requests only the caches writes the same cache rows;
* the whole caches equal the oracle's scatter (``oracle.kv_cache_write``) of the GPU's
  per-token rows into caches with the same fill, bit for bit (the scatter is byte work);
* the per-token rows themselves pass the staged parity check against the oracle
  (tests/parity.py) on sampled tokens.

Cases cover each row-kernel variant: one workgroup per token with split-K partials
(T <= 512), the generic kernel with a bf16 down projection and an fp32 tail (T=1000),
one wave per token (T=2048), the KV-Prolog mode and W8A8.
"""
import sys

import numpy as np
import pytest
import torch

import mla_prolog_amd as mlap
import oracle
import synth
from parity import check_prolog, run_staged, staged_names

pytestmark = pytest.mark.gpu
DEV = "cuda"

FILL = {"kv_cache": 0x7FC1, "kv_cache_i8": -128, "kv_cache_scale": -1.0, "kr_cache": 0x7FC1}
PER_TOKEN = oracle.CACHE_OF  # cache -> per-token output


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def fresh_caches(cfg, n):
    bf = lambda w: torch.full((n, w), FILL["kv_cache"], dtype=torch.int16).view(torch.bfloat16)
    return {"kv_cache": bf(cfg.kv_lora).to(DEV),
            "kv_cache_i8": torch.full((n, cfg.kv_lora), FILL["kv_cache_i8"], dtype=torch.int8, device=DEV),
            "kv_cache_scale": torch.full((n,), FILL["kv_cache_scale"], dtype=torch.float32, device=DEV),
            "kr_cache": bf(cfg.rope_dim).to(DEV)}


def ix(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.long)


def raw(t):
    """Bit patterns (bf16 as int16) for exact comparisons, NaN fills included."""
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


CASES = [("v2lite_kv_decode", None, 200),
         ("v3_decode", 64, 160),
         ("v3_decode", None, 1024),
         ("v3_prefill", 1000, 4096),
         ("v3_prefill", 2048, 4096),
         ("v3_w8a8", 130, 512),
         ("v4_decode", None, 64),        # the V4 shape (per-head q norm after q_b)
         ("v3_mxfp8", 300, 1024)]        # MXFP8 projections


@pytest.mark.parametrize("name,T,n_slots", CASES)
def test_kv_cache_write(name, T, n_slots):
    cfg = synth.get_config(name, T=T)
    T = cfg.T
    say("kv cache write", name, "T=%d slots=%d" % (T, n_slots))
    inp = synth.make_inputs(cfg)
    slots = synth.slot_mapping(T, n_slots, seed=T)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    dinp["slot_mapping"] = slots.to(DEV)
    p = mlap.Prolog.from_config(cfg)

    outs = p.alloc_outputs(T, want=staged_names(cfg))
    caches = fresh_caches(cfg, n_slots)
    _, outs0 = run_staged(p, cfg, dinp, outputs=dict(outs, **caches))

    s = slots.numpy()
    valid = (s >= 0) & (s < n_slots)
    toks, rows = np.nonzero(valid)[0], s[valid]
    untouched = np.setdiff1d(np.arange(n_slots), rows)
    for c, src in PER_TOKEN.items():
        cache, per_tok = raw(caches[c]), raw(outs[src])
        np.testing.assert_array_equal(cache[rows], per_tok[toks], err_msg=c)
        fill = np.asarray(FILL[c], dtype=cache.dtype)
        assert (cache[untouched] == fill).all(), "%s: a row no token maps to was written" % c
    say("  %d tokens cached, %d padding / out of range" % (toks.size, T - toks.size))

    # only the caches requested
    caches2 = fresh_caches(cfg, n_slots)
    p.run(dinp, outputs=caches2)
    torch.cuda.synchronize()
    for c in PER_TOKEN:
        np.testing.assert_array_equal(raw(caches2[c]), raw(caches[c]), err_msg=c + " (caches only)")

    # the oracle's scatter of the GPU's per-token rows, into caches with the same fill
    oc = {c: raw(fresh_caches(cfg, n_slots)[c]) for c in PER_TOKEN}
    oracle.kv_cache_write({src: raw(outs[src]) for src in PER_TOKEN.values()}, s, oc)
    for c in PER_TOKEN:
        np.testing.assert_array_equal(raw(caches[c]), oc[c], err_msg=c + " (oracle scatter)")

    # the per-token rows against the oracle, staged, on sampled tokens
    rng = np.random.default_rng(T)
    pick = toks if toks.size <= 48 else np.sort(rng.choice(toks, 48, replace=False))
    st = check_prolog(cfg, inp, outs, outs0, rows=pick)
    say("  caches = oracle scatter of the per-token rows; staged parity:",
        {k: v if isinstance(v, tuple) else round(v, 4) for k, v in st.items()})


def test_kv_cache_needs_slots():
    cfg = synth.get_config("v2lite_kv_decode", T=8)
    inp = {k: v.to(DEV) for k, v in synth.make_inputs(cfg).items()}
    p = mlap.Prolog.from_config(cfg)
    with pytest.raises(mlap.MlapError):
        p.run(inp, outputs=fresh_caches(cfg, 16))   # no slot_mapping
