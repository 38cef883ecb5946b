"""KV cache write on the GPU (the ScatterUpdate of the prolog's kv results into the cache:
[V32] page, section 2.4; [BLOG] page, step 2), through the C ABI.

Each case runs the prolog with caches pre-filled with values the path never produces
(bf16 NaN bits, code -128, scale -1) and a seeded slot mapping with padding (-1) and
out-of-range slots. Checks:

* every cache row a token maps to holds exactly that token's per-token output (bit for
  bit: the kernels store the same values twice), every other row keeps its fill;
* a run that requests only the caches writes the same cache rows;
* against the oracle (``oracle.kv_cache_write`` of the oracle's own per-token rows): on
  sampled tokens within the parity bounds (bf16 1e-3 + 1e-2|o| with the cast-point
  allowances of the stage-1 checks;
  codes +-1 with 99.9% exact, scales 1e-3), and for the small cases on whole caches,
  untouched rows included.

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
from parity import bits, check_bf16, check_quant_vs_oracle, norm_allowance, rope_allowance

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
         ("v3_w8a8", 130, 512)]


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

    outs = p.alloc_outputs(T)
    caches = fresh_caches(cfg, n_slots)
    p.run(dinp, outputs=dict(outs, **caches))
    torch.cuda.synchronize()

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

    # against the oracle on sampled tokens
    rng = np.random.default_rng(T)
    pick = toks if toks.size <= 48 else np.sort(rng.choice(toks, 48, replace=False))
    ref = oracle.prolog(cfg, inp, rows=pick)
    r = ix(s[pick])
    C = {k: v.detach().cpu() for k, v in caches.items()}
    check_bf16("kv_cache", C["kv_cache"][r], ref["kv_norm"], extra=norm_allowance(ref["kv_norm"]))
    check_bf16("kr_cache", C["kr_cache"][r], ref["k_pe"], extra=rope_allowance(ref["k_pe"], cfg.rope_dim))
    check_quant_vs_oracle("kv_cache_i8", bits(C["kv_cache"][r]), C["kv_cache_i8"][r].numpy(),
                          C["kv_cache_scale"][r].numpy(), ref["kv_norm"], ref["kv_i8"], ref["kv_scale"])

    # small runs: the oracle's whole caches, untouched rows included
    if T <= 64:
        full = oracle.prolog(cfg, inp)
        oc = {"kv_cache": np.full((n_slots, cfg.kv_lora), FILL["kv_cache"], np.uint16),
              "kv_cache_i8": np.full((n_slots, cfg.kv_lora), FILL["kv_cache_i8"], np.int8),
              "kv_cache_scale": np.full((n_slots,), FILL["kv_cache_scale"], np.float32),
              "kr_cache": np.full((n_slots, cfg.rope_dim), FILL["kr_cache"], np.uint16)}
        oracle.kv_cache_write(full, s, oc)
        for c in ("kv_cache", "kr_cache"):
            np.testing.assert_array_equal(bits(C[c])[untouched], oc[c][untouched])
        np.testing.assert_array_equal(C["kv_cache_i8"].numpy()[untouched], oc["kv_cache_i8"][untouched])
        np.testing.assert_array_equal(C["kv_cache_scale"].numpy()[untouched], oc["kv_cache_scale"][untouched])
        check_bf16("kv_cache[all]", C["kv_cache"][ix(rows)], oc["kv_cache"][rows],
                   extra=norm_allowance(oc["kv_cache"][rows]))
        check_bf16("kr_cache[all]", C["kr_cache"][ix(rows)], oc["kr_cache"][rows],
                   extra=rope_allowance(oc["kr_cache"][rows], cfg.rope_dim))
        check_quant_vs_oracle("kv_cache_i8[all]", bits(C["kv_cache"][ix(rows)]), C["kv_cache_i8"].numpy()[rows],
                              C["kv_cache_scale"].numpy()[rows], oc["kv_cache"][rows],
                              oc["kv_cache_i8"][rows], oc["kv_cache_scale"][rows])
    say("  cache rows match the per-token outputs bit for bit and the oracle within bounds")


def test_kv_cache_needs_slots():
    cfg = synth.get_config("v2lite_kv_decode", T=8)
    inp = {k: v.to(DEV) for k, v in synth.make_inputs(cfg).items()}
    p = mlap.Prolog.from_config(cfg)
    with pytest.raises(mlap.MlapError):
        p.run(inp, outputs=fresh_caches(cfg, 16))   # no slot_mapping
