"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Sizes: full configurations where the oracle finishes in seconds, with token
counts that leave ragged M tiles; at the largest sizes (T=8192 prefill,
T=16384 W8A8) the GPU runs the whole batch in the launch configuration the
benchmark times and the oracle computes a sample of token rows (first, last,
tile edges and random rows), which is exact because every output row depends
only on its own token.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import mla_prolog_amd as mlap
import oracle
import synth
from parity import check_bf16, check_prolog, run_staged, staged_names

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def run_gpu(cfg, inp, t_max=None, outputs=None):
    """One run with every output the staged check reads (q_norm and the taps included)."""
    p = mlap.Prolog.from_config(cfg, t_max=t_max)
    T = int(inp["x"].shape[0])
    out = p.run(to_dev(inp), outputs=outputs if outputs is not None else p.alloc_outputs(T, want=staged_names(cfg)))
    torch.cuda.synchronize()
    return out


def run_checked(cfg, inp, t_max=None, rows=None):
    """The run and its position-0 twin, then the staged parity check (tests/parity.py)."""
    p = mlap.Prolog.from_config(cfg, t_max=t_max)
    out, out0 = run_staged(p, cfg, to_dev(inp))
    return out, check_prolog(cfg, inp, out, out0, rows=rows)


def fmt(stats):
    return {k: (tuple(round(x, 4) for x in v) if isinstance(v, tuple) else round(v, 4)) for k, v in stats.items()}


# ------------------------------------------------------------- GEMM cores ----

@pytest.mark.parametrize("M,N,K", [(200, 264, 448), (1, 8, 64), (129, 2112, 1536)])
def test_gemm_bf16_core(M, N, K):
    say("gemm_bf16", M, N, K)
    g = torch.Generator().manual_seed(M * 7 + N)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    B = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16)
    C = mlap.gemm_bf16(A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16(synth.bf16_bits(A), synth.bf16_bits(B))
    exact = check_bf16("C", C, ref)
    assert exact > 0.99, exact


# The int32 export runs the W8A8 prolog's own tiles for an M-token batch: M > 512 the LDS-DMA
# 256 x 256 tiles (N = 2112: 8 of them plus the 64 x 64 remainder tiles; N = 24576: the q up
# projection's 96 column tiles), M <= 512 the small-batch register-staged tiles (N = 2112:
# 256 x 64; N = 24576: 128 x 192), at the V3 W8A8 projection shapes, ragged batches included.
@pytest.mark.parametrize("M,N,K", [(37, 200, 256), (130, 136, 7168), (1, 1, 128),
                                   (1000, 2112, 7168), (1000, 24576, 1536), (513, 2112, 7168),
                                   (130, 2112, 7168), (130, 24576, 1536), (600, 520, 256)])
def test_gemm_i8_core_bit_exact(M, N, K):
    say("gemm_i8", M, N, K)
    g = torch.Generator().manual_seed(M + N + K)
    A = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int8)
    B = torch.randint(-127, 128, (N, K), generator=g, dtype=torch.int8)
    Cg = mlap.gemm_i8_i32(A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cg.cpu().numpy(), oracle.gemm_i8(A.numpy(), B.numpy()))


def test_gemm_i8_core_extreme_accumulators():
    # every product at +-127^2 over K = 7168: the largest V3 magnitude, exact in int32
    K = 7168
    A = torch.full((64, K), 127, dtype=torch.int8)
    A[1::2] = -127
    B = torch.full((96, K), -127, dtype=torch.int8)
    Cg = mlap.gemm_i8_i32(A.to(DEV), B.to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(Cg, oracle.gemm_i8(A.numpy(), B.numpy()))
    assert abs(int(Cg[0, 0])) == K * 127 * 127


def _e4m3_table():
    return np.array([oracle.e4m3_value(c) for c in range(256)], np.float64)


@pytest.mark.parametrize("M,N,K,kind", [(200, 264, 1536, "weights"), (64, 128, 7168, "acts"),
                                        (300, 96, 512, "wide")])
def test_gemm_mxfp8_core(M, N, K, kind):
    """The block-scaled MFMA core against the exact sum of the dequantised products. The
    operand layout and the scale selection are exact (any slip is an O(1) error); the sum of
    the 64 products inside one instruction is the hardware's and not exact, so the bound is
    1e-3 of sum |products| per output (measured well below: ~1e-4 on operands spanning the whole
    E4M3 range, less on activation-like ones)."""
    say("gemm_mxfp8", M, N, K, kind)
    g = torch.Generator().manual_seed(M + N + K)
    tab = _e4m3_table()

    def codes(n, k):
        if kind == "wide":  # any non-NaN byte, subnormals included
            c = torch.randint(0, 256, (n, k), generator=g, dtype=torch.int32)
            c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
        else:
            c, _ = synth._mx_weight(g, n, k)
            return c
        return c.to(torch.uint8)

    A = codes(M, K)
    B = codes(N, K)
    if kind == "acts":  # A: MX conversion of N(0,1) rows (codes recovered from the oracle's values)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16)
        inv = {v: i for i, v in enumerate(tab) if not np.isnan(v)}
        rows, scs = [], []
        for r in synth.bf16_bits(x):
            deq, sc = oracle.mx_quant_row(r)
            q = oracle.f32(deq).astype(np.float64) / np.repeat(np.exp2(sc.astype(np.float64) - 127), 32)
            rows.append([inv[v] for v in q])
            scs.append(sc)
        A = torch.tensor(np.array(rows, np.uint8))
        As = torch.tensor(np.array(scs, np.uint8))
    else:
        As = torch.randint(120, 132, (M, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    Bs = torch.randint(118, 122, (N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    out = mlap.gemm_mxfp8_f32(A.cuda(), As.cuda(), B.cuda(), Bs.cuda())
    torch.cuda.synchronize()
    da = tab[A.numpy()] * np.repeat(np.exp2(As.numpy().astype(np.float64) - 127), 32, axis=1)
    db = tab[B.numpy()] * np.repeat(np.exp2(Bs.numpy().astype(np.float64) - 127), 32, axis=1)
    exact = da @ db.T
    mag = np.abs(da) @ np.abs(db).T
    err = np.abs(out.cpu().numpy().astype(np.float64) - exact)
    rel = err / np.maximum(mag, 1e-300)
    say("  max err / sum|products| = %.3g, median %.3g" % (rel.max(), np.median(rel)))
    assert rel.max() <= 1e-3


# --------------------------------------------------------- whole prolog -----

CASES = [
    ("tiny_kv", None),
    ("v2lite_kv_decode", None),
    ("v2lite_kv_decode", 1),
    ("v3_decode", 8),         # the smoke case
    ("v3_decode", 37),
    ("v3_decode", 64),        # last batch size of the 64-row weight-streaming tiles
    ("v3_decode", 65),        # first batch size of the 256-row weight-streaming tiles
    ("v3_decode", 200),       # 128-row head tiles with a ragged second row tile
    ("v3_decode", None),      # T = 256, every row
    ("v3_decode", 512),       # the largest weight-streaming batch
    ("v3_prefill", 513),      # the smallest batch on the large-batch tiles, ragged row tile
    ("v2lite_kv_decode", 200),
    ("v2lite_kv_decode", 300),  # two row tiles of the narrow kv_b tiles
    ("v3_w8a8", 37),
    ("v3_w8a8", 130),
]


@pytest.mark.parametrize("name,T", CASES)
def test_prolog_parity(name, T):
    cfg = synth.get_config(name, T=T)
    say("prolog parity", name, "T=%d" % cfg.T)
    inp = synth.make_inputs(cfg)
    out, stats = run_checked(cfg, inp)
    say("  bit-exact fractions / excused rows / e2e (inside, worst):", fmt(stats))


# Numeric variants (configuration flags): RMSNorm variant A, the QuantRope3D de-interleaved
# rope, per-(token, head) q quant; alone and together, on each path (weight streaming,
# 64-row tiles, KV-Prolog mode, W8A8).
ALL3 = dict(norm_rsqrt=True, rope_interleaved=True, q_quant_per_head=True)
VARIANTS = [("v3_decode", 64, ALL3),
            ("v3_decode", None, dict(rope_interleaved=True)),
            ("v3_decode", 200, dict(q_quant_per_head=True)),
            ("v3_decode", 37, dict(norm_rsqrt=True)),
            ("v2lite_kv_decode", None, dict(norm_rsqrt=True, rope_interleaved=True)),
            ("tiny_kv", None, dict(rope_interleaved=True)),
            ("v3_w8a8", 130, ALL3),
            # the large-batch 256 x 256 heads tile (16 x 16 x 32 MFMAs in bf16): q with every
            # variant, kv_b in KV-Prolog mode, the V4 q projection before its per-head norm
            ("v3_decode", 600, ALL3),
            ("v2lite_kv_decode", 700, dict(norm_rsqrt=True, rope_interleaved=True)),
            ("v4_decode", 700, dict(norm_rsqrt=True)),
            # the V4-shape prolog (per-head q RMSNorm after q_b), alone and with the variants
            ("v4_decode", None, {}),
            ("v4_decode", 100, dict(norm_rsqrt=True, rope_interleaved=True)),
            ("v4_decode", 64, dict(q_quant_per_head=True)),
            # MXFP8 projections (E4M3 weights, E8M0 scales per 32 of K, MX-converted activations)
            ("v3_mxfp8", 64, {}),
            ("v3_mxfp8", 37, ALL3),
            ("v2lite_kv_decode", None, dict(mxfp8=True)),
            ("tiny_kv", None, dict(mxfp8=True)),
            ("v4_decode", 64, dict(mxfp8=True)),
            # ... on the block-scaled MFMA: weight streaming (64- and 256-row tiles), KV-Prolog
            # mode, the V4 shape, and a config whose kv_b falls back to the decoded weights
            ("v3_mxfp8", 64, dict(mxfp8_mfma=True)),
            ("v3_mxfp8", 200, dict(ALL3, mxfp8_mfma=True)),
            ("v2lite_kv_decode", None, dict(mxfp8=True, mxfp8_mfma=True)),
            ("v4_decode", 64, dict(mxfp8=True, mxfp8_mfma=True)),
            ("tiny_kv", None, dict(mxfp8=True, mxfp8_mfma=True))]


@pytest.mark.parametrize("name,T,var", VARIANTS)
def test_prolog_variants_parity(name, T, var):
    cfg = synth.get_config(name, T=T, **var)
    say("prolog parity", name, "T=%d" % cfg.T, var)
    inp = synth.make_inputs(cfg)
    out, stats = run_checked(cfg, inp)
    say("  bit-exact fractions / excused rows / e2e (inside, worst):", fmt(stats))


# W8A8 with rows longer than 8192 values: the activation quant holds 8192 values of a row in
# registers between its amax and its codes and reads the rest again (hidden 8320 = 65 K-tiles
# of 128 int8), on the weight-streaming and the large-batch tiles.
@pytest.mark.parametrize("T", [37, 520])
def test_prolog_w8a8_long_rows_parity(T):
    cfg = dataclasses.replace(synth.get_config("v3_w8a8", T=T), hidden=8320)
    say("prolog parity", "v3_w8a8 hidden=8320", "T=%d" % cfg.T)
    inp = synth.make_inputs(cfg)
    out, stats = run_checked(cfg, inp)
    say("  bit-exact fractions / excused rows / e2e (inside, worst):", fmt(stats))


def sample_rows(T, n_random=40, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 127, 128, 129, T // 2, T - 129, T - 128, T - 2, T - 1]
    rows = set(r for r in edges if 0 <= r < T) | set(rng.integers(0, T, n_random).tolist())
    return np.array(sorted(rows), dtype=np.int32)


# Batches past the weight-streaming bucket run the large-batch GEMM (256 x 256 tiles):
# mid sizes with ragged last tiles, and the full benchmark sizes.
@pytest.mark.parametrize("name,T", [("v3_prefill", 1000), ("v3_w8a8", 700),
                                    ("v2lite_kv_decode", 1000), ("v3_prefill", None),
                                    ("v3_w8a8", None)])
def test_prolog_parity_full_size_sampled_rows(name, T):
    cfg = synth.get_config(name, T=T)
    say("prolog full-size", name, "T=%d" % cfg.T)
    inp = synth.make_inputs(cfg)
    rows = sample_rows(cfg.T)
    rows = np.union1d(rows, [r for r in (255, 256, 511, 512, 767, 768) if r < cfg.T]).astype(np.int32)
    out, stats = run_checked(cfg, inp, rows=rows)
    say("  rows", len(rows), fmt(stats))
    # every row with a nonzero amax reaches |code| = 127
    if "q_i8" in out:
        assert (out["q_i8"].abs().reshape(cfg.T, -1).amax(1) == 127).all()
    assert (out["kv_i8"].abs().amax(1) == 127).all()


# Batch sizes drawn from a seeded generator, per configuration one up to 64 tokens (the 32- and
# 64-row tiles), one in the 256-row weight-streaming bucket and one past it, each with a seeded
# choice of the numeric variants, so that parity does not rest on hand-picked edges alone; rows
# are sampled past 512 tokens (the full rows below that).
def _sweep():
    rng = np.random.default_rng(20261202)
    flag_sets = [{}, dict(norm_rsqrt=True), dict(rope_interleaved=True), dict(q_quant_per_head=True), ALL3]
    cases = []
    for name in ("v3_decode", "v3_w8a8", "v2lite_kv_decode", "v4_decode", "v3_mxfp8", "tiny_kv"):
        for lo, hi in ((1, 65), (65, 513), (513, 1201)):
            var = dict(flag_sets[int(rng.integers(0, len(flag_sets)))])
            if name in ("v2lite_kv_decode", "tiny_kv"):
                var.pop("q_quant_per_head", None)  # no q path in KV-Prolog mode
            cases.append((name, int(rng.integers(lo, hi)), var))
    return cases


@pytest.mark.parametrize("name,T,var", _sweep())
def test_prolog_parity_seeded_batch_sizes(name, T, var):
    cfg = synth.get_config(name, T=T, **var)
    say("prolog parity (seeded size)", name, "T=%d" % cfg.T, var)
    inp = synth.make_inputs(cfg)
    rows = sample_rows(cfg.T, n_random=24) if cfg.T > 512 else None
    out, stats = run_checked(cfg, inp, rows=rows)
    say("  rows", cfg.T if rows is None else len(rows), fmt(stats))


# ------------------------------------------------------------- invariants ----

def test_rope_keeps_pair_norms_against_position_zero():
    cfg = synth.get_config("v3_decode", T=16)
    inp = synth.make_inputs(cfg)
    a = run_gpu(cfg, inp)
    inp0 = dict(inp, positions=torch.zeros(cfg.T, dtype=torch.int32))
    b = run_gpu(cfg, inp0)
    h = cfg.rope_dim // 2
    for k in ("q_pe", "k_pe"):
        pa, pb = a[k].float().cpu(), b[k].float().cpu()
        na = pa[..., :h] ** 2 + pa[..., h:] ** 2
        nb = pb[..., :h] ** 2 + pb[..., h:] ** 2
        torch.testing.assert_close(na, nb, rtol=2e-2, atol=1e-4)
    # the nope part does not depend on the position at all
    torch.testing.assert_close(a["q_nope"], b["q_nope"], rtol=0, atol=0)
    torch.testing.assert_close(a["kv_norm"], b["kv_norm"], rtol=0, atol=0)


def test_position_zero_rope_is_identity_on_gpu():
    # at position 0, q_pe must equal the raw q_b rope slice: compare with a kv_b-free run whose
    # q_b weight has the rope rows copied into nope rows of another head
    cfg = synth.get_config("v3_decode", T=8)
    inp = synth.make_inputs(cfg)
    inp["positions"] = torch.zeros(cfg.T, dtype=torch.int32)
    w = inp["w_qb"].clone().view(cfg.n_heads, cfg.q_head, cfg.q_lora)
    w[1, : cfg.rope_dim] = w[0, cfg.nope_dim:]   # head 1 nope[0:64] = head 0 rope rows
    inp["w_qb"] = w.reshape(-1, cfg.q_lora).contiguous()
    out = run_gpu(cfg, inp)
    torch.testing.assert_close(out["q_pe"][:, 0], out["q_nope"][:, 1, : cfg.rope_dim],
                               rtol=0, atol=0)


def test_identical_kv_rows_normalise_to_gamma():
    cfg = synth.get_config("v3_decode", T=24)
    inp = synth.make_inputs(cfg)
    w = inp["w_kva"].clone()
    w[: cfg.kv_lora] = w[0]
    inp["w_kva"] = w
    out = run_gpu(cfg, inp)
    g = inp["gamma_kv"].float()
    kvn = out["kv_norm"].float().cpu()
    sign = torch.sign(kvn[:, :1])
    torch.testing.assert_close(kvn, sign * g[None, :], rtol=0, atol=0)


def test_zero_tokens_give_zero_outputs_and_zero_scales():
    cfg = synth.get_config("v3_decode", T=9)
    inp = synth.make_inputs(cfg)
    x = inp["x"].clone()
    x[3] = 0
    x[7] = 0
    inp["x"] = x
    out, _ = run_checked(cfg, inp)
    for k in ("q_nope", "q_pe", "kv_norm", "k_pe", "q_i8", "kv_i8"):
        assert not out[k][[3, 7]].float().abs().sum().item(), k
    assert out["q_scale"][[3, 7]].abs().sum().item() == 0
    assert out["kv_scale"][[3, 7]].abs().sum().item() == 0


def test_last_table_position_and_t_max():
    cfg = synth.get_config("v2lite_kv_decode", T=5)
    inp = synth.make_inputs(cfg)
    inp["positions"] = torch.full((5,), cfg.max_pos - 1, dtype=torch.int32)
    run_checked(cfg, inp, t_max=5)


def test_subset_of_outputs_and_repeatability():
    cfg = synth.get_config("v3_decode", T=33)
    inp = synth.make_inputs(cfg)
    p = mlap.Prolog.from_config(cfg)
    d = to_dev(inp)
    full = p.run(d)
    full2 = p.run(d)
    torch.cuda.synchronize()
    for k in full:  # bitwise deterministic run to run
        assert torch.equal(full[k], full2[k]), k
    only = p.alloc_outputs(cfg.T, want=["kv_norm", "q_scale", "k_pe"])
    p.run(d, outputs=only)
    torch.cuda.synchronize()
    for k in only:
        assert torch.equal(only[k], full[k]), k


def test_q_norm_output_matches_oracle():
    cfg = synth.get_config("v3_decode", T=20)
    inp = synth.make_inputs(cfg)
    p = mlap.Prolog.from_config(cfg)
    outs, outs0 = run_staged(p, cfg, to_dev(inp),
                             outputs=p.alloc_outputs(cfg.T, want=["q_norm", "q_nope", "q_pe", "q_i8",
                                                                  "q_scale", "a_proj"]))
    check_prolog(cfg, inp, outs, outs0)


def test_empty_batch_is_a_noop():
    cfg = synth.get_config("v3_decode", T=4)
    inp = synth.make_inputs(cfg)
    p = mlap.Prolog.from_config(cfg)
    d = to_dev(inp)
    out = p.alloc_outputs(4)
    for v in out.values():
        v.fill_(7)
    d0 = {k: (v[:0] if k in ("x", "positions") else v) for k, v in d.items()}
    p.run(d0, outputs={k: v[:0] for k, v in out.items()})
    torch.cuda.synchronize()
    for v in out.values():
        assert (v.float() == 7).all()


# the variants on the large-batch kernels: the 256 x 256 heads epilogue (late cos/sin in LDS),
# the k_pe columns of the large-batch down projection (eight extra columns per 256 x 256 tile
# at V3 width; a split-K tail launch on the block-scaled MXFP8 route and at other widths), the
# wave-per-token row kernel and the W8A8 token blocks with their forked quant
@pytest.mark.parametrize("name,T,var", [("v3_prefill", 1000, ALL3), ("v3_prefill", 2048, ALL3),
                                        ("v3_w8a8", 2048, ALL3), ("v4_decode", 1000, {}),
                                        ("v4_decode", 2048, ALL3), ("v3_mxfp8", None, {}),
                                        ("v3_mxfp8", 1000, ALL3),
                                        ("v3_mxfp8", None, dict(mxfp8_mfma=True)),
                                        ("v3_mxfp8", 1000, dict(ALL3, mxfp8_mfma=True))])
def test_prolog_variants_large_batch_sampled_rows(name, T, var):
    cfg = synth.get_config(name, T=T, **var)
    say("variants, sampled rows", name, "T=%d" % cfg.T)
    inp = synth.make_inputs(cfg)
    out, stats = run_checked(cfg, inp, rows=sample_rows(cfg.T, n_random=24))
    say("  bit-exact fractions / excused rows / e2e (inside, worst):", fmt(stats))

