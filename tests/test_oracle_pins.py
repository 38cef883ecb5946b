"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each check would fail for a plausible mistake in the oracle: a wrong rounding
rule, a transposed operand, a dropped term, a wrong sign or half in RoPE, a
wrong quantisation rule. None of them re-types the oracle's own formulas: they
use library routines (torch's bf16 conversion, numpy fp64 / complex128 maths,
exact rationals), closed forms and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

rng = np.random.default_rng(1234)


def to_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def from_bits(b):
    return oracle.f32(b)


def ulp_diff(a_bits, b_bits):
    """Distance in bf16 units between two bf16 bit arrays of the same sign."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    # map sign-magnitude to a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


# ------------------------------------------------------------------ bf16 ----

def test_bf16_rounding_matches_torch_library_conversion():
    # random values across many binades, plus exact ties, near-overflow, subnormals
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    base = to_bf16_bits(rng.standard_normal(5000).astype(np.float32)).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)            # exactly half-way between two bf16
    near_max = np.array([3.3895e38, 3.39e38, -3.3895e38, 3.3961e38], np.float32)
    subn = (rng.standard_normal(1000) * 1e-39).astype(np.float32)
    allv = np.concatenate([v, ties, near_max, subn, np.float32([0.0, -0.0, np.inf, -np.inf])])
    ours = oracle.bf16(allv)
    ref = to_bf16_bits(allv)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is half-way between 1 and 1+2^-7: even mantissa is 1.0
    assert oracle.bf16(np.float32([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is half-way between 1+2^-7 (odd) and 1+2^-6 (even): goes up
    assert oracle.bf16(np.float32([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert np.isnan(from_bits(oracle.bf16(np.float32([np.nan])))[0])


# ------------------------------------------------------------------ GEMM ----

def test_gemm_exact_rational_brute_force():
    M, N, K = 3, 5, 24
    X = to_bf16_bits(rng.standard_normal((M, K)))
    W = to_bf16_bits(rng.standard_normal((N, K)) * 0.05)
    Y = oracle.gemm_bf16(X, W)
    xf, wf = from_bits(X), from_bits(W)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(K))
            ref = to_bf16_bits(np.float32(float(exact)))
            assert Y[m, n] == ref, (m, n)


def test_gemm_selection_weights_return_columns_exactly():
    M, K, N = 7, 64, 40
    X = to_bf16_bits(rng.standard_normal((M, K)))
    sigma = rng.permutation(K)[:N]
    Wf = np.zeros((N, K), np.float32)
    Wf[np.arange(N), sigma] = 1.0
    Y = oracle.gemm_bf16(X, to_bf16_bits(Wf))
    np.testing.assert_array_equal(Y, X[:, sigma])


def test_gemm_against_numpy_fp64_and_orientation():
    M, N, K = 9, 33, 192
    X = to_bf16_bits(rng.standard_normal((M, K)))
    W = to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    Y = oracle.gemm_bf16(X, W)
    ref = to_bf16_bits((from_bits(X).astype(np.float64) @ from_bits(W).astype(np.float64).T)
                       .astype(np.float32))
    d = ulp_diff(Y, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    # identical weight rows give identical output columns; scaling W by 2 scales Y exactly
    W2 = W.copy()
    W2[5] = W2[3]
    Y2 = oracle.gemm_bf16(X, W2)
    np.testing.assert_array_equal(Y2[:, 5], Y2[:, 3])
    Y4 = oracle.gemm_bf16(X, to_bf16_bits(from_bits(W) * 2))
    np.testing.assert_array_equal(from_bits(Y4), from_bits(Y) * 2)


def test_gemm_i8_brute_force_and_bound():
    A = rng.integers(-127, 128, (4, 96)).astype(np.int8)
    B = rng.integers(-127, 128, (6, 96)).astype(np.int8)
    Cm = oracle.gemm_i8(A, B)
    for m in range(4):
        for n in range(6):
            assert Cm[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(96))
    # the largest V3 accumulator (K = 7168, all codes at 127) still fits int32
    A = np.full((1, 7168), 127, np.int8)
    assert oracle.gemm_i8(A, A)[0, 0] == 7168 * 127 * 127
    A = np.full((1, 140000), -127, np.int8)
    B = np.full((1, 140000), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i8(A, B)


# --------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_constant_row_gives_gamma():
    D = 512
    gamma = to_bf16_bits(rng.uniform(0.5, 1.5, D))
    for c in (1.0, -3.5, 0.25, 200.0):
        out = oracle.rmsnorm_row(to_bf16_bits(np.full(D, c)), gamma, 1e-6)
        np.testing.assert_array_equal(from_bits(out), np.sign(c) * from_bits(gamma))
    # where eps is not negligible against c^2 the closed form is gamma*c/sqrt(c^2+eps)
    c = 0.0078125
    out = oracle.rmsnorm_row(to_bf16_bits(np.full(D, c)), gamma, 1e-6)
    expect = from_bits(gamma).astype(np.float64) * c / np.sqrt(c * c + 1e-6)
    d = ulp_diff(out, to_bf16_bits(expect.astype(np.float32)))
    assert d.max() <= 1 and np.abs(from_bits(out) - expect).max() < 0.01


def test_rmsnorm_alternating_row_and_no_gamma():
    D = 1536
    row = np.where(np.arange(D) % 2 == 0, 0.75, -0.75)
    gamma = to_bf16_bits(rng.uniform(0.5, 1.5, D))
    out = oracle.rmsnorm_row(to_bf16_bits(row), gamma, 1e-6)
    np.testing.assert_array_equal(from_bits(out), np.sign(row) * from_bits(gamma))
    out = oracle.rmsnorm_row(to_bf16_bits(row), None, 1e-6)
    np.testing.assert_array_equal(from_bits(out), np.sign(row))


def test_rmsnorm_against_fp64_definition():
    D = 512
    for trial in range(20):
        y = from_bits(to_bf16_bits(rng.standard_normal(D) * rng.uniform(0.01, 10)))
        g = from_bits(to_bf16_bits(rng.uniform(0.5, 1.5, D)))
        ref = y.astype(np.float64) / np.sqrt(np.mean(y.astype(np.float64) ** 2) + 1e-6) * g
        out = oracle.rmsnorm_row(to_bf16_bits(y), to_bf16_bits(g), 1e-6)
        d = ulp_diff(out, to_bf16_bits(ref.astype(np.float32)))
        assert d.max() <= 1 and (d == 0).mean() > 0.98


def test_rmsnorm_eps_matters_for_tiny_rows():
    # mean square 1e-6 = eps: the norm must be 1/sqrt(2e-6), not 1/sqrt(1e-6)
    D = 64
    y = np.full(D, 1e-3, np.float32)
    out = from_bits(oracle.rmsnorm_row(to_bf16_bits(y), None, 1e-6))
    yb = from_bits(to_bf16_bits(y))[0].astype(np.float64)
    expect = yb / np.sqrt(yb * yb + 1e-6)
    np.testing.assert_allclose(out, expect, rtol=2 ** -8)
    assert abs(out[0] - 1.0) > 0.2


# ------------------------------------------------------------------ RoPE ----

def test_rope_position_zero_is_identity():
    R = 64
    cos, sin = synth.rope_table(4, R)
    u = to_bf16_bits(rng.standard_normal(R))
    out = oracle.rope_row(u, cos[0].numpy(), sin[0].numpy())
    np.testing.assert_array_equal(from_bits(out), from_bits(u))


def test_rope_matches_complex_rotation():
    # rotate-half RoPE = multiply (u_i + j u_{i+h}) by exp(j p theta_i)
    R, P = 64, 8192
    cos, sin = synth.rope_table(P, R)
    h = R // 2
    theta = np.array([10000.0 ** (-2.0 * i / R) for i in range(h)])
    for p in (1, 7, 1000, 8191):
        u = to_bf16_bits(rng.standard_normal(R))
        uf = from_bits(u).astype(np.float64)
        z = (uf[:h] + 1j * uf[h:]) * np.exp(1j * p * theta)
        ref = np.concatenate([z.real, z.imag]).astype(np.float32)
        out = oracle.rope_row(u, cos[p].numpy(), sin[p].numpy())
        np.testing.assert_allclose(from_bits(out), ref, rtol=2 ** -7, atol=1e-6)


def test_rope_unit_vectors_and_pair_norms():
    R, P = 16, 64
    cos, sin = synth.rope_table(P, R)
    h = R // 2
    p = 37
    for i in range(h):
        e = np.zeros(R, np.float32)
        e[i] = 1.0
        out = from_bits(oracle.rope_row(to_bf16_bits(e), cos[p].numpy(), sin[p].numpy()))
        np.testing.assert_array_equal(out[i], from_bits(to_bf16_bits(cos[p, i].numpy())))
        np.testing.assert_array_equal(out[i + h], from_bits(to_bf16_bits(sin[p, i].numpy())))
        # the other coordinates stay zero
        mask = np.ones(R, bool)
        mask[[i, i + h]] = False
        assert not out[mask].any()
    u = from_bits(to_bf16_bits(rng.standard_normal(R)))
    out = from_bits(oracle.rope_row(to_bf16_bits(u), cos[p].numpy(), sin[p].numpy()))
    n_in = u[:h] ** 2 + u[h:] ** 2
    n_out = out[:h] ** 2 + out[h:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=2 * 2 ** -7)


# ----------------------------------------------------------------- Quant ----

def test_quant_ties_to_even_when_multiplier_is_one():
    # amax = 127 makes the multiplier exactly 1: codes are the half-even integers of z
    z = np.float32([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 100.25, -126.75])
    codes, scale = oracle.quant_row(to_bf16_bits(z))
    np.testing.assert_array_equal(codes, [127, 2, 4, -2, -4, 0, 2, 0, 100, -127])
    assert scale == 1.0


def test_quant_zero_row_one_hot_and_symmetry():
    codes, scale = oracle.quant_row(np.zeros(64, np.uint16))
    assert scale == 0.0 and not codes.any()
    z = np.zeros(64, np.float32)
    z[9] = -0.3
    codes, scale = oracle.quant_row(to_bf16_bits(z))
    assert codes[9] == -127 and np.count_nonzero(codes) == 1
    assert scale == pytest.approx(from_bits(to_bf16_bits(z))[9] * -1 / 127, rel=1e-7)
    y = to_bf16_bits(rng.standard_normal(512))
    c1, s1 = oracle.quant_row(y)
    c2, s2 = oracle.quant_row(y ^ np.uint16(0x8000))
    np.testing.assert_array_equal(c1, -c2)
    assert s1 == s2


def test_quant_invariants_random_rows():
    for n in (512, 24576):
        for trial in range(5):
            z = to_bf16_bits(rng.standard_normal(n) * rng.uniform(0.01, 100))
            codes, scale = oracle.quant_row(z)
            zf = from_bits(z).astype(np.float64)
            assert np.abs(codes).max() == 127
            assert scale == pytest.approx(np.abs(zf).max() / 127, rel=1e-6)
            err = np.abs(zf - codes.astype(np.float64) * scale)
            assert err.max() <= scale / 2 * (1 + 1e-5)


# ---------------------------------------------------------------- Prolog ----

def _f64_prolog_kv(cfg, inp):
    """The KV Prolog in fp64 without any intermediate bf16 cast (numpy)."""
    x = from_bits(synth.bf16_bits(inp["x"])).astype(np.float64)
    Wkva = from_bits(synth.bf16_bits(inp["w_kva"])).astype(np.float64)
    Wkvb = from_bits(synth.bf16_bits(inp["w_kvb"])).astype(np.float64)
    g = from_bits(synth.bf16_bits(inp["gamma_kv"])).astype(np.float64)
    pos = inp["positions"].numpy()
    Lkv, R, H, Dn, Dv = cfg.kv_lora, cfg.rope_dim, cfg.n_heads, cfg.nope_dim, cfg.v_dim
    a = x @ Wkva.T
    ckv, kpe = a[:, :Lkv], a[:, Lkv:]
    kvn = ckv / np.sqrt((ckv ** 2).mean(1, keepdims=True) + cfg.eps) * g
    h = R // 2
    theta = np.array([10000.0 ** (-2.0 * i / R) for i in range(h)])
    z = (kpe[:, :h] + 1j * kpe[:, h:]) * np.exp(1j * pos[:, None] * theta[None, :])
    kpe_r = np.concatenate([z.real, z.imag], 1)
    kvb = (kvn @ Wkvb.T).reshape(-1, H, Dn + Dv)
    return dict(kv_norm=kvn, k_pe=kpe_r, k_nope=kvb[..., :Dn], value=kvb[..., Dn:])


def test_prolog_tiny_kv_against_fp64_without_casts():
    cfg = synth.get_config("tiny_kv")
    inp = synth.make_inputs(cfg)
    out = oracle.prolog(cfg, inp)
    ref = _f64_prolog_kv(cfg, inp)
    for k in ("kv_norm", "k_pe", "k_nope", "value"):
        got = from_bits(out[k]).astype(np.float64)
        # bf16 casts at three points: a few bf16 ulps of drift at most
        np.testing.assert_allclose(got, ref[k], rtol=3e-2, atol=2e-3, err_msg=k)
    # the kv quant reconstructs kv_norm within half a step
    kvn = from_bits(out["kv_norm"]).astype(np.float64)
    rec = out["kv_i8"].astype(np.float64) * out["kv_scale"][:, None]
    assert (np.abs(kvn - rec) <= out["kv_scale"][:, None] / 2 * (1 + 1e-5)).all()
    assert (np.abs(out["kv_i8"]).max(1) == 127).all()


def test_prolog_identical_kv_rows_give_gamma_and_position_zero_identity():
    cfg = synth.get_config("tiny_kv")
    inp = synth.make_inputs(cfg)
    w = inp["w_kva"].clone()
    w[: cfg.kv_lora] = w[0]                 # every c_kv column equal
    inp["w_kva"] = w
    inp["positions"] = torch.zeros(cfg.T, dtype=torch.int32)
    out = oracle.prolog(cfg, inp)
    g = from_bits(synth.bf16_bits(inp["gamma_kv"]))
    a0 = from_bits(oracle.gemm_bf16(synth.bf16_bits(inp["x"]), synth.bf16_bits(w[:1])))[:, 0]
    np.testing.assert_array_equal(from_bits(out["kv_norm"]), np.sign(a0)[:, None] * g[None, :])
    # RoPE at position 0 leaves the k_pe slice of the kv_a projection unchanged
    raw = oracle.gemm_bf16(synth.bf16_bits(inp["x"]), synth.bf16_bits(w[cfg.kv_lora:]))
    np.testing.assert_array_equal(from_bits(out["k_pe"]), from_bits(raw))


def test_prolog_v3_shape_small_T_invariants():
    cfg = synth.get_config("v3_decode", T=3)
    inp = synth.make_inputs(cfg)
    out = oracle.prolog(cfg, inp)
    H, Dn, R = cfg.n_heads, cfg.nope_dim, cfg.rope_dim
    assert out["q_nope"].shape == (3, H, Dn) and out["q_pe"].shape == (3, H, R)
    # q quant: one scale per token over [nope | rope] of every head
    qrow = np.concatenate([out["q_nope"], out["q_pe"]], axis=2).reshape(3, -1)
    qf = from_bits(qrow).astype(np.float64)
    np.testing.assert_allclose(out["q_scale"], np.abs(qf).max(1) / 127, rtol=1e-6)
    assert (np.abs(out["q_i8"]).reshape(3, -1).max(1) == 127).all()
    rec = out["q_i8"].reshape(3, -1).astype(np.float64) * out["q_scale"][:, None]
    assert (np.abs(qf - rec) <= out["q_scale"][:, None] / 2 * (1 + 1e-5)).all()
    # q path against fp64 without casts for the q_nope part (the chain x->q_a->norm->q_b)
    x = from_bits(synth.bf16_bits(inp["x"])).astype(np.float64)
    Wqa = from_bits(synth.bf16_bits(inp["w_qa"])).astype(np.float64)
    Wqb = from_bits(synth.bf16_bits(inp["w_qb"])).astype(np.float64)
    g = from_bits(synth.bf16_bits(inp["gamma_q"])).astype(np.float64)
    qa = x @ Wqa.T
    qn = qa / np.sqrt((qa ** 2).mean(1, keepdims=True) + cfg.eps) * g
    np.testing.assert_allclose(from_bits(out["q_norm"]), qn, rtol=2e-2, atol=1e-3)
    q = (qn @ Wqb.T).reshape(3, H, Dn + R)
    # bf16 casts of q_a and q_norm (~1.1e-3 rms relative each) feed a K=1536 sum and the
    # result is cast again: ~2e-3 rms drift on |q| ~ 0.8. A dropped gamma, eps or norm,
    # or a transposed weight, moves q by 1e-1 or more.
    err = np.abs(from_bits(out["q_nope"]) - q[..., :Dn])
    assert err.max() < 2.5e-2 and np.sqrt((err ** 2).mean()) < 4e-3


def test_prolog_rows_subset_is_rowwise():
    cfg = synth.get_config("v2lite_kv_decode", T=9)
    inp = synth.make_inputs(cfg)
    full = oracle.prolog(cfg, inp)
    sub = oracle.prolog(cfg, inp, rows=[7, 2, 2])
    for k in full:
        np.testing.assert_array_equal(sub[k], full[k][[7, 2, 2]], err_msg=k)


def test_prolog_w8a8_against_integer_brute_force():
    cfg = synth.get_config("v3_w8a8", T=2)
    inp = synth.make_inputs(cfg)
    out = oracle.prolog(cfg, inp, rows=[1])
    # q_norm from the dequantised q_a projection, rebuilt from exact integer products
    xq, xs = oracle.quant_row(synth.bf16_bits(inp["x"][1]))
    acc = inp["w_qa"].numpy().astype(np.int64) @ xq.astype(np.int64)
    qa = acc.astype(np.float64) * xs * inp["w_qa_scale"].numpy().astype(np.float64)
    g = from_bits(synth.bf16_bits(inp["gamma_q"])).astype(np.float64)
    qn = qa / np.sqrt((qa ** 2).mean() + cfg.eps) * g
    np.testing.assert_allclose(from_bits(out["q_norm"][0]), qn, rtol=2e-2, atol=1e-3)


def test_golden_v2lite_case_shapes():
    """Shapes of the pages' mla_prolog_001 case (minimal prefill)."""
    import json
    import os
    case = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "v2lite_mla_prolog_001_shapes.json")))
    cfg = synth.get_config("v2lite_kv_decode", T=case["hidden_states"][0] * case["hidden_states"][1])
    assert cfg.hidden == case["hidden_size"] and cfg.kv_lora == case["kv_lora_rank"]
    assert cfg.rope_dim == case["rope_dim"] and cfg.n_heads * cfg.kv_head == case["kv_b_weight"][1]
    inp = synth.make_inputs(cfg)
    # the pages give kv_a as [K, N] = [2048, 576]; ours is the [N, K] layout of the same matrix
    assert list(inp["w_kva"].shape[::-1]) == case["kv_a_weight"]
    assert list(inp["w_kvb"].shape[::-1]) == case["kv_b_weight"]
    out = oracle.prolog(cfg, inp)
    b, s = case["hidden_states"][:2]
    assert [b, cfg.n_heads, s, cfg.nope_dim] == case["k_nope"]
    assert [b, cfg.n_heads, s, cfg.v_dim] == case["value"]
    assert [b, 1, s, cfg.rope_dim] == case["k_pe"]
    assert out["k_nope"].shape == (b * s, cfg.n_heads, cfg.nope_dim)
    assert out["value"].shape == (b * s, cfg.n_heads, cfg.v_dim)
    assert out["k_pe"].shape == (b * s, cfg.rope_dim)
    assert case["eps"] == cfg.eps


# ------------------------------------------------------------------ KV cache ----

def test_cache_scatter_hand_example():
    """The cache write on a hand-made run: token rows land at their slots; padding (-1) and
    out-of-range slots write nothing; the other rows keep their contents."""
    rows = np.array([[11, 12, 13], [21, 22, 23], [31, 32, 33], [41, 42, 43], [51, 52, 53]],
                    dtype=np.uint16)
    slots = [4, -1, 0, 6, 2]          # 6 is past a 5-row cache
    cache = np.full((5, 3), 7, dtype=np.uint16)
    oracle.cache_scatter(slots, rows, cache)
    expect = np.array([[31, 32, 33], [7, 7, 7], [51, 52, 53], [7, 7, 7], [11, 12, 13]],
                      dtype=np.uint16)
    np.testing.assert_array_equal(cache, expect)
    # one value per row (the scales) and int8 rows take the same path
    sc = np.zeros(5, np.float32)
    oracle.cache_scatter(slots, np.array([1.5, 2.5, 3.5, 4.5, 5.5], np.float32), sc)
    np.testing.assert_array_equal(sc, [3.5, 0, 5.5, 0, 1.5])
    c8 = np.zeros((5, 2), np.int8)
    oracle.cache_scatter(slots, np.array([[1, -1], [2, -2], [3, -3], [4, -4], [5, -5]], np.int8), c8)
    np.testing.assert_array_equal(c8, [[3, -3], [0, 0], [5, -5], [0, 0], [1, -1]])


def test_cache_scatter_rejects_repeated_slots():
    with pytest.raises(ValueError):
        oracle.cache_scatter([1, 3, 1], np.zeros((3, 2), np.uint16), np.zeros((4, 2), np.uint16))
    # padding may repeat
    oracle.cache_scatter([-1, 3, -1], np.ones((3, 2), np.uint16), np.zeros((4, 2), np.uint16))


def test_slot_mapping_generator():
    s = synth.slot_mapping(300, 1024, seed=3).numpy()
    valid = s[(s >= 0) & (s < 1024)]
    assert len(np.unique(valid)) == valid.size          # distinct in-range slots
    assert (s == -1).any() and (s >= 1024).sum() == 2   # padding and out-of-range tokens
    np.testing.assert_array_equal(s, synth.slot_mapping(300, 1024, seed=3).numpy())


# ------------------------------------------------------- numeric variants ----

def test_rmsnorm_variant_a_closed_forms():
    """Variant A (rsqrt, 1/D after the sum): constant and alternating rows give +-gamma, the
    eps closed form holds, and it agrees with the fp64 definition within one bf16 ulp."""
    D = 512
    gamma = to_bf16_bits(rng.uniform(0.5, 1.5, D))
    for c in (1.0, -3.5, 0.25, 200.0):
        out = oracle.rmsnorm_row_rsqrt(to_bf16_bits(np.full(D, c)), gamma, 1e-6)
        np.testing.assert_array_equal(from_bits(out), np.sign(c) * from_bits(gamma))
    row = np.where(np.arange(D) % 2 == 0, 0.75, -0.75)
    np.testing.assert_array_equal(from_bits(oracle.rmsnorm_row_rsqrt(to_bf16_bits(row), None, 1e-6)),
                                  np.sign(row))
    y = np.full(64, 1e-3, np.float32)
    yb = from_bits(to_bf16_bits(y))[0].astype(np.float64)
    np.testing.assert_allclose(from_bits(oracle.rmsnorm_row_rsqrt(to_bf16_bits(y), None, 1e-6)),
                               yb / np.sqrt(yb * yb + 1e-6), rtol=2 ** -8)
    for trial in range(20):
        y = from_bits(to_bf16_bits(rng.standard_normal(D) * rng.uniform(0.01, 10)))
        g = from_bits(to_bf16_bits(rng.uniform(0.5, 1.5, D)))
        ref = y.astype(np.float64) / np.sqrt(np.mean(y.astype(np.float64) ** 2) + 1e-6) * g
        out = oracle.rmsnorm_row_rsqrt(to_bf16_bits(y), to_bf16_bits(g), 1e-6)
        d = ulp_diff(out, to_bf16_bits(ref.astype(np.float32)))
        assert d.max() <= 1 and (d == 0).mean() > 0.98
        # the two variants differ only in the last bits
        assert ulp_diff(out, oracle.rmsnorm_row(to_bf16_bits(y), to_bf16_bits(g), 1e-6)).max() <= 1


def test_chunked_rope_position_zero_deinterleaves():
    """QuantRope3D with chunk 2 at cos = 1, sin = 0: the output is the input with adjacent
    pairs split into the two halves (u0 u2 u4 ... | u1 u3 u5 ...)."""
    R = 64
    cos, sin = synth.rope_table(4, R)
    u = to_bf16_bits(rng.standard_normal(R))
    out = oracle.rope_row_chunked(u, cos[0].numpy(), sin[0].numpy(), 2)
    np.testing.assert_array_equal(from_bits(out), np.concatenate([from_bits(u)[0::2], from_bits(u)[1::2]]))
    # chunk = R is one chunk: no transpose, plain rotate-half
    p = 3
    np.testing.assert_array_equal(oracle.rope_row_chunked(u, cos[p].numpy(), sin[p].numpy(), R),
                                  oracle.rope_row(u, cos[p].numpy(), sin[p].numpy()))


def test_chunked_rope_is_the_interleaved_pair_rotation():
    """With chunk 2, pair (u_2i, u_2i+1) is rotated by p*theta_i as the complex number
    u_2i + j u_2i+1 (the interleaved-pair RoPE), real parts to column i, imaginary to i + R/2."""
    R, P = 64, 8192
    cos, sin = synth.rope_table(P, R)
    h = R // 2
    theta = np.array([10000.0 ** (-2.0 * i / R) for i in range(h)])
    for p in (1, 7, 1000, 8191):
        u = to_bf16_bits(rng.standard_normal(R))
        uf = from_bits(u).astype(np.float64)
        z = (uf[0::2] + 1j * uf[1::2]) * np.exp(1j * p * theta)
        ref = np.concatenate([z.real, z.imag]).astype(np.float32)
        out = oracle.rope_row_chunked(u, cos[p].numpy(), sin[p].numpy(), 2)
        np.testing.assert_allclose(from_bits(out), ref, rtol=2 ** -7, atol=1e-6)


def test_per_head_q_quant():
    """Per-(token, head) q quant: each head's [nope | pe] row is quantised on its own; every
    head reaches code 127 and the token's q row reconstructs within half a scale per head
    (plus the fp32 rounding of z * 127/amax, at most 127 * 2^-24 code units)."""
    cfg = synth.get_config("v3_decode", T=2, q_quant_per_head=True)
    inp = synth.make_inputs(cfg)
    out = oracle.prolog(cfg, inp, rows=np.array([1], np.int32))
    H, QH = cfg.n_heads, cfg.nope_dim + cfg.rope_dim
    q = np.concatenate([from_bits(out["q_nope"][0]), from_bits(out["q_pe"][0])], axis=1)  # [H, QH]
    codes = out["q_i8"][0].reshape(H, QH).astype(np.float64)
    sc = out["q_scale"][0]
    assert sc.shape == (H,)
    assert (np.abs(codes).max(1) == 127).all()
    np.testing.assert_allclose(sc, np.abs(q).max(1) / 127.0, rtol=1e-7)
    assert (np.abs(q - codes * sc[:, None]) <= sc[:, None] * (0.5 + 2.0 ** -16)).all()
    # the per-token form of the same run has one scale: the largest head's
    tok = oracle.prolog(synth.get_config("v3_decode", T=2), inp, rows=np.array([1], np.int32))
    assert tok["q_scale"][0] == sc.max()


# ----------------------------------------------------- V4-shape head norm ----

def test_golden_v4_case_shapes():
    """Sizes of the card's V4 test case; the q row reshapes to (num_heads, head_dim)."""
    import json
    import os
    case = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "v4_mla_prolog_t16_shapes.json")))
    cfg = synth.get_config("v4_decode")
    assert (cfg.T, cfg.n_heads, cfg.hidden, cfg.q_lora) == (case["t"], case["num_heads"], case["h"],
                                                           case["q_lora_rank"])
    assert cfg.nope_dim + cfg.rope_dim == case["head_dim"] and cfg.rope_dim == case["qk_rope_head_dim"]
    inp = synth.make_inputs(cfg)
    assert list(inp["w_qb"].shape) == [case["num_heads"] * case["head_dim"], case["q_lora_rank"]]
    out = oracle.prolog(cfg, inp, rows=np.array([0, 15], np.int32))
    assert out["q_nope"].shape[1:] == (case["num_heads"], case["head_dim"] - case["qk_rope_head_dim"])
    assert out["q_pe"].shape[1:] == (case["num_heads"], case["qk_rope_head_dim"])


def test_head_norm_is_scale_invariant_per_head():
    """With eps = 0 the per-head RMSNorm undoes a power-of-two scale of one head's q_b rows
    bit for bit (every step scales exactly); without the head norm the head scales by it."""
    from dataclasses import replace
    cfg = replace(synth.get_config("v4_decode", T=3), eps=0.0)
    inp = synth.make_inputs(cfg)
    QH = cfg.nope_dim + cfg.rope_dim
    h = 5
    scaled = dict(inp)
    w = inp["w_qb"].clone()
    w[h * QH:(h + 1) * QH] *= 8
    scaled["w_qb"] = w
    rows = np.array([0, 2], np.int32)
    a, b = oracle.prolog(cfg, inp, rows=rows), oracle.prolog(cfg, scaled, rows=rows)
    for k in ("q_nope", "q_pe", "q_i8", "q_scale"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    plain = replace(cfg, q_head_norm=False)
    a, b = oracle.prolog(plain, inp, rows=rows), oracle.prolog(plain, scaled, rows=rows)
    np.testing.assert_array_equal(from_bits(b["q_nope"][:, h]), 8 * from_bits(a["q_nope"][:, h]))


def test_head_norm_gives_unit_rms_heads():
    """At position 0 (RoPE is the identity) every head of q has mean square 1 up to the bf16
    rounding of its values."""
    cfg = synth.get_config("v4_decode", T=2)
    inp = synth.make_inputs(cfg)
    inp["positions"] = torch.zeros_like(inp["positions"])
    out = oracle.prolog(cfg, inp)
    q = np.concatenate([from_bits(out["q_nope"]), from_bits(out["q_pe"])], axis=2).astype(np.float64)
    ms = (q ** 2).mean(axis=2)
    assert np.abs(ms - 1).max() < 2.0 ** -7


# ------------------------------------------------------------------ MXFP8 ----

def test_e4m3_decode_all_codes():
    """Every E4M3FN byte decodes as torch's float8_e4m3fn does (NaN at 0x7F and 0xFF)."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_rounding_matches_torch_and_saturates():
    """Nearest E4M3 value, ties to even, against torch's conversion inside the finite range
    (grid points, midpoints, subnormals, random values); beyond 448 the MX conversion
    saturates to 448."""
    grid = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    grid = np.unique(grid[~np.isnan(grid)])
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([grid, mids, rng.uniform(-440, 440, 2000), rng.uniform(-0.02, 0.02, 2000)])
    vals = vals[np.abs(vals) < 448]
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_round(float(np.float32(v))) for v in vals])
    np.testing.assert_array_equal(got, ref)
    for v in (448.0, 449.0, 470.0, 511.9, 1e6):
        assert oracle.e4m3_round(v) == 448.0 and oracle.e4m3_round(-v) == -448.0


def test_mx_block_scale_rule():
    """Shared exponent floor(log2(amax)) - 8: amax 1.0 gives E8M0 119; the block's largest value
    lands in [256, 512) before rounding; an all-zero block gives zeros (scale byte 0); values
    on the E4M3 grid times a power of two come back exactly when the block's largest
    mantissa is at most 1.75 (1.875 * 2^e lands on 480 > 448 and saturates to 1.75 * 2^e)."""
    v = np.zeros(128, np.float32)
    v[:32] = rng.uniform(-1, 1, 32)
    v[0] = 1.0
    v[32:64] = rng.uniform(-3e-3, 3e-3, 32)
    codes = [0x38] + list(range(0x40, 0x5F))                             # 1.0 and 2 .. 28
    grid = np.array([oracle.e4m3_value(c) for c in codes])
    v[64:96] = (grid * 2.0 ** -12).astype(np.float32)
    v[96:128] = v[64:96]
    v[96] = 30 * 2.0 ** -12                                              # 1.875 * 2^4
    bitsv = to_bf16_bits(v)
    deq, sc = oracle.mx_quant_row(bitsv)
    assert sc[0] == 119
    b = from_bits(bitsv[32:64]).astype(np.float64)
    assert 256 <= np.abs(b).max() / 2.0 ** (int(sc[1]) - 127) < 512
    np.testing.assert_array_equal(from_bits(deq[64:96]), from_bits(bitsv[64:96]))
    assert from_bits(deq[96:97])[0] == 28 * 2.0 ** -12
    z, zs = oracle.mx_quant_row(to_bf16_bits(np.zeros(32, np.float32)))
    assert (z == 0).all() and zs[0] == 0


def test_mx_projection_is_the_bf16_gemm_of_dequantised_operands():
    """An MXFP8 projection equals the bf16 GEMM definition on its dequantised operands: the
    MX-converted activation row and the weights decoded with torch's E4M3 type times their
    E8M0 scales (exact in bf16 here). Checked on k_pe at position 0, where RoPE is the
    identity, of a small KV-Prolog configuration."""
    from dataclasses import replace
    cfg = replace(synth.get_config("tiny_kv"), mxfp8=True)
    inp = synth.make_inputs(cfg)
    assert int(inp["positions"][0]) == 0
    out = oracle.prolog(cfg, inp, rows=np.array([0], np.int32))
    xd, _ = oracle.mx_quant_row(synth.bf16_bits(inp["x"][0]))
    w = inp["w_kva"].view(torch.float8_e4m3fn).double()
    s = torch.exp2(inp["w_kva_mxscale"].double() - 127).repeat_interleave(32, dim=1)
    wd = to_bf16_bits((w * s).float().numpy())
    assert np.array_equal(from_bits(wd).astype(np.float64), (w * s).numpy())   # exact in bf16
    ref = oracle.gemm_bf16(xd.reshape(1, -1), wd)[0]
    np.testing.assert_array_equal(out["k_pe"][0], ref[cfg.kv_lora:cfg.kv_lora + cfg.rope_dim])


# ------------------------------------------------- W8A8 dequant and wiring ----

def _ulp_within(got_bits, exact_f64, n_ulp=1):
    """Every bf16 value within n_ulp bf16 steps of the exact value: a wrong factor (a dropped or
    squared activation scale, another channel's weight scale) moves it by far more."""
    got = from_bits(got_bits).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact_f64), 2.0 ** -126))) - 7)
    err = np.abs(got - exact_f64)
    assert (err <= n_ulp * ulp).all(), "worst %g ulp" % float((err / ulp).max())
    return err / ulp


def test_w8a8_dequant_k_pe_row_at_position_zero():
    """AT-10 card, section 四: y = dequant(int32 x_q . w_q, x_scale, w_scale). At position 0
    RoPE is the identity, so the W8A8 k_pe row is the dequantised kv_a projection of the rope
    channels itself: the exact product (integer brute force) times x_scale times each channel's
    w_scale, within one bf16 step."""
    cfg = synth.get_config("v3_w8a8", T=3)
    inp = synth.make_inputs(cfg)
    inp["positions"] = torch.zeros(cfg.T, dtype=torch.int32)
    out = oracle.prolog(cfg, inp)
    wq = inp["w_kva"].numpy().astype(np.int64)[cfg.kv_lora:]       # the rope channels
    ws = inp["w_kva_scale"].numpy().astype(np.float64)[cfg.kv_lora:]
    for t in range(cfg.T):
        xq, xs = oracle.quant_row(synth.bf16_bits(inp["x"][t]))
        assert 0.005 < xs < 0.2                                       # far from 1: a dropped scale shows
        acc = wq @ xq.astype(np.int64)
        _ulp_within(out["k_pe"][t], acc.astype(np.float64) * xs * ws)


def test_w8a8_dequant_q_nope_row_of_the_q_b_stage():
    """The q_b stage of the W8A8 path on a given q_norm row: per-token quant of that row, exact
    int32 products, dequant with the row's scale and each output channel's scale."""
    cfg = synth.get_config("v3_w8a8", T=2)
    inp = synth.make_inputs(cfg)
    qn = to_bf16_bits(rng.standard_normal((cfg.T, cfg.q_lora)) * 1.7)
    out = oracle.prolog(cfg, inp, q_norm=qn)
    H, Dn, QH = cfg.n_heads, cfg.nope_dim, cfg.q_head
    wq = inp["w_qb"].numpy().astype(np.int64)
    ws = inp["w_qb_scale"].numpy().astype(np.float64)
    nope_rows = (np.arange(H)[:, None] * QH + np.arange(Dn)[None, :]).reshape(-1)
    for t in range(cfg.T):
        codes, sc = oracle.quant_row(qn[t])
        acc = wq[nope_rows] @ codes.astype(np.int64)
        _ulp_within(out["q_nope"][t].reshape(-1), acc.astype(np.float64) * sc * ws[nope_rows])


def test_q_pe_of_the_v3_chain_against_fp64_rotation():
    """q_pe = RoPE(q_b projection of q_norm) per head at the token's position: the raw rope
    slice from an exact fp64 GEMM (rounded once to bf16 by torch), rotated as complex numbers
    by the table's cos/sin, within one bf16 step of the oracle; catches a wrong head offset,
    slice, pairing, sign or table row."""
    cfg = synth.get_config("v3_decode", T=3)
    inp = synth.make_inputs(cfg)
    assert (inp["positions"] > 0).all()
    out = oracle.prolog(cfg, inp)
    H, Dn, R, QH = cfg.n_heads, cfg.nope_dim, cfg.rope_dim, cfg.q_head
    h = R // 2
    qn = from_bits(out["q_norm"]).astype(np.float64)
    W = from_bits(synth.bf16_bits(inp["w_qb"])).astype(np.float64)
    raw = from_bits(to_bf16_bits((qn @ W.T).astype(np.float32))).reshape(cfg.T, H, QH)[..., Dn:]
    pos = inp["positions"].numpy()
    c = inp["cos"].numpy().astype(np.float64)[pos][:, None, :]
    s = inp["sin"].numpy().astype(np.float64)[pos][:, None, :]
    lo = raw[..., :h] * c[..., :h] - raw[..., h:] * s[..., :h]
    hi = raw[..., h:] * c[..., h:] + raw[..., :h] * s[..., h:]
    d = _ulp_within(out["q_pe"], np.concatenate([lo, hi], axis=-1))
    assert (d < 0.5 + 1e-9).mean() > 0.99       # nearly all are the correctly rounded value
    # the rope slice really moved (the positions are not 0): the raw slice differs
    assert (out["q_pe"] != to_bf16_bits(raw.astype(np.float32))).mean() > 0.9


def _selection_config(**kw):
    return synth.Config("sel", T=2, hidden=1040, q_lora=512, kv_lora=512, rope_dim=16,
                        nope_dim=16, v_dim=0, n_heads=2, max_pos=4, positions="arange", **kw)


def _row_where_variants_differ(g, lo, hi):
    """A bf16 row whose [lo, hi) segment RMSNorm variants A and B round differently."""
    for _ in range(5000):
        x = to_bf16_bits(rng.standard_normal(1040) * rng.uniform(0.05, 20))
        if (oracle.rmsnorm_row_rsqrt(x[lo:hi], g, 1e-6) != oracle.rmsnorm_row(x[lo:hi], g, 1e-6)).any():
            return x
    raise AssertionError("no row found")


def test_rmsnorm_variant_routing_on_rows_where_the_variants_differ():
    """With one-hot weights the down projection returns x's columns exactly (pinned above), so
    q_norm and kv_norm are RMSNorm of given rows. Token 0's q segment and token 1's kv segment
    are rows on which variant A (rsqrt) and variant B (sqrt, divide) round differently: the
    default configuration must give B and the rsqrt flag A, on both branches."""
    gq = to_bf16_bits(rng.uniform(0.5, 1.5, 512))
    gkv = to_bf16_bits(rng.uniform(0.5, 1.5, 512))
    x = np.stack([_row_where_variants_differ(gq, 0, 512), _row_where_variants_differ(gkv, 512, 1024)])
    eye = torch.zeros(1040, 1040, dtype=torch.bfloat16)
    eye[torch.arange(1040), torch.arange(1040)] = 1
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    inp = {"x": bf(x), "positions": torch.zeros(2, dtype=torch.int32),
           "w_qa": eye[:512].contiguous(), "w_kva": eye[512:].contiguous(),
           "w_qb": (torch.randn(2 * 32, 512) * 0.02).to(torch.bfloat16),
           "gamma_q": bf(gq), "gamma_kv": bf(gkv)}
    inp["cos"], inp["sin"] = synth.rope_table(4, 16)
    for rsqrt, fn in ((False, oracle.rmsnorm_row), (True, oracle.rmsnorm_row_rsqrt)):
        o = oracle.prolog(_selection_config(norm_rsqrt=rsqrt), inp)
        for t in range(2):
            np.testing.assert_array_equal(o["q_norm"][t], fn(x[t, :512], gq, 1e-6))
            np.testing.assert_array_equal(o["kv_norm"][t], fn(x[t, 512:1024], gkv, 1e-6))


def test_staging_hooks_reproduce_the_unstaged_chain():
    """Feeding the oracle its own intermediate rows (the down projection, q_norm, the raw q_b
    heads, the pre-RoPE slices) reproduces its unstaged outputs bit for bit, with and without the
    de-interleaved RoPE and the per-head norm (the hooks change where a row comes from, not the
    arithmetic)."""
    for var in ({}, {"rope_interleaved": True}, {"q_head_norm": True, "rope_interleaved": True}):
        name = "v4_decode" if var.get("q_head_norm") else "v3_decode"
        cfg = synth.get_config(name, T=2, **var)
        inp = synth.make_inputs(cfg)
        ref = oracle.prolog(cfg, inp, taps=True)
        st = oracle.prolog(cfg, inp, a=ref["a_proj"], q_norm=ref["q_norm"], q_raw=ref["q_proj"],
                           q_pe_in=ref["q_pre"], taps=True)
        for k in ref:
            np.testing.assert_array_equal(st[k], ref[k], err_msg="%s %s" % (var, k))
    # the tap of the down projection is the bf16 GEMM of x with [W_qa ; W_kva]
    cfg = synth.get_config("v3_decode", T=2)
    inp = synth.make_inputs(cfg)
    ref = oracle.prolog(cfg, inp, taps=True)
    W = np.concatenate([synth.bf16_bits(inp["w_qa"]), synth.bf16_bits(inp["w_kva"])])
    np.testing.assert_array_equal(ref["a_proj"], oracle.gemm_bf16(synth.bf16_bits(inp["x"]), W))
