"""Seeded synthetic inputs for the MLA Prolog workloads.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``mla_prolog_amd``). It only draws random numbers and lays them out; it holds
none of the method's arithmetic (no GEMM, norm, RoPE or quantisation).

The shapes follow the MLA configurations the pages describe:

* the DeepSeek-V2-Lite KV Prolog (hidden 2048, kv_a 2048->576, RMSNorm over
  the 512-wide compressed KV, kv_b 512->16x(128+128)), from "DeepSeek-V2-Lite-Chat
  MLA KV Prolog 迁移指南", section 精度验证 (the mla_prolog_001 case);
* the DeepSeek-V3 MLA Prolog (hidden 7168, q_lora 1536, kv_lora 512, rope 64,
  nope 128, 128 heads), the q_a -> RMSNorm -> q_b chain of "PyPTO-Gym 算子设计模式
  AT-10 ... MLAProlog 实战", section 五.

No public dataset or benchmark is involved; the pages only run a chat model
whose trained weights are not available, so random weights and activations of
the same shapes and scale stand in for them.

Draws: activations x ~ N(0, 1); bf16 weights ~ N(0, 0.02); gamma ~ U(0.5, 1.5);
positions uniform in [0, max_pos) for decode, 0..T-1 for prefill. The prefill
workload also scales 1% of the hidden channels (a seeded choice) by 20 before
rounding to bf16, to stress the per-token amax. Everything is drawn in fp32 from
``torch.Generator().manual_seed(seed)`` and rounded to bf16 by torch (round to
nearest even), so both sides read identical bytes.

For the W8A8 workload the int8 weight codes and their per-output-channel fp32
scales are drawn directly (codes = clamp(round(N(0,1) * 127/4.5), -127, 127),
scale = 0.02 * 4.5/127 * U(0.9, 1.1)): they are inputs of the method, not
something it computes.

The RoPE table is an input too: cos/sin of shape [max_pos, rope_dim] fp32,
built in fp64 from theta_i = 10000^(-2i/rope_dim), i < rope_dim/2, with the two
halves duplicated (the usual rotate-half table layout).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict, replace

import torch

__all__ = ["Config", "CONFIGS", "get_config", "make_inputs", "rope_table", "seed_for",
           "slot_mapping"]


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    hidden: int
    q_lora: int          # 0: no q path (KV-Prolog mode)
    kv_lora: int
    rope_dim: int
    nope_dim: int
    v_dim: int           # 0: no kv_b projection
    n_heads: int
    max_pos: int
    eps: float = 1e-6
    w8a8: bool = False
    positions: str = "uniform"   # "uniform" in [0, max_pos) or "arange"
    outlier_frac: float = 0.0    # fraction of hidden channels scaled by outlier_scale
    outlier_scale: float = 20.0
    index: int = 0               # seed = 1000 + index
    # numeric variants (flags of the prolog, not of the inputs)
    norm_rsqrt: bool = False        # RMSNorm variant A
    rope_interleaved: bool = False  # rope slices de-interleaved before rotate-half
    q_quant_per_head: bool = False  # q codes / scales per (token, head)
    q_head_norm: bool = False       # RMSNorm of every q head after q_b (the V4-shape prolog)
    mxfp8: bool = False             # MXFP8 weights (E4M3 codes + E8M0 block scales)
    mxfp8_mfma: bool = False        # run MXFP8 on the GPU's block-scaled MFMA (same method)

    def asdict(self):
        return asdict(self)

    @property
    def n1(self) -> int:
        """Width of the fused down-projection output [q_a | c_kv | k_pe]."""
        return self.q_lora + self.kv_lora + self.rope_dim

    @property
    def q_head(self) -> int:
        return self.nope_dim + self.rope_dim

    @property
    def kv_head(self) -> int:
        return self.nope_dim + self.v_dim


CONFIGS = {
    # Tiny KV Prolog: checks the whole chain at a size brute force can follow.
    "tiny_kv": Config("tiny_kv", T=4, hidden=256, q_lora=0, kv_lora=64, rope_dim=16,
                      nope_dim=32, v_dim=32, n_heads=2, max_pos=4, positions="arange",
                      index=0),
    # DeepSeek-V2-Lite KV Prolog, decode batch.
    "v2lite_kv_decode": Config("v2lite_kv_decode", T=64, hidden=2048, q_lora=0, kv_lora=512,
                               rope_dim=64, nope_dim=128, v_dim=128, n_heads=16,
                               max_pos=4096, positions="uniform", index=1),
    # DeepSeek-V3 full MLA Prolog, decode batch.
    "v3_decode": Config("v3_decode", T=256, hidden=7168, q_lora=1536, kv_lora=512, rope_dim=64,
                        nope_dim=128, v_dim=0, n_heads=128, max_pos=8192,
                        positions="uniform", index=2),
    # Same shape in prefill, with 1% outlier channels x20.
    "v3_prefill": Config("v3_prefill", T=8192, hidden=7168, q_lora=1536, kv_lora=512,
                         rope_dim=64, nope_dim=128, v_dim=0, n_heads=128, max_pos=8192,
                         positions="arange", outlier_frac=0.01, index=3),
    # The V4-shape MLA Prolog of the AT-10 card's test case (t=16, 64 heads of 512 with a
    # 64-wide rope slice, hidden 4096, q_lora 1024) with the per-head q RMSNorm after q_b; the
    # card gives no kv dimensions: kv_lora 512 and the same rope width.
    "v4_decode": Config("v4_decode", T=16, hidden=4096, q_lora=1024, kv_lora=512, rope_dim=64,
                        nope_dim=448, v_dim=0, n_heads=64, max_pos=8192, positions="uniform",
                        q_head_norm=True, index=5),
    # Same shape with MXFP8 projections (E4M3 weights, one E8M0 scale per 32 of K), a
    # mid-size batch and the decode batch.
    "v3_mxfp8": Config("v3_mxfp8", T=4096, hidden=7168, q_lora=1536, kv_lora=512, rope_dim=64,
                       nope_dim=128, v_dim=0, n_heads=128, max_pos=8192, positions="arange",
                       mxfp8=True, index=6),
    "v3_mxfp8_decode": Config("v3_mxfp8_decode", T=256, hidden=7168, q_lora=1536, kv_lora=512,
                              rope_dim=64, nope_dim=128, v_dim=0, n_heads=128, max_pos=8192,
                              positions="uniform", mxfp8=True, index=7),
    # Same shape with int8 W8A8 projections.
    "v3_w8a8": Config("v3_w8a8", T=16384, hidden=7168, q_lora=1536, kv_lora=512, rope_dim=64,
                      nope_dim=128, v_dim=0, n_heads=128, max_pos=16384,
                      positions="arange", w8a8=True, index=4),
}


def get_config(name: str, T: int | None = None, **variants) -> Config:
    """A named configuration, optionally with another token count and variant flags
    (norm_rsqrt, rope_interleaved, q_quant_per_head, q_head_norm, mxfp8, mxfp8_mfma)."""
    cfg = CONFIGS[name]
    if T is not None:
        cfg = replace(cfg, T=int(T))
    if variants:
        cfg = replace(cfg, **variants)
    return cfg


def seed_for(cfg: Config) -> int:
    return 1000 + cfg.index


def rope_table(max_pos: int, rope_dim: int, base: float = 10000.0):
    """cos/sin [max_pos, rope_dim] fp32 with duplicated halves (built in fp64)."""
    half = rope_dim // 2
    inv = torch.tensor([base ** (-2.0 * i / rope_dim) for i in range(half)], dtype=torch.float64)
    pos = torch.arange(max_pos, dtype=torch.float64)
    ang = pos[:, None] * inv[None, :]
    ang = torch.cat([ang, ang], dim=1)
    return torch.cos(ang).to(torch.float32).contiguous(), torch.sin(ang).to(torch.float32).contiguous()


def slot_mapping(T: int, n_slots: int, seed: int = 0, pad_frac: float = 0.08,
                 out_of_range: int = 2):
    """KV cache slots [T] int32 for a run of T tokens: distinct rows of a cache of n_slots
    (n_slots >= T) in random order, about pad_frac of them -1 (padding tokens), and
    `out_of_range` tokens at n_slots or beyond (not written)."""
    g = torch.Generator().manual_seed(int(seed))
    slots = torch.randperm(n_slots, generator=g)[:T].to(torch.int32)
    pad = torch.rand(T, generator=g) < pad_frac
    slots[pad] = -1
    if T > 0 and out_of_range > 0:
        idx = torch.randperm(T, generator=g)[:out_of_range]
        slots[idx] = n_slots + torch.arange(idx.numel(), dtype=torch.int32) * 7
    return slots.contiguous()


def _mx_weight(g, n, k):
    """MXFP8 weight [n, k]: E4M3 bytes drawn directly (random sign, exponent field 3..10,
    mantissa 0..7, so no NaN codes) and one E8M0 byte per 32 of k (2^-9 .. 2^-7): magnitudes
    from about 1e-4 to 0.12, around the size of the bf16 weights."""
    sign = torch.randint(0, 2, (n, k), generator=g, dtype=torch.int32) << 7
    exp = torch.randint(3, 11, (n, k), generator=g, dtype=torch.int32) << 3
    man = torch.randint(0, 8, (n, k), generator=g, dtype=torch.int32)
    codes = (sign | exp | man).to(torch.uint8).contiguous()
    scales = torch.randint(127 - 9, 127 - 6, (n, k // 32), generator=g, dtype=torch.int32)
    return codes, scales.to(torch.uint8).contiguous()


def _normal(g, shape, std):
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * std)


def _bf16_weight(g, n, k, std=0.02):
    return _normal(g, (n, k), std).to(torch.bfloat16).contiguous()


def _int8_weight(g, n, k):
    codes = torch.round(torch.randn(n, k, generator=g, dtype=torch.float32) * (127.0 / 4.5))
    codes = codes.clamp_(-127, 127).to(torch.int8).contiguous()
    scale = (0.02 * 4.5 / 127.0) * (0.9 + 0.2 * torch.rand(n, generator=g, dtype=torch.float32))
    return codes, scale.contiguous()


def make_inputs(cfg: Config, seed: int | None = None, weights_seed: int | None = None):
    """Return a dict of CPU tensors for ``cfg``.

    Keys: x [T,hidden] bf16, positions [T] int32, gamma_kv [kv_lora] bf16,
    w_kva [kv_lora+rope, hidden], optionally gamma_q, w_qa [q_lora, hidden],
    w_qb [H*(nope+rope), q_lora], w_kvb [H*(nope+v), kv_lora] (bf16, or int8
    with a matching ``*_scale`` fp32 [N] entry for W8A8), cos/sin [max_pos, rope] fp32.

    ``weights_seed`` draws the weights from a separate stream so that several
    weight sets of one shape can be made (used to defeat the last-level cache
    when timing).
    """
    seed = seed_for(cfg) if seed is None else int(seed)
    g = torch.Generator().manual_seed(seed)
    gw = g if weights_seed is None else torch.Generator().manual_seed(int(weights_seed))
    T, Hd = cfg.T, cfg.hidden
    out = {}

    x = torch.randn(T, Hd, generator=g, dtype=torch.float32)
    if cfg.outlier_frac > 0:
        n_out = int(round(cfg.outlier_frac * Hd))
        ch = torch.randperm(Hd, generator=g)[:n_out]
        x[:, ch] *= cfg.outlier_scale
        out["outlier_channels"] = ch.sort().values.to(torch.int32)
    out["x"] = x.to(torch.bfloat16).contiguous()

    if cfg.positions == "arange":
        pos = torch.arange(T, dtype=torch.int32) % cfg.max_pos
    else:
        pos = torch.randint(0, cfg.max_pos, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    out["positions"] = pos.contiguous()

    def weight(name, n, k):
        if cfg.mxfp8:
            codes, scales = _mx_weight(gw, n, k)
            out[name] = codes
            out[name + "_mxscale"] = scales
        elif cfg.w8a8:
            codes, scale = _int8_weight(gw, n, k)
            out[name] = codes
            out[name + "_scale"] = scale
        else:
            out[name] = _bf16_weight(gw, n, k)

    if cfg.q_lora > 0:
        weight("w_qa", cfg.q_lora, Hd)
        out["gamma_q"] = (0.5 + torch.rand(cfg.q_lora, generator=gw)).to(torch.bfloat16)
        weight("w_qb", cfg.n_heads * cfg.q_head, cfg.q_lora)
    weight("w_kva", cfg.kv_lora + cfg.rope_dim, Hd)
    out["gamma_kv"] = (0.5 + torch.rand(cfg.kv_lora, generator=gw)).to(torch.bfloat16)
    if cfg.v_dim > 0:
        weight("w_kvb", cfg.n_heads * cfg.kv_head, cfg.kv_lora)

    cos, sin = rope_table(cfg.max_pos, cfg.rope_dim)
    out["cos"], out["sin"] = cos, sin
    return out


def bf16_bits(t: torch.Tensor):
    """A bf16 tensor's raw 16-bit patterns as a numpy uint16 array (no arithmetic)."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
