// row_kernels.hip -- per-token row stages of the MLA Prolog on gfx950.
//
// These stages are tiny next to the GEMMs (a few hundred bytes per token) and
// are latency work: one 256-thread workgroup owns one token row, keeps it in
// registers, and reduces across the row with wave-wide butterfly shuffles plus
// a 4-entry LDS exchange in a fixed order (so results do not depend on timing).
//
// RMSNorm follows variant B of the AT-10 card ("PyPTO-Gym 算子设计模式 AT-10 ...
// MLAProlog 实战", section 三): fp32 x^2, times 1/D, row sum, +eps, sqrt, 1/std
// by an IEEE divide, x*rstd; then *fp32(gamma) and the bf16 cast (section 五).
// RoPE is rotate-half with one cos/sin row per token ("PyPTO Operator 深度解析",
// section 3.3). The INT8 quant is the per-row PrologQuant of the same page,
// section 3.1: multiplier 127/amax, round half to even, saturate, scale amax/127.
#include "common.hpp"
#include <algorithm>

#include "launch.hpp"

namespace mlap {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kMaxChunks = 4;  // 8-element chunks per thread and segment: widths <= 8192

__device__ __forceinline__ float block_sum(float v, float* sh) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) t += sh[w];
    return t;
}

__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) t = fmaxf(t, sh[w]);
    return t;
}

// Cache row of token t: slots[t] when the run writes a KV cache and the slot is in range,
// else -1.
__device__ __forceinline__ int cache_row(const NormArgs& a, int t) {
    if (!a.slots) return -1;
    const int s = a.slots[t];
    return (s >= 0 && s < a.n_slots) ? s : -1;
}

// 1/rms of a row from its sum s: variant B (the default) summed x^2/D and takes
// 1/sqrt(s + eps); variant A (rsqrt) summed x^2, scales the sum by 1/D, then rsqrt.
__device__ __forceinline__ float norm_rstd(const NormArgs& a, float s, float invD) {
    return a.rsqrt ? rsqrtf(s * invD + a.eps) : 1.0f / sqrtf(s + a.eps);
}

// Store v at element `off` of row t of `out` and, for a token with a cache row, of row `cr`
// of `cache` (the same row width); either pointer may be null.
template <typename E, typename V>
__device__ __forceinline__ void put_row(E* out, E* cache, int t, int cr, int width, int off, const V& v) {
    if (out) *reinterpret_cast<V*>(out + static_cast<size_t>(t) * width + off) = v;
    if (cache && cr >= 0) *reinterpret_cast<V*>(cache + static_cast<size_t>(cr) * width + off) = v;
}

// Sum over `splits` split-K fp32 partials (8 values at p + sp * stride each, split 0 first)
// then round to bf16 (the GEMM's output cast point). Loads go out in groups of eight so a
// group costs one memory latency; the additions stay in split order.
__device__ __forceinline__ void sum_partials8(const float* p, size_t stride, int splits, float* f) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += 8) {
        float4 x[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sp = min(s0 + j, splits - 1);
            const float4* q = reinterpret_cast<const float4*>(p + static_cast<size_t>(sp) * stride);
            x[j][0] = q[0];
            x[j][1] = q[1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s0 + j < splits) {
                s[0] += x[j][0].x; s[1] += x[j][0].y; s[2] += x[j][0].z; s[3] += x[j][0].w;
                s[4] += x[j][1].x; s[5] += x[j][1].y; s[6] += x[j][1].z; s[7] += x[j][1].w;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = bf2f(f2bf(s[e]));
}

// sum_partials8 with the split count known at compile time: straight-line code, so the
// loads of several chunks can all be in flight before the first sum.
template <int SPL>
__device__ __forceinline__ void sum_partials8_n(const float* p, size_t stride, float* f) {
    float4 x[SPL][2];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const float4* q = reinterpret_cast<const float4*>(p + static_cast<size_t>(j) * stride);
        x[j][0] = q[0];
        x[j][1] = q[1];
    }
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        s[0] += x[j][0].x; s[1] += x[j][0].y; s[2] += x[j][0].z; s[3] += x[j][0].w;
        s[4] += x[j][1].x; s[5] += x[j][1].y; s[6] += x[j][1].z; s[7] += x[j][1].w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = bf2f(f2bf(s[e]));
}

// 8 consecutive down-projection outputs of token t starting at column col, as the fp32
// values of their bf16 rounding (the GEMM's bf16 output cast point).
__device__ __forceinline__ void load_a8(const NormArgs& a, int t, int col, float* f) {
    if (a.tail_f32 && col >= a.tail_c0) {
        const int w = a.N1 - a.tail_c0;
        sum_partials8(a.tail_f32 + static_cast<size_t>(t) * w + (col - a.tail_c0),
                      static_cast<size_t>(a.T) * w, a.tail_splits, f);
        return;
    }
    if (!a.a_f32) {
        unpack8(*reinterpret_cast<const uint4*>(a.a_bf16 + static_cast<size_t>(t) * a.N1 + col), f);
        return;
    }
    sum_partials8(a.a_f32 + static_cast<size_t>(t) * a.N1 + col, static_cast<size_t>(a.T) * a.N1,
                  a.k_splits, f);
}

__global__ __launch_bounds__(kRowThreads) void norm_rope_kernel(NormArgs a) {
    __shared__ float red[kRowWaves];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nq = a.Lq >> 3, nkv = a.Lkv >> 3;
    const int cache_r = cache_row(a, t);

    float qv[kMaxChunks][8], kv[kMaxChunks][8];
    float sq = 0.f, skv = 0.f;
    const float invq = a.Lq > 0 ? 1.0f / static_cast<float>(a.Lq) : 0.f;
    const float invkv = 1.0f / static_cast<float>(a.Lkv);
    const float eq = a.rsqrt ? 1.0f : invq, ekv = a.rsqrt ? 1.0f : invkv;  // per-element 1/D (B)
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
        const int c = tid + i * kRowThreads;
        if (c < nq) {
            load_a8(a, t, c * 8, qv[i]);
            if (a.a_proj) *reinterpret_cast<uint4*>(a.a_proj + static_cast<size_t>(t) * a.N1 + c * 8) = pack8(qv[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = qv[i][e] * qv[i][e];
                sq += p * eq;
            }
        }
        if (c < nkv) {
            load_a8(a, t, a.Lq + c * 8, kv[i]);
            if (a.a_proj) *reinterpret_cast<uint4*>(a.a_proj + static_cast<size_t>(t) * a.N1 + a.Lq + c * 8) = pack8(kv[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = kv[i][e] * kv[i][e];
                skv += p * ekv;
            }
        }
    }
    const float msq = (a.Lq > 0) ? block_sum(sq, red) : 0.f;
    const float mskv = block_sum(skv, red);
    const float rstd_q = norm_rstd(a, msq, invq);
    const float rstd_kv = norm_rstd(a, mskv, invkv);

    float qmax = 0.f, kvmax = 0.f;
    uint4 qo[kMaxChunks], kvo[kMaxChunks];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
        const int c = tid + i * kRowThreads;
        if (c < nq) {
            float g[8], o[8];
            unpack8(*reinterpret_cast<const uint4*>(a.gamma_q + c * 8), g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y = qv[i][e] * rstd_q;
                o[e] = y * g[e];
            }
            qo[i] = pack8(o);
            if (a.q_norm)
                *reinterpret_cast<uint4*>(a.q_norm + static_cast<size_t>(t) * a.Lq + c * 8) = qo[i];
            qmax = fmaxf(qmax, absmax8(qo[i]));
        }
        if (c < nkv) {
            float g[8], o[8];
            unpack8(*reinterpret_cast<const uint4*>(a.gamma_kv + c * 8), g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y = kv[i][e] * rstd_kv;
                o[e] = y * g[e];
            }
            kvo[i] = pack8(o);
            put_row(a.kv_norm, a.kv_cache, t, cache_r, a.Lkv, c * 8, kvo[i]);
            kvmax = fmaxf(kvmax, absmax8(kvo[i]));
        }
    }

    // rotate-half RoPE of the k_pe slice (pairs i, i + R/2), one cos/sin row per token
    const int half = a.R >> 1;
    if ((a.k_pe || a.kr_cache || a.a_proj) && tid < (half >> 3)) {
        const int i0 = tid * 8;
        const int p = clamp_pos(a.positions[t], a.max_pos);
        MLAP_CHECK(a.dbg, a.positions[t] >= 0 && a.positions[t] < a.max_pos, kDbgPos);
        MLAP_CHECK(a.dbg, t < a.T && a.Lq + a.Lkv + a.R <= a.N1, kDbgRow);
        const float* cr = a.cos + static_cast<size_t>(p) * a.R;
        const float* sr = a.sin + static_cast<size_t>(p) * a.R;
        float x1[8], x2[8], lo[8], hi[8];
        load_a8(a, t, a.Lq + a.Lkv + i0, x1);
        load_a8(a, t, a.Lq + a.Lkv + half + i0, x2);
        if (a.a_proj) {
            uint16_t* ar = a.a_proj + static_cast<size_t>(t) * a.N1 + a.Lq + a.Lkv;
            *reinterpret_cast<uint4*>(ar + i0) = pack8(x1);
            *reinterpret_cast<uint4*>(ar + half + i0) = pack8(x2);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float p1 = x1[e] * cr[i0 + e];
            float p2 = (-x2[e]) * sr[i0 + e];
            lo[e] = p1 + p2;
            float p3 = x2[e] * cr[half + i0 + e];
            float p4 = x1[e] * sr[half + i0 + e];
            hi[e] = p3 + p4;
        }
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, i0, pack8(lo));
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, half + i0, pack8(hi));
    }

    // per-token INT8 quant of kv_norm
    if (a.kv_i8 || a.kv_scale || a.kv_i8_b || a.kv_scale_b || a.kv_cache_i8 || a.kv_cache_scale) {
        const float amax = block_max(kvmax, red);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
        for (int i = 0; i < kMaxChunks; ++i) {
            const int c = tid + i * kRowThreads;
            if (c < nkv) {
                const uint2 codes = quant8(kvo[i], mult);
                put_row(a.kv_i8, a.kv_cache_i8, t, cache_r, a.Lkv, c * 8, codes);
                if (a.kv_i8_b) *reinterpret_cast<uint2*>(a.kv_i8_b + static_cast<size_t>(t) * a.Lkv + c * 8) = codes;
            }
        }
        if (tid == 0) {
            const float sc = amax / 127.0f;
            if (a.kv_scale) a.kv_scale[t] = sc;
            if (a.kv_scale_b) a.kv_scale_b[t] = sc;
            if (a.kv_cache_scale && cache_r >= 0) a.kv_cache_scale[cache_r] = sc;
        }
    }
    // W8A8: per-token activation quant of q_norm for the int8 up projection
    if (a.qn_i8) {
        const float amax = block_max(qmax, red);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
        for (int i = 0; i < kMaxChunks; ++i) {
            const int c = tid + i * kRowThreads;
            if (c < nq)
                *reinterpret_cast<uint2*>(a.qn_i8 + static_cast<size_t>(t) * a.Lq + c * 8) =
                    quant8(qo[i], mult);
        }
        if (tid == 0) a.qn_scale[t] = amax / 127.0f;
    }
}

// The same stage for small batches, one workgroup per token, shaped for latency: the
// token's whole input (down-projection values, gamma chunks, the rope slice and its
// position) is requested in one burst before anything is reduced, and the cos/sin row
// right after the position returns, so a token costs two memory round trips instead of
// one per dependent step. Thread i owns q chunks i + 256 c (c < QC) and kv chunks
// i + 256 c (c < KC); chunk indexes past a segment are clamped for the loads (in bounds,
// straight-line code) and masked out of the sums and stores. SPL > 0 selects SPL fp32
// split-K partials as input, SPL = 0 the bf16 down-projection output; no tail partials.
template <int QC, int KC, int SPL>
__device__ __forceinline__ void norm_rope_block_body(const NormArgs& a, float* red) {
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int cache_r = cache_row(a, t);
    const int nq = a.Lq >> 3, nkv = a.Lkv >> 3;
    const int half = a.R >> 1;
    // A chunk's raw input: up to 8 splits of float4 pairs (one fetch group), or one uint4 of
    // bf16. More than 8 splits are fetched in groups of 8 (a round trip per group) so the
    // registers in flight stay bounded; the sums still run in split order.
    constexpr int GS = SPL > 8 ? 8 : (SPL > 0 ? SPL : 1);
    constexpr int NG = SPL > 0 ? (SPL + 7) / 8 : 1;
    struct Raw {
        float4 x[GS][2];
        uint4 b;
    };
    auto fetch = [&](int col, Raw& r, auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        if constexpr (SPL > 0) {
            constexpr int n = SPL - 8 * g < GS ? SPL - 8 * g : GS;
            const float* p = a.a_f32 + static_cast<size_t>(t) * a.N1 + col;
            const size_t stride = static_cast<size_t>(a.T) * a.N1;
#pragma unroll
            for (int j = 0; j < n; ++j) {
                const float4* q = reinterpret_cast<const float4*>(p + static_cast<size_t>(8 * g + j) * stride);
                r.x[j][0] = q[0];
                r.x[j][1] = q[1];
            }
        } else {
            r.b = *reinterpret_cast<const uint4*>(a.a_bf16 + static_cast<size_t>(t) * a.N1 + col);
        }
    };
    // add fetch group g to the running split sums s8 (split order)
    auto accum = [&](const Raw& r, float* s8, auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        if constexpr (SPL > 0) {
            constexpr int n = SPL - 8 * g < GS ? SPL - 8 * g : GS;
#pragma unroll
            for (int j = 0; j < n; ++j) {
                s8[0] += r.x[j][0].x; s8[1] += r.x[j][0].y; s8[2] += r.x[j][0].z; s8[3] += r.x[j][0].w;
                s8[4] += r.x[j][1].x; s8[5] += r.x[j][1].y; s8[6] += r.x[j][1].z; s8[7] += r.x[j][1].w;
            }
        } else {
            unpack8(r.b, s8);
        }
    };
    // the chunk's 8 values as the fp32 of their bf16 rounding (the GEMM's output cast)
    auto finish = [&](float* s8) __attribute__((always_inline)) {
        if constexpr (SPL > 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = bf2f(f2bf(s8[e]));
        }
    };

    const bool rope = (a.k_pe != nullptr || a.kr_cache != nullptr || a.a_proj != nullptr) && half >= 8;
    const int pos = rope ? clamp_pos(a.positions[t], a.max_pos) : 0;
    MLAP_CHECK(a.dbg, !rope || (a.positions[t] >= 0 && a.positions[t] < a.max_pos), kDbgPos);
    MLAP_CHECK(a.dbg, t < a.T && a.Lq + a.Lkv + a.R <= a.N1 && (cache_r < 0 || cache_r < a.n_slots), kDbgRow);
    const bool roper = rope && tid < (half >> 3);
    const int i0 = rope ? min(tid, (half >> 3) - 1) * 8 : 0;
    float qv[QC > 0 ? QC : 1][8], kv[KC][8], x1[8], x2[8];
    static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[decltype(c_c)::value][e] = 0.f;
    });
    static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[decltype(c_c)::value][e] = 0.f;
    });
#pragma unroll
    for (int e = 0; e < 8; ++e) x1[e] = x2[e] = 0.f;
    uint4 gq[QC > 0 ? QC : 1], gkv[KC];
    float4 cl[2], ch_[2], sl[2], sh[2];
    static_for<NG>([&](auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        // one round trip: every load of this group (and, with the first, γ and the position)
        // is requested before any of them is used
        Raw rq[QC > 0 ? QC : 1], rkv[KC], r1, r2;
        static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
            constexpr int c = decltype(c_c)::value;
            const int ch = min(tid + kRowThreads * c, nq - 1);
            fetch(ch * 8, rq[c], g_c);
            if constexpr (g == 0) gq[c] = *reinterpret_cast<const uint4*>(a.gamma_q + ch * 8);
        });
        static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
            constexpr int c = decltype(c_c)::value;
            const int ch = min(tid + kRowThreads * c, nkv - 1);
            fetch(a.Lq + ch * 8, rkv[c], g_c);
            if constexpr (g == 0) gkv[c] = *reinterpret_cast<const uint4*>(a.gamma_kv + ch * 8);
        });
        if (rope) {
            fetch(a.Lq + a.Lkv + i0, r1, g_c);
            fetch(a.Lq + a.Lkv + half + i0, r2, g_c);
        }
        if constexpr (g == 0) {
            // the token's cos/sin row, requested as soon as the position is back
            if (rope) {
                const float* cr = a.cos + static_cast<size_t>(pos) * a.R;
                const float* sr = a.sin + static_cast<size_t>(pos) * a.R;
                cl[0] = *reinterpret_cast<const float4*>(cr + i0);
                cl[1] = *reinterpret_cast<const float4*>(cr + i0 + 4);
                ch_[0] = *reinterpret_cast<const float4*>(cr + half + i0);
                ch_[1] = *reinterpret_cast<const float4*>(cr + half + i0 + 4);
                sl[0] = *reinterpret_cast<const float4*>(sr + i0);
                sl[1] = *reinterpret_cast<const float4*>(sr + i0 + 4);
                sh[0] = *reinterpret_cast<const float4*>(sr + half + i0);
                sh[1] = *reinterpret_cast<const float4*>(sr + half + i0 + 4);
            }
        }
        static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
            accum(rq[decltype(c_c)::value], qv[decltype(c_c)::value], g_c);
        });
        static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
            accum(rkv[decltype(c_c)::value], kv[decltype(c_c)::value], g_c);
        });
        if (rope) {
            accum(r1, x1, g_c);
            accum(r2, x2, g_c);
        }
    });
    static_for<QC>([&](auto c_c) __attribute__((always_inline)) { finish(qv[decltype(c_c)::value]); });
    static_for<KC>([&](auto c_c) __attribute__((always_inline)) { finish(kv[decltype(c_c)::value]); });
    finish(x1);
    finish(x2);
    if (a.a_proj) {  // the down-projection row as read (the GEMM's bf16 cast point)
        uint16_t* ar = a.a_proj + static_cast<size_t>(t) * a.N1;
        static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
            const int ch = tid + kRowThreads * decltype(c_c)::value;
            if (ch < nq) *reinterpret_cast<uint4*>(ar + ch * 8) = pack8(qv[decltype(c_c)::value]);
        });
        static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
            const int ch = tid + kRowThreads * decltype(c_c)::value;
            if (ch < nkv) *reinterpret_cast<uint4*>(ar + a.Lq + ch * 8) = pack8(kv[decltype(c_c)::value]);
        });
        if (roper) {
            *reinterpret_cast<uint4*>(ar + a.Lq + a.Lkv + i0) = pack8(x1);
            *reinterpret_cast<uint4*>(ar + a.Lq + a.Lkv + half + i0) = pack8(x2);
        }
    }

    // RMS statistics: per thread in element order, then the fixed-order block sum
    float sq = 0.f, skv = 0.f;
    const float invq = a.Lq > 0 ? 1.0f / static_cast<float>(a.Lq) : 0.f;
    const float invkv = 1.0f / static_cast<float>(a.Lkv);
    const float eq = a.rsqrt ? 1.0f : invq, ekv = a.rsqrt ? 1.0f : invkv;  // per-element 1/D (B)
    static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
        constexpr int c = decltype(c_c)::value;
        if (tid + kRowThreads * c < nq) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = qv[c][e] * qv[c][e];
                sq += p * eq;
            }
        }
    });
    static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
        constexpr int c = decltype(c_c)::value;
        if (tid + kRowThreads * c < nkv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = kv[c][e] * kv[c][e];
                skv += p * ekv;
            }
        }
    });
    const float msq = QC > 0 ? block_sum(sq, red) : 0.f;
    const float mskv = block_sum(skv, red);
    const float rstd_q = norm_rstd(a, msq, invq);
    const float rstd_kv = norm_rstd(a, mskv, invkv);

    float qmax = 0.f, kvmax = 0.f;
    uint4 qo[QC > 0 ? QC : 1], kvo[KC];
    static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
        constexpr int c = decltype(c_c)::value;
        const int ch = tid + kRowThreads * c;
        float g[8], o[8];
        unpack8(gq[c], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = qv[c][e] * rstd_q;
            o[e] = y * g[e];
        }
        qo[c] = pack8(o);
        if (ch < nq) {
            if (a.q_norm) *reinterpret_cast<uint4*>(a.q_norm + static_cast<size_t>(t) * a.Lq + ch * 8) = qo[c];
            qmax = fmaxf(qmax, absmax8(qo[c]));
        }
    });
    static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
        constexpr int c = decltype(c_c)::value;
        const int ch = tid + kRowThreads * c;
        float g[8], o[8];
        unpack8(gkv[c], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = kv[c][e] * rstd_kv;
            o[e] = y * g[e];
        }
        kvo[c] = pack8(o);
        if (ch < nkv) {
            put_row(a.kv_norm, a.kv_cache, t, cache_r, a.Lkv, ch * 8, kvo[c]);
            kvmax = fmaxf(kvmax, absmax8(kvo[c]));
        }
    });

    // rotate-half RoPE of the k_pe slice (pairs i, i + R/2)
    if (roper) {
        const float cv[8] = {cl[0].x, cl[0].y, cl[0].z, cl[0].w, cl[1].x, cl[1].y, cl[1].z, cl[1].w};
        const float chv[8] = {ch_[0].x, ch_[0].y, ch_[0].z, ch_[0].w, ch_[1].x, ch_[1].y, ch_[1].z, ch_[1].w};
        const float sv[8] = {sl[0].x, sl[0].y, sl[0].z, sl[0].w, sl[1].x, sl[1].y, sl[1].z, sl[1].w};
        const float shv[8] = {sh[0].x, sh[0].y, sh[0].z, sh[0].w, sh[1].x, sh[1].y, sh[1].z, sh[1].w};
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float p1 = x1[e] * cv[e];
            float p2 = (-x2[e]) * sv[e];
            lo[e] = p1 + p2;
            float p3 = x2[e] * chv[e];
            float p4 = x1[e] * shv[e];
            hi[e] = p3 + p4;
        }
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, i0, pack8(lo));
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, half + i0, pack8(hi));
    }

    // per-token INT8 quant of kv_norm
    if (a.kv_i8 || a.kv_scale || a.kv_i8_b || a.kv_scale_b || a.kv_cache_i8 || a.kv_cache_scale) {
        const float amax = block_max(kvmax, red);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
        static_for<KC>([&](auto c_c) __attribute__((always_inline)) {
            constexpr int c = decltype(c_c)::value;
            const int ch = tid + kRowThreads * c;
            if (ch < nkv) {
                const uint2 codes = quant8(kvo[c], mult);
                put_row(a.kv_i8, a.kv_cache_i8, t, cache_r, a.Lkv, ch * 8, codes);
                if (a.kv_i8_b) *reinterpret_cast<uint2*>(a.kv_i8_b + static_cast<size_t>(t) * a.Lkv + ch * 8) = codes;
            }
        });
        if (tid == 0) {
            const float sc = amax / 127.0f;
            if (a.kv_scale) a.kv_scale[t] = sc;
            if (a.kv_scale_b) a.kv_scale_b[t] = sc;
            if (a.kv_cache_scale && cache_r >= 0) a.kv_cache_scale[cache_r] = sc;
        }
    }
    // W8A8: per-token activation quant of q_norm for the int8 up projection
    if (QC > 0 && a.qn_i8) {
        const float amax = block_max(qmax, red);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
        static_for<QC>([&](auto c_c) __attribute__((always_inline)) {
            constexpr int c = decltype(c_c)::value;
            const int ch = tid + kRowThreads * c;
            if (ch < nq)
                *reinterpret_cast<uint2*>(a.qn_i8 + static_cast<size_t>(t) * a.Lq + ch * 8) = quant8(qo[c], mult);
        });
        if (tid == 0) a.qn_scale[t] = amax / 127.0f;
    }
}

template <int QC, int KC, int SPL>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void norm_rope_block_kernel(NormArgs a) {
    __shared__ float red[kRowWaves];
    norm_rope_block_body<QC, KC, SPL>(a, red);
}

// Same stage with one 64-wide wave per token (four tokens per workgroup) for segment
// widths up to 64 * 8 * QC (q) and 64 * 8 * KC (kv), for a bf16 down-projection output
// (with an optional fp32 split-K tail): every reduction is a wave butterfly, there is no
// workgroup barrier, and 2048 workgroups of four short waves fill the chip. Every input
// of the token is requested before any is used; when the rope slice lies in the split-K
// tail, its chunk x split partials are spread one per lane and summed across lanes in
// split order. Rows of four or more chunks per lane (V3: three q and one kv) hold too many
// values for four workgroups per CU (128 registers: they spilled to scratch) and run three.
template <int QC, int KC>
__global__ __launch_bounds__(256, QC + KC >= 4 ? 3 : 4) void norm_rope_wave_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;  // the whole wave leaves; nothing below synchronises the workgroup
    const int cache_r = cache_row(a, t);
    const int nq = a.Lq >> 3, nkv = a.Lkv >> 3;
    const int half = a.R >> 1;
    const int rc = half >> 3;  // rope chunks per half
    const bool rope = (a.k_pe != nullptr || a.kr_cache != nullptr || a.a_proj != nullptr) && rc > 0;
    const uint16_t* arow = a.a_bf16 + static_cast<size_t>(t) * a.N1;
    const int c_rope = a.Lq + a.Lkv;  // first column of the rope slice
    // rope slice from the tail partials, one (chunk, split) pair per lane
    const int S = a.tail_splits;
    const bool lane_tail = rope && a.tail_f32 && c_rope >= a.tail_c0 && 2 * rc * S <= 64;

    // ---- one burst of loads: rows, gamma, position, rope inputs
    const int pos = rope ? clamp_pos(a.positions[t], a.max_pos) : 0;
    MLAP_CHECK(a.dbg, !rope || (a.positions[t] >= 0 && a.positions[t] < a.max_pos), kDbgPos);
    MLAP_CHECK(a.dbg, a.Lq + a.Lkv + a.R <= a.N1 && (cache_r < 0 || cache_r < a.n_slots), kDbgRow);
    uint4 rq[QC > 0 ? QC : 1], rkv[KC], gq[QC > 0 ? QC : 1], gkv[KC];
#pragma unroll
    for (int i = 0; i < QC; ++i) {
        const int c = min(lane + 64 * i, nq - 1);
        rq[i] = *reinterpret_cast<const uint4*>(arow + c * 8);
        gq[i] = *reinterpret_cast<const uint4*>(a.gamma_q + c * 8);
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int c = min(lane + 64 * i, nkv - 1);
        rkv[i] = *reinterpret_cast<const uint4*>(arow + a.Lq + c * 8);
        gkv[i] = *reinterpret_cast<const uint4*>(a.gamma_kv + c * 8);
    }
    const int i0 = rope ? min(lane, rc - 1) * 8 : 0;
    float4 tp[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    float x1[8], x2[8];
    if (lane_tail) {
        const int j = min(lane / S, 2 * rc - 1), sp = lane - j * S;
        if (sp < S) {
            const int w = a.N1 - a.tail_c0;
            const float* pp = a.tail_f32 + (static_cast<size_t>(sp) * a.T + t) * w + (c_rope - a.tail_c0) + 8 * j;
            tp[0] = *reinterpret_cast<const float4*>(pp);
            tp[1] = *reinterpret_cast<const float4*>(pp + 4);
        }
    } else if (rope) {
        load_a8(a, t, c_rope + i0, x1);
        load_a8(a, t, c_rope + half + i0, x2);
    }
    float4 cl[2], chh[2], sl[2], shh[2];
    if (rope) {
        const float* cr = a.cos + static_cast<size_t>(pos) * a.R;
        const float* sr = a.sin + static_cast<size_t>(pos) * a.R;
        cl[0] = *reinterpret_cast<const float4*>(cr + i0);
        cl[1] = *reinterpret_cast<const float4*>(cr + i0 + 4);
        chh[0] = *reinterpret_cast<const float4*>(cr + half + i0);
        chh[1] = *reinterpret_cast<const float4*>(cr + half + i0 + 4);
        sl[0] = *reinterpret_cast<const float4*>(sr + i0);
        sl[1] = *reinterpret_cast<const float4*>(sr + i0 + 4);
        shh[0] = *reinterpret_cast<const float4*>(sr + half + i0);
        shh[1] = *reinterpret_cast<const float4*>(sr + half + i0 + 4);
    }

    if (a.a_proj) {  // the down-projection row as read (q and kv segments; rope slice below)
        uint16_t* ar = a.a_proj + static_cast<size_t>(t) * a.N1;
#pragma unroll
        for (int i = 0; i < QC; ++i)
            if (lane + 64 * i < nq) *reinterpret_cast<uint4*>(ar + (lane + 64 * i) * 8) = rq[i];
#pragma unroll
        for (int i = 0; i < KC; ++i)
            if (lane + 64 * i < nkv) *reinterpret_cast<uint4*>(ar + a.Lq + (lane + 64 * i) * 8) = rkv[i];
    }

    // ---- RMSNorm of both segments
    float qv[QC > 0 ? QC : 1][8], kv[KC][8];
    float sq = 0.f, skv = 0.f;
    const float invq = a.Lq > 0 ? 1.0f / static_cast<float>(a.Lq) : 0.f;
    const float invkv = 1.0f / static_cast<float>(a.Lkv);
    const float eq = a.rsqrt ? 1.0f : invq, ekv = a.rsqrt ? 1.0f : invkv;  // per-element 1/D (B)
#pragma unroll
    for (int i = 0; i < QC; ++i) {
        unpack8(rq[i], qv[i]);
        if (lane + 64 * i < nq) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = qv[i][e] * qv[i][e];
                sq += p * eq;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        unpack8(rkv[i], kv[i]);
        if (lane + 64 * i < nkv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = kv[i][e] * kv[i][e];
                skv += p * ekv;
            }
        }
    }
    const float msq = QC > 0 ? wave_sum(sq) : 0.f;
    const float mskv = wave_sum(skv);
    const float rstd_q = norm_rstd(a, msq, invq);
    const float rstd_kv = norm_rstd(a, mskv, invkv);

    float qmax = 0.f, kvmax = 0.f;
    uint4 qo[QC > 0 ? QC : 1], kvo[KC];
#pragma unroll
    for (int i = 0; i < QC; ++i) {
        const int c = lane + 64 * i;
        float g[8], o[8];
        unpack8(gq[i], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = qv[i][e] * rstd_q;
            o[e] = y * g[e];
        }
        qo[i] = pack8(o);
        if (c < nq) {
            if (a.q_norm) *reinterpret_cast<uint4*>(a.q_norm + static_cast<size_t>(t) * a.Lq + c * 8) = qo[i];
            qmax = fmaxf(qmax, absmax8(qo[i]));
        }
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int c = lane + 64 * i;
        float g[8], o[8];
        unpack8(gkv[i], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = kv[i][e] * rstd_kv;
            o[e] = y * g[e];
        }
        kvo[i] = pack8(o);
        if (c < nkv) {
            put_row(a.kv_norm, a.kv_cache, t, cache_r, a.Lkv, c * 8, kvo[i]);
            kvmax = fmaxf(kvmax, absmax8(kvo[i]));
        }
    }

    // ---- rotate-half RoPE of the k_pe slice (pairs i, i + R/2)
    if (lane_tail) {
        // chunk j's sum over its S splits, in split order, in every lane of its group; then
        // lane i < rc takes chunks i (x1) and i + rc (x2), rounded to bf16 (the GEMM's cast)
        const int j = min(lane / S, 2 * rc - 1);
        float v[8] = {tp[0].x, tp[0].y, tp[0].z, tp[0].w, tp[1].x, tp[1].y, tp[1].z, tp[1].w};
        float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < S; ++sp) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += __shfl(v[e], j * S + sp);
        }
        const int il = min(lane, rc - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x1[e] = bf2f(f2bf(__shfl(sum[e], il * S)));
            x2[e] = bf2f(f2bf(__shfl(sum[e], (il + rc) * S)));
        }
    }
    if (rope && lane < rc && a.a_proj) {
        uint16_t* ar = a.a_proj + static_cast<size_t>(t) * a.N1 + c_rope;
        *reinterpret_cast<uint4*>(ar + i0) = pack8(x1);
        *reinterpret_cast<uint4*>(ar + half + i0) = pack8(x2);
    }
    if (rope && lane < rc) {
        const float cv[8] = {cl[0].x, cl[0].y, cl[0].z, cl[0].w, cl[1].x, cl[1].y, cl[1].z, cl[1].w};
        const float chv[8] = {chh[0].x, chh[0].y, chh[0].z, chh[0].w, chh[1].x, chh[1].y, chh[1].z, chh[1].w};
        const float sv[8] = {sl[0].x, sl[0].y, sl[0].z, sl[0].w, sl[1].x, sl[1].y, sl[1].z, sl[1].w};
        const float shv[8] = {shh[0].x, shh[0].y, shh[0].z, shh[0].w, shh[1].x, shh[1].y, shh[1].z, shh[1].w};
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float p1 = x1[e] * cv[e];
            float p2 = (-x2[e]) * sv[e];
            lo[e] = p1 + p2;
            float p3 = x2[e] * chv[e];
            float p4 = x1[e] * shv[e];
            hi[e] = p3 + p4;
        }
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, i0, pack8(lo));
        put_row(a.k_pe, a.kr_cache, t, cache_r, a.R, half + i0, pack8(hi));
    }

    // ---- per-token INT8 quant of kv_norm
    if (a.kv_i8 || a.kv_scale || a.kv_i8_b || a.kv_scale_b || a.kv_cache_i8 || a.kv_cache_scale) {
        const float amax = wave_max(kvmax);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int c = lane + 64 * i;
            if (c < nkv) {
                const uint2 codes = quant8(kvo[i], mult);
                put_row(a.kv_i8, a.kv_cache_i8, t, cache_r, a.Lkv, c * 8, codes);
                if (a.kv_i8_b) *reinterpret_cast<uint2*>(a.kv_i8_b + static_cast<size_t>(t) * a.Lkv + c * 8) = codes;
            }
        }
        if (lane == 0) {
            const float sc = amax / 127.0f;
            if (a.kv_scale) a.kv_scale[t] = sc;
            if (a.kv_scale_b) a.kv_scale_b[t] = sc;
            if (a.kv_cache_scale && cache_r >= 0) a.kv_cache_scale[cache_r] = sc;
        }
    }
    // W8A8: per-token activation quant of q_norm for the int8 up projection
    if (QC > 0 && a.qn_i8) {
        const float amax = wave_max(qmax);
        const float mult = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
        for (int i = 0; i < QC; ++i) {
            const int c = lane + 64 * i;
            if (c < nq)
                *reinterpret_cast<uint2*>(a.qn_i8 + static_cast<size_t>(t) * a.Lq + c * 8) =
                    quant8(qo[i], mult);
        }
        if (lane == 0) a.qn_scale[t] = amax / 127.0f;
    }
}

__global__ __launch_bounds__(kRowThreads) void act_quant_kernel(const uint16_t* x, int K,
                                                                int8_t* codes, float* scale) {
    __shared__ float red[kRowWaves];
    const int t = blockIdx.x;
    const uint16_t* row = x + static_cast<size_t>(t) * K;
    int8_t* crow = codes + static_cast<size_t>(t) * K;
    const int nc = K >> 3;
    // The row stays in registers between its amax and its codes (x is read once; a second
    // pass missed L2 often enough to cost 18% of the kernel): up to kHold 16-byte chunks per
    // thread, rows of up to 8192 values; longer rows read the rest again.
    constexpr int kHold = 4;
    uint4 v[kHold];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < kHold; ++k) {
        const int c = threadIdx.x + k * kRowThreads;
        v[k] = *reinterpret_cast<const uint4*>(row + min(c, nc - 1) * 8);
        if (c < nc) m = fmaxf(m, absmax8(v[k]));
    }
    for (int c = threadIdx.x + kHold * kRowThreads; c < nc; c += kRowThreads)
        m = fmaxf(m, absmax8(*reinterpret_cast<const uint4*>(row + c * 8)));
    const float amax = block_max(m, red);
    const float mult = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
    for (int k = 0; k < kHold; ++k) {
        const int c = threadIdx.x + k * kRowThreads;
        if (c < nc) *reinterpret_cast<uint2*>(crow + c * 8) = quant8(v[k], mult);
    }
    for (int c = threadIdx.x + kHold * kRowThreads; c < nc; c += kRowThreads)
        *reinterpret_cast<uint2*>(crow + c * 8) = quant8(*reinterpret_cast<const uint4*>(row + c * 8), mult);
    if (threadIdx.x == 0) scale[t] = amax / 127.0f;
}

// kHeld q chunks per thread are fetched before the amax is known (a small batch has one
// workgroup per CU and lives on latency); kHeld = 0 streams the row after the amax, which
// keeps registers low and occupancy high for large batches.
template <int kHeld>
__global__ __launch_bounds__(kRowThreads) void quant_q_kernel(QuantQArgs a) {
    __shared__ float red[kRowWaves];
    // `parts` workgroups per token (small batches: more workgroups in flight), each with the
    // token's amax from all partials and its own share [c0, c1) of the row's chunks
    const int parts = a.parts > 0 ? a.parts : 1;
    const int t = blockIdx.x / parts, part = blockIdx.x - t * parts;
    const int QH = a.Dn + a.R;
    const int cph = QH >> 3, cn = a.Dn >> 3;
    const int total_all = a.H * cph;
    const int per = (total_all + parts - 1) / parts;
    const int c0 = part * per;
    const int total = min(total_all, c0 + per);  // chunks [c0, total) belong to this workgroup
    auto chunk_at = [&](int c) -> const uint4* {
        c = min(c, total_all - 1);
        const int h = c / cph, j = c - h * cph;
        const size_t th = static_cast<size_t>(t) * a.H + h;
        return (j < cn) ? reinterpret_cast<const uint4*>(a.q_nope + th * a.Dn + j * 8)
                        : reinterpret_cast<const uint4*>(a.q_pe + th * a.R + (j - cn) * 8);
    };
    if (!a.q_i8) {  // scale only
        float m = 0.f;
        for (int i = threadIdx.x; i < a.n_tiles; i += kRowThreads)
            m = fmaxf(m, a.part_amax[static_cast<size_t>(t) * a.n_tiles + i]);
        const float amax = block_max(m, red);
        if (threadIdx.x == 0 && part == 0 && a.q_scale) a.q_scale[t] = amax / 127.0f;
        return;
    }
    // The partial amaxes go out first and the token's q values right behind them (they do
    // not depend on the amax), so the amax reduction runs while the row is in flight.
    // Clamped indexes keep the loads unconditional (straight-line code, exact waits): a
    // repeated partial amax does not change the max, repeated chunks are not stored.
    const int i0 = threadIdx.x;
    const float pa = a.part_amax[static_cast<size_t>(t) * a.n_tiles + min(i0, a.n_tiles - 1)];
    uint4 held[kHeld > 0 ? kHeld : 1];
#pragma unroll
    for (int k = 0; k < kHeld; ++k) held[k] = *chunk_at(c0 + static_cast<int>(threadIdx.x) + k * kRowThreads);
    float m = pa;
    for (int i = i0 + kRowThreads; i < a.n_tiles; i += kRowThreads)
        m = fmaxf(m, a.part_amax[static_cast<size_t>(t) * a.n_tiles + i]);
    const float amax = block_max(m, red);
    if (threadIdx.x == 0 && part == 0 && a.q_scale) a.q_scale[t] = amax / 127.0f;
    const float mult = amax > 0.f ? 127.0f / amax : 0.f;
    auto store = [&](int c, const uint4& v) {
        const int h = c / cph, j = c - h * cph;
        const size_t th = static_cast<size_t>(t) * a.H + h;
        MLAP_CHECK(a.dbg, t < a.T && h < a.H && (th * QH + j * 8 + 8) <= static_cast<size_t>(a.T) * a.H * QH, kDbgQuant);
        store_nt8(a.q_i8 + th * QH + j * 8, quant8(v, mult));
    };
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        const int c = c0 + threadIdx.x + k * kRowThreads;
        if (c < total) store(c, held[k]);
    }
    // the rest of the row in batches of kBatch chunks per thread, all loads of a batch in
    // flight before its first store (a V3 row is 12 chunks per thread: one batch; measured
    // against batches of four: the large-batch quant 3% faster at T=8192 and T=16384)
    constexpr int kBatch = 12;
    int c = c0 + threadIdx.x + kHeld * kRowThreads;
    for (; c + (kBatch - 1) * kRowThreads < total; c += kBatch * kRowThreads) {
        uint4 v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) v[k] = *chunk_at(c + k * kRowThreads);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) store(c + k * kRowThreads, v[k]);
    }
    for (; c < total; c += kRowThreads) store(c, *chunk_at(c));
}

// Per-(token, head) INT8 quant of q: each head's [q_nope | q_pe] row on its own (the row
// max of the [t, heads, d] q tensor over its last axis). One workgroup per token holds the
// whole row (kHeld chunks per thread); chunk maxima go through LDS to one maximum per head.
template <int kHeld>
__global__ __launch_bounds__(kRowThreads) void quant_q_head_kernel(QuantQArgs a) {
    __shared__ float cmax[kHeld * kRowThreads];
    __shared__ float hmax[kMaxQuantHeads];
    const int t = blockIdx.x;
    const int QH = a.Dn + a.R;
    const int cph = QH >> 3, cn = a.Dn >> 3;
    const int total = a.H * cph;
    auto chunk_at = [&](int c) -> const uint4* {
        const int h = c / cph, j = c - h * cph;
        const size_t th = static_cast<size_t>(t) * a.H + h;
        return (j < cn) ? reinterpret_cast<const uint4*>(a.q_nope + th * a.Dn + j * 8)
                        : reinterpret_cast<const uint4*>(a.q_pe + th * a.R + (j - cn) * 8);
    };
    uint4 held[kHeld];
#pragma unroll
    for (int k = 0; k < kHeld; ++k) held[k] = *chunk_at(min(static_cast<int>(threadIdx.x) + k * kRowThreads, total - 1));
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        const int c = threadIdx.x + k * kRowThreads;
        if (c < total) cmax[c] = absmax8(held[k]);
    }
    __syncthreads();
    for (int h = threadIdx.x; h < a.H; h += kRowThreads) {
        float m = 0.f;
        for (int j = 0; j < cph; ++j) m = fmaxf(m, cmax[h * cph + j]);
        hmax[h] = m;
        if (a.q_scale) a.q_scale[static_cast<size_t>(t) * a.H + h] = m / 127.0f;
    }
    __syncthreads();
    if (!a.q_i8) return;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        const int c = threadIdx.x + k * kRowThreads;
        if (c < total) {
            const int h = c / cph, j = c - h * cph;
            const float m = hmax[h];
            const float mult = m > 0.f ? 127.0f / m : 0.f;
            store_nt8(a.q_i8 + (static_cast<size_t>(t) * a.H + h) * QH + j * 8, quant8(held[k], mult));
        }
    }
}

// One workgroup per token: the q row (H heads of Dn + R raw values) is held in registers; each
// chunk's sum of squares goes to LDS and one thread per head adds its chunks in order; the
// normalised rope chunks are staged in LDS so each can read its rotate-half partner (R/2
// columns away in the same head); the token's |q| max closes the kernel.
__global__ __launch_bounds__(kRowThreads) void q_head_norm_kernel(QHeadNormArgs a) {
    __shared__ float csq[kHeadNormChunks * kRowThreads];
    __shared__ float hrstd[kMaxQuantHeads];
    __shared__ uint4 pe_stage[kHeadNormPeChunks];
    __shared__ float red[kRowWaves];
    // `groups` workgroups per token (small batches), each with a whole-head share of the row:
    // heads [h0, h0 + hg), chunks [c0, total)
    const int G = a.groups > 0 ? a.groups : 1;
    const int t = blockIdx.x / G, grp = blockIdx.x - t * G;
    const int QH = a.Dn + a.R;
    const int cph = QH >> 3, cn = a.Dn >> 3, cr = a.R >> 3;
    const int hg = a.H / G, h0 = grp * hg;
    const int c0 = h0 * cph;
    const int total = c0 + hg * cph;
    const float invD = 1.0f / static_cast<float>(QH);
    const float e = a.rsqrt ? 1.0f : invD;  // per-element 1/D (variant B)
    auto chunk_ptr = [&](int c) -> uint16_t* {
        const int h = c / cph, j = c - h * cph;
        const size_t th = static_cast<size_t>(t) * a.H + h;
        return (j < cn) ? a.q_nope + th * a.Dn + j * 8 : a.q_pe + th * a.R + (j - cn) * 8;
    };
    const int p = clamp_pos(a.positions[t], a.max_pos);
    MLAP_CHECK(a.dbg, a.positions[t] >= 0 && a.positions[t] < a.max_pos, kDbgPos);
    uint4 held[kHeadNormChunks];
#pragma unroll
    for (int k = 0; k < kHeadNormChunks; ++k)
        held[k] = *reinterpret_cast<const uint4*>(chunk_ptr(min(c0 + static_cast<int>(threadIdx.x) + k * kRowThreads, total - 1)));
#pragma unroll
    for (int k = 0; k < kHeadNormChunks; ++k) {
        const int c = c0 + threadIdx.x + k * kRowThreads;
        if (c < total) {
            if (a.q_proj) *reinterpret_cast<uint4*>(a.q_proj + static_cast<size_t>(t) * a.H * QH + c * 8) = held[k];
            float f[8], s = 0.f;
            unpack8(held[k], f);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float sq = f[q] * f[q];
                s += sq * e;
            }
            csq[c - c0] = s;
        }
    }
    __syncthreads();
    for (int hl = threadIdx.x; hl < hg; hl += kRowThreads) {
        float s = 0.f;
        for (int j = 0; j < cph; ++j) s += csq[hl * cph + j];
        hrstd[hl] = a.rsqrt ? rsqrtf(s * invD + a.eps) : 1.0f / sqrtf(s + a.eps);
    }
    __syncthreads();
    // normalise (bf16 cast point); rope chunks go to LDS for their partners
#pragma unroll
    for (int k = 0; k < kHeadNormChunks; ++k) {
        const int c = c0 + threadIdx.x + k * kRowThreads;
        if (c < total) {
            const int h = c / cph, j = c - h * cph;
            const float r = hrstd[h - h0];
            float f[8];
            unpack8(held[k], f);
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = f[q] * r;
            held[k] = pack8(f);
            if (j >= cn) pe_stage[(h - h0) * cr + (j - cn)] = held[k];
        }
    }
    __syncthreads();
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < kHeadNormChunks; ++k) {
        const int c = c0 + threadIdx.x + k * kRowThreads;
        if (c < total) {
            const int h = c / cph, j = c - h * cph;
            uint4 o = held[k];
            if (j >= cn) {
                // lo = x1*cos - x2*sin (first half), hi = x2*cos + x1*sin (second half), cos/sin
                // at this chunk's own columns; the partner is the other half
                const int jr = j - cn;
                const bool low = jr < (cr >> 1);
                const uint4 pv = pe_stage[(h - h0) * cr + (low ? jr + (cr >> 1) : jr - (cr >> 1))];
                float own[8], oth[8], res[8];
                unpack8(o, own);
                unpack8(pv, oth);
                const float* cs = a.cos + static_cast<size_t>(p) * a.R + jr * 8;
                const float* sn = a.sin + static_cast<size_t>(p) * a.R + jr * 8;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float t1 = own[q] * cs[q];
                    const float t2 = (low ? -oth[q] : oth[q]) * sn[q];
                    res[q] = t1 + t2;
                }
                o = pack8(res);
            }
            *reinterpret_cast<uint4*>(chunk_ptr(c)) = o;
            mx = fmaxf(mx, absmax8(o));
        }
    }
    if (a.part_amax) {
        const float amax = block_max(mx, red);
        if (threadIdx.x == 0) a.part_amax[static_cast<size_t>(t) * G + grp] = amax;
    }
}

hipError_t launch_q_head_norm(const QHeadNormArgs& a_in, hipStream_t s) {
    QHeadNormArgs a = a_in;
    a.dbg = debug_word();
    if (a.T <= 0) return hipSuccess;
    if (a.H > kMaxQuantHeads || a.H * ((a.Dn + a.R) >> 3) > kHeadNormChunks * kRowThreads ||
        a.H * (a.R >> 3) > kHeadNormPeChunks || (a.R >> 3) % 2)
        return hipErrorInvalidValue;
    const int G = a.groups > 0 ? a.groups : 1;
    if (a.H % G) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q_head_norm_kernel, dim3(a.T * G), dim3(kRowThreads), 0, s, a);
    return hipGetLastError();
}

// ---- MXFP8: E4M3 data with one E8M0 scale (2^(e-127)) per 32 values along K ----

// Value of an OCP E4M3FN byte (0x7F / 0xFF are NaN).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15, m = c & 7;
    float v = (e == 0) ? ldexpf(static_cast<float>(m), -9) : ldexpf(1.0f + 0.125f * m, static_cast<int>(e) - 7);
    if (e == 15 && m == 7) v = __builtin_nanf("");
    return (c & 0x80) ? -v : v;
}

// Nearest E4M3 value to v (|v| < 2^10), ties to even, saturating at +-448; every step is exact
// in fp32 (scalings by powers of two and a round to an integer).
__device__ __forceinline__ float e4m3_round(float v) {
    const float a = fabsf(v);
    float q;
    if (a >= 448.0f) {
        q = 448.0f;
    } else if (a < 0x1p-6f) {
        q = rintf(a * 512.0f) * 0x1p-9f;  // subnormal grid: steps of 2^-9
    } else {
        const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFF) - 127;  // a in [2^e, 2^(e+1))
        q = ldexpf(rintf(ldexpf(a, 3 - e)), e - 3);
        q = fminf(q, 448.0f);
    }
    return copysignf(q, v);
}

// Weights: E4M3 bytes [N, K] with E8M0 bytes [N, K/32] -> bf16 [N, K] (exact within bf16's
// exponent range); 16 values per thread.
__global__ __launch_bounds__(256) void mx_dequant_kernel(const uint8_t* codes, const uint8_t* scales,
                                                         size_t n16, int K, uint16_t* out) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const size_t e0 = i * 16;
        const size_t row = e0 / K;
        const int col = static_cast<int>(e0 - row * K);
        const uint4 c = *reinterpret_cast<const uint4*>(codes + e0);
        const int sh = static_cast<int>(scales[row * (K / 32) + col / 32]) - 127;
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
        float f[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = ldexpf(e4m3_value((w[j >> 2] >> (8 * (j & 3))) & 0xFF), sh);
        uint4* o = reinterpret_cast<uint4*>(out + e0);
        o[0] = pack8(f);
        o[1] = pack8(f + 8);
    }
}

// Activations: the MX conversion of a bf16 matrix [T, K], block by block (32 values, one
// thread each): shared exponent floor(log2(amax)) - 8 clamped to E8M0's range, values divided
// by 2^shared rounded to E4M3; writes the dequantised values (exact in bf16) for the bf16
// MFMA GEMM that follows.
__global__ __launch_bounds__(256) void mx_act_kernel(const uint16_t* x, size_t nblocks, uint16_t* out) {
    for (size_t b = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; b < nblocks;
         b += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
        float f[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(src[j], f + 8 * j);
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
        int sh = -127;
        if (amax > 0.f) {
            const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // floor(log2)
            sh = min(127, max(-127, e - 8));
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) f[j] = amax > 0.f ? ldexpf(e4m3_round(ldexpf(f[j], -sh)), sh) : 0.f;
        uint4* dst = reinterpret_cast<uint4*>(out + b * 32);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = pack8(f + 8 * j);
    }
}

// E4M3FN byte of a value already on the E4M3 grid (|v| <= 448, as e4m3_round returns).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const float a = fabsf(v);
    uint32_t c;
    if (a < 0x1p-6f) {
        c = static_cast<uint32_t>(a * 512.0f);  // subnormal: m * 2^-9 (0 for zero)
    } else {
        const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFF) - 127;
        const uint32_t m = (__float_as_uint(a) >> 20) & 7;  // the three mantissa bits
        c = (static_cast<uint32_t>(e + 7) << 3) | m;
    }
    return c | (v < 0.f ? 0x80u : 0u);
}

// Activations to MXFP8 operands: the conversion of mx_act_kernel, written as E4M3 codes and
// one E8M0 byte per 32-value block; one block per thread.
__global__ __launch_bounds__(256) void mx_act_codes_kernel(const uint16_t* x, size_t nblocks, uint8_t* codes,
                                                           uint8_t* scales) {
    for (size_t b = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; b < nblocks;
         b += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
        float f[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(src[j], f + 8 * j);
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
        int sh = -127;
        if (amax > 0.f) {
            const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // floor(log2)
            sh = min(127, max(-127, e - 8));
        }
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float y = amax > 0.f ? e4m3_round(ldexpf(f[4 * j + q], -sh)) : 0.f;
                v |= e4m3_code(y) << (8 * q);
            }
            w[j] = v;
        }
        uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[b] = static_cast<uint8_t>(sh + 127);
    }
}

hipError_t launch_mx_act_codes(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (K % 32) return hipErrorInvalidValue;
    const size_t nb = static_cast<size_t>(T) * K / 32;
    const int grid = static_cast<int>(std::min<size_t>((nb + 255) / 256, 8192));
    hipLaunchKernelGGL(mx_act_codes_kernel, dim3(grid), dim3(256), 0, s, x, nb, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, int N, int K, uint16_t* out,
                             hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    if (K % 32) return hipErrorInvalidValue;
    const size_t n16 = static_cast<size_t>(N) * K / 16;
    const int grid = static_cast<int>(std::min<size_t>((n16 + 255) / 256, 8192));
    hipLaunchKernelGGL(mx_dequant_kernel, dim3(grid), dim3(256), 0, s, codes, scales, n16, K, out);
    return hipGetLastError();
}

hipError_t launch_mx_act(const uint16_t* x, int T, int K, uint16_t* out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (K % 32) return hipErrorInvalidValue;
    const size_t nb = static_cast<size_t>(T) * K / 32;
    const int grid = static_cast<int>(std::min<size_t>((nb + 255) / 256, 8192));
    hipLaunchKernelGGL(mx_act_kernel, dim3(grid), dim3(256), 0, s, x, nb, out);
    return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a_in, hipStream_t s) {
    NormArgs a = a_in;
    a.dbg = debug_word();
    if (a.T <= 0) return hipSuccess;
    const int qc = (a.Lq / 8 + 63) / 64, kc = (a.Lkv / 8 + 63) / 64;
    const dim3 grid((a.T + 3) / 4), block(kRowThreads);
    // A wave per token needs thousands of tokens to fill 256 CUs; small batches keep a
    // whole workgroup per token.
    if (a.T >= 2048 && !a.a_f32 && a.R <= 1024 && kc >= 1 && kc <= 4 && qc <= 4) {
#define MLAP_NORM_WAVE(Q, K)                                                  \
    if (qc == Q && kc == K) {                                                 \
        hipLaunchKernelGGL((norm_rope_wave_kernel<Q, K>), grid, block, 0, s, a); \
        return hipGetLastError();                                             \
    }
        MLAP_NORM_WAVE(0, 1) MLAP_NORM_WAVE(0, 2) MLAP_NORM_WAVE(0, 3) MLAP_NORM_WAVE(0, 4)
        MLAP_NORM_WAVE(1, 1) MLAP_NORM_WAVE(2, 1) MLAP_NORM_WAVE(3, 1) MLAP_NORM_WAVE(4, 1)
        MLAP_NORM_WAVE(3, 2) MLAP_NORM_WAVE(4, 2) MLAP_NORM_WAVE(2, 2) MLAP_NORM_WAVE(1, 2)
#undef MLAP_NORM_WAVE
    }
    const int qb = (a.Lq / 8 + kRowThreads - 1) / kRowThreads, kb = (a.Lkv / 8 + kRowThreads - 1) / kRowThreads;
    const int spl = a.a_f32 ? a.k_splits : 0;
    if (!a.tail_f32 && a.R / 16 <= kRowThreads && kb == 1 && qb <= 1) {
#define MLAP_NORM_BLOCK(Q, P)                                                                      \
    if (qb == Q && spl == P) {                                                                     \
        hipLaunchKernelGGL((norm_rope_block_kernel<Q, 1, P>), dim3(a.T), dim3(kRowThreads), 0, s, a); \
        return hipGetLastError();                                                                  \
    }
        MLAP_NORM_BLOCK(0, 0) MLAP_NORM_BLOCK(1, 0) MLAP_NORM_BLOCK(0, 1) MLAP_NORM_BLOCK(1, 1)
        MLAP_NORM_BLOCK(0, 2) MLAP_NORM_BLOCK(1, 2) MLAP_NORM_BLOCK(0, 4) MLAP_NORM_BLOCK(1, 4)
        MLAP_NORM_BLOCK(0, 7) MLAP_NORM_BLOCK(1, 7) MLAP_NORM_BLOCK(0, 8) MLAP_NORM_BLOCK(1, 8)
        MLAP_NORM_BLOCK(0, 14) MLAP_NORM_BLOCK(1, 14) MLAP_NORM_BLOCK(0, 16) MLAP_NORM_BLOCK(1, 16)
#undef MLAP_NORM_BLOCK
    }
    hipLaunchKernelGGL(norm_rope_kernel, dim3(a.T), dim3(kRowThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* x, int T, int K, int8_t* codes, float* scale,
                            hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(act_quant_kernel, dim3(T), dim3(kRowThreads), 0, s, x, K, codes, scale);
    return hipGetLastError();
}

hipError_t launch_quant_q(const QuantQArgs& a_in, hipStream_t s) {
    QuantQArgs a = a_in;
    a.dbg = debug_word();
    if (a.T <= 0) return hipSuccess;
    if (a.per_head) {
        if (a.H > kMaxQuantHeads || a.H * ((a.Dn + a.R) >> 3) > kQuantHeadChunks * kRowThreads)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(quant_q_head_kernel<kQuantHeadChunks>, dim3(a.T), dim3(kRowThreads), 0, s, a);
        return hipGetLastError();
    }
    if (a.T >= 1024) {
        QuantQArgs b = a;
        b.parts = 1;
        hipLaunchKernelGGL(quant_q_kernel<0>, dim3(a.T), dim3(kRowThreads), 0, s, b);
    } else {
        // at most 64 tokens: four workgroups per token (measured: 1.5 us less at 16 tokens,
        // 1 us more at 256 tokens with two)
        QuantQArgs b = a;
        b.parts = a.T <= 64 ? 4 : 1;
        hipLaunchKernelGGL(quant_q_kernel<16>, dim3(a.T * b.parts), dim3(kRowThreads), 0, s, b);
    }
    return hipGetLastError();
}

}  // namespace mlap
