// gemm_big.hpp -- GEMM C = A . B^T on gfx950 matrix cores with global->LDS DMA staging.
//
// A [M, K] holds token activations, B [N, K] the weights (the AT-10 card's b_trans
// layout), both K-contiguous. One workgroup of WM x WN 64-wide waves computes a BM x BN
// output tile; each wave owns a (BM/WM) x (BN/WN) block held in accumulator registers.
// Shapes in use: 256 x 256 with 4 x 2 waves for large token batches (64 x 128 per wave,
// two waves per SIMD), and 256-row tiles 64 or 96 columns wide with 4 x 1 waves for
// weight streaming at small batches.
//
// Operand staging. A K-stage is KB bytes of every tile row (KB = 128: 64 bf16 or 128
// int8), (BM + BN) rows x KB bytes; S stages form a ring in LDS. Every stage is copied
// global -> LDS directly by the load unit (global_load_lds_dwordx4: each lane moves 16
// bytes and a wave writes 1 KB of consecutive LDS), so no register holds operands in
// flight. A lane fetches the global chunk that lands on its fixed LDS slot: 16-byte
// chunk c of tile row r lives at chunk c ^ swz(r), which spreads the 128-bit operand
// reads of the 16 lanes the LDS serves per cycle over distinct banks.
//
// Per stage a wave runs KB / 32 k-steps of v_mfma_f32_32x32x16_bf16 (or
// v_mfma_i32_32x32x32_i8). The weight fragment is the MFMA's first operand and the
// activation fragment its second, so the accumulator is the transposed tile: lane l,
// register 4g + q holds token (l % 32) and output column 8g + 4(l / 32) + q. Every lane
// therefore owns runs of four consecutive output columns of its tokens. The bf16 256 x 256
// heads tile (the large-batch q and kv_b up projections; the q projection runs at the board's
// power limit) uses v_mfma_f32_16x16x32_bf16 instead, 2 x 2 blocks of 16 x 16 per 32 x 32
// fragment: less energy per FLOP, so a higher clock under the limit (the kernel's M16 path).
//
// The k-step schedule is explicit (waits placed by hand, fenced slots): one MFMA, then
// the LDS reads of the next k-step's fragments and the copy instructions that fall on that
// slot, so LDS latency and copy issue hide under the matrix pipe and the copies never
// queue up behind the address unit; one workgroup barrier per stage, placed inside the
// last k-step. (The block-scaled MXFP8 tile keeps sched_group_barrier templates.)
#pragma once

#include "gemm.hpp"

namespace mlap {
namespace big {

// Chunk swizzle of a tile row of KB bytes (KB / 16 chunks of 16 bytes), chosen by
// measurement on gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT over this kernel's fragment read
// pattern): with 64-byte rows (r >> 2) & 3 reads conflict-free where the unswizzled layout
// is 4-way; with 128-byte rows (r >> 1) & 7 is conflict-free where unswizzled is 8-way.
// Both are invariant under r -> r + 32, so every 32-row fragment shares the lane's swizzle.
template <int KB>
__device__ __forceinline__ int swz(int r) {
    if constexpr (KB == 64)
        return (r >> 2) & 3;
    else
        return (r >> 1) & 7;
}

// Epilogue LDS: the bf16 tile with rows padded by 16 bytes, then one row-amax word per row
// and wave column.
constexpr int epi_pitch(int bn) { return bn * 2 + 16; }
constexpr int epi_lds(int bm, int bn, int wn) { return bm * epi_pitch(bn) + wn * bm * 4; }

// XR extra weight rows per stage follow the BM + BN tile rows (kStoreBf16X).
template <int BM, int BN, int WM, int WN, int KB, int S, int XR = 0>
struct Shape {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;  // per-wave block
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int KS = KB / 32;                // MFMA k-steps per stage (32 bytes each)
    static constexpr int LPR = KB / 16;               // copy lanes per tile row
    static constexpr int ROWS = BM + BN;
    static constexpr int RROWS = NT / LPR;            // rows one workgroup-wide copy round fills
    static constexpr int ROUNDS = ROWS / RROWS;
    static constexpr int STAGE = (ROWS + XR) * KB;
    static constexpr int MAIN = S * STAGE;
    static constexpr int EPI = epi_lds(BM, BN, WN);           // staged tile + row amaxes
    static constexpr int LDS = MAIN > EPI ? MAIN : EPI;
    static_assert(KB == 64 || KB == 128, "stage row bytes");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave block must be whole 32x32 fragments");
    static_assert(BM % RROWS == 0 && BN % RROWS == 0, "tile rows must fill whole copy rounds");
    static_assert(S >= 2 && LDS <= 160 * 1024, "LDS budget");
    static_assert((S - 2) * ROUNDS < 64, "vmcnt range");
};

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier that orders LDS traffic without waiting for outstanding global
// loads (a __syncthreads() fence would drain the copy ring). s_barrier itself does not
// wait for this wave's LDS operations, so they are drained first (lgkmcnt(0)): without
// that, a write issued just before the barrier (a staged tile chunk, a cleared row amax)
// can land after another wave's access that the barrier was meant to order behind it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// One 4-byte-per-lane copy global -> LDS (global_load_lds_dword): lane l writes lds + 4 l
// (`lds` wave-uniform); lanes outside the exec mask write nothing.
__device__ __forceinline__ void copy4_to_lds(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)(lds), 4, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l holds row l % 16 of the 16 x 32 first operand and column
// l % 16 of the 32 x 16 second one, K values 8 (l / 16) + [0, 8) of both (one 16-byte chunk);
// the result's lane l holds rows 4 (l / 16) + [0, 4) of column l % 16 (layout checked on
// gfx950 with exact small-integer operands).
__device__ __forceinline__ f32x4 mma16x16(const i32x4& a, const i32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
// v_mfma_i32_16x16x64_i8: the same lanes, 16 int8 K values 16 (l / 16) + [0, 16) per lane
// (checked the same way).
__device__ __forceinline__ i32x4 mma16x16(const i32x4& a, const i32x4& b, const i32x4& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// One 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4); `lds` must be
// wave-uniform: lane l writes lds + 16 l. A device function rather than a lambda body:
// lambdas are host-device in HIP, and a device builtin inside one suppresses the
// kernel's host-side launch stub.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)(lds), 16, 0, 0);
}

// An empty statement that needs `v` in VGPRs (an allocation hint, no instruction).
__device__ __forceinline__ void pin_vgpr(i32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_vgpr(i32x8& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // v_cvt_pk_bf16_f32, RNE
    return __builtin_bit_cast(uint32_t, v);
}

// 16-byte store marked non-temporal: output tiles are written once and not read again by
// the kernel, so they should not displace operand lines from the L2.
__device__ __forceinline__ void store_nt(void* p, const uint4& v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace big

// Operands of the in-register rotate-half of the heads epilogue (64-wide rope slices that
// start on a 32-column fragment). Lane l holds, for each of its FM tokens, columns
// 8g + 4(l / 32) + q of both 32-column halves of a slice: their cos/sin values depend on
// the token and the column only. The positions are read when the workgroup starts; the
// cos/sin values under the last K-stage (gather) on shapes with registers to hold them,
// else the epilogue stages the tile's cos/sin rows in LDS.
template <int FM>
struct RopeOps {
    bool on;        // the tile holds a rope slice (wave-uniform)
    int pos[FM];
    float4 c[FM][2][4], s[FM][2][4];  // [token fragment][half][column group g]
    __device__ __forceinline__ void fetch_positions(const GemmArgs& g, int mb) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            pos[i] = g.positions[min(mb + 32 * i, g.M - 1)];
            MLAP_CHECK(g.dbg, pos[i] >= 0 && pos[i] < g.max_pos, kDbgPos);
        }
    }
    // every token fragment's cos/sin (shapes with registers to hold them)
    __device__ __forceinline__ void gather(const GemmArgs& g, int lh) {
        if (!on) return;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const size_t row = static_cast<size_t>(clamp_pos(pos[i], g.max_pos)) * 64 + 4 * lh;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    c[i][h][gq] = *reinterpret_cast<const float4*>(g.cos + row + 32 * h + 8 * gq);
                    s[i][h][gq] = *reinterpret_cast<const float4*>(g.sin + row + 32 * h + 8 * gq);
                }
        }
    }
};
template <>
struct RopeOps<0> {
    static constexpr bool on = false;
    __device__ __forceinline__ void fetch_positions(const GemmArgs&, int) {}
    __device__ __forceinline__ void gather(const GemmArgs&, int) {}
};

// Output stage of a BM x BN tile held in the transposed accumulator layout (lane l,
// register 4g + q of fragment (j, i): token 32 i + l % 32 of the wave's rows, column
// 32 j + 8 g + 4 (l / 32) + q of its columns). `smem` must hold
// big::epi_lds(BM, BN, WN) bytes and be free: every wave is done with the operand stages.
// EARLY: the cos/sin operands were gathered under the last K-stage (else the epilogue
// copies the tile's cos/sin rows into LDS while it packs the accumulators). W8A8: `scl`
// holds the tile's dequantisation scales in LDS, a_scale of rows m0 + [0, BM) then b_scale
// of columns n0 + [0, BN) (through b_row; rows and columns past the matrix edge clamped).
// M16 (the 16 x 16 x 32 heads tile): register 4 gq + q of fragment (j, i) holds token
// 32 i + 16 (gq / 2) + l % 16 and column 32 j + 16 (gq % 2) + 4 (l / 16) + q instead.
template <typename Tin, int BM, int BN, int WM, int WN, Epi EPI, bool EARLY, bool M16, typename AccT, int FN,
          int FM, int RF>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, AccT (&acc)[FN][FM], char* smem,
                                              const float* scl, int m0, int n0, int n_tile, int split,
                                              RopeOps<RF>& rope_ops) {
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    static_assert(FM == TM / 32 && FN == TN / 32, "accumulator shape");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, lh = lane >> 5;
    const int l16 = lane & 15, lq = lane >> 4;  // M16 lane view
    static_assert(!M16 || (EPI == Epi::kHeads && RF > 0 && !EARLY), "the 16 x 16 form is the large heads tile");
    // Lane view of the transposed accumulator: token m = mb + 32 i + lr, columns
    // nb + 32 j + 8 g + 4 lh + q for register 4 g + q.
    const int mb = m0 + wm * TM + lr;
    const int nb = n0 + wn * TN + 4 * lh;

    // W8A8 dequantisation scales of this lane's rows and columns, from the tile's copy in
    // LDS: a_scale of each of its FM tokens, b_scale of its 4-column runs.
    constexpr bool DEQ = kIsI8<Tin> && EPI != Epi::kStoreI32;  // int32 export: raw accumulators
    float asc[DEQ ? FM : 1];
    float4 bsc[DEQ ? FN : 1][4];
    if constexpr (DEQ) {
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            asc[i] = scl[min(mb + 32 * i, g.M - 1) - m0];
        });
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                bsc[j][gq] = *reinterpret_cast<const float4*>(scl + BM + (nb - n0) + 32 * j + 8 * gq);
        });
    }

    // Fragment (j, i) as eight packed bf16 pairs (the GEMM's bf16 output cast), with the
    // W8A8 dequantisation f32(acc) * (a_scale[m] * b_scale[n]) applied first.
    auto frag_bf16 = [&](auto j_c, auto i_c, uint32_t* w) __attribute__((always_inline)) {
        constexpr int j = decltype(j_c)::value, i = decltype(i_c)::value;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            float v[4];
            if constexpr (DEQ) {
                const float as = asc[i];
                const float bs[4] = {bsc[j][gq].x, bsc[j][gq].y, bsc[j][gq].z, bsc[j][gq].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float sc = as * bs[q];
                    v[q] = static_cast<float>(acc[j][i][4 * gq + q]) * sc;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = acc[j][i][4 * gq + q];
            }
            w[2 * gq] = big::pack_bf16x2(v[0], v[1]);
            w[2 * gq + 1] = big::pack_bf16x2(v[2], v[3]);
        }
    };

    if constexpr (EPI == Epi::kStoreI32) {
        // the raw int32 accumulators [M, ldo] (the W8A8 core's test export): four consecutive
        // columns per lane, element by element past the last whole run of N
        static_assert(kIsI8<Tin>, "int32 output needs int8 operands");
        int32_t* out = static_cast<int32_t*>(g.out);
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                const int m = mb + 32 * i;
                if (m < g.M) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int n = nb + 32 * j + 8 * gq;
                        int32_t* o = out + static_cast<size_t>(m) * g.ldo + n;
                        if (n + 3 < g.N && g.ldo % 4 == 0) {
                            *reinterpret_cast<int4*>(o) = make_int4(acc[j][i][4 * gq], acc[j][i][4 * gq + 1],
                                                                    acc[j][i][4 * gq + 2], acc[j][i][4 * gq + 3]);
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (n + q < g.N) o[q] = acc[j][i][4 * gq + q];
                        }
                    }
                }
            });
        });
        return;
    }
    if constexpr (EPI == Epi::kStoreF32) {
        // split-K partial sums, fp32 [k_splits][M][ldo]: four consecutive columns per lane
        float* out = static_cast<float*>(g.out) + static_cast<size_t>(split) * g.M * g.ldo;
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                const int m = mb + 32 * i;
                if (m < g.M) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int n = nb + 32 * j + 8 * gq;
                        MLAP_CHECK(g.dbg, n >= g.N || (n + 4 <= g.ldo && split < g.k_splits), kDbgStore);
                        if (n < g.N)  // N is a multiple of 4
                            *reinterpret_cast<float4*>(out + static_cast<size_t>(m) * g.ldo + n) =
                                make_float4(acc[j][i][4 * gq], acc[j][i][4 * gq + 1],
                                            acc[j][i][4 * gq + 2], acc[j][i][4 * gq + 3]);
                    }
                }
            });
        });
        return;
    }

    // The bf16 tile is transposed through LDS (the stage buffers are free now) so that
    // stores leave as whole 16-byte chunks, a row's chunks on consecutive lanes. Rows are
    // padded by 16 bytes against bank conflicts.
    constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
    constexpr int PITCH = big::epi_pitch(BN);
    auto stage_frag = [&](int row, int col, const uint32_t* w) __attribute__((always_inline)) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<uint2*>(smem + row * PITCH + (col + 8 * gq) * 2) = make_uint2(w[2 * gq], w[2 * gq + 1]);
    };
    big::lds_barrier();  // every wave is done reading the last stage
    if constexpr (EPI == Epi::kStoreBf16 || EPI == Epi::kStoreBf16X) {
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                uint32_t w[8];
                frag_bf16(j_c, i_c, w);
                stage_frag(wm * TM + 32 * decltype(i_c)::value + lr, wn * TN + 32 * j + 4 * lh, w);
            });
        });
        big::lds_barrier();
        uint16_t* out = static_cast<uint16_t*>(g.out);
        for (int idx = tid; idx < BM * CPR; idx += NT) {
            const int row = idx / CPR, c = idx - row * CPR;
            const int m = m0 + row, n = n0 + 8 * c;
            if (m < g.M && n < g.N) {  // N is a multiple of 8
                MLAP_CHECK(g.dbg, n + 8 <= g.ldo, kDbgStore);
                big::store_nt(out + static_cast<size_t>(m) * g.ldo + n,
                              *reinterpret_cast<const uint4*>(smem + row * PITCH + c * 16));
            }
        }
    } else if constexpr (EPI == Epi::kHeads) {
        // The heads work is done in registers before the tile is staged. A rope slice is 64
        // columns that start on a 32-column fragment j, so its two halves are fragments j and
        // j + 1 of the same lane (one register apart per value). A token's amax over the tile
        // is a lane-local max, one exchange with lane l ^ 32 (the other column runs), and
        // with several wave columns a max over their per-row entries in LDS.
        float* wave_amax = reinterpret_cast<float*>(smem + BM * PITCH);  // [WN][BM]
        const int cw = n0 + wn * TN;  // first column of this wave
        // Fragment sj starts this wave's rope slice, or sj = -1 (wave-uniform). Slices are
        // at least 128 columns apart, so a wave's columns hold at most one.
        int sj = -1;
        if constexpr (RF > 0) {
            if (rope_ops.on)
                for (int j = 0; j + 1 < FN; ++j) {
                    const int cj = cw + 32 * j;
                    if (sj < 0 && cj + 64 <= g.N && cj % g.head_w == g.d0) sj = j;
                }
        }
        auto absmax_frag = [&](const uint32_t* w) __attribute__((always_inline)) {
            // |bf16| values: clear the sign bits, then compare as floats
            float mx = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t a = w[e] & 0x7fff7fffu;
                mx = fmaxf(mx, fmaxf(big::lo_bf(a), big::hi_bf(a)));
            }
            return mx;
        };
        // |max| of the four packed words w[w0 .. w0 + 4) (M16: one token's eight columns)
        auto absmax_words = [&](const uint32_t* w, int w0) __attribute__((always_inline)) {
            float mx = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a = w[w0 + e] & 0x7fff7fffu;
                mx = fmaxf(mx, fmaxf(big::lo_bf(a), big::hi_bf(a)));
            }
            return mx;
        };
        float amx16[M16 ? FM : 1][2] = {};
        // lo = x1*cos - x2*sin (first half), hi = x2*cos + x1*sin (second half), cos/sin at
        // each value's own column: cc/ss[half][g] hold columns 32 half + 8 g + 4 (l / 32) + q
        // (M16: columns 32 half + 16 (g % 2) + 4 (l / 16) + q of token 16 (g / 2) + l % 16)
        auto rotate = [&](uint32_t(&lo)[8], uint32_t(&hi)[8], const float4(&cc)[2][4],
                          const float4(&ss)[2][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const float4 cl = cc[0][gq], ch = cc[1][gq], sl = ss[0][gq], sh = ss[1][gq];
                const float c_lo[4] = {cl.x, cl.y, cl.z, cl.w}, c_hi[4] = {ch.x, ch.y, ch.z, ch.w};
                const float s_lo[4] = {sl.x, sl.y, sl.z, sl.w}, s_hi[4] = {sh.x, sh.y, sh.z, sh.w};
                float x1[4], x2[4], r1[4], r2[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    x1[2 * h] = big::lo_bf(lo[2 * gq + h]);
                    x1[2 * h + 1] = big::hi_bf(lo[2 * gq + h]);
                    x2[2 * h] = big::lo_bf(hi[2 * gq + h]);
                    x2[2 * h + 1] = big::hi_bf(hi[2 * gq + h]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    r1[q] = x1[q] * c_lo[q] + (-x2[q]) * s_lo[q];
                    r2[q] = x2[q] * c_hi[q] + x1[q] * s_hi[q];
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    lo[2 * gq + h] = big::pack_bf16x2(r1[2 * h], r1[2 * h + 1]);
                    hi[2 * gq + h] = big::pack_bf16x2(r2[2 * h], r2[2 * h + 1]);
                }
            }
        };
        float amx[FM];
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) { amx[decltype(i_c)::value] = 0.f; });
        if constexpr (RF > 0 && !EARLY) {
            // Two waves per SIMD: no registers to hold cos/sin through the main loop. The
            // tile's cos and sin rows (256 B each per token) are copied into the free LDS
            // by the load unit while the accumulators are packed: per wave row, cos rows of
            // its TM tokens then sin rows, one table per wave column, 16-byte chunk c of
            // token row t at chunk c ^ (t % 16) so that 16 lanes reading 16 consecutive
            // tokens' chunk hit distinct banks. Each row is fetched once per tile (instead of
            // once per rope slice and wave, scattered over 32 tokens per load).
            constexpr int CS_ROWS = 2 * TM;                  // rows per wave row
            constexpr int PER = CS_ROWS * 256 / 1024 / WN;   // 1 KB copies per wave
            static_assert(WN == 2 && 4 * PER == TM, "one table per wave column");
            static_assert(BM * 512 <= big::epi_lds(BM, BN, WN), "cos/sin rows fit the epilogue LDS");
            char* const cs_lds = smem;
            if (rope_ops.on) {  // tile-uniform
                const float* table = wn == 0 ? g.cos : g.sin;
                char* const dst = cs_lds + (wm * CS_ROWS + wn * TM) * 256;
                static_for<PER>([&](auto k_c) __attribute__((always_inline)) {
                    constexpr int k = decltype(k_c)::value;
                    const int t = 4 * k + (lane >> 4);  // token within the wave row
                    const int p = clamp_pos(__shfl(rope_ops.pos[k / 8], (4 * k) % 32 + (lane >> 4)), g.max_pos);
                    const int c = (lane & 15) ^ (t & 15);
                    big::copy16_to_lds(table + static_cast<size_t>(p) * 64 + c * 4, dst + k * 1024);
                });
            }
            uint32_t w[FN][FM][8];
            static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
                static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                    frag_bf16(j_c, i_c, w[decltype(j_c)::value][decltype(i_c)::value]);
                });
            });
            big::wait_vmcnt<0>();
            big::lds_barrier();  // every wave's cos/sin rows have landed
            if (sj >= 0) {
                static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    float4 cc[2][4], ss[2][4];
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        // the token and the 4-column chunk of group gq (16 B chunks of the row)
                        const int t = M16 ? 32 * i + 16 * (gq >> 1) + l16 : 32 * i + lr;
                        const int ch = M16 ? 4 * (gq & 1) + lq : 2 * gq + lh;
                        const char* crow = cs_lds + (wm * CS_ROWS + t) * 256;
                        const char* srow = crow + TM * 256;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int off = ((8 * h + ch) ^ (t & 15)) * 16;
                            cc[h][gq] = *reinterpret_cast<const float4*>(crow + off);
                            ss[h][gq] = *reinterpret_cast<const float4*>(srow + off);
                        }
                    }
                    static_for<FN - 1>([&](auto j_c) __attribute__((always_inline)) {
                        constexpr int j = decltype(j_c)::value;
                        if (j == sj) rotate(w[j][i], w[j + 1][i], cc, ss);
                    });
                });
            }
            big::lds_barrier();  // every wave is done reading cos/sin: the tile goes over them
            static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int j = decltype(j_c)::value;
                static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    if constexpr (M16) {
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const int row = wm * TM + 32 * i + 16 * (gq >> 1) + l16;
                            const int col = wn * TN + 32 * j + 16 * (gq & 1) + 4 * lq;
                            *reinterpret_cast<uint2*>(smem + row * PITCH + col * 2) =
                                make_uint2(w[j][i][2 * gq], w[j][i][2 * gq + 1]);
                        }
                        // token halves: words 0..3 (first 16 tokens), 4..7 (second 16)
                        amx16[i][0] = fmaxf(amx16[i][0], absmax_words(w[j][i], 0));
                        amx16[i][1] = fmaxf(amx16[i][1], absmax_words(w[j][i], 4));
                    } else {
                        stage_frag(wm * TM + 32 * i + lr, wn * TN + 32 * j + 4 * lh, w[j][i]);
                        amx[i] = fmaxf(amx[i], absmax_frag(w[j][i]));
                    }
                });
            });
        } else {
            // Every fragment is packed and staged at once, its |max| folded into the token's
            // running max; only the rope slice's two fragments are kept for the rotation,
            // with the cos/sin values gathered under the last K-stage.
            uint32_t sw[RF > 0 ? 2 : 1][FM][8];
            static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int j = decltype(j_c)::value;
                static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    uint32_t w[8];
                    frag_bf16(j_c, i_c, w);
                    bool keep = false;
                    if constexpr (RF > 0) {
                        if (sj >= 0 && (j == sj || j == sj + 1)) {
                            keep = true;
#pragma unroll
                            for (int e = 0; e < 8; ++e) sw[j == sj ? 0 : 1][i][e] = w[e];
                        }
                    }
                    if (!keep) {
                        stage_frag(wm * TM + 32 * i + lr, wn * TN + 32 * j + 4 * lh, w);
                        amx[i] = fmaxf(amx[i], absmax_frag(w));
                    }
                });
            });
            if constexpr (RF > 0) {
                if (sj >= 0) {
                    static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                        constexpr int i = decltype(i_c)::value;
                        rotate(sw[0][i], sw[1][i], rope_ops.c[i], rope_ops.s[i]);
                        const int row = wm * TM + 32 * i + lr;
                        stage_frag(row, wn * TN + 32 * sj + 4 * lh, sw[0][i]);
                        stage_frag(row, wn * TN + 32 * (sj + 1) + 4 * lh, sw[1][i]);
                        amx[i] = fmaxf(amx[i], fmaxf(absmax_frag(sw[0][i]), absmax_frag(sw[1][i])));
                    });
                }
            }
        }
        if (M16 && g.part_amax) {
            // a token's maxima are spread over the four lanes l % 16 + 16 k
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
#pragma unroll
                for (int si = 0; si < 2; ++si) {
                    float mx = amx16[M16 ? i : 0][si];
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    if (lq == 0) wave_amax[wn * BM + wm * TM + 32 * i + 16 * si + l16] = mx;
                }
            });
        } else if (g.part_amax) {
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                const float mx = fmaxf(amx[i], __shfl_xor(amx[i], 32));
                const int row = wm * TM + 32 * i + lr;
                if constexpr (WN == 1) {
                    const int m = m0 + row;
                    if (lh == 0 && m < g.M) g.part_amax[static_cast<size_t>(m) * g.n_tiles + n_tile] = mx;
                } else {
                    if (lh == 0) wave_amax[wn * BM + row] = mx;
                }
            });
        }
        big::lds_barrier();
        if constexpr (WN > 1) {
            if (g.part_amax)
                for (int r = tid; r < BM; r += NT)
                    if (m0 + r < g.M) {
                        float mx = wave_amax[r];
#pragma unroll
                        for (int k = 1; k < WN; ++k) mx = fmaxf(mx, wave_amax[k * BM + r]);
                        g.part_amax[static_cast<size_t>(m0 + r) * g.n_tiles + n_tile] = mx;
                    }
        }
        // Per head [seg0 (d0 columns) | seg1 (d1 columns)]; the host picks tiles whose
        // 8-column chunks each lie inside one segment. A thread keeps one chunk column c for
        // the whole tile and walks the rows, RPP rows per pass.
        constexpr int RPP = NT / CPR;
        constexpr int PASSES = (BM + RPP - 1) / RPP;
        const int HW = g.head_w, d0 = g.d0, d1 = g.d1;
        uint16_t* out0 = static_cast<uint16_t*>(g.out0);
        uint16_t* out1 = static_cast<uint16_t*>(g.out1);
        const int c = tid % CPR, r_in = tid / CPR;
        const int n = n0 + 8 * c;
        const bool nok = tid < RPP * CPR && n < g.N;
        const int h = n / HW;
        const int d = n - h * HW;
        const bool seg0 = d < d0;
        uint16_t* const dst = seg0 ? out0 : out1;
        const int dw = seg0 ? d0 : d1, dd = seg0 ? d : d - d0;
        if (nok && dst) {
            static_for<PASSES>([&](auto p_c) __attribute__((always_inline)) {
                constexpr int p = decltype(p_c)::value;
                const int row = p * RPP + r_in;
                const int m = m0 + row;
                if (row < BM && m < g.M) {
                    MLAP_CHECK(g.dbg, h < g.n_heads && dd + 8 <= dw, kDbgStore);
                    big::store_nt(dst + (static_cast<size_t>(m) * g.n_heads + h) * dw + dd,
                                  *reinterpret_cast<const uint4*>(smem + row * PITCH + c * 16));
                }
            });
        }
    }
}

template <typename Tin, int BM, int BN, int WM, int WN, int KB, int S, Epi EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_big_kernel(GemmArgs g) {
    // kStoreBf16X: XR = 8 extra weight rows per stage (rows BM + BN .. + 7 of the stage), the
    // eight extra output columns of this column tile; see xcols below
    constexpr int XR = EPI == Epi::kStoreBf16X ? 8 : 0;
    static_assert(XR == 0 || ((std::is_same<Tin, uint16_t>::value || kIsI8<Tin>) && BM == 256 && WM == 4 &&
                              WN == 2 && S == 2 && KB == 128),
                  "extra columns: the 256 x 256 bf16 / int8 tile with a two-slot ring only");
    using SH = big::Shape<BM, BN, WM, WN, KB, S, XR>;
    using Op = MfmaOp<Tin>;
    unsigned long long clk0 = 0, wall0 = 0;  // measurement only (g.clk, sampled workgroups)
    if (g.clk && (blockIdx.x & 15) == 0) {
        clk0 = clock64();
        wall0 = wall_clock64();
    }
    // MXFP8: a k-step is one 64-deep block-scaled MFMA, 64 bytes of every row, read as two
    // 16-byte chunks per lane
    constexpr bool MX = kIsMx<Tin>;
    constexpr int RPK = MX ? 2 : 1;  // LDS reads per fragment per k-step
    constexpr int TM = SH::TM, TN = SH::TN, FM = SH::FM, FN = SH::FN, KS = MX ? KB / 64 : SH::KS;
    constexpr int ROUNDS = SH::ROUNDS, LPR = SH::LPR;
    // W8A8: the tile's dequantisation scales (BM + BN floats) follow the stage / epilogue LDS
    constexpr bool DEQ = kIsI8<Tin> && EPI != Epi::kStoreI32;
    constexpr int SCL = DEQ ? (BM + BN) * 4 : 0;
    static_assert(SH::LDS % 16 == 0 && SH::LDS + SCL <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[SH::LDS + SCL];
    float* const scl = reinterpret_cast<float*>(smem + SH::LDS);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tiles_m = (g.M + BM - 1) / BM;
    const int tiles_n = (g.N + BN - 1) / BN;
    int m_tile, n_tile, split;
    if (g.n_major)
        tile_of(blockIdx.x, tiles_n, tiles_m, g.k_splits, g.group_m, n_tile, m_tile, split);
    else
        tile_of(blockIdx.x, tiles_m, tiles_n, g.k_splits, g.group_m, m_tile, n_tile, split);
    const int m0 = m_tile * BM;
    const int n0 = n_tile * BN;
    // W8A8: the tile's scales go to LDS now, one dword per lane and 64 per wave; the main
    // loop's first stage wait and barrier cover them (they are the oldest loads)
    if constexpr (DEQ) {
        static_assert(BM % 64 == 0 && BN % 64 == 0, "whole waves of scales");
        for (int c = wave; c < (BM + BN) / 64; c += WM * WN) {
            const int idx = 64 * c + lane;
            if (idx < BM) {  // wave-uniform
                if (m0 + idx < g.M) big::copy4_to_lds(g.a_scale + m0 + idx, scl + 64 * c);
            } else {
                const int nn = b_row(g, min(n0 + idx - BM, g.N - 1));
                MLAP_CHECK(g.dbg, nn >= 0 && nn < g.N + XR * tiles_n, kDbgBRow);
                big::copy4_to_lds(nn < g.b_split ? g.b_scale0 + nn : g.b_scale1 + (nn - g.b_split), scl + 64 * c);
            }
        }
    }
    // In-register rope operands of the heads epilogue: whether the columns hold a 64-wide
    // rope slice, and if so the tokens' positions now. With one wave per SIMD (a
    // 512-register budget) each wave with a slice gathers its cos/sin values under the last
    // K-stage; the two-waves-per-SIMD shape has no registers to spare there, and all of
    // its waves copy the tile's cos/sin rows into LDS in the epilogue if any wave needs
    // them.
    constexpr int RF = EPI == Epi::kHeads && FN > 1 ? FM : 0;
    constexpr bool EARLY = WM * WN <= 4 && SH::FM <= 2;
    // The bf16 256 x 256 heads tile (the large-batch q and kv_b up projections) runs on
    // v_mfma_f32_16x16x32_bf16 instead of the 32 x 32 x 16 form: the same operand bytes and
    // FLOPs per cycle, but about 20% less energy per FLOP (the accumulator traffic of a
    // 16 x 16 block is half that of a 32 x 32 one per FLOP), which the power-limited prefill
    // step turns into clock.
    constexpr bool M16 = std::is_same<Tin, uint16_t>::value && EPI == Epi::kHeads && BM == 256 && BN == 256 &&
                         WM == 4 && WN == 2 && KB == 128 && S == 2 && XR == 0;
    RopeOps<RF> rope_ops;
    if constexpr (RF > 0) {
        rope_ops.on = false;
        if (g.rope && g.d1 == 64) {
            const int c0 = EARLY ? n0 + wn * TN : n0;  // this wave's columns, or the tile's
            constexpr int NF = EARLY ? FN : BN / 32;
            for (int j = 0; j + 1 < NF; ++j) {
                const int cj = c0 + 32 * j;
                rope_ops.on |= cj + 64 <= g.N && cj % g.head_w == g.d0;
            }
        }
        if (rope_ops.on) rope_ops.fetch_positions(g, m0 + wm * TM + (lane & 31));
    }
    // split-K (fp32 partial epilogue only): this workgroup covers K bytes
    // [split * kbs, (split + 1) * kbs) of every row
    const int kbs = g.K * static_cast<int>(sizeof(Tin)) / g.k_splits;
    const int nk = kbs / KB;
    // Weight-streaming shapes (three-stage rings) run their K-stages in a per-tile rotated
    // order, so that the workgroups sharing activation rows (every tile of the launch) do not
    // all fetch the same lines at once. The large-batch tiles keep the common order: there,
    // tiles running side by side share their operand rows through L2 (rotated, the kernel's
    // HBM traffic grew 12% at T=8192 for no gain in time).
    const int krot = S > 2 ? (n_tile + m_tile) % (nk > 0 ? nk : 1) : 0;
    auto kphys = [&](int kt) __attribute__((always_inline)) { return kt + krot < nk ? kt + krot : kt + krot - nk; };
    const size_t k0 = static_cast<size_t>(split) * kbs;
    MLAP_CHECK(g.dbg, kbs % KB == 0 && split < g.k_splits && k0 + kbs <= static_cast<size_t>(g.K) * sizeof(Tin), kDbgK);

    // Copy sources: round i moves tile row i*RROWS + tid/LPR, physical chunk tid%LPR.
    // Rows past the matrix edge re-read its last row; their results are never stored.
    const char* src[ROUNDS];
    {
        const size_t lda_b = static_cast<size_t>(g.lda) * sizeof(Tin);
        const size_t ldb_b = static_cast<size_t>(g.ldb) * sizeof(Tin);
        static_for<ROUNDS>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            const int r = i * SH::RROWS + tid / LPR;
            const int c = (tid % LPR) ^ big::swz<KB>(r);
            if constexpr (i * SH::RROWS < BM) {
                const int m = min(m0 + r, g.M - 1);
                MLAP_CHECK(g.dbg, m >= 0 && m < g.M, kDbgARow);
                src[i] = static_cast<const char*>(g.A) + static_cast<size_t>(m) * lda_b + k0 + c * 16;
            } else {
                const int n = b_row(g, min(n0 + r - BM, g.N - 1));
                MLAP_CHECK(g.dbg, n >= 0 && n < g.N + XR * tiles_n, kDbgBRow);
                const char* row = n < g.b_split
                                      ? static_cast<const char*>(g.B0) + static_cast<ptrdiff_t>(n) * static_cast<ptrdiff_t>(ldb_b)
                                      : static_cast<const char*>(g.B1) +
                                            static_cast<ptrdiff_t>(n - g.b_split) * static_cast<ptrdiff_t>(ldb_b);
                src[i] = row + k0 + c * 16;
            }
        });
    }
    // kStoreBf16X: the extra columns g.N + XR n_tile + [0, XR) come from weight rows of the
    // same index (through b_row), staged after the tile rows of every stage. The XR rows of
    // 128 bytes are one wave-wide copy: wave 0 moves them, lane l physical chunk l % 8 of
    // extra row l / 8.
    const char* xsrc = nullptr;
    if constexpr (XR > 0) {
        const int r = lane >> 3;
        const int c = (lane & 7) ^ big::swz<KB>(BM + BN + r);
        const int n = b_row(g, g.N + XR * n_tile + r);
        MLAP_CHECK(g.dbg, n >= 0 && n < g.N + XR * tiles_n, kDbgBRow);
        const ptrdiff_t ldb_b = static_cast<ptrdiff_t>(g.ldb) * static_cast<ptrdiff_t>(sizeof(Tin));
        const char* row = n < g.b_split ? static_cast<const char*>(g.B0) + static_cast<ptrdiff_t>(n) * ldb_b
                                        : static_cast<const char*>(g.B1) + static_cast<ptrdiff_t>(n - g.b_split) * ldb_b;
        xsrc = row + k0 + c * 16;
    }
    auto issue_x = [&](int kt, int slot) __attribute__((always_inline)) {
        if constexpr (XR > 0) {
            if (wave == 0) big::copy16_to_lds(xsrc + kphys(kt) * KB, smem + slot * SH::STAGE + (BM + BN) * KB);
        }
    };
    // Copy rounds [R0, R1) of stage kt into `slot`.
    auto issue_part = [&](int kt, int slot, auto r0_c, auto r1_c) __attribute__((always_inline)) {
        constexpr int R0 = decltype(r0_c)::value, R1 = decltype(r1_c)::value;
        char* dst = smem + slot * SH::STAGE + wave * 1024;
        const int koff = kphys(kt) * KB;
        static_for<R1 - R0>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = R0 + decltype(i_c)::value;
            big::copy16_to_lds(src[i] + koff, dst + i * SH::RROWS * KB);
        });
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
        issue_part(kt, slot, std::integral_constant<int, 0>{}, std::integral_constant<int, ROUNDS>{});
    };

    // LDS read offsets of this lane's operands: row (l % 32) of each 32-row fragment,
    // logical 16-byte chunk 2*ks + l/32 (MXFP8: chunks 4*ks + l/32 and 4*ks + 2 + l/32).
    const int lr = lane & 31, lh = lane >> 5;
    int a_rd[KS][RPK], b_rd[KS][RPK];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h = 0; h < RPK; ++h) {
            const int logical = MX ? 4 * ks + 2 * h + lh : 2 * ks + lh;
            const int chunk = (logical ^ big::swz<KB>(lr)) * 16;
            a_rd[ks][h] = (wm * TM + lr) * KB + chunk;
            b_rd[ks][h] = (BM + wn * TN + lr) * KB + chunk;
        }

    // MXFP8 block scales: per stage, one 32-bit word per fragment row holding the E8M0
    // bytes of its four 32-value blocks, loaded a stage ahead into registers; shifted by
    // 8 (l / 32) so that byte 2*ks is this lane's block of k-step ks.
    const uint8_t* a_sp[MX ? FM : 1];
    const uint8_t* b_sp[MX ? FN : 1];
    uint32_t sx[MX ? FM : 1], sw[MX ? FN : 1], sx_n[MX ? FM : 1], sw_n[MX ? FN : 1];
    if constexpr (MX) {
        const size_t srow = static_cast<size_t>(g.K / 32);
        const size_t kblk = k0 / 32;
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            const int m = min(m0 + wm * TM + 32 * i + lr, g.M - 1);
            a_sp[i] = g.a_mx + static_cast<size_t>(m) * srow + kblk;
        });
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            const int n = b_row(g, min(n0 + wn * TN + 32 * j + lr, g.N - 1));
            b_sp[j] = n < g.b_split ? g.b_mx0 + static_cast<ptrdiff_t>(n) * static_cast<ptrdiff_t>(srow) + kblk
                                    : g.b_mx1 + static_cast<ptrdiff_t>(n - g.b_split) * static_cast<ptrdiff_t>(srow) + kblk;
        });
    }
    auto load_scales = [&](int kt) __attribute__((always_inline)) {
        if constexpr (MX) {
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                sx_n[i] = *reinterpret_cast<const uint32_t*>(a_sp[i] + 4 * kphys(kt));
            });
            static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int j = decltype(j_c)::value;
                sw_n[j] = *reinterpret_cast<const uint32_t*>(b_sp[j] + 4 * kphys(kt));
            });
        }
    };
    auto take_scales = [&]() __attribute__((always_inline)) {
        if constexpr (MX) {
            static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                sx[i] = sx_n[i] >> (8 * lh);
            });
            static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int j = decltype(j_c)::value;
                sw[j] = sw_n[j] >> (8 * lh);
            });
        }
    };

    // kStoreBf16X operands, 16 x 16 MFMA layout (mma16x16): the XR extra weight rows as
    // the first operand (lanes with l % 16 >= 8 repeat rows 0..7; those result rows are
    // dropped) and this wave's 32 tokens wm TM + 32 wn + [0, 32) as two 16-token groups, for
    // the two 32-deep halves of a stage; 16-byte chunk 4 h + l / 16 of each row.
    int xw_rd[2] = {0, 0}, xx_rd[2][2] = {{0, 0}, {0, 0}};
    using XAcc = typename std::conditional<kIsI8<Tin>, i32x4, f32x4>::type;
    XAcc acc_x[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    i32x4 xw[2], xx[2][2];
    if constexpr (XR > 0) {
        const int xq = lane & 15, xk = lane >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int wr = BM + BN + (xq & 7);
            xw_rd[h] = wr * KB + ((4 * h + xk) ^ big::swz<KB>(wr)) * 16;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const int xr = wm * TM + 32 * wn + 16 * gi + xq;
                xx_rd[gi][h] = xr * KB + ((4 * h + xk) ^ big::swz<KB>(xr)) * 16;
            }
        }
    }
    auto xread = [&](const char* base) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            xw[h] = *reinterpret_cast<const i32x4*>(base + xw_rd[h]);
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) xx[gi][h] = *reinterpret_cast<const i32x4*>(base + xx_rd[gi][h]);
        }
    };
    auto xmultiply = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) acc_x[gi] = big::mma16x16(xw[h], xx[gi][h], acc_x[gi]);
    };

    typename Op::acc_t acc[FN][FM];
    static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            acc[decltype(j_c)::value][decltype(i_c)::value] = Op::zero();
        });
    });

    // One k-step's operands: FN weight and FM activation fragments.
    using FragT = typename std::conditional<MX, i32x8, i32x4>::type;
    struct Frags {
        FragT w[FN], x[FM];
    };
    auto frag_at = [&](const char* p, const int (&rd)[RPK]) __attribute__((always_inline)) {
        if constexpr (MX) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(p + rd[0]);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(p + rd[1]);
            return FragT{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        } else {
            return *reinterpret_cast<const i32x4*>(p + rd[0]);
        }
    };
    auto read = [&](const char* base, auto ks_c, Frags& f) __attribute__((always_inline)) {
        constexpr int ks = decltype(ks_c)::value;
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            f.w[j] = frag_at(base + j * 32 * KB, b_rd[ks]);
        });
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            f.x[i] = frag_at(base + i * 32 * KB, a_rd[ks]);
        });
    };
    // Pin a k-step's operand fragments to VGPRs: left to itself the register allocator
    // may park them in AGPRs, which the accumulators fill. The pins sit at the head of a
    // k-step (an empty asm is an ordering point for memory instructions), so the reads
    // and copies after them stay free to interleave with the MFMAs.
    auto pin = [&](Frags& f) __attribute__((always_inline)) {
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
            big::pin_vgpr(f.w[decltype(j_c)::value]);
        });
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            big::pin_vgpr(f.x[decltype(i_c)::value]);
        });
    };
    // One MFMA (weight fragment idx / FM against activation fragment idx % FM) and one
    // fragment read (idx < FN: weight fragment idx, else activation fragment idx - FN).
    auto mma_one = [&](Frags& f, auto ks_c, auto idx_c) __attribute__((always_inline)) {
        constexpr int idx = decltype(idx_c)::value, j = idx / FM, i = idx % FM;
        if constexpr (MX)
            Op::template mma<2 * decltype(ks_c)::value>(acc[j][i], f.w[j], f.x[i], static_cast<int>(sw[j]),
                                                        static_cast<int>(sx[i]));
        else
            Op::mma(acc[j][i], f.w[j], f.x[i]);
    };
    auto read_one = [&](const char* base, auto ks_c, auto idx_c, Frags& f) __attribute__((always_inline)) {
        constexpr int ks = decltype(ks_c)::value, idx = decltype(idx_c)::value;
        if constexpr (idx < FN)
            f.w[idx] = frag_at(base + idx * 32 * KB, b_rd[ks]);
        else
            f.x[idx - FN] = frag_at(base + (idx - FN) * 32 * KB, a_rd[ks]);
    };

    // Stage j goes to slot j % S and is copied S - 1 stages ahead. The k-steps are written
    // as explicit slots: MFMA m, then the fragment reads and copy rounds that fall on slot
    // m, then a scheduling fence, so the order is the one written here. Every k-step first
    // waits for its own fragments (read during the previous k-step) and spreads the next
    // k-step's reads over its slots. The copies of stage kt + S - 1 go out one per slot over
    // the first CSPAN slots of stage kt: each 1 KB global_load_lds occupies the CU's
    // address unit for ~16 cycles, so a burst of them at the head of a stage stalls the
    // issuing wave (in-order issue) and with it the MFMA pipe; one per MFMA keeps the
    // copies early (two slots leave a stage to land) without that stall. The stage barrier
    // sits inside the last k-step after half of its MFMAs: it certifies that stage kt + 1
    // has landed for every wave (each wave first waits for its own copies) and that every
    // wave is done reading slot kt % S, which the copy issued in the next stage reuses; the
    // next stage's first reads then run under the second half.
    constexpr int NR = FN + FM, NM = FN * FM;
    constexpr int PRE = (KS - 1) * NM + NM / 2;  // MFMA slots of a stage before its barrier
    constexpr int CSPAN = PRE < 8 ? PRE : 8;  // (small tiles put several copies on a slot)
    // MFMAs [M0, M0 + N) of k-step ks on fragments fc, stage slots G0 + [0, N); with RD the
    // NR reads of k-step rks's fragments from rbase into fn, spread over these slots; with
    // CP the copy rounds of stage ckt into ring slot cslot whose stage slot falls here.
    auto slots = [&](Frags& fc, auto ks_c, auto m0_c, auto n_c, auto g0_c, auto rd_c, const char* rbase, auto rks_c,
                     Frags& fn, auto cp_c, int ckt, int cslot) __attribute__((always_inline)) {
        constexpr int M0 = decltype(m0_c)::value, N = decltype(n_c)::value, G0 = decltype(g0_c)::value;
        constexpr bool RD = decltype(rd_c)::value, CP = decltype(cp_c)::value;
        const int koff = kphys(ckt) * KB;
        char* dst = smem + cslot * SH::STAGE + wave * 1024;
        static_for<N>([&](auto m_c) __attribute__((always_inline)) {
            constexpr int m = decltype(m_c)::value;
            mma_one(fc, ks_c, std::integral_constant<int, M0 + m>{});
            if constexpr (RD) {
                static_for<NR>([&](auto r_c) __attribute__((always_inline)) {
                    constexpr int r = decltype(r_c)::value;
                    if constexpr ((r * N) / NR == m) read_one(rbase, rks_c, r_c, fn);
                });
            }
            if constexpr (CP) {
                static_for<ROUNDS>([&](auto c_c) __attribute__((always_inline)) {
                    constexpr int c = decltype(c_c)::value;
                    if constexpr ((c * CSPAN) / ROUNDS == G0 + m)
                        big::copy16_to_lds(src[c] + koff, dst + c * SH::RROWS * KB);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // (the first stage's scales go out ahead of the copies, so the waits below cover them)
    if (nk > 0) load_scales(0);
    static_for<S - 1>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        if (s < nk) {
            issue(s, s);
            issue_x(s, s);
        }
    });
    Frags f[2];
    if (!M16 && nk > 0) {
        if (nk >= S - 1) big::wait_vmcnt<(S - 2) * ROUNDS>(); else big::wait_vmcnt<0>();
        big::lds_barrier();
        take_scales();
        read(smem, std::integral_constant<int, 0>{}, f[0]);
    }
    // MXFP8 k-step (the block-scaled tile: its 32-byte fragments in VGPRs beside 256 AGPRs
    // of accumulators leave no registers for the slot order, which spills there): the copy
    // share of this k-step at its head (with two ring slots the whole copy on k-step 0),
    // then the MFMAs, with scheduling groups that put one fragment read, then one copy,
    // after each MFMA.
    auto mma_range = [&](Frags& fc, auto ks_c, auto m0_c, auto n_c) __attribute__((always_inline)) {
        static_for<decltype(n_c)::value>([&](auto m_c) __attribute__((always_inline)) {
            mma_one(fc, ks_c, std::integral_constant<int, decltype(m0_c)::value + decltype(m_c)::value>{});
        });
    };
    auto groups = [&](auto n_c, auto nr_c, auto nc_c) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value, NRG = decltype(nr_c)::value, NCG = decltype(nc_c)::value;
        static_for<N>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if constexpr (i < NRG)
                __builtin_amdgcn_sched_group_barrier(0x100, RPK, 0);  // DS read(s)
            else if constexpr (i - NRG < NCG)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (the copy)
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    auto mx_kstep = [&](int kt, auto ks_c, const char* base, int cslot, int nslot, auto cp_c) __attribute__((always_inline)) {
        constexpr int ks = decltype(ks_c)::value;
        constexpr int SPREAD = S == 2 ? 1 : KS;
        constexpr int r0 = ks < SPREAD ? ROUNDS * ks / SPREAD : ROUNDS;
        constexpr int r1 = ks < SPREAD ? ROUNDS * (ks + 1) / SPREAD : ROUNDS;
        constexpr int NC = decltype(cp_c)::value ? r1 - r0 : 0;
        using I0 = std::integral_constant<int, 0>;
        if constexpr (NC > 0)
            issue_part(kt + S - 1, cslot, std::integral_constant<int, r0>{}, std::integral_constant<int, r1>{});
        if constexpr (ks + 1 < KS) {
            read(base, std::integral_constant<int, ks + 1>{}, f[(ks + 1) & 1]);
            mma_range(f[ks & 1], ks_c, I0{}, std::integral_constant<int, NM>{});
            groups(std::integral_constant<int, NM>{}, std::integral_constant<int, NR>{}, std::integral_constant<int, NC>{});
        } else {
            mma_range(f[ks & 1], ks_c, I0{}, std::integral_constant<int, NM / 2>{});
            groups(std::integral_constant<int, NM / 2>{}, I0{}, std::integral_constant<int, NC>{});
            const bool more = kt + 1 < nk;
            if (more) {
                if (decltype(cp_c)::value) big::wait_vmcnt<(S - 2) * ROUNDS>(); else big::wait_vmcnt<0>();
                big::lds_barrier();
            }
            __builtin_amdgcn_sched_barrier(0);
            if (more) read(smem + nslot * SH::STAGE, I0{}, f[(ks + 1) & 1]);
            mma_range(f[ks & 1], ks_c, std::integral_constant<int, NM / 2>{}, std::integral_constant<int, NM - NM / 2>{});
            groups(std::integral_constant<int, NM - NM / 2>{}, std::integral_constant<int, NR>{}, I0{});
        }
    };
    int slot = 0;  // kt % S
    auto stage = [&](int kt, auto copy_c) __attribute__((always_inline)) {
        using CP = std::integral_constant<bool, decltype(copy_c)::value>;
        using T_ = std::true_type;
        using F_ = std::false_type;
        using I0 = std::integral_constant<int, 0>;
        using IH = std::integral_constant<int, NM / 2>;
        using IR = std::integral_constant<int, NM - NM / 2>;
        using INONE = std::integral_constant<int, PRE>;  // stage slots past every copy
        const int cslot = slot == 0 ? S - 1 : slot - 1;
        const int nslot = slot + 1 == S ? 0 : slot + 1;
        const char* base = smem + slot * SH::STAGE;
        if constexpr (CP::value) issue_x(kt + S - 1, cslot);  // extra rows (the stage-end wait covers them)
        // the next stage's scales, ahead of this stage's copies (the stage-end wait covers them)
        if (kt + 1 < nk) load_scales(kt + 1);
        static_for<KS>([&](auto ks_c) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_c)::value;
            using G0 = std::integral_constant<int, ks * NM>;
            big::wait_lgkmcnt0();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (XR > 0 && ks == 1) {
                xread(base);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (XR > 0 && ks == 2) {
                xmultiply();
                __builtin_amdgcn_sched_barrier(0);
            }
            pin(f[ks & 1]);
            if constexpr (MX) {
                mx_kstep(kt, ks_c, base, cslot, nslot, CP{});
            } else if constexpr (ks + 1 < KS) {
                slots(f[ks & 1], ks_c, I0{}, std::integral_constant<int, NM>{}, G0{}, T_{}, base,
                      std::integral_constant<int, ks + 1>{}, f[(ks + 1) & 1], CP{}, kt + S - 1, cslot);
            } else {
                slots(f[ks & 1], ks_c, I0{}, IH{}, G0{}, F_{}, base, I0{}, f[(ks + 1) & 1], CP{}, kt + S - 1, cslot);
                const bool more = kt + 1 < nk;
                if (more) {
                    if (CP::value) big::wait_vmcnt<(S - 2) * ROUNDS>(); else big::wait_vmcnt<0>();
                    big::lds_barrier();
                }
                __builtin_amdgcn_sched_barrier(0);
                if (more)
                    slots(f[ks & 1], ks_c, IH{}, IR{}, INONE{}, T_{}, smem + nslot * SH::STAGE, I0{}, f[(ks + 1) & 1],
                          F_{}, kt, cslot);
                else
                    slots(f[ks & 1], ks_c, IH{}, IR{}, INONE{}, F_{}, base, I0{}, f[(ks + 1) & 1], F_{}, kt, cslot);
            }
        });
        take_scales();  // the next stage's (its loads were covered by the stage-end wait)
        slot = nslot;
    };
    if constexpr (M16) {
        // 16 x 16 x 32 MFMAs (mma16x16). A k-step is 32 of K (64 bytes of every row); a
        // 32-row fragment unit is two 16-row sub-fragments, lane l reading row 16 s + l % 16,
        // logical chunk 4 ks + l / 16 (the swizzle of row l % 16 holds for every unit and
        // half). Block (sj, si) of unit (j, i), weight half sj times token half si, lives in
        // registers 4 (2 si + sj) + [0, 4) of acc[j][i]: lane l holds token
        // 32 i + 16 si + l % 16 and columns 32 j + 16 sj + 4 (l / 16) + [0, 4).
        // A k-step's 32 MFMAs go weight sub-fragment by weight sub-fragment, each against
        // the four token sub-fragments; the weight sub-fragments stream through a ring of
        // LEAD + 1 registers, each read LEAD sub-fragments (4 LEAD MFMAs) ahead of its
        // first use, into the registers of the one whose last use just passed, so a k-step
        // holds four of its eight at a time; the token sub-fragments of the next k-step are
        // read during this one (two sets). Slots as in the 32 x 32 form: MFMA m, the reads
        // and copy rounds that fall on it, a scheduling fence. The stage barrier follows the
        // slot that reads the stage's last weight sub-fragment; the next stage's first reads
        // come after it.
        constexpr int XS = 2 * FM;         // token sub-fragments per k-step
        constexpr int WS = 2 * FN;         // weight sub-fragments per k-step
        constexpr int KS2 = KB / 64;       // k-steps per stage
        constexpr int MK = WS * XS;        // MFMAs per k-step
        constexpr int MS = KS2 * MK;       // MFMAs per stage
        constexpr int NWS = KS2 * WS;      // weight sub-fragments per stage
        constexpr int LEAD = 3;
        constexpr int RING = LEAD + 1;
        constexpr int PRE16 = (NWS - 1 - LEAD) * XS + 1;  // slots up to the last read of the stage
        static_assert(XS == 4 && KS2 == 2 && NWS % RING == 0 && ROUNDS <= PRE16 && PRE16 + XS <= MS && S == 2,
                      "schedule written for the 4 x 2 wave tile and a two-slot ring");
        const int lq = lane >> 4, l16 = lane & 15;
        int wo[KS2][2], xo[KS2][2];
#pragma unroll
        for (int k2 = 0; k2 < KS2; ++k2)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int chunk = ((4 * k2 + lq) ^ big::swz<KB>(l16)) * 16;
                wo[k2][h] = (BM + wn * TN + 16 * h + l16) * KB + chunk;
                xo[k2][h] = (wm * TM + 16 * h + l16) * KB + chunk;
            }
        i32x4 xa[2][XS];  // [k-step parity][2 i + si]
        i32x4 wr[RING];   // weight sub-fragment n of a stage (n = WS k-step + 2 j + sj) in wr[n % RING]
        auto read_w = [&](const char* base, auto n_c) __attribute__((always_inline)) {
            constexpr int n = decltype(n_c)::value, k2 = n / WS, ws = n % WS;
            wr[n % RING] = *reinterpret_cast<const i32x4*>(base + (ws >> 1) * 32 * KB + wo[k2][ws & 1]);
        };
        auto read_x = [&](const char* base, auto k2_c, auto q_c) __attribute__((always_inline)) {
            constexpr int k2 = decltype(k2_c)::value, q = decltype(q_c)::value;
            xa[k2 & 1][q] = *reinterpret_cast<const i32x4*>(base + (q >> 1) * 32 * KB + xo[k2][q & 1]);
        };
        auto mma16 = [&](auto m_c) __attribute__((always_inline)) {
            constexpr int m = decltype(m_c)::value, k2 = m / MK, ws = (m % MK) / XS, q = m % XS;
            constexpr int j = ws >> 1, i = q >> 1, b = 2 * (q & 1) + (ws & 1);
            f32x4 t = {acc[j][i][4 * b], acc[j][i][4 * b + 1], acc[j][i][4 * b + 2], acc[j][i][4 * b + 3]};
            t = big::mma16x16(wr[(k2 * WS + ws) % RING], xa[k2 & 1][q], t);
            acc[j][i][4 * b] = t[0];
            acc[j][i][4 * b + 1] = t[1];
            acc[j][i][4 * b + 2] = t[2];
            acc[j][i][4 * b + 3] = t[3];
        };
        // slots [LO, HI) of a stage; NX: the next stage's first reads (from nbase) after the
        // barrier; CP: the copy rounds of stage ckt into ring slot cslot, one per slot
        auto slots16 = [&](auto lo_c, auto hi_c, auto nx_c, auto cp_c, const char* base, const char* nbase, int ckt,
                           int cslot) __attribute__((always_inline)) {
            constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
            constexpr bool NX = decltype(nx_c)::value, CP = decltype(cp_c)::value;
            const int koff = kphys(ckt) * KB;
            char* dst = smem + cslot * SH::STAGE + wave * 1024;
            static_for<HI - LO>([&](auto k_c) __attribute__((always_inline)) {
                constexpr int m = LO + decltype(k_c)::value;
                mma16(std::integral_constant<int, m>{});
                __builtin_amdgcn_sched_barrier(0);  // the slot's reads after its MFMA
                if constexpr (m % XS == 0 && m < PRE16 && m / XS + LEAD < NWS)
                    read_w(base, std::integral_constant<int, m / XS + LEAD>{});
                if constexpr (m < MK && m % XS == 2 && m / XS < XS)  // the second k-step's tokens
                    read_x(base, std::integral_constant<int, 1>{}, std::integral_constant<int, m / XS>{});
                if constexpr (NX && m >= PRE16) {
                    if constexpr (m - PRE16 < XS)
                        read_x(nbase, std::integral_constant<int, 0>{}, std::integral_constant<int, m - PRE16>{});
                    if constexpr (m % XS == 0 && m / XS + LEAD >= NWS)
                        read_w(nbase, std::integral_constant<int, m / XS + LEAD - NWS>{});
                }
                if constexpr (CP) {
                    static_for<ROUNDS>([&](auto c_c) __attribute__((always_inline)) {
                        constexpr int c = decltype(c_c)::value;
                        if constexpr (c == m) big::copy16_to_lds(src[c] + koff, dst + c * SH::RROWS * KB);
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        using I0 = std::integral_constant<int, 0>;
        using IP = std::integral_constant<int, PRE16>;
        using IE = std::integral_constant<int, MS>;
        auto stage16 = [&](int kt, auto cp_c) __attribute__((always_inline)) {
            using CP = std::integral_constant<bool, decltype(cp_c)::value>;
            const int cslot = slot == 0 ? S - 1 : slot - 1;
            const int nslot = slot + 1 == S ? 0 : slot + 1;
            const char* base = smem + slot * SH::STAGE;
            const char* nbase = smem + nslot * SH::STAGE;
            // with a two-slot ring the stages that copy ahead are exactly those another stage
            // follows: the loops below pass that as a constant, so the steady-state stage has
            // no branch and the compiler's LDS wait counts stay exact across iterations
            slots16(I0{}, IP{}, F_{}, CP{}, base, nbase, kt + S - 1, cslot);
            if constexpr (CP::value) {
                big::wait_vmcnt<0>();
                big::lds_barrier();
            }
            __builtin_amdgcn_sched_barrier(0);
            slots16(IP{}, IE{}, CP{}, F_{}, base, nbase, kt, cslot);
            slot = nslot;
        };
        if (nk > 0) {
            if (nk >= S - 1) big::wait_vmcnt<(S - 2) * ROUNDS>(); else big::wait_vmcnt<0>();
            big::lds_barrier();
            static_for<XS>([&](auto q_c) __attribute__((always_inline)) { read_x(smem, I0{}, q_c); });
            static_for<LEAD>([&](auto n_c) __attribute__((always_inline)) { read_w(smem, n_c); });
        }
        int kt = 0;
        for (; kt + S - 1 < nk; ++kt) stage16(kt, std::true_type{});
        for (; kt < nk; ++kt) stage16(kt, std::false_type{});
    } else {
        int kt = 0;
        for (; kt + S - 1 < nk; ++kt) stage(kt, std::true_type{});
        for (; kt < nk; ++kt) {
            if (EARLY && kt + 1 == nk) rope_ops.gather(g, lh);  // lands under the last stage's MFMAs
            stage(kt, std::false_type{});
        }
        if (EARLY && nk == 0) rope_ops.gather(g, lh);
    }

    tile_epilogue<Tin, BM, BN, WM, WN, EPI, EARLY, M16>(g, acc, smem, scl, m0, n0, n_tile, split, rope_ops);
    if constexpr (XR > 0) {
        // lane l < 32 holds extra columns 4 (l / 16) + [0, 4) of token l % 16 of each group;
        // W8A8 dequantises them like the tile, f32(acc) * (a_scale[m] * b_scale[n])
        if (lane < 32) {
            uint16_t* out = static_cast<uint16_t*>(g.out);
            const int col = g.N + XR * n_tile + 4 * (lane >> 4);
            MLAP_CHECK(g.dbg, col + 4 <= g.ldo, kDbgStore);
            float bs[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (kIsI8<Tin>) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nn = b_row(g, col + q);
                    bs[q] = nn < g.b_split ? g.b_scale0[nn] : g.b_scale1[nn - g.b_split];
                }
            }
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const int m = m0 + wm * TM + 32 * wn + 16 * gi + (lane & 15);
                if (m < g.M) {
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (kIsI8<Tin>) {
                            const float sc = g.a_scale[m] * bs[q];
                            v[q] = static_cast<float>(acc_x[gi][q]) * sc;
                        } else {
                            v[q] = acc_x[gi][q];
                        }
                    }
                    *reinterpret_cast<uint2*>(out + static_cast<size_t>(m) * g.ldo + col) =
                        make_uint2(big::pack_bf16x2(v[0], v[1]), big::pack_bf16x2(v[2], v[3]));
                }
            }
        }
    }
    if (g.clk && threadIdx.x == 0 && (blockIdx.x & 15) == 0) {
        atomicAdd(g.clk, clock64() - clk0);
        atomicAdd(g.clk + 1, wall_clock64() - wall0);
    }
}

}  // namespace mlap
