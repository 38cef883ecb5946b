// gemm.hpp -- GEMM arguments, tile order and MFMA wrappers shared by the GEMM kernels,
// and the register-staged MFMA GEMM for gfx950, C = A . B^T with A [M,K], B [N,K], which
// serves the int8 small-batch projections, the test exports and shapes the LDS-DMA kernel
// (gemm_big.hpp) does not cover.
//
// Both operands are K-contiguous (activations [T, K], weights [N, K] as the
// AT-10 card's b_trans layout), so every lane fetches 16-byte runs along K for
// both MFMA operands and no transpose is needed anywhere.
//
// One K-tile is 128 bytes of every row: 64 bf16 or 128 int8. The tile is read
// from HBM into registers (16-byte loads, 8 lanes per 128-byte row segment),
// written to LDS with a 16-byte row pad (rows 144 bytes apart, so the 128-bit
// LDS reads of consecutive rows hit distinct banks), and consumed by
// v_mfma_f32_32x32x16_bf16 or v_mfma_i32_32x32x32_i8: each instruction eats 32
// bytes of K per row, so a K-tile is four MFMA k-steps for either type. The
// next K-tile is fetched into registers while the current one is multiplied.
//
// Accumulator layout of a 32x32 MFMA block (lane l, register r in 0..15):
// column l % 32, row 8*(r/4) + 4*(l/32) + r%4.
//
// Epilogues: bf16 store, fp32 split-K partial store, int32 store (test export),
// and the per-head epilogue of the up projection (split into two segments per
// head, rotate-half RoPE of the second, per-tile partial row amax for the
// per-token INT8 quant). The bf16 cast happens once, when accumulators are
// staged to LDS, which is exactly the GEMM's bf16 output cast point.
#pragma once

#include "common.hpp"

namespace mlap {

// kStoreBf16X: kStoreBf16 for the BN tile columns plus eight extra columns per column
// tile, g.N + 8 n_tile + [0, 8), from the weight rows of the same index (the 256 x 256 bf16
// tile only): a narrow column slice that rides on the operand rows already staged.
enum class Epi : int { kStoreBf16 = 0, kStoreF32 = 1, kStoreI32 = 2, kHeads = 3, kStoreBf16X = 4 };

struct GemmArgs {
    int M, N, K;
    // A [M, lda] and B rows: row n < b_split comes from B0 + n*ldb, else B1 + (n-b_split)*ldb.
    const void* A;
    int lda;
    const void* B0;
    const void* B1;
    int b_split;
    int ldb;
    int k_splits;  // each split covers K/k_splits (kStoreF32 only)
    int group_m;   // M-tiles per group in the workgroup -> tile order
    int n_major;   // large-batch kernel: split the tile space over XCDs by N rather than M
                   // (each XCD then streams a 1/8 share of B and all of A)
    // W8A8 dequant: y = f32(acc) * (a_scale[m] * b_scale[n]); b_scale split like B.
    const float* a_scale;
    const float* b_scale0;
    const float* b_scale1;
    // plain stores: out [M, ldo] (kStoreF32: [k_splits][M][ldo])
    void* out;
    int ldo;
    // per-head epilogue
    int head_w, d0, d1, rope, n_heads;
    void* out0;  // [M, n_heads, d0] bf16
    void* out1;  // [M, n_heads, d1] bf16
    const int* positions;
    const float* cos;
    const float* sin;
    int max_pos;
    float* part_amax;  // [M, n_tiles] or null
    int n_tiles;
    // Rope slices read in de-interleaved order (pe_w > 0): in every period of pe_period
    // columns of the whole projection, columns [pe_off, pe_off + pe_w) take weight rows
    // pe_off + 2i (first half, i < pe_w/2) and pe_off + 2i + 1 (second half) of their
    // period, so the output holds the slice of the interleaved-pair layout split into its
    // halves. pe_c0: the projection column of this launch's column 0 (B, b_scale and out
    // are offset to it).
    int pe_period, pe_off, pe_w, pe_c0;
    // MXFP8 operands (E4M3 bytes in A and B): E8M0 block scales, one byte per 32 values
    // of K, rows of K/32 bytes: a_mx [M, K/32]; b_mx split like B (rows remapped like B).
    const uint8_t* a_mx;
    const uint8_t* b_mx0;
    const uint8_t* b_mx1;
    // Measurement (LDS-DMA kernel): when set, every 16th workgroup adds the shader-clock
    // cycles and the 100 MHz constant-clock ticks it ran for to clk[0] and clk[1] (a sample:
    // from every workgroup, the atomics on two addresses serialised and slowed launches of
    // a thousand one-wave workgroups from 15 to 37 us).
    unsigned long long* clk;
    unsigned int* dbg;  // debug build: bounds-check flags (see MLAP_CHECK), else null
};

// Weight row (and per-channel scale) feeding output column n of this launch, relative to
// its B base; a remapped row may lie outside the launch's own columns (a slice cut by the
// launch boundary) but stays in the slice, inside one weight segment.
__device__ __forceinline__ int b_row(const GemmArgs& g, int n) {
    if (g.pe_w == 0) return n;
    const int c = n + g.pe_c0;
    const int h = c / g.pe_period;
    const int d = c - h * g.pe_period - g.pe_off;
    if (d < 0 || d >= g.pe_w) return n;
    const int half = g.pe_w >> 1;
    return h * g.pe_period + g.pe_off + (d < half ? 2 * d : 2 * (d - half) + 1) - g.pe_c0;
}

// An OCP E4M3FN byte (the element type of the MXFP8 operands).
struct fp8e4m3 {
    uint8_t bits;
};

template <typename Tin>
constexpr bool kIsI8 = std::is_same<Tin, int8_t>::value;
template <typename Tin>
constexpr bool kIsMx = std::is_same<Tin, fp8e4m3>::value;

template <typename Tin>
struct MfmaOp;

// MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0). Operand
// layout (checked on gfx950): lane l holds row l % 32, its 32 bytes being K values
// 16 (l / 32) + [0, 16) and 32 + 16 (l / 32) + [0, 16) of the 64; the scale operand of
// lane l is the E8M0 byte of row l % 32 and 32-value block l / 32, taken from byte OPSEL
// of the 32-bit register. The products are exact and the hardware adds the 64 of them
// into the fp32 accumulator.
template <>
struct MfmaOp<fp8e4m3> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t zero() {
        acc_t z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
        return z;
    }
    template <int OPSEL>
    static __device__ __forceinline__ void mma(acc_t& c, const i32x8& a, const i32x8& b, int sa, int sb) {
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
    }
};

template <>
struct MfmaOp<uint16_t> {  // bf16
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t zero() {
        acc_t z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
        return z;
    }
    static __device__ __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x4& b) {
        bf16x8 av = __builtin_bit_cast(bf16x8, a);
        bf16x8 bv = __builtin_bit_cast(bf16x8, b);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
    }
};

template <>
struct MfmaOp<int8_t> {  // int8
    typedef i32x16 acc_t;
    static __device__ __forceinline__ acc_t zero() {
        acc_t z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0;
        return z;
    }
    static __device__ __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x4& b) {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

constexpr int kTileKBytes = 128;
constexpr int kLdsRow = kTileKBytes + 16;  // padded row pitch in bytes

// Tile geometry. BM x BN output tile per workgroup of WM x WN waves; each wave owns a
// (BM/WM) x (BN/WN) block of 32x32 MFMA fragments. P K-tiles are kept in flight in
// registers ahead of the one being multiplied; LDS holds two K-tiles.
template <int BM, int BN, int WM, int WN, int P>
struct TileShape {
    static constexpr int NT = kWave * WM * WN;
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int FM = TM / 32;
    static constexpr int FN = TN / 32;
    static constexpr int A_PER = BM * 8 / NT;  // 16-byte chunks per thread per K-tile
    static constexpr int B_PER = BN * 8 / NT;
    static constexpr int CH = A_PER + B_PER;
    static constexpr int STAGE_LDS = (BM + BN) * kLdsRow;
    static constexpr int MAIN_LDS = 2 * STAGE_LDS;
    static constexpr int EPI_ROWS = TM;                      // rows staged per epilogue pass
    static constexpr int EPI_PITCH = BN + 8;                 // bf16 elements per staged row
    static constexpr int EPI_LDS = EPI_ROWS * EPI_PITCH * 2 + EPI_ROWS * 4;
    static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32-aligned");
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile rows must split over threads");
    static_assert(P >= 1 && P <= 4, "prefetch depth");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Workgroup -> tile order. The hardware hands workgroup i to XCD i % 8; this makes
// each XCD own one contiguous range of the (split, tile) space, walked in groups of
// `group_m` M-tiles, so the workgroups that run together on an XCD share A and B
// rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int lin, int tiles_m, int tiles_n, int splits, int group_m,
                                        int& m_tile, int& n_tile, int& split) {
    const int total = tiles_m * tiles_n * splits;
    const int x = lin & 7, j = lin >> 3;
    const int q = total >> 3, r = total & 7;
    const int t2 = x * q + (x < r ? x : r) + j;
    const int tiles = tiles_m * tiles_n;
    split = t2 / tiles;
    const int t = t2 - split * tiles;
    const int gsz_full = group_m * tiles_n;
    const int grp = t / gsz_full;
    const int first_m = grp * group_m;
    const int gsz = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int within = t - grp * gsz_full;
    m_tile = first_m + within % gsz;
    n_tile = within / gsz;
}

// Per-head epilogue on one staged pass of rows [r0, r0+rows) of the tile.
// The staged tile holds the GEMM output already rounded to bf16.
template <int BM, int BN, int WM, int WN, int P>
__device__ __forceinline__ void heads_epilogue(const GemmArgs& g, const uint16_t* cs,
                                               uint32_t* row_amax, int m_base, int n0,
                                               int rows, int tid) {
    using S = TileShape<BM, BN, WM, WN, P>;
    const int HW = g.head_w, d0 = g.d0, d1 = g.d1;
    const int heads_in_tile = BN / HW;
    const int h0 = n0 / HW;
    const int c0 = d0 >> 3;
    const int half = d1 >> 1;
    const int c1 = g.rope ? (half >> 3) : (d1 >> 3);
    const int per_head = c0 + c1;
    const int items = rows * heads_in_tile * per_head;
    uint16_t* out0 = static_cast<uint16_t*>(g.out0);
    uint16_t* out1 = static_cast<uint16_t*>(g.out1);
    for (int it = tid; it < items; it += S::NT) {
        const int lr = it / (heads_in_tile * per_head);
        const int rem = it - lr * heads_in_tile * per_head;
        const int hh = rem / per_head;
        const int j = rem - hh * per_head;
        const int m = m_base + lr;
        const int h = h0 + hh;
        if (m >= g.M || h >= g.n_heads) continue;
        const uint16_t* src = cs + lr * S::EPI_PITCH + hh * HW;
        float amax;
        if (j < c0) {
            uint4 v = *reinterpret_cast<const uint4*>(src + j * 8);
            if (out0)
                *reinterpret_cast<uint4*>(out0 + (static_cast<size_t>(m) * g.n_heads + h) * d0 +
                                          j * 8) = v;
            amax = absmax8(v);
        } else if (g.rope) {
            const int i0 = (j - c0) * 8;
            const int p = clamp_pos(g.positions[m], g.max_pos);
            const float* cr = g.cos + static_cast<size_t>(p) * d1;
            const float* sr = g.sin + static_cast<size_t>(p) * d1;
            float x1[8], x2[8], lo[8], hi[8];
            unpack8(*reinterpret_cast<const uint4*>(src + d0 + i0), x1);
            unpack8(*reinterpret_cast<const uint4*>(src + d0 + half + i0), x2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // rotate_half(x) = (-x2, x1): out = x*cos + rotate_half(x)*sin
                float a = x1[e] * cr[i0 + e];
                float b = (-x2[e]) * sr[i0 + e];
                lo[e] = a + b;
                float c = x2[e] * cr[half + i0 + e];
                float d = x1[e] * sr[half + i0 + e];
                hi[e] = c + d;
            }
            uint4 vlo = pack8(lo), vhi = pack8(hi);
            if (out1) {
                uint16_t* dst = out1 + (static_cast<size_t>(m) * g.n_heads + h) * d1;
                *reinterpret_cast<uint4*>(dst + i0) = vlo;
                *reinterpret_cast<uint4*>(dst + half + i0) = vhi;
            }
            amax = fmaxf(absmax8(vlo), absmax8(vhi));
        } else {
            const int i0 = (j - c0) * 8;
            uint4 v = *reinterpret_cast<const uint4*>(src + d0 + i0);
            if (out1)
                *reinterpret_cast<uint4*>(out1 + (static_cast<size_t>(m) * g.n_heads + h) * d1 +
                                          i0) = v;
            amax = absmax8(v);
        }
        if (g.part_amax) atomicMax(row_amax + lr, __float_as_uint(amax));
    }
}

template <typename Tin, int BM, int BN, int WM, int WN, int P, Epi EPI>
__global__ __launch_bounds__(kWave* WM* WN) void gemm_nt_kernel(GemmArgs g) {
    using S = TileShape<BM, BN, WM, WN, P>;
    using Op = MfmaOp<Tin>;
    __shared__ __attribute__((aligned(16))) char smem[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int tiles_m = (g.M + BM - 1) / BM;
    const int tiles_n = (g.N + BN - 1) / BN;
    int m_tile, n_tile, split;
    tile_of(blockIdx.x, tiles_m, tiles_n, g.k_splits, g.group_m, m_tile, n_tile, split);
    const int m0 = m_tile * BM;
    const int n0 = n_tile * BN;

    const int kbytes_split = g.K * static_cast<int>(sizeof(Tin)) / g.k_splits;
    const int n_ktiles = kbytes_split / kTileKBytes;
    const size_t lda_b = static_cast<size_t>(g.lda) * sizeof(Tin);
    const size_t ldb_b = static_cast<size_t>(g.ldb) * sizeof(Tin);

    // Workgroup-uniform row bases (the host keeps every B tile inside one segment) and
    // per-thread row/chunk coordinates. Thread t copies 16-byte chunk (t % 8) of rows
    // t/8 + i*NT/8. Rows past the matrix edge re-read its last row: their results land
    // in tile rows/columns that are never stored.
    const char* a_base = static_cast<const char*>(g.A) + static_cast<size_t>(m0) * lda_b +
                         static_cast<size_t>(split) * kbytes_split;
    const bool seg0 = n0 < g.b_split;
    const char* b_base = (seg0 ? static_cast<const char*>(g.B0) + static_cast<size_t>(n0) * ldb_b
                               : static_cast<const char*>(g.B1) +
                                     static_cast<size_t>(n0 - g.b_split) * ldb_b) +
                         static_cast<size_t>(split) * kbytes_split;
    const int a_last = g.M - 1 - m0;
    const int b_last = g.N - 1 - n0;
    const int row0 = tid >> 3;
    const int cc16 = (tid & 7) * 16;
    constexpr int R8 = S::NT / 8;  // rows covered by one pass of the workgroup
    const uint32_t lda32 = static_cast<uint32_t>(lda_b);
    // byte offsets of this thread's B rows from b_base (signed: a row remapped for a
    // de-interleaved rope slice may come from outside the tile)
    int64_t b_off[S::CH > S::A_PER ? S::CH - S::A_PER : 1];
    static_for<S::CH - S::A_PER>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        const int r = row0 + i * R8;
        const int n = n0 + (r < b_last ? r : b_last);
        b_off[i] = static_cast<int64_t>(b_row(g, n) - n0) * static_cast<int64_t>(ldb_b) + cc16;
    });

    i32x4 pre[P][S::CH];
    auto fetch = [&](int kt, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        const char* ap = a_base + kt * kTileKBytes;
        const char* bp = b_base + kt * kTileKBytes;
        static_for<S::CH>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            if constexpr (i < S::A_PER) {
                const int r = row0 + i * R8;
                const uint32_t off = static_cast<uint32_t>(r < a_last ? r : a_last) * lda32 + cc16;
                pre[slot][i] = *reinterpret_cast<const i32x4*>(ap + off);
            } else {
                pre[slot][i] = *reinterpret_cast<const i32x4*>(bp + b_off[i - S::A_PER]);
            }
        });
    };
    const int lds_w = row0 * kLdsRow + cc16;
    auto stash = [&](auto slot_c, int buf) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        char* base = smem + buf * S::STAGE_LDS + lds_w;
        static_for<S::CH>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            constexpr int off = (i < S::A_PER) ? i * R8 * kLdsRow
                                               : (BM + (i - S::A_PER) * R8) * kLdsRow;
            *reinterpret_cast<i32x4*>(base + off) = pre[slot][i];
        });
    };

    typename Op::acc_t acc[S::FM][S::FN];
    static_for<S::FM>([&](auto i_c) __attribute__((always_inline)) {
        static_for<S::FN>([&](auto j_c) __attribute__((always_inline)) {
            acc[decltype(i_c)::value][decltype(j_c)::value] = Op::zero();
        });
    });

    // LDS read offsets of this lane's MFMA operands (row l%32, 16-byte half l/32).
    const int a_rd = (wm * S::TM + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
    const int b_rd = BM * kLdsRow + (wn * S::TN + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const char* base = smem + buf * S::STAGE_LDS;
        static_for<4>([&](auto ks_c) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_c)::value;
            i32x4 af[S::FM], bfr[S::FN];
            static_for<S::FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                af[i] = *reinterpret_cast<const i32x4*>(base + a_rd + i * 32 * kLdsRow + ks * 32);
            });
            static_for<S::FN>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int j = decltype(j_c)::value;
                bfr[j] = *reinterpret_cast<const i32x4*>(base + b_rd + j * 32 * kLdsRow + ks * 32);
            });
            static_for<S::FM>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                static_for<S::FN>([&](auto j_c) __attribute__((always_inline)) {
                    constexpr int j = decltype(j_c)::value;
                    Op::mma(acc[i][j], af[i], bfr[j]);
                });
            });
        });
    };

    // K-tile j travels HBM -> registers (slot j % P) -> LDS buffer j % 2 -> MFMA.
    // (prologue loads are clamped to the last K-tile: always valid, never used past the end)
    static_for<P>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        fetch(s < n_ktiles ? s : n_ktiles - 1, s_c);
    });
    stash(std::integral_constant<int, 0>{}, 0);
    fetch(P < n_ktiles ? P : n_ktiles - 1, std::integral_constant<int, 0>{});
    __syncthreads();
    // Steady state without guards (every sub-step stashes and refills), so the compiler's
    // wait counts stay exact and P K-tiles really are in flight; then a guarded tail.
    int kt0 = 0;
    for (; kt0 + 2 * P < n_ktiles; kt0 += P) {
        static_for<P>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            constexpr int nslot = (s + 1) % P;
            const int kt = kt0 + s;
            compute(kt & 1);
            stash(std::integral_constant<int, nslot>{}, (kt + 1) & 1);
            fetch(kt + 1 + P, std::integral_constant<int, nslot>{});
            __syncthreads();
        });
    }
    for (; kt0 < n_ktiles; kt0 += P) {
        static_for<P>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            constexpr int nslot = (s + 1) % P;
            const int kt = kt0 + s;
            if (kt < n_ktiles) {
                compute(kt & 1);
                if (kt + 1 < n_ktiles) stash(std::integral_constant<int, nslot>{}, (kt + 1) & 1);
                if (kt + 1 + P < n_ktiles) fetch(kt + 1 + P, std::integral_constant<int, nslot>{});
                __syncthreads();
            }
        });
    }

    // ------------------------------------------------------------- epilogues --
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);

    if constexpr (EPI == Epi::kStoreI32 || EPI == Epi::kStoreF32) {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * S::TM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                    const int n = n0 + wn * S::TN + j * 32 + col_l;
                    if (m < g.M && n < g.N) {
                        if constexpr (EPI == Epi::kStoreI32) {
                            static_cast<int32_t*>(g.out)[static_cast<size_t>(m) * g.ldo + n] = acc[i][j][r];
                        } else {
                            static_cast<float*>(g.out)[(static_cast<size_t>(split) * g.M + m) * g.ldo + n] =
                                acc[i][j][r];
                        }
                    }
                }
        return;
    } else {
        uint16_t* cs = reinterpret_cast<uint16_t*>(smem);
        uint32_t* row_amax = reinterpret_cast<uint32_t*>(smem + S::EPI_ROWS * S::EPI_PITCH * 2);
        for (int pass = 0; pass < WM; ++pass) {
            // stage rows [pass*TM, pass*TM + TM) of the tile as bf16
            if (wm == pass) {
#pragma unroll
                for (int i = 0; i < S::FM; ++i)
#pragma unroll
                    for (int j = 0; j < S::FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int lr = i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                            const int lc = wn * S::TN + j * 32 + col_l;
                            float v;
                            if constexpr (sizeof(Tin) == 1) {
                                const int m = m0 + pass * S::TM + lr;
                                const int n = b_row(g, n0 + lc);
                                const float as = (m < g.M) ? g.a_scale[m] : 0.f;
                                const float bs = (n0 + lc < g.N) ? ((n < g.b_split) ? g.b_scale0[n]
                                                                                   : g.b_scale1[n - g.b_split])
                                                                : 0.f;
                                const float sc = as * bs;
                                v = static_cast<float>(acc[i][j][r]) * sc;
                            } else {
                                v = acc[i][j][r];
                            }
                            cs[lr * S::EPI_PITCH + lc] = f2bf(v);
                        }
            }
            if (tid < S::EPI_ROWS) row_amax[tid] = 0u;
            __syncthreads();
            const int m_base = m0 + pass * S::TM;
            if constexpr (EPI == Epi::kStoreBf16) {
                constexpr int CPR = BN / 8;  // 16-byte chunks per row
                uint16_t* out = static_cast<uint16_t*>(g.out);
                for (int c = tid; c < S::EPI_ROWS * CPR; c += S::NT) {
                    const int lr = c / CPR, cc = c % CPR;
                    const int m = m_base + lr, n = n0 + cc * 8;
                    if (m < g.M && n < g.N)  // N is a multiple of 8
                        *reinterpret_cast<uint4*>(out + static_cast<size_t>(m) * g.ldo + n) =
                            *reinterpret_cast<const uint4*>(cs + lr * S::EPI_PITCH + cc * 8);
                }
            } else {
                heads_epilogue<BM, BN, WM, WN, P>(g, cs, row_amax, m_base, n0, S::EPI_ROWS, tid);
                if (g.part_amax) {
                    __syncthreads();
                    if (tid < S::EPI_ROWS && m_base + tid < g.M)
                        g.part_amax[static_cast<size_t>(m_base + tid) * g.n_tiles + n_tile] =
                            __uint_as_float(row_amax[tid]);
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace mlap
