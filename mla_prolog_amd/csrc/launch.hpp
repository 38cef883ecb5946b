// launch.hpp -- host-side launch interface of the gfx950 MLA Prolog kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace mlap {

// The debug build's bounds-check word on the current device (null in release builds); every
// launcher passes it to its kernels.
unsigned int* debug_word();


enum class InType : int { kBf16 = 0, kInt8 = 1, kFp8 = 2 };  // kFp8: MXFP8 (E4M3 + E8M0 block scales)

// Output tile rows x columns and K-tiles of register prefetch.
struct GemmTile {
    int bm, bn, prefetch;
};

// Launch C = A . B^T with the given tile shape and epilogue on a 1-D grid of
// tiles x k_splits workgroups. The B operand's segment split (b_split) must be a
// multiple of the tile width or >= N. Returns hipErrorInvalidValue for a
// (type, tile, epilogue) combination that has no instantiation.
hipError_t launch_gemm(const GemmArgs& g, InType t, const GemmTile& tile, Epi epi, hipStream_t s);

// LDS-DMA GEMM (gemm_big.hpp) in four shapes (the bf16 ones also on MXFP8 E4M3 operands):
//   kWide        -- 256 x 256 tiles, eight waves (large batches, MFMA-bound; four waves of
//                   128 x 128 with MXFP8); kStoreBf16 and
//                   kHeads (head width and d0 multiples of 64, a 64-wide rope slice);
//   kHalfHead    -- 96-column tiles: one per half of a 192-wide q head, the whole batch in
//                   one tile row (bf16, kHeads);
//   kSplitK      -- 64-column tiles, split-K fp32 partials (bf16, kStoreF32);
//   kNarrowHeads -- 32-column tiles that stay inside one head segment, no rope (bf16,
//                   kHeads; the kv_b projection of small batches).
// The weight-streaming shapes (all but kWide) use 256-row tiles with four waves, or 64-row
// tiles with two waves when M <= 64. A ragged column remainder of a kWide kStoreBf16 launch
// runs on 64 x 64 tiles. With kHeads, g.n_tiles must be ceil(N / big_tile_n(shape)) (one
// partial amax per token and tile). gemm_big_fits says whether the shapes suit it (K a whole
// number of 128-byte stages per split).
enum class BigShape : int { kWide = 0, kHalfHead = 1, kSplitK = 2, kNarrowHeads = 3 };
constexpr int kBigTile = 256;
int big_tile_n(BigShape shape);
bool gemm_big_fits(const GemmArgs& g, InType t, Epi epi, BigShape shape = BigShape::kWide);
hipError_t launch_gemm_big(const GemmArgs& g, InType t, Epi epi, hipStream_t s,
                           BigShape shape = BigShape::kWide);

// Per-token row stage after the down projection: RMSNorm*gamma -> bf16 for the q and kv
// segments, rotate-half RoPE of the k_pe segment, per-token INT8 quant of kv_norm and (W8A8)
// of q_norm. One wave per token for large batches, one workgroup per token otherwise.
struct NormArgs {
    int T, Lq, Lkv, R, N1, k_splits;
    int rsqrt;  // RMSNorm variant A (sum, x 1/D, rsqrt) instead of B (x^2/D summed, sqrt, divide)
    const uint16_t* a_bf16;  // [T, N1] bf16 down-projection output, or
    const float* a_f32;      // [k_splits, T, N1] fp32 split-K partial sums (used when set)
    // Columns [tail_c0, N1) of the down projection, when set, come from their own split-K
    // fp32 partials [tail_splits, T, N1 - tail_c0] instead (tail_c0 a multiple of 8).
    const float* tail_f32;
    int tail_c0, tail_splits;
    const uint16_t* gamma_q;
    const uint16_t* gamma_kv;
    float eps;
    const int* positions;
    const float* cos;
    const float* sin;
    int max_pos;
    uint16_t* q_norm;    // [T, Lq] or null
    uint16_t* kv_norm;   // [T, Lkv] or null
    uint16_t* k_pe;      // [T, R] or null
    int8_t* kv_i8;       // [T, Lkv] or null
    float* kv_scale;     // [T] or null
    int8_t* kv_i8_b;     // second destination of the kv codes (W8A8 kv_b input) or null
    float* kv_scale_b;
    int8_t* qn_i8;       // [T, Lq] W8A8 activation codes of q_norm, or null
    float* qn_scale;     // [T]
    // KV cache rows: token t's kv_norm / codes and scale / k_pe also go to row slots[t] of
    // these when 0 <= slots[t] < n_slots (each pointer optional)
    const int* slots;
    int n_slots;
    uint16_t* kv_cache;     // [n_slots, Lkv]
    int8_t* kv_cache_i8;    // [n_slots, Lkv]
    float* kv_cache_scale;  // [n_slots]
    uint16_t* kr_cache;     // [n_slots, R]
    // diagnostic tap: the down-projection row as read, [T, N1] bf16 (rope slice in rotate-half
    // order), or null
    uint16_t* a_proj;
    unsigned int* dbg;  // debug build: bounds-check flags (set by the launcher)
};
hipError_t launch_norm(const NormArgs& a, hipStream_t s);

// Per-token dynamic INT8 quant of a bf16 matrix [T, K] (W8A8 activation quant of x).
hipError_t launch_act_quant(const uint16_t* x, int T, int K, int8_t* codes, float* scale,
                            hipStream_t s);

// Per-token INT8 quant of q = [q_nope | q_pe] per head, from the per-tile partial amax the
// up-projection epilogue wrote.
struct QuantQArgs {
    int T, H, Dn, R, n_tiles;
    const float* part_amax;   // [T, n_tiles]
    const uint16_t* q_nope;   // [T, H, Dn]
    const uint16_t* q_pe;     // [T, H, R]
    int8_t* q_i8;             // [T, H, Dn+R] or null
    float* q_scale;           // [T] or null; [T, H] with per_head
    int per_head;             // one scale per (token, head) instead of per token
    int parts;                // per-token quant: workgroups per token (set by the launcher)
    unsigned int* dbg;        // debug build: bounds-check flags (set by the launcher)
};
// Limits of the per-head q quant (one workgroup holds a token's row).
constexpr int kMaxQuantHeads = 1024;
constexpr int kQuantHeadChunks = 16;  // 16-byte chunks per thread: H*(Dn+R) <= 16*8*256
hipError_t launch_quant_q(const QuantQArgs& a, hipStream_t s);

// Per-head RMSNorm (no gamma) of q after the up projection, then rotate-half RoPE of each
// head's rope slice, in place on q_nope / q_pe (the raw projection output), and the token's
// |q| max as a single partial amax (the V4-shape prolog: q_b -> reshape to heads -> RMSNorm).
struct QHeadNormArgs {
    int T, H, Dn, R;
    float eps;
    int rsqrt;                // RMSNorm variant A instead of B
    const int* positions;
    const float* cos;
    const float* sin;
    int max_pos;
    uint16_t* q_nope;         // [T, H, Dn], in place
    uint16_t* q_pe;           // [T, H, R], in place
    float* part_amax;         // [T, groups] or null
    int groups;               // workgroups per token, each a whole-head share (H % groups == 0)
    uint16_t* q_proj;         // diagnostic tap: the raw heads as read, [T, H, Dn+R], or null
    unsigned int* dbg;        // debug build: bounds-check flags (set by the launcher)
};
// Limits of the per-head norm (one workgroup holds a token's q row): H*(Dn+R) <= 32768 and
// H*R <= 8192 (the rope chunks staged in LDS).
constexpr int kHeadNormChunks = 16;
constexpr int kHeadNormPeChunks = 1024;
hipError_t launch_q_head_norm(const QHeadNormArgs& a, hipStream_t s);

// MXFP8 operands for the bf16 MFMA GEMMs: E4M3 weights [N, K] with E8M0 scales [N, K/32]
// decoded to bf16 (exact), and the MX conversion of bf16 activations [T, K] (K a multiple of
// 32), written back as the dequantised bf16 values.
hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, int N, int K, uint16_t* out,
                             hipStream_t s);
hipError_t launch_mx_act(const uint16_t* x, int T, int K, uint16_t* out, hipStream_t s);
// The same conversion, written as E4M3 codes [T, K] and E8M0 block scales [T, K/32] (the
// operands of the block-scaled MFMA).
hipError_t launch_mx_act_codes(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);

}  // namespace mlap
