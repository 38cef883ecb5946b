// gemm_kernels.hip -- tile choice of the gfx950 MFMA GEMMs. The kernels are the LDS-DMA
// GEMM of gemm_big.hpp (256 x 256 tiles, eight waves, operands copied HBM -> LDS directly in
// 128-byte row stages, for large batches; narrow weight-streaming tiles for small ones) and
// the register-staged GEMM of gemm.hpp; their instantiations live in gemm_big_*.hip and
// gemm_nt.hip.
#include "gemm_inst.hpp"

namespace mlap {

namespace {

hipError_t launch_big_typed(const GemmArgs& g, InType t, Epi epi, BigTile tile, hipStream_t s) {
    switch (t) {
        case InType::kBf16: return launch_big_bf16(g, epi, tile, s);
        case InType::kInt8: return launch_big_i8(g, epi, tile, s);
        case InType::kFp8: return launch_big_fp8(g, epi, tile, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int big_tile_n(BigShape shape) {
    switch (shape) {
        case BigShape::kWide: return 256;
        case BigShape::kHalfHead: return 96;
        case BigShape::kSplitK: return 64;
        case BigShape::kNarrowHeads: return 32;
    }
    return 0;
}

bool gemm_big_fits(const GemmArgs& g, InType t, Epi epi, BigShape shape) {
    const int kbytes = g.K * (t == InType::kBf16 ? 2 : 1);
    const int splits = g.k_splits > 0 ? g.k_splits : 1;
    if (g.K <= 0 || kbytes % (128 * splits)) return false;  // whole 128-byte stages per split
    if (splits > 1 && epi != Epi::kStoreF32) return false;
    switch (shape) {
        case BigShape::kWide:
            if (epi == Epi::kStoreBf16) return g.N % 8 == 0 && g.ldo % 8 == 0;
            if (epi == Epi::kStoreBf16X)  // whole column tiles; the output rows hold the extras
                return t != InType::kFp8 && g.k_splits <= 1 && g.N % kBigTile == 0 &&
                       g.ldo >= g.N + 8 * (g.N / kBigTile) && g.ldo % 4 == 0;
            if (epi == Epi::kStoreI32) return t == InType::kInt8;
            if (epi == Epi::kHeads) {
                if (g.head_w % 64 || g.d0 % 64) return false;
                return g.rope ? g.d1 == 64 : g.d1 % 8 == 0;
            }
            return false;
        case BigShape::kHalfHead:
            // 96-column tiles, two per head: [0, 96) all seg0, [96, 192) the rest of seg0
            // (32 columns) and the 64-wide rope slice, rotated in registers
            return t != InType::kInt8 && epi == Epi::kHeads && g.head_w == 192 && g.rope &&
                   g.d0 == 128 && g.d1 == 64;
        case BigShape::kSplitK:
            return t != InType::kInt8 && epi == Epi::kStoreF32 && g.N % 4 == 0 && g.ldo % 4 == 0;
        case BigShape::kNarrowHeads:
            // 32-column tiles that never straddle a segment; no rotate-half pairs
            return t != InType::kInt8 && epi == Epi::kHeads && !g.rope && g.head_w % 32 == 0 &&
                   g.d0 % 32 == 0 && g.d1 % 8 == 0;
    }
    return false;
}

hipError_t launch_gemm_big(const GemmArgs& g, InType t, Epi epi, hipStream_t s, BigShape shape) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (shape == BigShape::kWide && (epi == Epi::kStoreBf16 || epi == Epi::kStoreI32) && g.N > kBigTile &&
        g.N % kBigTile && g.N % 64 == 0) {
        // A ragged last column tile would cost a whole extra round of 256x256 tiles: run the
        // full-width columns here and the remainder with 64 x 64 tiles.
        const int nm = g.N / kBigTile * kBigTile;
        GemmArgs a = g;
        a.N = nm;
        hipError_t e = launch_gemm_big(a, t, epi, s, shape);
        if (e != hipSuccess) return e;
        GemmArgs r = g;
        r.N = g.N - nm;
        r.pe_c0 = g.pe_c0 + nm;
        const size_t eb = t == InType::kBf16 ? 2 : 1;
        const size_t mxrow = static_cast<size_t>(g.K / 32);  // E8M0 bytes per B row (MXFP8)
        if (nm >= g.b_split) {  // the remainder rows all come from the second segment
            r.B0 = r.B1 = static_cast<const char*>(g.B1) + static_cast<size_t>(nm - g.b_split) * g.ldb * eb;
            r.b_scale0 = r.b_scale1 = g.b_scale1 ? g.b_scale1 + (nm - g.b_split) : nullptr;
            r.b_mx0 = r.b_mx1 = g.b_mx1 ? g.b_mx1 + static_cast<size_t>(nm - g.b_split) * mxrow : nullptr;
            r.b_split = r.N;
        } else {
            r.B0 = static_cast<const char*>(g.B0) + static_cast<size_t>(nm) * g.ldb * eb;
            r.b_scale0 = g.b_scale0 ? g.b_scale0 + nm : nullptr;
            r.b_mx0 = g.b_mx0 ? g.b_mx0 + static_cast<size_t>(nm) * mxrow : nullptr;
            r.b_split = g.b_split - nm;
        }
        r.out = static_cast<char*>(g.out) + static_cast<size_t>(nm) * (epi == Epi::kStoreI32 ? 4 : 2);
        // 64 x 64 tiles: one per 64 tokens, so the narrow remainder still spreads over the CUs
        if ((static_cast<size_t>(r.K) * eb) % 128 == 0) return launch_big_typed(r, t, epi, BigTile::kRem64, s);
        if (epi == Epi::kStoreI32) return hipErrorInvalidValue;
        return launch_gemm(r, t, GemmTile{256, 64, 1}, Epi::kStoreBf16, s);
    }
    if (!gemm_big_fits(g, t, epi, shape)) return hipErrorInvalidValue;
    // Weight-streaming shapes cover the whole batch in one row tile; at most 64 tokens take
    // 64-row tiles (two waves), so no copy bandwidth goes to clamped duplicate rows.
    // At most 32 tokens take the 32-row (one-wave) forms where they exist (bf16).
    const bool m64 = g.M <= 64, m32 = g.M <= 32 && t == InType::kBf16;
    BigTile tile = BigTile::kWide;
    switch (shape) {
        case BigShape::kWide: tile = BigTile::kWide; break;
        case BigShape::kHalfHead: tile = m64 ? BigTile::kHalfHead64 : BigTile::kHalfHead; break;
        case BigShape::kSplitK:
            tile = m32 ? BigTile::kSplitK32 : m64 ? BigTile::kSplitK64 : BigTile::kSplitK;
            break;
        case BigShape::kNarrowHeads:
            tile = m32 ? BigTile::kNarrowHeads32 : m64 ? BigTile::kNarrowHeads64 : BigTile::kNarrowHeads;
            break;
    }
    return launch_big_typed(g, t, epi, tile, s);
}

hipError_t launch_gemm(const GemmArgs& g, InType type, const GemmTile& t, Epi epi, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (type == InType::kFp8) return hipErrorInvalidValue;  // MXFP8 runs on the LDS-DMA kernel only
    return type == InType::kBf16 ? launch_nt_bf16(g, t, epi, s) : launch_nt_i8(g, t, epi, s);
}

}  // namespace mlap
