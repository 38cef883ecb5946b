// gemm_kernels.hip -- instantiations of the gfx950 MFMA GEMM and their launcher.
//
// Tile shapes (rows x columns of the output tile, K-tiles of prefetch in flight):
//   256 x {64..256}, 1 ahead  -- large batches (prefill): 128x128 (or 64x64) per wave,
//                                enough MFMA work per LDS byte to stay MFMA-bound;
//   128 x {64..256}, 3 ahead  -- small batches (decode): weight streaming, where the
//                                bytes in flight per workgroup set the bandwidth;
//   256 x 64, 3 ahead         -- the split-K down projection of small batches;
//   128 x 128, 1 ahead        -- the GEMM-core test exports.
// and the large-batch kernel of gemm_big.hpp: 256 x 256 tiles, eight waves, operands
// copied HBM -> LDS directly in 128-byte row stages, two stages in LDS.
#include "gemm.hpp"
#include "gemm_big.hpp"
#include "launch.hpp"

namespace mlap {

namespace {

template <typename Tin, int BM, int BN, int WM, int WN, int P, Epi EPI>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.k_splits;
    hipLaunchKernelGGL((gemm_nt_kernel<Tin, BM, BN, WM, WN, P, EPI>), dim3(tiles),
                       dim3(kWave * WM * WN), 0, s, g);
    return hipGetLastError();
}

template <typename Tin>
hipError_t dispatch(const GemmArgs& g, const GemmTile& t, Epi epi, hipStream_t s) {
    const int BM = t.bm, BN = t.bn, P = t.prefetch;
    switch (epi) {
        case Epi::kStoreBf16:
            if (BM == 128 && BN == 128 && P == 1) return launch_one<Tin, 128, 128, 2, 2, 1, Epi::kStoreBf16>(g, s);
            if (BM == 256 && BN == 192 && P == 1) return launch_one<Tin, 256, 192, 2, 2, 1, Epi::kStoreBf16>(g, s);
            if (BM == 256 && BN == 64 && P == 1) return launch_one<Tin, 256, 64, 4, 1, 1, Epi::kStoreBf16>(g, s);
            break;
        case Epi::kStoreF32:
            if constexpr (sizeof(Tin) == 2)
                if (BM == 256 && BN == 64 && P == 3) return launch_one<Tin, 256, 64, 4, 1, 3, Epi::kStoreF32>(g, s);
            break;
        case Epi::kStoreI32:
            if constexpr (sizeof(Tin) == 1)
                if (BM == 128 && BN == 128 && P == 1) return launch_one<Tin, 128, 128, 2, 2, 1, Epi::kStoreI32>(g, s);
            break;
        case Epi::kHeads:
            if (BM == 128 && P == 3) {
                if (BN == 64) return launch_one<Tin, 128, 64, 2, 2, 3, Epi::kHeads>(g, s);
                if (BN == 128) return launch_one<Tin, 128, 128, 2, 2, 3, Epi::kHeads>(g, s);
                if (BN == 192) return launch_one<Tin, 128, 192, 2, 2, 3, Epi::kHeads>(g, s);
                if (BN == 256) return launch_one<Tin, 128, 256, 2, 2, 3, Epi::kHeads>(g, s);
            }
            if (BM == 256 && P == 1) {
                if (BN == 64) return launch_one<Tin, 256, 64, 4, 1, 1, Epi::kHeads>(g, s);
                if (BN == 128) return launch_one<Tin, 256, 128, 2, 2, 1, Epi::kHeads>(g, s);
                if (BN == 192) return launch_one<Tin, 256, 192, 2, 2, 1, Epi::kHeads>(g, s);
                if (BN == 256) return launch_one<Tin, 256, 256, 2, 2, 1, Epi::kHeads>(g, s);
            }
            break;
    }
    return hipErrorInvalidValue;
}

template <typename Tin, int BM, int BN, int WM, int WN, int S, Epi EPI>
hipError_t launch_big_one(const GemmArgs& g, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.k_splits;
    hipLaunchKernelGGL((gemm_big_kernel<Tin, BM, BN, WM, WN, 128, S, EPI>), dim3(tiles),
                       dim3(64 * WM * WN), 0, s, g);
    return hipGetLastError();
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
    if (shape == BigShape::kWide && epi == Epi::kStoreBf16 && g.N > kBigTile && g.N % kBigTile &&
        g.N % 64 == 0) {
        // A ragged last column tile would cost a whole extra round of 256x256 tiles: run the
        // full-width columns here and the remainder with 256 x 64 tiles.
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
        r.out = static_cast<uint16_t*>(g.out) + nm;
        // 64 x 64 tiles: one per 64 tokens, so the narrow remainder still spreads over the CUs
        if ((static_cast<size_t>(r.K) * eb) % 128 == 0) {
            if (t == InType::kFp8) return launch_big_one<fp8e4m3, 64, 64, 2, 1, 3, Epi::kStoreBf16>(r, s);
            return t == InType::kInt8 ? launch_big_one<int8_t, 64, 64, 2, 1, 3, Epi::kStoreBf16>(r, s)
                                      : launch_big_one<uint16_t, 64, 64, 2, 1, 3, Epi::kStoreBf16>(r, s);
        }
        return launch_gemm(r, t, GemmTile{256, 64, 1}, Epi::kStoreBf16, s);
    }
    if (!gemm_big_fits(g, t, epi, shape)) return hipErrorInvalidValue;
    // Weight-streaming shapes cover the whole batch in one row tile; at most 64 tokens take
    // 64-row tiles (two waves), so no copy bandwidth goes to clamped duplicate rows.
    const bool m64 = g.M <= 64;
    if (t == InType::kFp8) {  // MXFP8: the same shapes on E4M3 operands
        switch (shape) {
            case BigShape::kWide:
                return epi == Epi::kStoreBf16 ? launch_big_one<fp8e4m3, 256, 256, 2, 2, 2, Epi::kStoreBf16>(g, s)
                                              : launch_big_one<fp8e4m3, 256, 256, 2, 2, 2, Epi::kHeads>(g, s);
            case BigShape::kHalfHead:
                return m64 ? launch_big_one<fp8e4m3, 64, 96, 2, 1, 3, Epi::kHeads>(g, s)
                           : launch_big_one<fp8e4m3, 256, 96, 4, 1, 3, Epi::kHeads>(g, s);
            case BigShape::kSplitK:
                return m64 ? launch_big_one<fp8e4m3, 64, 64, 2, 1, 3, Epi::kStoreF32>(g, s)
                           : launch_big_one<fp8e4m3, 256, 64, 4, 1, 3, Epi::kStoreF32>(g, s);
            case BigShape::kNarrowHeads:
                return m64 ? launch_big_one<fp8e4m3, 64, 32, 2, 1, 3, Epi::kHeads>(g, s)
                           : launch_big_one<fp8e4m3, 256, 32, 4, 1, 3, Epi::kHeads>(g, s);
        }
        return hipErrorInvalidValue;
    }
    switch (shape) {
        case BigShape::kWide:
            if (t == InType::kBf16)
                return epi == Epi::kStoreBf16 ? launch_big_one<uint16_t, 256, 256, 4, 2, 2, Epi::kStoreBf16>(g, s)
                                              : launch_big_one<uint16_t, 256, 256, 4, 2, 2, Epi::kHeads>(g, s);
            return epi == Epi::kStoreBf16 ? launch_big_one<int8_t, 256, 256, 4, 2, 2, Epi::kStoreBf16>(g, s)
                                          : launch_big_one<int8_t, 256, 256, 4, 2, 2, Epi::kHeads>(g, s);
        case BigShape::kHalfHead:
            return m64 ? launch_big_one<uint16_t, 64, 96, 2, 1, 3, Epi::kHeads>(g, s)
                       : launch_big_one<uint16_t, 256, 96, 4, 1, 3, Epi::kHeads>(g, s);
        case BigShape::kSplitK:
            return m64 ? launch_big_one<uint16_t, 64, 64, 2, 1, 3, Epi::kStoreF32>(g, s)
                       : launch_big_one<uint16_t, 256, 64, 4, 1, 3, Epi::kStoreF32>(g, s);
        case BigShape::kNarrowHeads:
            return m64 ? launch_big_one<uint16_t, 64, 32, 2, 1, 3, Epi::kHeads>(g, s)
                       : launch_big_one<uint16_t, 256, 32, 4, 1, 3, Epi::kHeads>(g, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& g, InType type, const GemmTile& t, Epi epi, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (type == InType::kFp8) return hipErrorInvalidValue;  // MXFP8 runs on the LDS-DMA kernel only
    return type == InType::kBf16 ? dispatch<uint16_t>(g, t, epi, s) : dispatch<int8_t>(g, t, epi, s);
}

}  // namespace mlap
