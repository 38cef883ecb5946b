// gemm_nt.hip -- instantiations of the register-staged MFMA GEMM (gemm.hpp): the int8
// small-batch projections, the GEMM-core test exports and the shapes the LDS-DMA kernel
// does not take.
//
// Tile shapes (rows x columns of the output tile, K-tiles of register prefetch in flight):
//   256 x {64..256}, 1 ahead  -- large batches: 128x128 (or 64x64) per wave;
//   128 x {64..256}, 3 ahead  -- small batches (weight streaming): bytes in flight per
//                                workgroup set the bandwidth;
//   256 x 64, 3 ahead         -- split-K fp32 partials;
//   128 x 128, 1 ahead        -- the bf16 GEMM-core test export.
#include "gemm_inst.hpp"

namespace mlap {

namespace {

template <typename Tin, int BM, int BN, int WM, int WN, int P, Epi EPI>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.k_splits;
    GemmArgs a = g;
    a.dbg = debug_word();
    hipLaunchKernelGGL((gemm_nt_kernel<Tin, BM, BN, WM, WN, P, EPI>), dim3(tiles),
                       dim3(kWave * WM * WN), 0, s, a);
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
            // the int8 small-batch projections' own tiles (the int32 test export runs them)
            if constexpr (sizeof(Tin) == 1) {
                if (BM == 256 && BN == 64 && P == 1) return launch_one<Tin, 256, 64, 4, 1, 1, Epi::kStoreI32>(g, s);
                if (BM == 128 && BN == 192 && P == 3) return launch_one<Tin, 128, 192, 2, 2, 3, Epi::kStoreI32>(g, s);
            }
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

}  // namespace

hipError_t launch_nt_bf16(const GemmArgs& g, const GemmTile& t, Epi epi, hipStream_t s) {
    return dispatch<uint16_t>(g, t, epi, s);
}

hipError_t launch_nt_i8(const GemmArgs& g, const GemmTile& t, Epi epi, hipStream_t s) {
    return dispatch<int8_t>(g, t, epi, s);
}

}  // namespace mlap
