// gemm_kernels.hip -- instantiations of the gfx950 MFMA GEMM and their launcher.
#include "gemm.hpp"
#include "launch.hpp"

namespace mlap {

namespace {

template <typename Tin, int BM, int BN, int WM, int WN, Epi EPI>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
    const dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.k_splits);
    hipLaunchKernelGGL((gemm_nt_kernel<Tin, BM, BN, WM, WN, EPI>), grid, dim3(kWave * WM * WN), 0, s,
                       g);
    return hipGetLastError();
}

template <typename Tin>
hipError_t dispatch(const GemmArgs& g, int BM, int BN, Epi epi, hipStream_t s) {
    if (BM != 128) return hipErrorInvalidValue;
    switch (epi) {
        case Epi::kStoreBf16:
            if (BN == 128) return launch_one<Tin, 128, 128, 2, 2, Epi::kStoreBf16>(g, s);
            break;
        case Epi::kStoreF32:
            if constexpr (sizeof(Tin) == 2)
                if (BN == 128) return launch_one<Tin, 128, 128, 2, 2, Epi::kStoreF32>(g, s);
            break;
        case Epi::kStoreI32:
            if constexpr (sizeof(Tin) == 1)
                if (BN == 128) return launch_one<Tin, 128, 128, 2, 2, Epi::kStoreI32>(g, s);
            break;
        case Epi::kHeads:
            if (BN == 64) return launch_one<Tin, 128, 64, 2, 2, Epi::kHeads>(g, s);
            if (BN == 128) return launch_one<Tin, 128, 128, 2, 2, Epi::kHeads>(g, s);
            if (BN == 192) return launch_one<Tin, 128, 192, 2, 2, Epi::kHeads>(g, s);
            if (BN == 256) return launch_one<Tin, 128, 256, 2, 2, Epi::kHeads>(g, s);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, InType t, int BM, int BN, Epi epi, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    return t == InType::kBf16 ? dispatch<uint16_t>(g, BM, BN, epi, s)
                              : dispatch<int8_t>(g, BM, BN, epi, s);
}

}  // namespace mlap
