// gemm_big_i8.hip -- int8 (W8A8) instantiations of the LDS-DMA GEMM (gemm_big.hpp): the
// large-batch tiles of the W8A8 projections and their raw int32 form (the test export).
#include "gemm_big_launch.hpp"

namespace mlap {

hipError_t launch_big_i8(const GemmArgs& g, Epi epi, BigTile t, hipStream_t s) {
    using T = int8_t;
    switch (t) {
        case BigTile::kWide:
            if (epi == Epi::kStoreBf16) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kStoreBf16>(g, s);
            if (epi == Epi::kStoreBf16X) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kStoreBf16X>(g, s);
            if (epi == Epi::kHeads) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kHeads>(g, s);
            if (epi == Epi::kStoreI32) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kStoreI32>(g, s);
            break;
        case BigTile::kRem64:
            if (epi == Epi::kStoreBf16) return launch_big_one<T, 64, 64, 2, 1, 3, Epi::kStoreBf16>(g, s);
            if (epi == Epi::kStoreI32) return launch_big_one<T, 64, 64, 2, 1, 3, Epi::kStoreI32>(g, s);
            break;
        default:
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mlap
