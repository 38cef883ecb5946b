// gemm_big_bf16.hip -- bf16 instantiations of the LDS-DMA GEMM (gemm_big.hpp).
#include "gemm_big_launch.hpp"

namespace mlap {

hipError_t launch_big_bf16(const GemmArgs& g, Epi epi, BigTile t, hipStream_t s) {
    using T = uint16_t;
    switch (t) {
        case BigTile::kWide:
            if (epi == Epi::kStoreBf16) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kStoreBf16>(g, s);
            if (epi == Epi::kStoreBf16X) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kStoreBf16X>(g, s);
            if (epi == Epi::kHeads) return launch_big_one<T, 256, 256, 4, 2, 2, Epi::kHeads>(g, s);
            break;
        case BigTile::kHalfHead:
            if (epi == Epi::kHeads) return launch_big_one<T, 256, 96, 4, 1, 3, Epi::kHeads>(g, s);
            break;
        case BigTile::kHalfHead64:
            if (epi == Epi::kHeads) return launch_big_one<T, 64, 96, 2, 1, 3, Epi::kHeads>(g, s);
            break;
        case BigTile::kSplitK:
            if (epi == Epi::kStoreF32) return launch_big_one<T, 256, 64, 4, 1, 3, Epi::kStoreF32>(g, s);
            break;
        case BigTile::kSplitK64:
            if (epi == Epi::kStoreF32) return launch_big_one<T, 64, 64, 2, 1, 3, Epi::kStoreF32>(g, s);
            break;
        case BigTile::kNarrowHeads:
            if (epi == Epi::kHeads) return launch_big_one<T, 256, 32, 4, 1, 3, Epi::kHeads>(g, s);
            break;
        case BigTile::kNarrowHeads64:
            if (epi == Epi::kHeads) return launch_big_one<T, 64, 32, 2, 1, 3, Epi::kHeads>(g, s);
            break;
        case BigTile::kRem64:
            if (epi == Epi::kStoreBf16) return launch_big_one<T, 64, 64, 2, 1, 3, Epi::kStoreBf16>(g, s);
            break;
        case BigTile::kSplitK32:
            if (epi == Epi::kStoreF32) return launch_big_one<T, 32, 64, 1, 1, 3, Epi::kStoreF32>(g, s);
            break;
        case BigTile::kNarrowHeads32:
            if (epi == Epi::kHeads) return launch_big_one<T, 32, 32, 1, 1, 3, Epi::kHeads>(g, s);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mlap
