// gemm_inst.hpp -- per-operand-type launchers of the GEMM kernels. Each operand type's
// instantiations live in a translation unit of their own (gemm_big_bf16.hip,
// gemm_big_i8.hip, gemm_big_fp8.hip, gemm_nt.hip) so they compile in parallel;
// gemm_kernels.hip picks the tile and calls these.
#pragma once

#include "gemm.hpp"
#include "launch.hpp"

namespace mlap {

// Tiles of the LDS-DMA kernel (gemm_big.hpp): the BigShape families, their 64-row forms for
// batches of at most 64 tokens (32-row forms of two of them for at most 32), and the 64 x 64
// tiles of a ragged column remainder.
enum class BigTile : int {
    kWide = 0,       // 256 x 256 (bf16, int8: 4 x 2 waves; E4M3: 2 x 2 waves)
    kHalfHead,       // 256 x 96, 4 x 1 waves, 3 stages
    kHalfHead64,     // 64 x 96, 2 x 1 waves
    kSplitK,         // 256 x 64, 4 x 1 waves, 3 stages
    kSplitK64,       // 64 x 64, 2 x 1 waves
    kNarrowHeads,    // 256 x 32, 4 x 1 waves, 3 stages
    kNarrowHeads64,  // 64 x 32, 2 x 1 waves
    kRem64,          // 64 x 64, 2 x 1 waves, 3 stages (column remainder of a kWide launch)
    kSplitK32,       // 32 x 64, one wave, 3 stages (batches of at most 32 tokens)
    kNarrowHeads32   // 32 x 32, one wave, 3 stages
};

// Launch tile `t` with epilogue `epi` on a 1-D grid of tiles x k_splits workgroups; returns
// hipErrorInvalidValue for a combination that has no instantiation.
hipError_t launch_big_bf16(const GemmArgs& g, Epi epi, BigTile t, hipStream_t s);
hipError_t launch_big_i8(const GemmArgs& g, Epi epi, BigTile t, hipStream_t s);
hipError_t launch_big_fp8(const GemmArgs& g, Epi epi, BigTile t, hipStream_t s);

// The register-staged kernel (gemm.hpp) for bf16 and int8 operands.
hipError_t launch_nt_bf16(const GemmArgs& g, const GemmTile& t, Epi epi, hipStream_t s);
hipError_t launch_nt_i8(const GemmArgs& g, const GemmTile& t, Epi epi, hipStream_t s);

template <typename Tin, int BM, int BN, int WM, int WN, int S, Epi EPI>
hipError_t launch_big_one(const GemmArgs& g, hipStream_t s);

}  // namespace mlap
