// gemm_big_launch.hpp -- the launch of one LDS-DMA GEMM instantiation (included by the
// per-type translation units only).
#pragma once

#include "gemm_big.hpp"
#include "gemm_inst.hpp"

namespace mlap {

template <typename Tin, int BM, int BN, int WM, int WN, int S, Epi EPI>
hipError_t launch_big_one(const GemmArgs& g, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.k_splits;
    GemmArgs a = g;
    a.dbg = debug_word();
    hipLaunchKernelGGL((gemm_big_kernel<Tin, BM, BN, WM, WN, 128, S, EPI>), dim3(tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

}  // namespace mlap
