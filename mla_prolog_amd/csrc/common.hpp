// common.hpp -- device helpers shared by the gfx950 MLA Prolog kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace mlap {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1. Every index seen
// by the body is a constant, so register arrays it touches are never demoted to memory.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf2f(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// Unpack 8 bf16 from a 16-byte chunk.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    uint4 v;
    v.x = pack_bf2(f[0], f[1]);
    v.y = pack_bf2(f[2], f[3]);
    v.z = pack_bf2(f[4], f[5]);
    v.w = pack_bf2(f[6], f[7]);
    return v;
}

// Largest |bf16| among 8 packed values, computed on the bit patterns (exact).
__device__ __forceinline__ float absmax8(const uint4& v) {
    float f[8];
    unpack8(v, f);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// Wave-wide reductions over 64 lanes (butterfly through DPP/permute via shfl).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Symmetric INT8 code of fp32 value v under multiplier m = 127/amax:
// round half to even (v_rndne_f32), then saturate to [-127, 127].
__device__ __forceinline__ int8_t quant_code(float v, float m) {
    float r = __builtin_rintf(v * m);
    r = fminf(fmaxf(r, -127.f), 127.f);
    return static_cast<int8_t>(static_cast<int>(r));
}

// Pack 8 int8 codes of 8 bf16 values (one 16-byte chunk) into 8 bytes.
__device__ __forceinline__ uint2 quant8(const uint4& v, float m) {
    float f[8];
    unpack8(v, f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t c = static_cast<uint8_t>(quant_code(f[i], m));
        w[i >> 2] |= c << (8 * (i & 3));
    }
    return make_uint2(w[0], w[1]);
}

// 8-byte store marked non-temporal (a final output, not read again by the path).
__device__ __forceinline__ void store_nt8(void* p, const uint2& v) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, static_cast<u32x2*>(p));
}

__device__ __forceinline__ int clamp_pos(int p, int max_pos) {
    return p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
}

// Bounds checks of the debug build (compiled with MLAP_DEBUG): a failed check sets its bit
// in *dbg with a vector atomic and the kernel carries on (the access it describes is
// clamped or guarded anyway); release builds compile the checks away. mlap_debug_flags
// reads and clears the word.
enum : unsigned {
    kDbgARow = 1u,     // GEMM operand row past the activation rows
    kDbgBRow = 2u,     // GEMM weight row outside the rows the launch may read
    kDbgK = 4u,        // GEMM K range past the row length
    kDbgStore = 8u,    // output index past its row or tensor
    kDbgRow = 16u,     // row-kernel token or column index out of range
    kDbgQuant = 32u,   // q quant chunk or store index out of range
    kDbgPos = 64u,     // an input position outside [0, max_pos) (clamped: a precondition)
};
#ifdef MLAP_DEBUG
#define MLAP_CHECK(dbg, cond, bit)                        \
    do {                                                  \
        if (!(cond) && (dbg) != nullptr) atomicOr((dbg), (bit)); \
    } while (0)
#else
#define MLAP_CHECK(dbg, cond, bit) \
    do {                           \
    } while (0)
#endif

}  // namespace mlap
