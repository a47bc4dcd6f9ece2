// common.h -- device helpers shared by the gfx950 sink-attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, one wave64):
//   A (32 x 16):  lane l holds row l%32, k = (l/32)*8 + e for its 8 bf16 e.
//   B (16 x 32):  lane l holds col l%32, k = (l/32)*8 + e.
//   C (32 x 32):  lane l, register i holds row (i/4)*8 + (l/32)*4 + i%4, col l%32.
// The contraction index of A and B only has to agree between the two operands,
// so every kernel is free to map (k-step, lane half, element) to any head-dim
// or key index it likes; the comments at each use say which mapping it takes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace sinkattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDqk = 192;
constexpr int kDv = 128;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_uint4(const bf16x8 &b) { return __builtin_bit_cast(uint4, b); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// Two floats -> one dword holding (lo, hi) bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the two 32-lane halves of a wave (lanes l and l^32 hold the same column).
__device__ __forceinline__ float max_across_halves(float x) {
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float sum_across_halves(float x) { return x + __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o, 64);
    return x;
}

// Row of the 32x32 C tile held by register i of a lane in half `hh` (= lane/32).
__device__ __forceinline__ int c_row(int i, int hh) { return (i >> 2) * 8 + hh * 4 + (i & 3); }

// Key order inside a 32-key block: the A-operand row r that must hold key kk so
// that register i of lane half hh ends up holding key 16*hh + i.
__host__ __device__ __forceinline__ int row_of_key(int kk) {
    const int hh = kk >> 4, a = (kk >> 2) & 3, b = kk & 3;
    return a * 8 + hh * 4 + b;
}
__host__ __device__ __forceinline__ int key_of_row(int r) {
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

}  // namespace sinkattn
