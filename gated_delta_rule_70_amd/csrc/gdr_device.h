// Device-side helpers shared by the gfx950 kernels of libgdr: vector types, element
// conversions, and thin wrappers over the CDNA4 matrix-core (MFMA) builtins.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Raw 16-bit storage of bf16 inputs.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Split an fp32 value into a bf16 high part and a bf16 remainder (round to nearest even
// on both), so that hi + lo carries ~16 significant bits with fp32's exponent range.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// D(16x16, fp32) += A(16x32) * B(32x16), fp16 operands.  Per lane l (g = l / 16):
//   A: row l % 16, 8 consecutive reduction slots of group g;  B: column l % 16, same slots;
//   D: rows 4g .. 4g+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_f16(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reduction-slot permutation used for every fragment that meets an accumulator tile.
// Slot jj (0..7) of lane group g inside a 32-wide reduction step maps to index
//   16 * (jj / 4) + 4 * g + (jj % 4)
// which is exactly the set of rows an accumulator lane holds in the two 16-row tiles
// of that step.  Accumulators can therefore feed the B operand of the next product with
// no data movement; the A operand reads its columns in the same order.
__device__ __forceinline__ int perm_slot(int g, int jj) { return 16 * (jj >> 2) + 4 * g + (jj & 3); }

}  // namespace gdr
