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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw 16-bit storage of bf16 inputs.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Four consecutive log-decay values (index i a multiple of 4) as fp32, from fp32 or bf16
// storage (bf16 widens exactly).
__device__ __forceinline__ f32x4 load_g4(const float* g, size_t i) {
    return *reinterpret_cast<const f32x4*>(g + i);
}
__device__ __forceinline__ f32x4 load_g4(const bf16_t* g, size_t i) {
    const uint2 u = *reinterpret_cast<const uint2*>(g + i);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
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

// Buffer resource over `nbytes` bytes at `base` (raw, stride 0).  Buffer loads and stores
// take a 32-bit per-lane offset plus a wave-uniform offset held in an SGPR, which keeps
// address arithmetic off the vector ALU; a load whose per-lane offset is past `nbytes`
// returns zero and such a store is dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                             0x00020000);
}
__device__ __forceinline__ half8 buf_load_half8(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ f32x4 buf_load_f32x4(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Raw bits of one q/k/v element (fp32 bits, or bf16 bits zero-extended); converted by
// raw_to_f32 only where the value is used, so the load stays in flight until then.
__device__ __forceinline__ uint32_t buf_load_raw(rsrc_t r, int voff, int soff, float) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load_raw(rsrc_t r, int voff, int soff, bf16_t) {
    return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
__device__ __forceinline__ float raw_to_f32(uint32_t x, float) { return __uint_as_float(x); }
__device__ __forceinline__ float raw_to_f32(uint32_t x, bf16_t) { return __uint_as_float(x << 16); }
__device__ __forceinline__ void buf_store_f32(float x, rsrc_t r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store_f32x4(f32x4 x, rsrc_t r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, soff, 0);
}
// Cache-policy operand (the gfx950 non-temporal bit) of the accesses whose data no later
// kernel of the prefill reads: the outputs o, stored by the carry, and the log-decays g
// (fp32), loaded once by the prep.  That way neither displaces the chunk records from the
// last-level cache, which the prep writes and the carry reads right after.  Measured at
// HV = 32, 128 x 128, C = 64: o streamed, the carry takes 84.5 instead of 94 us at B = 1,
// T = 4097 and 57.6 instead of 64 us at B = 8, T = 512; g streamed as well, 62.6 instead of
// 72.1 us at B = 1, T = 4097 (the whole prefill 122 instead of 132 us) and 55.6 instead of
// 61.0 us at B = 8, T = 512, the prep unchanged.  Where the records outgrow the cache
// (B = 2, T = 4097; B = 1, T = 32768) neither changes anything.  Streaming q and k as well
// slows the prep by 10-17 % (each key head's rows serve the G value heads of its group
// through L2), v in the column-split carry by 13 % (its 8 column groups share each v
// line), v in the whole-head carry by up to 30 %; a bf16 g streamed slows the prep by 9 %
// (59.9 against 65.1 us at B = 1, T = 4097) and is read with the default policy.
constexpr int kStream = 2;
__device__ __forceinline__ void buf_store_f32x4_stream(f32x4 x, rsrc_t r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, soff, kStream);
}

// ---- outputs o: fp32, or bf16 when the caller asks for it (obf) ----------------------------
// A bf16 output is the fp32 result rounded to the nearest bf16, ties to even (the hardware
// conversion in the default rounding mode), as it is stored.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 bf16x4_bits(f32x4 x) {
    const bf16x4v b = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]), static_cast<__bf16>(x[2]),
                       static_cast<__bf16>(x[3])};
    return __builtin_bit_cast(u32x2, b);
}
// Bytes per output element.
__device__ __forceinline__ int o_elt(int obf) { return obf ? 2 : 4; }
// Four consecutive outputs, given the byte offsets (voff, soff) they have in fp32 storage;
// in bf16 storage they sit at half those offsets.  An offset beyond the buffer range drops
// the store either way.
__device__ __forceinline__ void store_o4_stream(f32x4 x, rsrc_t r, int voff, int soff, int obf) {
    if (obf)
        __builtin_amdgcn_raw_buffer_store_b64(bf16x4_bits(x), r, voff >> 1, soff >> 1, kStream);
    else
        buf_store_f32x4_stream(x, r, voff, soff);
}
// Four consecutive outputs at element index i of o (i a multiple of 4, o 16-byte aligned).
__device__ __forceinline__ void store_o4(void* o, size_t i, f32x4 x, int obf) {
    if (obf)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + i) = bf16x4_bits(x);
    else
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + i) = x;
}
// One output at element index i of o.
__device__ __forceinline__ void store_o1(void* o, size_t i, float x, int obf) {
    if (obf)
        static_cast<__bf16*>(o)[i] = static_cast<__bf16>(x);
    else
        static_cast<float*>(o)[i] = x;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global/buffer loads (vmcnt), so prefetches stay in flight across it.  The empty asm
// statements stop the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- magnitude reductions and power-of-two scaling --------------------------------------
// Operands of the fp16 matrix-core products are brought into fp16's range by exact
// power-of-two factors; these helpers find the exponents.

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// max(x[l], x[l ^ 16]) and max(x[l], x[l ^ 32]) in every lane (gfx950 lane-swap moves)
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] in every lane: the four lane groups' sum
__device__ __forceinline__ float sum_over_groups(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(u[0]) + __uint_as_float(u[1]);
}

// ---- fused input prologue ---------------------------------------------------------------
// Keys given raw are used as k / max(|k|_2, 1e-12) (per token and key head); gate logits a
// give the log-decay g = -softplus(a) = -log(1 + e^a).
constexpr float kKeyNormEps = 1e-12f;
__device__ __forceinline__ float inv_key_norm(float sum_sq) {
    return 1.f / fmaxf(__builtin_sqrtf(sum_sq), kKeyNormEps);
}
// -softplus(a) in log2 units (g * log2(e)), stable for either sign of a
__device__ __forceinline__ float neg_softplus_log2(float a) {
    const float u = a * 1.4426950408889634f;
    return -(fmaxf(u, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(u))));
}
// -softplus(a) in natural units: the log-decay g from a gate logit a
__device__ __forceinline__ float neg_softplus(float a) { return neg_softplus_log2(a) * 0.6931471805599453f; }
// exp(-softplus(a)) = 1 / (1 + e^a): the per-token decay factor from a gate logit
__device__ __forceinline__ float decay_from_logit(float a) { return 1.f / (1.f + __expf(a)); }

// Maximum over the four lanes l % 16 + 16 * g (g = 0..3): one column of an accumulator tile.
__device__ __forceinline__ float max_over_groups(float x) { return max_xor32(max_xor16(x)); }
// Maximum over the whole wave, in every lane.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_mov<0x124>(x));  // row_ror:4
    x = fmaxf(x, dpp_mov<0x128>(x));  // row_ror:8
    return max_over_groups(x);
}
// Exponent e with m = f * 2^e, f in [0.5, 1) (0 for m == 0, inf or NaN).
__device__ __forceinline__ int exponent_of(float m) { return __builtin_amdgcn_frexp_expf(m); }
// x * 2^e, exact while the result stays a normal fp32 number
__device__ __forceinline__ float ldexp2(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }
// 2^e as fp16 for e in [-24, 15] (0 below), the exact factor that aligns two scaled operands
__device__ __forceinline__ _Float16 half_pow2(int e) {
    if (e < -24) return static_cast<_Float16>(0.f);
    return static_cast<_Float16>(ldexp2(1.f, e));
}

// Reduction-slot permutation used for every fragment that meets an accumulator tile.
// Slot jj (0..7) of lane group g inside a 32-wide reduction step maps to index
//   16 * (jj / 4) + 4 * g + (jj % 4)
// which is exactly the set of rows an accumulator lane holds in the two 16-row tiles
// of that step.  Accumulators can therefore feed the B operand of the next product with
// no data movement; the A operand reads its columns in the same order.
__device__ __forceinline__ int perm_slot(int g, int jj) { return 16 * (jj >> 2) + 4 * g + (jj & 3); }

}  // namespace gdr
