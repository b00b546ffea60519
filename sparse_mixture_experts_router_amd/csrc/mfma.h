// MFMA step shared by the router and the grouped GEMMs (gfx950).
//
// Every operand fragment is 16 contiguous bytes of one row, taken at byte
// offset 16 * (lane / 16) of a 64-byte slice of the reduction dimension:
//   row  = lane % 16 of the 16-row block (A: token row, B: weight row)
//   bf16 : 8 elements -> one v_mfma_f32_16x16x32_bf16 covers the 32 elements
//          of the slice (lane group q supplies elements 8q .. 8q+7);
//   fp32 : 4 elements -> four v_mfma_f32_16x16x4_f32, the j-th taking element
//          j of every lane's four, so together they cover the 16 elements of
//          the slice (lane group q supplies elements 4q .. 4q+3).
// A and B use the same element-to-lane assignment, so each MFMA sums matching
// products.  The 16x16 fp32 result lives in lane l, register r as
// C[4 * (l / 16) + r][l % 16].
#pragma once

#include "moe_internal.h"

namespace moe {

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
    return c;
  }
};

// The same bf16 step with the accumulator pinned to AGPRs.  Used where a
// wavefront holds 256 accumulator registers: the compiler's own MFMA form would
// split them between VGPRs and AGPRs and copy them back and forth every
// iteration.  Because the compiler cannot see that this asm is an MFMA, the
// caller issues mfma_drain() before anything else reads the accumulators.
__device__ __forceinline__ void mfma_bf16_agpr(f32x4& c, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// The same, for an operand that a VALU instruction may have just written (a
// widened FP8 fragment).  CDNA3/4 need two wait states between a VALU write of
// a VGPR and an MFMA reading it; the compiler inserts them only before MFMAs it
// recognises, so the asm form carries its own.
__device__ __forceinline__ void mfma_bf16_agpr_after_valu(f32x4& c, u32x4 a, u32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// 8 FP8 E4M3 codes (bytes 0..7 of v, little endian) -> 8 bf16, one 16-byte
// MFMA operand chunk.  Every finite E4M3 value is exact in bf16 (3 of its 7
// mantissa bits, exponents 2^-9 .. 2^8); the conversion's scale is 1.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
  return r;
}

// Wait states between the last MFMA writing an accumulator and any other
// instruction reading it (covers the longest 16x16x32 bf16 latency).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// Byte offset of 16-byte chunk `ch` (0..7) of row `r` in an LDS tile whose
// rows are 128 bytes: the chunk index is XOR-ed with the row's low 3 bits so
// that 8 consecutive rows read at the same logical chunk hit 8 different
// 16-byte bank groups.
__device__ __forceinline__ int lds_swz(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

}  // namespace moe
