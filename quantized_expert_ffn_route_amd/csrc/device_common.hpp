// Device helpers shared by the HIP kernels: operand types, loads, block
// dequantisation into MFMA operands, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 activations are carried as their uint16 bit patterns.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float f16_lo(uint32_t p) { return (float)__builtin_bit_cast(half2_t, p).x; }
__device__ __forceinline__ float f16_hi(uint32_t p) { return (float)__builtin_bit_cast(half2_t, p).y; }

// ---------------------------------------------------------------------------
// Block dequantisation.
//
// A lane owns one block of 32 codes.  Masking a code field word leaves, in
// each 16-bit half, one code q at bit offset o; read as an fp16 subnormal that
// half is q * 2^(o-24) exactly.  One fused multiply-add with the fp32 scale
// d * 2^(24-o) (exact: d is fp16) and the min m then gives the float32
// rounding of the exact d*q + m -- the dequantised weight -- in a single
// instruction (v_fma_mix_f32).  Pairs come out in code order: the low half of
// a word holds the even code, the high half the next odd code.
// ---------------------------------------------------------------------------

struct BlockScale {
  float m;
  float s16, s18, s20, s21, s22, s24;
};

__device__ __forceinline__ BlockScale block_scale(uint32_t dm) {
  const float d = f16_lo(dm);
  BlockScale b;
  b.m = f16_hi(dm);
  b.s16 = d * 65536.0f;
  b.s18 = d * 262144.0f;
  b.s20 = d * 1048576.0f;
  b.s21 = d * 2097152.0f;
  b.s22 = d * 4194304.0f;
  b.s24 = d * 16777216.0f;
  return b;
}

// Emits the dequantised pair (codes 2j, 2j+1) hidden in `p` with scale `s`.
template <typename Sink>
__device__ __forceinline__ void emit_pair(Sink& sink, int j, uint32_t p, float s, float m) {
  sink(j, __builtin_fmaf(s, f16_lo(p), m), __builtin_fmaf(s, f16_hi(p), m));
}

// Dequantise the 32 codes of one block (code field words w[0..bits-1]) and
// hand pairs j = 0..15 (codes 2j, 2j+1) to `sink(j, lo, hi)`.
template <int BITS, typename Sink>
__device__ __forceinline__ void dequant_block(const uint32_t* w, uint32_t dm, Sink& sink) {
  const BlockScale b = block_scale(dm);
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t t = w[i] >> 8;
      emit_pair(sink, 4 * i + 0, w[i] & 0x000F000Fu, b.s24, b.m);
      emit_pair(sink, 4 * i + 1, w[i] & 0x00F000F0u, b.s20, b.m);
      emit_pair(sink, 4 * i + 2, t & 0x000F000Fu, b.s24, b.m);
      emit_pair(sink, 4 * i + 3, t & 0x00F000F0u, b.s20, b.m);
    }
  } else if constexpr (BITS == 3) {
#pragma unroll
    for (int i = 0; i < 3; i++) {
      const uint32_t t = w[i] >> 9;
      emit_pair(sink, 5 * i + 0, w[i] & 0x00070007u, b.s24, b.m);
      emit_pair(sink, 5 * i + 1, w[i] & 0x00380038u, b.s21, b.m);
      emit_pair(sink, 5 * i + 2, w[i] & 0x01C001C0u, b.s18, b.m);
      emit_pair(sink, 5 * i + 3, t & 0x00070007u, b.s24, b.m);
      emit_pair(sink, 5 * i + 4, t & 0x00380038u, b.s21, b.m);
    }
    // codes 30 and 31: bit r of each sits in bit 15 / 31 of word r
    const uint32_t last = ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
                          ((w[2] >> 13) & 0x00040004u);
    emit_pair(sink, 15, last, b.s24, b.m);
  } else {
    static_assert(BITS == 2, "bits must be 2, 3 or 4");
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t t = w[i] >> 10;
      emit_pair(sink, 8 * i + 0, w[i] & 0x00030003u, b.s24, b.m);
      emit_pair(sink, 8 * i + 1, w[i] & 0x000C000Cu, b.s22, b.m);
      emit_pair(sink, 8 * i + 2, w[i] & 0x00300030u, b.s20, b.m);
      emit_pair(sink, 8 * i + 3, w[i] & 0x00C000C0u, b.s18, b.m);
      emit_pair(sink, 8 * i + 4, w[i] & 0x03000300u, b.s16, b.m);
      emit_pair(sink, 8 * i + 5, t & 0x00030003u, b.s24, b.m);
      emit_pair(sink, 8 * i + 6, t & 0x000C000Cu, b.s22, b.m);
      emit_pair(sink, 8 * i + 7, t & 0x00300030u, b.s20, b.m);
    }
  }
}

// Sink that rounds pairs to packed bf16 (MFMA operand words).
struct SinkBf16 {
  uint32_t v[16];
  __device__ __forceinline__ void operator()(int j, float lo, float hi) { v[j] = pack_bf16(lo, hi); }
};

// Sink that keeps fp32 values (fp32 activations).
struct SinkF32 {
  float v[32];
  __device__ __forceinline__ void operator()(int j, float lo, float hi) {
    v[2 * j] = lo;
    v[2 * j + 1] = hi;
  }
};

// Loads the code field of a block: `BITS` dwords.
template <int BITS>
__device__ __forceinline__ void load_field(const uint8_t* p, uint32_t* w) {
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 3) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2];
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  }
}

// ---------------------------------------------------------------------------
// MFMA wrappers.  Lane l of a 16x16 tile: operand row/column l % 16, k-group
// l / 16; accumulator element i is C[4*(l/16) + i][l % 16].
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4_t mfma_bf16(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                             uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3,
                                             f32x4_t c) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 A = {a0, a1, a2, a3};
  u32x4 B = {b0, b1, b2, b3};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                 __builtin_bit_cast(bf16x8_t, B), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Wave reductions (butterfly: every lane ends with the same value).
// ---------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
