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

// ---------------------------------------------------------------------------
// MXFP4 blocks: byte j of the 16-byte field holds codes 2j (low nibble) and
// 2j + 1 (high nibble), and the block scale is the E8M0 byte X + 127.  The
// CDNA4 conversion v_cvt_scalef32_pk_{bf16,f32}_fp4 turns one byte's two
// E2M1 codes, times an fp32 scale, into a bf16 or fp32 pair; with the scale
// 2^X (X in [-125, 125]) the product is exact in either type.  One
// instruction per two weights.
// ---------------------------------------------------------------------------

// The E8M0 byte X + 127 as the float 2^X (a normal float for X >= -126).
__device__ __forceinline__ float mx_scale(uint32_t e) { return __uint_as_float(e << 23); }

template <int B>
__device__ __forceinline__ uint32_t mx_pair_bf16(uint32_t w, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, B));
}

template <int B, typename Sink>
__device__ __forceinline__ void mx_pair(Sink& sink, int j, uint32_t w, float s) {
  if constexpr (Sink::kBf16) {
    sink.put(j, mx_pair_bf16<B>(w, s));
  } else {
    const auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, B);
    sink(j, p[0], p[1]);
  }
}

template <typename Sink>
__device__ __forceinline__ void dequant_block_mx(const uint32_t* w, uint32_t e, Sink& sink) {
  const float s = mx_scale(e);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    mx_pair<0>(sink, 4 * i + 0, w[i], s);
    mx_pair<1>(sink, 4 * i + 1, w[i], s);
    mx_pair<2>(sink, 4 * i + 2, w[i], s);
    mx_pair<3>(sink, 4 * i + 3, w[i], s);
  }
}

template <int BITS, typename Sink>
__device__ __forceinline__ void dequant_block_affine(const uint32_t* w, uint32_t dm, Sink& sink);

// Dequantise the 32 codes of one block (code field words w[0..bits-1]) and
// hand pairs j = 0..15 (codes 2j, 2j+1) to the sink: `sink(j, lo, hi)` as
// floats, or, for bf16 sinks (Sink::kBf16), `sink.put(j, packed bf16 pair)`.
// `dm` is the block's (d, m) word, or its E8M0 byte for MXFP4.
template <int BITS, typename Sink>
__device__ __forceinline__ void dequant_block(const uint32_t* w, uint32_t dm, Sink& sink) {
  if constexpr (BITS == kMx4) {
    dequant_block_mx(w, dm, sink);
  } else {
    dequant_block_affine<BITS>(w, dm, sink);
  }
}

template <int BITS, typename Sink>
__device__ __forceinline__ void dequant_block_affine(const uint32_t* w, uint32_t dm, Sink& sink) {
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
  } else if constexpr (BITS == 2) {
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
  } else {
    static_assert(BITS == 2, "format must be 2, 3, 4 bits or MXFP4");
  }
}

// Sink that rounds pairs to packed bf16 (MFMA operand words).
struct SinkBf16 {
  static constexpr bool kBf16 = true;
  uint32_t v[16];
  __device__ __forceinline__ void operator()(int j, float lo, float hi) { v[j] = pack_bf16(lo, hi); }
  __device__ __forceinline__ void put(int j, uint32_t p) { v[j] = p; }
};

// Sink that keeps only pairs 4K .. 4K + 3 of a block (the 8 codes of MFMA
// k-step K), as packed bf16; the other pairs are dead code once inlined.
template <int K>
struct SinkBf16Step {
  static constexpr bool kBf16 = true;
  uint32_t v[4];
  __device__ __forceinline__ void operator()(int j, float lo, float hi) {
    if ((j >> 2) == K) v[j & 3] = pack_bf16(lo, hi);
  }
  __device__ __forceinline__ void put(int j, uint32_t p) {
    if ((j >> 2) == K) v[j & 3] = p;
  }
};

// The bf16 MFMA operand words of k-step k (0..3) of one block.
template <int BITS>
__device__ __forceinline__ void dequant_kstep(int k, const uint32_t* w, uint32_t dm,
                                              uint32_t (&out)[4]) {
  if constexpr (BITS == kMx4) {
    // k-step k is exactly field word k: four conversions
    const float s = mx_scale(dm);
    out[0] = mx_pair_bf16<0>(w[k], s);
    out[1] = mx_pair_bf16<1>(w[k], s);
    out[2] = mx_pair_bf16<2>(w[k], s);
    out[3] = mx_pair_bf16<3>(w[k], s);
    return;
  }
  switch (k) {
    case 0: { SinkBf16Step<0> s; dequant_block<BITS>(w, dm, s); for (int i = 0; i < 4; i++) out[i] = s.v[i]; break; }
    case 1: { SinkBf16Step<1> s; dequant_block<BITS>(w, dm, s); for (int i = 0; i < 4; i++) out[i] = s.v[i]; break; }
    case 2: { SinkBf16Step<2> s; dequant_block<BITS>(w, dm, s); for (int i = 0; i < 4; i++) out[i] = s.v[i]; break; }
    default: { SinkBf16Step<3> s; dequant_block<BITS>(w, dm, s); for (int i = 0; i < 4; i++) out[i] = s.v[i]; break; }
  }
}

// Sink that keeps fp32 values (fp32 activations).
struct SinkF32 {
  static constexpr bool kBf16 = false;
  float v[32];
  __device__ __forceinline__ void operator()(int j, float lo, float hi) {
    v[2 * j] = lo;
    v[2 * j + 1] = hi;
  }
};

// Loads the code field of a block: `BITS` dwords (4 for MXFP4).  A kernel
// reads each weight block once, so the loads carry the non-temporal hint.
template <int BITS>
__device__ __forceinline__ void load_field(const uint8_t* p, uint32_t* w) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (BITS == 4 || BITS == kMx4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 3) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = __builtin_nontemporal_load(q);
    w[1] = __builtin_nontemporal_load(q + 1);
    w[2] = __builtin_nontemporal_load(q + 2);
  } else {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = v.x; w[1] = v.y;
  }
}

// The code field of block `idx` of a table and its scale entry: the (d, m)
// word, or the zero-extended E8M0 byte of an MXFP4 table.
template <int BITS>
__device__ __forceinline__ const uint8_t* field_ptr(const uint8_t* codes, size_t idx) {
  return codes + idx * field_bytes(BITS);
}
template <int BITS>
__device__ __forceinline__ uint32_t load_scale(const uint32_t* dm, size_t idx) {
  if constexpr (BITS == kMx4) return reinterpret_cast<const uint8_t*>(dm)[idx];
  else return dm[idx];
}

// Copies n uint4 from global memory into LDS with the whole workgroup,
// eight loads per thread in flight before their stores (a plain strided loop
// would wait for each load before the next).  `src_at(i)` gives the address
// of element i.
template <typename SrcAt>
__device__ __forceinline__ void copy_to_lds(uint4* __restrict__ dst, int n, SrcAt src_at) {
  const int nt = blockDim.x;
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * nt) {
    // unconditional loads from clamped indices, no branch between them; the
    // eight words are named values, not an array, so they stay in registers
    const auto ld = [&](int j) { return *src_at(min(i0 + j * nt, n - 1)); };
    const uint4 v0 = ld(0), v1 = ld(1), v2 = ld(2), v3 = ld(3);
    const uint4 v4 = ld(4), v5 = ld(5), v6 = ld(6), v7 = ld(7);
    const auto st = [&](int j, const uint4& v) {
      const int i = i0 + j * nt;
      if (i < n) dst[i] = v;
    };
    st(0, v0); st(1, v1); st(2, v2); st(3, v3);
    st(4, v4); st(5, v5); st(6, v6); st(7, v7);
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

// Wave sums of 8 candidates at once: p[c] is this lane's partial of
// candidate c.  Each exchange hands the half of the candidates this lane does
// not keep to its partner, so candidate c's total ends in lanes 8c .. 8c + 7
// after 10 fp64 exchanges instead of 48.  Every addition pairs the same two
// partial sums as wave_sum_f64 (partners at distance 32, 16, 8, 4, 2, 1), so
// each total is bit-identical to wave_sum_f64 of that candidate's partials.
__device__ __forceinline__ double wave_sum8_f64(const double (&p)[8], int lane) {
  // every element read at a constant index, and every choice made between
  // values: a select between two elements of p would otherwise be folded into
  // one load at a lane-dependent index, which keeps p in scratch memory
  const double p0 = p[0], p1 = p[1], p2 = p[2], p3 = p[3];
  const double p4 = p[4], p5 = p[5], p6 = p[6], p7 = p[7];
  const bool h32 = (lane >> 5) & 1, h16 = (lane >> 4) & 1, h8 = (lane >> 3) & 1;
  const double q0 = (h32 ? p4 : p0) + __shfl_xor(h32 ? p0 : p4, 32, 64);
  const double q1 = (h32 ? p5 : p1) + __shfl_xor(h32 ? p1 : p5, 32, 64);
  const double q2 = (h32 ? p6 : p2) + __shfl_xor(h32 ? p2 : p6, 32, 64);
  const double q3 = (h32 ? p7 : p3) + __shfl_xor(h32 ? p3 : p7, 32, 64);
  const double r0 = (h16 ? q2 : q0) + __shfl_xor(h16 ? q0 : q2, 16, 64);
  const double r1 = (h16 ? q3 : q1) + __shfl_xor(h16 ? q1 : q3, 16, 64);
  double v = (h8 ? r1 : r0) + __shfl_xor(h8 ? r0 : r1, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

// silu(z) = z / (1 + e^-z) from the hardware 2^x and reciprocal (v_exp_f32,
// v_rcp_f32, about 1 ulp each): a few fp32 ulp in all, far below the bf16
// rounding of h that follows, at a third of the instructions of expf and an
// IEEE division.  z -> -inf gives -0 (e^-z = inf, 1/inf = 0); NaN stays NaN.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Top-K ordering and a DPP wave argmax.
// ---------------------------------------------------------------------------

// Monotone map of a key to uint64: larger key -> larger value; -0 == +0;
// NaN maps to 0, below every number.
__device__ __forceinline__ uint64_t order_key(double k) {
  if (k != k) return 0ull;
  if (k == 0.0) k = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(k);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Inverse of order_key (0 -> NaN).
__device__ __forceinline__ double key_of_order(uint64_t u) {
  if (u == 0ull) return __longlong_as_double(0x7FF8000000000000ll);
  const uint64_t b = (u >> 63) ? (u & 0x7FFFFFFFFFFFFFFFull) : ~u;
  return __longlong_as_double((long long)b);
}

// (key descending, id ascending)
__device__ __forceinline__ bool ranks_before(uint64_t au, uint32_t aid, uint64_t bu, uint32_t bid) {
  return au > bu || (au == bu && aid < bid);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(uint64_t& u, uint32_t& id) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)u);
  const uint32_t hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  const uint32_t oid = dpp_u32<CTRL>(id);
  const uint64_t ou = ((uint64_t)hi << 32) | lo;
  if (ranks_before(ou, oid, u, id)) {
    u = ou;
    id = oid;
  }
}

__device__ __forceinline__ void argmax_readlane(uint64_t& bu, uint32_t& bid, uint64_t u, uint32_t id,
                                                int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  const uint32_t oid = (uint32_t)__builtin_amdgcn_readlane((int)id, lane);
  const uint64_t ou = ((uint64_t)hi << 32) | lo;
  if (ranks_before(ou, oid, bu, bid)) {
    bu = ou;
    bid = oid;
  }
}

// Wave-wide best (key, id) pair: quads, then rows of 16 by two row
// rotations, then the four rows through readlane.  Returns the same result
// in every lane.
__device__ __forceinline__ void wave_argmax(uint64_t& u, uint32_t& id) {
  argmax_dpp_step<0xB1>(u, id);   // quad_perm [1,0,3,2]
  argmax_dpp_step<0x4E>(u, id);   // quad_perm [2,3,0,1]
  argmax_dpp_step<0x124>(u, id);  // row_ror:4
  argmax_dpp_step<0x128>(u, id);  // row_ror:8
  uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 0) << 32) |
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 0);
  uint32_t bid = (uint32_t)__builtin_amdgcn_readlane((int)id, 0);
  argmax_readlane(bu, bid, u, id, 16);
  argmax_readlane(bu, bid, u, id, 32);
  argmax_readlane(bu, bid, u, id, 48);
  u = bu;
  id = bid;
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Sorted-list top-K of one wave.  Each lane holds KPL (key, id) pairs
// (expert ids lane, lane+64, ...), sorts them once (descending by
// (key, -id)), and every round takes the wave argmax of the lane heads; the
// winning lane (ids are unique) shifts its list.  Lanes r < rounds end with
// the r-th best id in *sel_id and its order key in *sel_u.
// ---------------------------------------------------------------------------

template <int KPL>
struct SortedKeys {
  uint64_t u[KPL];
  uint32_t id[KPL];
  __device__ __forceinline__ void cswap(int a, int b) {
    if (ranks_before(u[b], id[b], u[a], id[a])) {
      const uint64_t tu = u[a];
      const uint32_t ti = id[a];
      u[a] = u[b];
      id[a] = id[b];
      u[b] = tu;
      id[b] = ti;
    }
  }
  __device__ __forceinline__ void sort() {
    if constexpr (KPL == 2) {
      cswap(0, 1);
    } else if constexpr (KPL == 4) {
      cswap(0, 1); cswap(2, 3); cswap(0, 2); cswap(1, 3); cswap(1, 2);
    } else if constexpr (KPL == 8) {
      // 19-comparator optimal network (depth 6)
      cswap(0, 2); cswap(1, 3); cswap(4, 6); cswap(5, 7);
      cswap(0, 4); cswap(1, 5); cswap(2, 6); cswap(3, 7);
      cswap(0, 1); cswap(2, 3); cswap(4, 5); cswap(6, 7);
      cswap(2, 4); cswap(3, 5);
      cswap(1, 4); cswap(3, 6);
      cswap(1, 2); cswap(3, 4); cswap(5, 6);
    }
  }
};

// Mixing weights over the K selected keys (lane r holds key r): softmax in
// float64, stored fp32.
__device__ __forceinline__ float topk_weight(double key, int lane, int K) {
  const double k0 = __shfl(key, 0, 64);
  const double z = lane < K ? exp(key - k0) : 0.0;
  const double sum = wave_sum_f64(z);
  return (float)(z / sum);
}

template <int KPL>
__device__ __forceinline__ void topk_sorted(const double* __restrict__ krow, int E, int rounds,
                                            int lane, int* sel_id, uint64_t* sel_u) {
  static_assert(KPL == 1 || KPL == 2 || KPL == 4 || KPL == 8, "KPL");
  SortedKeys<KPL> L;
  // unconditional loads (clamped index), so all KPL are in flight at once
  double kv[KPL];
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const int e = lane + 64 * j;
    kv[j] = krow[e < E ? e : E - 1];
  }
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const int e = lane + 64 * j;
    L.u[j] = e < E ? order_key(kv[j]) : 0ull;
    L.id[j] = e < E ? (uint32_t)e : 0xFFFFFFFFu;
  }
  L.sort();
  int my_id = -1;
  uint64_t my_u = 0;
  for (int r = 0; r < rounds; r++) {
    uint64_t bu = L.u[0];
    uint32_t bid = L.id[0];
    wave_argmax(bu, bid);
    if (lane == r) {
      my_id = (int)bid;
      my_u = bu;
    }
    if (L.id[0] == bid) {  // this lane's head won: drop it
#pragma unroll
      for (int j = 0; j + 1 < KPL; j++) {
        L.u[j] = L.u[j + 1];
        L.id[j] = L.id[j + 1];
      }
      L.u[KPL - 1] = 0ull;
      L.id[KPL - 1] = 0xFFFFFFFFu;
    }
  }
  *sel_id = my_id;
  *sel_u = my_u;
}


// Helpers of the threshold top-K below.
template <int CTRL>
__device__ __forceinline__ double dpp_max_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return fmax(v, __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-wide maximum of a and of b (all 64 lanes active), the two chains
// interleaved: quads, rows of 16, then the four rows.
__device__ __forceinline__ void wave_max2_f64(double& a, double& b) {
  a = dpp_max_f64<0xB1>(a);  b = dpp_max_f64<0xB1>(b);    // quad_perm [1,0,3,2]
  a = dpp_max_f64<0x4E>(a);  b = dpp_max_f64<0x4E>(b);    // quad_perm [2,3,0,1]
  a = dpp_max_f64<0x124>(a); b = dpp_max_f64<0x124>(b);   // row_ror:4
  a = dpp_max_f64<0x128>(a); b = dpp_max_f64<0x128>(b);   // row_ror:8
  a = fmax(fmax(readlane_f64(a, 0), readlane_f64(a, 16)), fmax(readlane_f64(a, 32), readlane_f64(a, 48)));
  b = fmax(fmax(readlane_f64(b, 0), readlane_f64(b, 16)), fmax(readlane_f64(b, 32), readlane_f64(b, 48)));
}

// Number of keys >= th over the wave (empty slots hold -inf), wave-uniform.
template <int KPL>
__device__ __forceinline__ int count_ge(const double (&kv)[KPL], double th) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < KPL; j++) c += __popcll(__ballot(kv[j] >= th));
  return c;
}

// ---------------------------------------------------------------------------
// Threshold top-K of one wave (E <= 64 * KPL keys, lane l holding ids
// l + 64 j).  The keys are counted into 256 value bins of equal width between
// the smallest and the largest key; one scan from the top bin down finds the
// bin that holds the rounds-th key, and the keys in it and above are the
// candidates.  When that leaves more than 64 (clustered keys), a value
// threshold is bisected with ballot counts until between `rounds` and
// rounds + 8 keys reach it.  The candidates are compacted one per lane and
// each is ranked exactly by (key desc, id asc) against the others, read from
// the other lanes' registers.  The result equals the sorted-list selection
// above, which remains the fallback when the field cannot be narrowed to 64
// keys (many equal keys) or holds NaN or infinite keys.  `scratch` is 64 slots of
// LDS owned by this wave.  Lanes r < rounds end with the r-th best id and its
// order key; the other lanes with -1 and 0.
// ---------------------------------------------------------------------------

struct TopkSlot {
  uint64_t u;
  uint32_t id;
  uint32_t pad;
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exact top-`rounds` of nc <= 64 candidates held one per lane (lane i < nc:
// order key mu, id mid_): each candidate's rank (key desc, id asc) is counted
// against the others, read from their registers; lane r < rounds ends with
// the r-th best.  `scratch`: 64 slots of LDS owned by this wave.
__device__ __forceinline__ void rank_select(uint64_t mu, uint32_t mid_, int nc, int rounds,
                                            int lane, TopkSlot* __restrict__ scratch,
                                            int* sel_id, uint64_t* sel_u) {
  int rank = 0;
  for (int i = 0; i < nc; i++) {
    const uint32_t ulo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mu, i);
    const uint32_t uhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mu >> 32), i);
    const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)mid_, i);
    rank += ranks_before(((uint64_t)uhi << 32) | ulo, id, mu, mid_) ? 1 : 0;
  }
  if (lane < nc && rank < rounds) {
    scratch[rank].u = mu;
    scratch[rank].id = mid_;
  }
  wave_sync_lds();
  if (lane < rounds) {
    *sel_u = scratch[lane].u;
    *sel_id = (int)scratch[lane].id;
  } else {
    *sel_u = 0;
    *sel_id = -1;
  }
  wave_sync_lds();
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): four
// shifts inside each row of 16, then the row totals broadcast upwards.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

template <int KPL>
__device__ __forceinline__ void topk_threshold(const double* __restrict__ krow, int E, int rounds,
                                               int lane, TopkSlot* __restrict__ scratch,
                                               int* sel_id, uint64_t* sel_u) {
  static_assert(KPL == 1 || KPL == 2 || KPL == 4 || KPL == 8, "KPL");
  double kv[KPL];
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const int e = lane + 64 * j;
    kv[j] = krow[e < E ? e : E - 1];
  }
  double mx = -INFINITY, nmn = -INFINITY;   // max and -min over the valid keys
  bool bad = false;
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const bool ok = lane + 64 * j < E;
    bad |= ok && !(fabs(kv[j]) < INFINITY);   // NaN or infinite
    if (!ok) kv[j] = -INFINITY;
    if (ok) {
      mx = fmax(mx, kv[j]);
      nmn = fmax(nmn, -kv[j]);
    }
  }
  bad = __ballot(bad) != 0;
  const int want = rounds + 8 < 64 ? rounds + 8 : 64;
  // Candidate set: the keys in value bin >= cb (histogram pass), else the
  // keys >= th (bisection).  Either way every key outside the set is smaller
  // than every key inside it, so the top `rounds` are among the candidates.
  bool found = false, use_bins = false;
  int cb = 0;
  double th = 0.0;
  int bin[KPL];
#pragma unroll
  for (int j = 0; j < KPL; j++) bin[j] = -1;
  if (!bad) {
    wave_max2_f64(mx, nmn);
    double lo = -nmn, hi = mx;               // count(>= lo) = E >= rounds
    if (E <= want) {
      th = lo;
      found = true;
    } else if (hi > lo) {
      // 256 bins of equal width over [lo, hi] (the bin index is monotone in
      // the key), counted in an LDS histogram that aliases the scratch slots;
      // one scan from the top bin down finds the bin holding the rounds-th key
      uint32_t* hist = reinterpret_cast<uint32_t*>(scratch);
      reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
      wave_sync_lds();
      const double scale = 256.0 / (hi - lo);
#pragma unroll
      for (int j = 0; j < KPL; j++) {
        const double f = fmin(fmax((kv[j] - lo) * scale, 0.0), 255.0);
        if (lane + 64 * j < E) {
          bin[j] = (int)f;
          atomicAdd(&hist[bin[j]], 1u);
        }
      }
      wave_sync_lds();
      int cum = 0;
      cb = -1;
      for (int pass = 0; pass < 4 && cb < 0; pass++) {
        const int c = wave_incl_scan((int)hist[255 - 64 * pass - lane]) + cum;
        const uint64_t m = __ballot(c >= rounds);
        if (m) cb = 255 - 64 * pass - (int)__builtin_ctzll(m);
        else cum = __builtin_amdgcn_readlane(c, 63);
      }
      wave_sync_lds();
      int nb = 0;
#pragma unroll
      for (int j = 0; j < KPL; j++) nb += __popcll(__ballot(bin[j] >= 0 && bin[j] >= cb));
      if (cb >= 0 && nb >= rounds && nb <= 64) {
        use_bins = true;
        found = true;
      }
    }
    if (!found && hi > lo) {
      for (int it = 0; it < 64 && !found; it++) {
        const double mid = lo + (hi - lo) * 0.5;
        if (!(mid > lo && mid < hi)) break;   // no room left: equal keys
        const int c = count_ge<KPL>(kv, mid);
        if (c < rounds) hi = mid;
        else if (c > want) lo = mid;
        else { th = mid; found = true; }
      }
    }
    if (!found && count_ge<KPL>(kv, lo) <= 64) {   // ties: take the wider set
      th = lo;
      found = true;
    }
  }
  if (!found) {
    topk_sorted<KPL>(krow, E, rounds, lane, sel_id, sel_u);
    return;
  }
  // compact the candidates: candidate i goes to lane i
  int nc = 0;
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const bool c = use_bins ? (bin[j] >= 0 && bin[j] >= cb) : kv[j] >= th;
    const uint64_t m = __ballot(c);
    if (c) {
      const int pos = nc + __popcll(m & ((1ull << lane) - 1ull));
      scratch[pos].u = order_key(kv[j]);
      scratch[pos].id = (uint32_t)(lane + 64 * j);
    }
    nc += __popcll(m);
  }
  wave_sync_lds();
  uint64_t mu = 0;
  uint32_t mid_ = 0xFFFFFFFFu;
  if (lane < nc) {
    mu = scratch[lane].u;
    mid_ = scratch[lane].id;
  }
  wave_sync_lds();
  rank_select(mu, mid_, nc, rounds, lane, scratch, sel_id, sel_u);
}

}  // namespace moe
