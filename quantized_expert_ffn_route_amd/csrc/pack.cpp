// Host-side block quantiser and code packer.  Pure C++: no HIP calls, so the
// tier build can run (and be tested) on a machine without a GPU.
//
// Compiled with -ffp-contract=off: every step below is one IEEE fp32
// operation rounded to nearest-even, as the block format specifies.

#include <cmath>
#include <cstring>

#include "internal.hpp"

namespace moe {

namespace {

inline uint16_t f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest, ties to even
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

inline float f16_value(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}

inline bool f16_finite(uint16_t b) { return (b & 0x7C00u) != 0x7C00u; }

}  // namespace

// Affine block of 32 weights with an fp16 scale and fp16 min.  Storing each
// weight with fewer bits is the method's compression (P1, "a small
// dictionary before we start"; "step 4: three shelves, all on the GPU").
int quantise_block(const float* x, int bits, uint16_t* d_out, uint16_t* m_out, uint8_t* q) {
  const int L = (1 << bits) - 1;
  float lo = x[0], hi = x[0];
  for (int i = 0; i < 32; i++) {
    if (!std::isfinite(x[i])) return MOE_EINVAL;
    lo = x[i] < lo ? x[i] : lo;
    hi = x[i] > hi ? x[i] : hi;
  }
  const uint16_t mb = f16_bits(lo);
  volatile float span = hi - lo;  // one fp32 rounding
  volatile float step = span / (float)L;
  const uint16_t db = f16_bits(step);
  if (!f16_finite(mb) || !f16_finite(db)) return MOE_EINVAL;
  const float m = f16_value(mb), d = f16_value(db);
  for (int i = 0; i < 32; i++) {
    if (d == 0.0f) {
      q[i] = 0;
      continue;
    }
    volatile float diff = x[i] - m;
    volatile float t = diff / d;
    float r = std::nearbyint(t);  // default rounding mode: ties to even
    r = r < 0.0f ? 0.0f : (r > (float)L ? (float)L : r);
    q[i] = (uint8_t)r;
  }
  *d_out = db;
  *m_out = mb;
  return MOE_OK;
}

// MXFP4 block (OCP Microscaling v1.0; the pages' low down tier, P1 "step 4:
// three shelves, all on the GPU"): 32 E2M1 codes sharing the scale 2^X with
// X = floor(log2(max|x|)) - 2, clamped to [-125, 125] so that every element
// is a normal float (X = -125 for an all-zero block).  Each code is the E2M1
// value nearest to x / 2^X (exact in double), ties to the even mantissa,
// magnitudes above 6 saturating to 6; zero is code 0.
int quantise_block_mx(const float* x, uint8_t* e_out, uint8_t* q) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) {
    if (!std::isfinite(x[i])) return MOE_EINVAL;
    amax = std::fabs(x[i]) > amax ? std::fabs(x[i]) : amax;
  }
  int X = -125;
  if (amax > 0.0f) {
    int ex;
    std::frexp(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    X = ex - 1 - 2;
  }
  X = X < -125 ? -125 : (X > 125 ? 125 : X);
  // E2M1 magnitudes by code; a magnitude moves up to code k past the midpoint
  // of codes k-1 and k, or at it when k is even (the even mantissa)
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  for (int i = 0; i < 32; i++) {
    const double t = std::ldexp((double)x[i], -X);
    const double a = std::fabs(t);
    int k = 0;
    if (a > 6.0) {
      k = 7;
    } else {
      for (int c = 1; c < 8; c++) {
        const double mid = 0.5 * (mag[c - 1] + mag[c]);
        if (a > mid || (a == mid && (c & 1) == 0)) k = c;
      }
    }
    q[i] = (uint8_t)(k | (t < 0.0 && k > 0 ? 8 : 0));
  }
  *e_out = (uint8_t)(X + 127);
  return MOE_OK;
}

// Code field of one block: `bits` little-endian 32-bit words.  In every word
// the low half holds even-numbered codes and the high half the following odd
// codes at the same offsets, packed from bit 0.  4 bits: word i holds codes
// 8i..8i+7; 2 bits: word i holds codes 16i..16i+15; 3 bits: word i holds
// codes 10i..10i+9 and the top bit of each half-word of words 0..2 carries
// one bit of codes 30 (low halves) and 31 (high halves).
// MXFP4: 16 bytes, code k in bits 4k..4k+3 (byte k/2, low nibble for even k).
void encode_codes(const uint8_t* q, int bits, uint8_t* field) {
  if (bits == kMx4) {
    for (int j = 0; j < 16; j++) field[j] = (uint8_t)((q[2 * j] & 15u) | (q[2 * j + 1] & 15u) << 4);
    return;
  }
  uint32_t w[4] = {0, 0, 0, 0};
  if (bits == 4) {
    for (int k = 0; k < 32; k++) {
      int i = k / 8, p = (k % 8) / 2, s = k % 2;
      w[i] |= (uint32_t)(q[k] & 15u) << (16 * s + 4 * p);
    }
  } else if (bits == 2) {
    for (int k = 0; k < 32; k++) {
      int i = k / 16, p = (k % 16) / 2, s = k % 2;
      w[i] |= (uint32_t)(q[k] & 3u) << (16 * s + 2 * p);
    }
  } else {  // bits == 3
    for (int k = 0; k < 30; k++) {
      int i = k / 10, p = (k % 10) / 2, s = k % 2;
      w[i] |= (uint32_t)(q[k] & 7u) << (16 * s + 3 * p);
    }
    for (int s = 0; s < 2; s++)
      for (int r = 0; r < 3; r++) w[r] |= (uint32_t)((q[30 + s] >> r) & 1u) << (16 * s + 15);
  }
  for (int i = 0; i < bits; i++) {
    field[4 * i + 0] = (uint8_t)(w[i]);
    field[4 * i + 1] = (uint8_t)(w[i] >> 8);
    field[4 * i + 2] = (uint8_t)(w[i] >> 16);
    field[4 * i + 3] = (uint8_t)(w[i] >> 24);
  }
}

}  // namespace moe
