// Decode path (A5, A6): a group of up to 16 tokens, streamed once over the
// union of its experts.
//
// Every contraction runs as 16x16 MFMA tiles with the group's tokens on the
// M side (rows >= T are zero) and 16 weight rows on the N side.  A lane owns
// one quantised block (32 weights) of one weight row per 128-wide super-step:
// it loads the block's code field and (d, m) word with one coalesced
// wave-wide read of a tile (64 blocks, 16 rows x 4 blocks), dequantises it
// in registers straight into MFMA operand words, and never stages weights in
// LDS.  The pages fuse gate, up and the activation into one decode kernel
// (P1, "step 4: three shelves, all on the GPU"; "the four bugs, briefly"),
// as done here; each work item carries its tier and slot explicitly instead
// of a tag on a graph node.
#include "device_common.hpp"

namespace moe {

namespace {

// ---- one lane's share of a 128-wide super-step -------------------------------

// A operand: 32 consecutive activations of token row `row` (zeros if !valid).
template <typename A>
struct Frag;

template <>
struct Frag<bf16_t> {
  uint32_t v[16];  // 32 bf16, packed pairs
  __device__ __forceinline__ void load_act(const bf16_t* p, bool valid) {
    if (valid) {
      const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 t = q[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) v[i] = 0u;
    }
  }
  template <int BITS>
  __device__ __forceinline__ void load_quant(const uint8_t* codes, const uint32_t* dm, size_t idx) {
    uint32_t w[4];
    load_field<BITS>(codes + idx * (4 * BITS), w);
    SinkBf16 sink;
    dequant_block<BITS>(w, dm[idx], sink);
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = sink.v[i];
  }
};

template <>
struct Frag<float> {
  float v[32];
  __device__ __forceinline__ void load_act(const float* p, bool valid) {
    if (valid) {
      const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float4 t = q[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; i++) v[i] = 0.0f;
    }
  }
  template <int BITS>
  __device__ __forceinline__ void load_quant(const uint8_t* codes, const uint32_t* dm, size_t idx) {
    uint32_t w[4];
    load_field<BITS>(codes + idx * (4 * BITS), w);
    SinkF32 sink;
    dequant_block<BITS>(w, dm[idx], sink);
#pragma unroll
    for (int i = 0; i < 32; i++) v[i] = sink.v[i];
  }
};

// acc += A(16 x 128) * B(128 x 16) for one super-step.
__device__ __forceinline__ f32x4_t mma_step(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x4_t acc) {
#pragma unroll
  for (int i = 0; i < 4; i++)
    acc = mfma_bf16(a.v[4 * i], a.v[4 * i + 1], a.v[4 * i + 2], a.v[4 * i + 3], b.v[4 * i],
                    b.v[4 * i + 1], b.v[4 * i + 2], b.v[4 * i + 3], acc);
  return acc;
}

__device__ __forceinline__ f32x4_t mma_step(const Frag<float>& a, const Frag<float>& b, f32x4_t acc) {
#pragma unroll
  for (int s = 0; s < 32; s++) acc = mfma_f32(a.v[s], b.v[s], acc);
  return acc;
}

template <typename A>
__device__ __forceinline__ void store_act(A* p, float v);
template <>
__device__ __forceinline__ void store_act<bf16_t>(bf16_t* p, float v) { *p = to_bf16(v); }
template <>
__device__ __forceinline__ void store_act<float>(float* p, float v) { *p = v; }

// ---- A5: gate + up + SwiGLU --------------------------------------------------

// Shared expert: dense weights in the act dtype, row-major [I][H].
template <typename A>
__device__ __forceinline__ void gateup_loop_dense(const A* __restrict__ x, int T, int H, int rg,
                                                  const Tables& tb, int wave, int lane,
                                                  f32x4_t& accg, f32x4_t& accu) {
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = H / 128;
  const A* wg = reinterpret_cast<const A*>(tb.dense[MOE_GATE]);
  const A* wu = reinterpret_cast<const A*>(tb.dense[MOE_UP]);
  for (int c = wave; c < nbg; c += 4) {
    Frag<A> xa, bg, bu;
    const size_t off = (size_t)(rg * 16 + lm) * H + 128 * c + 32 * lg;
    bg.load_act(wg + off, true);
    bu.load_act(wu + off, true);
    xa.load_act(x + (size_t)lm * H + 128 * c + 32 * lg, lm < T);
    accg = mma_step(xa, bg, accg);
    accu = mma_step(xa, bu, accu);
  }
}

template <typename A, int BITS>
__device__ __forceinline__ void gateup_loop_q(const A* __restrict__ x, int T, int H, int I, int rg,
                                              int tier, int slot, const Tables& tb, int wave,
                                              int lane, f32x4_t& accg, f32x4_t& accu) {
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = H / 128, nrg = I / 16;
  const uint8_t* cg = tb.codes[tier][MOE_GATE];
  const uint8_t* cu = tb.codes[tier][MOE_UP];
  const uint32_t* dg = tb.dm[tier][MOE_GATE];
  const uint32_t* du = tb.dm[tier][MOE_UP];
  const size_t tile0 = ((size_t)slot * nrg + rg) * nbg;
  for (int c = wave; c < nbg; c += 4) {
    Frag<A> xa, bg, bu;
    const size_t idx = (tile0 + c) * 64 + lane;
    bg.template load_quant<BITS>(cg, dg, idx);
    bu.template load_quant<BITS>(cu, du, idx);
    xa.load_act(x + (size_t)lm * H + 128 * c + 32 * lg, lm < T);
    accg = mma_step(xa, bg, accg);
    accu = mma_step(xa, bu, accu);
  }
}

template <typename A>
__global__ __launch_bounds__(256) void k_decode_gateup(const Item* __restrict__ items,
                                                       const int32_t* __restrict__ n_items,
                                                       const A* __restrict__ x, int T, Tables tb,
                                                       A* __restrict__ h, int H, int I) {
  __shared__ float red[4][8][64];
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  if (u >= *n_items) return;
  const int tier = items[u].tier;
  if (tier < 0) return;
  const int slot = items[u].slot, bits = items[u].bits;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  if (tier == kDenseTier)
    gateup_loop_dense<A>(x, T, H, rg, tb, wave, lane, accg, accu);
  else if (bits == 4)
    gateup_loop_q<A, 4>(x, T, H, I, rg, tier, slot, tb, wave, lane, accg, accu);
  else if (bits == 3)
    gateup_loop_q<A, 3>(x, T, H, I, rg, tier, slot, tb, wave, lane, accg, accu);
  else
    gateup_loop_q<A, 2>(x, T, H, I, rg, tier, slot, tb, wave, lane, accg, accu);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    red[wave][i][lane] = accg[i];
    red[wave][4 + i][lane] = accu[i];
  }
  __syncthreads();
  if (wave != 0) return;
  const int lm = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float g = 0.f, up = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      g += red[w][i][lane];
      up += red[w][4 + i][lane];
    }
    const int t = 4 * lg + i;
    if (t < T) {
      const int r = items[u].route[t];
      if (r >= 0) store_act<A>(h + (size_t)r * I + rg * 16 + lm, silu_f32(g) * up);
    }
  }
}

// ---- A6: down + weighted combine --------------------------------------------

template <typename A, int BITS>
__device__ __forceinline__ f32x4_t down_pair(const A* __restrict__ h, int r, int H, int I, int rg,
                                             int c, int tier, int slot, const Tables& tb, int lane) {
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128, nrg = H / 16;
  Frag<A> ha, bd;
  if constexpr (BITS == 0) {
    const size_t off = (size_t)(rg * 16 + lm) * I + 128 * c + 32 * lg;
    bd.load_act(reinterpret_cast<const A*>(tb.dense[MOE_DOWN]) + off, true);
  } else {
    const size_t idx = (((size_t)slot * nrg + rg) * nbg + c) * 64 + lane;
    bd.template load_quant<BITS>(tb.codes[tier][MOE_DOWN], tb.dm[tier][MOE_DOWN], idx);
  }
  ha.load_act(h + (size_t)(r < 0 ? 0 : r) * I + 128 * c + 32 * lg, r >= 0);
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return mma_step(ha, bd, z);
}

template <typename A, typename Y>
__global__ __launch_bounds__(512) void k_decode_down(const Item* __restrict__ items,
                                                     const int32_t* __restrict__ n_items,
                                                     const A* __restrict__ h, int T, Tables tb,
                                                     Y* __restrict__ y, int H, int I) {
  __shared__ float red[8][4][64];
  const int rg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128;
  const int npairs = *n_items * nbg;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = wave; p < npairs; p += 8) {
    const int u = p / nbg, c = p % nbg;
    const Item& it = items[u];
    const int tier = it.tier;
    if (tier < 0) continue;
    const int r = lm < T ? it.route[lm] : -1;
    f32x4_t part;
    if (tier == kDenseTier)
      part = down_pair<A, 0>(h, r, H, I, rg, c, tier, 0, tb, lane);
    else if (it.bits == 4)
      part = down_pair<A, 4>(h, r, H, I, rg, c, tier, it.slot, tb, lane);
    else if (it.bits == 3)
      part = down_pair<A, 3>(h, r, H, I, rg, c, tier, it.slot, tb, lane);
    else
      part = down_pair<A, 2>(h, r, H, I, rg, c, tier, it.slot, tb, lane);
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] += it.gw[4 * lg + i] * part[i];
  }
#pragma unroll
  for (int i = 0; i < 4; i++) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 8; w++) s += red[w][i][lane];
    const int t = 4 * lg + i;
    if (t < T) {
      Y* out = y + (size_t)t * H + rg * 16 + lm;
      if constexpr (sizeof(Y) == 4) *out = s; else *out = to_bf16(s);
    }
  }
}

}  // namespace

void launch_decode_gateup(int act, const Item* items, const int32_t* n_items, int max_items,
                          const void* x, int T, const Tables& tb, void* h, int H, int I,
                          hipStream_t s) {
  dim3 grid(max_items * (I / 16));
  if (act == MOE_BF16)
    MOE_LAUNCH(MOE_K_DECODE_GATEUP, k_decode_gateup<bf16_t>, grid, dim3(256), 0, s, items, n_items,
                       (const bf16_t*)x, T, tb, (bf16_t*)h, H, I);
  else
    MOE_LAUNCH(MOE_K_DECODE_GATEUP, k_decode_gateup<float>, grid, dim3(256), 0, s, items, n_items,
                       (const float*)x, T, tb, (float*)h, H, I);
}

void launch_decode_down(int act, int y_dt, const Item* items, const int32_t* n_items,
                        int max_items, const void* h, int T, const Tables& tb, void* y, int H,
                        int I, hipStream_t s) {
  (void)max_items;
  dim3 grid(H / 16);
  if (act == MOE_BF16) {
    if (y_dt == MOE_BF16)
      MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<bf16_t, bf16_t>), grid, dim3(512), 0, s, items, n_items,
                         (const bf16_t*)h, T, tb, (bf16_t*)y, H, I);
    else
      MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<bf16_t, float>), grid, dim3(512), 0, s, items, n_items,
                         (const bf16_t*)h, T, tb, (float*)y, H, I);
  } else {
    MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<float, float>), grid, dim3(512), 0, s, items, n_items,
                       (const float*)h, T, tb, (float*)y, H, I);
  }
}

}  // namespace moe
