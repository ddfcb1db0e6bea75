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

// Raw (not yet dequantised) B-operand data of one lane for one super-step:
// a quantised block's code field and (d, m) word, or 32 dense act values.
template <typename A>
struct Raw {
  uint32_t v[16 * sizeof(A) / 2];  // dense: 32 act values; quantised: w[0..3], dm in v[4]
};

template <typename A, int BITS>
__device__ __forceinline__ void load_raw(Raw<A>& r, const uint8_t* codes, const uint32_t* dm,
                                         size_t idx) {
  load_field<BITS>(codes + idx * (4 * BITS), r.v);
  r.v[4] = dm[idx];
}

template <typename A>
__device__ __forceinline__ void load_raw_dense(Raw<A>& r, const A* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(A) * 2); i++) {
    const uint4 t = q[i];
    r.v[4 * i] = t.x; r.v[4 * i + 1] = t.y; r.v[4 * i + 2] = t.z; r.v[4 * i + 3] = t.w;
  }
}

// Raw -> MFMA operand fragment.
template <typename A, int BITS>
__device__ __forceinline__ void to_frag(Frag<A>& f, const Raw<A>& r) {
  if constexpr (BITS == 0) {
#pragma unroll
    for (int i = 0; i < (int)(16 * sizeof(A) / 2); i++) {
      if constexpr (sizeof(A) == 2) f.v[i] = r.v[i]; else f.v[i] = __uint_as_float(r.v[i]);
    }
  } else if constexpr (sizeof(A) == 2) {
    SinkBf16 sink;
    dequant_block<BITS>(r.v, r.v[4], sink);
#pragma unroll
    for (int i = 0; i < 16; i++) f.v[i] = sink.v[i];
  } else {
    SinkF32 sink;
    dequant_block<BITS>(r.v, r.v[4], sink);
#pragma unroll
    for (int i = 0; i < 32; i++) f.v[i] = sink.v[i];
  }
}

// ---- A5: gate + up + SwiGLU --------------------------------------------------
//
// Workgroup = (work item, 16 rows of gate and up); wave w takes the 128-wide
// super-steps c = w, w + NW, ... (NC of them) of the contraction.  Every load
// of the wave -- both matrices and the tokens -- is issued before the first
// dequantisation, so the whole kernel's traffic is in flight at once.

template <typename A, int BITS, int NC>
__device__ __forceinline__ void gateup_wave(const A* __restrict__ x, int T, int H, int I, int rg,
                                            int tier, int slot, const Tables& tb, int wave, int NW,
                                            int lane, f32x4_t& accg, f32x4_t& accu) {
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = H / 128, nrg = I / 16;
  Raw<A> rg_[NC], ru_[NC];
  Frag<A> xa[NC];
  if constexpr (BITS == 0) {
    const A* wg = reinterpret_cast<const A*>(tb.dense[MOE_GATE]);
    const A* wu = reinterpret_cast<const A*>(tb.dense[MOE_UP]);
#pragma unroll
    for (int j = 0; j < NC; j++) {
      const int c = wave + NW * j;
      if (c < nbg) {
        const size_t off = (size_t)(rg * 16 + lm) * H + 128 * c + 32 * lg;
        load_raw_dense<A>(rg_[j], wg + off);
        load_raw_dense<A>(ru_[j], wu + off);
      }
    }
  } else {
    const size_t tile0 = ((size_t)slot * nrg + rg) * nbg;
#pragma unroll
    for (int j = 0; j < NC; j++) {
      const int c = wave + NW * j;
      if (c < nbg) {
        const size_t idx = (tile0 + c) * 64 + lane;
        load_raw<A, BITS>(rg_[j], tb.codes[tier][MOE_GATE], tb.dm[tier][MOE_GATE], idx);
        load_raw<A, BITS>(ru_[j], tb.codes[tier][MOE_UP], tb.dm[tier][MOE_UP], idx);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NC; j++) {
    const int c = wave + NW * j;
    if (c < nbg) xa[j].load_act(x + (size_t)lm * H + 128 * c + 32 * lg, lm < T);
  }
#pragma unroll
  for (int j = 0; j < NC; j++) {
    const int c = wave + NW * j;
    if (c < nbg) {
      Frag<A> b;
      to_frag<A, BITS>(b, rg_[j]);
      accg = mma_step(xa[j], b, accg);
      to_frag<A, BITS>(b, ru_[j]);
      accu = mma_step(xa[j], b, accu);
    }
  }
}

template <typename A, int NC>
__global__ __launch_bounds__(1024) void k_decode_gateup(const Item* __restrict__ items,
                                                        const int32_t* __restrict__ n_items,
                                                        const A* __restrict__ x, int T, Tables tb,
                                                        A* __restrict__ h, int H, int I) {
  __shared__ float red[16][8][64];
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  // the count and this item's header (always inside the items array) in one trip
  const int n = *n_items;
  const int tier = items[u].tier;
  const int slot = items[u].slot, bits = items[u].bits;
  const int4 routes = *reinterpret_cast<const int4*>(&items[u].route[4 * (lane >> 4)]);
  if (u >= n || tier < 0) return;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  if (tier == kDenseTier)
    gateup_wave<A, 0, NC>(x, T, H, I, rg, 0, 0, tb, wave, NW, lane, accg, accu);
  else if (bits == 4)
    gateup_wave<A, 4, NC>(x, T, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  else if (bits == 3)
    gateup_wave<A, 3, NC>(x, T, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  else
    gateup_wave<A, 2, NC>(x, T, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    red[wave][i][lane] = accg[i];
    red[wave][4 + i][lane] = accu[i];
  }
  __syncthreads();
  for (int v = wave; v < 8; v += NW) {  // slot v summed over the waves, in wave order
    float sum = 0.f;
    for (int w = 0; w < NW; w++) sum += red[w][v][lane];
    red[0][v][lane] = sum;
  }
  __syncthreads();
  if (wave != 0) return;
  const int lm = lane & 15, lg = lane >> 4;
  const int rt[4] = {routes.x, routes.y, routes.z, routes.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = 4 * lg + i;
    if (t < T && rt[i] >= 0)
      store_act<A>(h + (size_t)rt[i] * I + rg * 16 + lm, silu_f32(red[0][i][lane]) * red[0][4 + i][lane]);
  }
}

// ---- A2 + A3 + A5 for one token ----------------------------------------------
//
// Batch-1 decode.  Work item u < K is the token's rank-u expert, item K the
// shared expert, so workgroup (u, rg) needs only the first u + 1 ranks of the
// top-K: wave 0 runs those rounds on the keys while the other waves prefetch
// the tier map into LDS, and the shared-expert workgroups skip routing.  The
// workgroup (K - 1, 0) runs all K rounds and publishes ids, weights and the
// work items for the down kernel.

template <typename A, int NC, int KPL>
__global__ __launch_bounds__(1024) void k_decode1_gateup(const double* __restrict__ keys, int E, int K,
                                                         const int32_t* __restrict__ tier_map,
                                                         int3 n_slots, int3 tier_bits, int has_shared,
                                                         const A* __restrict__ x, Tables tb,
                                                         A* __restrict__ h, int H, int I,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts,
                                                         Item* __restrict__ items,
                                                         int32_t* __restrict__ n_items) {
  __shared__ float red[16][8][64];
  __shared__ int32_t s_tm[4096];
  __shared__ int32_t s_sel;
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  int tier = kDenseTier, slot = 0, bits = 0;
  if (u < K) {
    const bool writer = u == K - 1 && rg == 0;
    if (wave == 0) {
      int sid;
      uint64_t su;
      topk_sorted<KPL>(keys, E, writer ? K : u + 1, lane, &sid, &su);
      if (lane == u) s_sel = sid;
      if (writer) {
        const double key = lane < K ? key_of_order(su) : 0.0;
        const float g = topk_weight(key, lane, K);
        if (lane < K) {
          ids[lane] = sid;
          wts[lane] = g;
          const int tm = tier_map[sid];
          const int t = tm >> 16, sl = tm & 0xFFFF;
          const int ns = t == 0 ? n_slots.x : (t == 1 ? n_slots.y : n_slots.z);
          const bool ok = t >= 0 && t < 3 && sl < ns;
          Item& it = items[lane];
          it.expert = sid;
          it.tier = ok ? t : -1;
          it.slot = ok ? sl : 0;
          it.bits = ok ? (t == 0 ? tier_bits.x : (t == 1 ? tier_bits.y : tier_bits.z)) : 0;
          it.route[0] = lane;
          it.gw[0] = g;
#pragma unroll
          for (int j = 1; j < kGroup; j++) {
            it.route[j] = -1;
            it.gw[j] = 0.0f;
          }
        }
        if (lane == 0) {
          if (has_shared) {
            Item& it = items[K];
            it.expert = -1;
            it.tier = kDenseTier;
            it.slot = 0;
            it.bits = 0;
            it.route[0] = K;
            it.gw[0] = 1.0f;
#pragma unroll
            for (int j = 1; j < kGroup; j++) {
              it.route[j] = -1;
              it.gw[j] = 0.0f;
            }
          }
          *n_items = K + (has_shared ? 1 : 0);
        }
      }
    } else {
      for (int e = threadIdx.x - 64; e < E; e += blockDim.x - 64) s_tm[e] = tier_map[e];
    }
    __syncthreads();
    const int tm = s_tm[s_sel];
    const int t = tm >> 16, sl = tm & 0xFFFF;
    const int ns = t == 0 ? n_slots.x : (t == 1 ? n_slots.y : n_slots.z);
    if (t < 0 || t > 2 || sl >= ns) return;
    tier = t;
    slot = sl;
    bits = t == 0 ? tier_bits.x : (t == 1 ? tier_bits.y : tier_bits.z);
  } else if (!has_shared) {
    return;
  }
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  if (tier == kDenseTier)
    gateup_wave<A, 0, NC>(x, 1, H, I, rg, 0, 0, tb, wave, NW, lane, accg, accu);
  else if (bits == 4)
    gateup_wave<A, 4, NC>(x, 1, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  else if (bits == 3)
    gateup_wave<A, 3, NC>(x, 1, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  else
    gateup_wave<A, 2, NC>(x, 1, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    red[wave][i][lane] = accg[i];
    red[wave][4 + i][lane] = accu[i];
  }
  __syncthreads();
  for (int v = wave; v < 8; v += NW) {
    float sum = 0.f;
    for (int w = 0; w < NW; w++) sum += red[w][v][lane];
    red[0][v][lane] = sum;
  }
  __syncthreads();
  // token 0 sits in accumulator element 0 of lanes 0..15; its h row is u
  if (threadIdx.x < 16)
    store_act<A>(h + (size_t)u * I + rg * 16 + lane, silu_f32(red[0][0][lane]) * red[0][4][lane]);
}

// ---- A6: down + weighted combine --------------------------------------------
//
// Workgroup = 16 output rows; its (item, super-step) pairs are dealt to the
// waves round-robin and processed in batches of kBatch, all loads of a batch
// issued first.  Each pair's 16x16 partial is scaled by the tokens' weights
// and added in a fixed order, then the waves are summed in wave order: the
// result is deterministic (no atomics).

constexpr int kBatch = 2;

template <typename A, typename Y>
__global__ __launch_bounds__(1024) void k_decode_down(const Item* __restrict__ items,
                                                      const int32_t* __restrict__ n_items,
                                                      int max_pairs, const A* __restrict__ h, int T,
                                                      Tables tb, Y* __restrict__ y, int H, int I) {
  __shared__ float red[16][4][64];
  const int rg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128, nrg = H / 16;
  const int npairs = *n_items * nbg;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // the first batch's headers are read in the same trip as the count (the
  // items array always holds max_items entries)
  for (int p0 = wave; p0 < max_pairs; p0 += NW * kBatch) {
    if (p0 >= npairs) break;
    int tier[kBatch], bits[kBatch], route[kBatch], cc[kBatch];
    size_t idx[kBatch];
    float4 gw[kBatch];
    Raw<A> raw[kBatch];
    Frag<A> ha[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; j++) {
      const int p = p0 + NW * j;
      tier[j] = -1;
      if (p < max_pairs) {
        const int u = p / nbg;
        cc[j] = p % nbg;
        const Item& it = items[u];
        tier[j] = it.tier;
        bits[j] = it.bits;
        route[j] = lm < T ? it.route[lm] : -1;
        gw[j] = *reinterpret_cast<const float4*>(&it.gw[4 * lg]);
        idx[j] = (((size_t)it.slot * nrg + rg) * nbg + cc[j]) * 64 + lane;
        if (p >= npairs) tier[j] = -1;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; j++) {
      const int t = tier[j];
      if (t < 0) continue;
      if (t == kDenseTier)
        load_raw_dense<A>(raw[j], reinterpret_cast<const A*>(tb.dense[MOE_DOWN]) +
                                      (size_t)(rg * 16 + lm) * I + 128 * cc[j] + 32 * lg);
      else if (bits[j] == 4)
        load_raw<A, 4>(raw[j], tb.codes[t][MOE_DOWN], tb.dm[t][MOE_DOWN], idx[j]);
      else if (bits[j] == 3)
        load_raw<A, 3>(raw[j], tb.codes[t][MOE_DOWN], tb.dm[t][MOE_DOWN], idx[j]);
      else
        load_raw<A, 2>(raw[j], tb.codes[t][MOE_DOWN], tb.dm[t][MOE_DOWN], idx[j]);
      const int r = route[j];
      ha[j].load_act(h + (size_t)(r < 0 ? 0 : r) * I + 128 * cc[j] + 32 * lg, r >= 0);
    }
#pragma unroll
    for (int j = 0; j < kBatch; j++) {
      const int t = tier[j];
      if (t < 0) continue;
      Frag<A> b;
      if (t == kDenseTier) to_frag<A, 0>(b, raw[j]);
      else if (bits[j] == 4) to_frag<A, 4>(b, raw[j]);
      else if (bits[j] == 3) to_frag<A, 3>(b, raw[j]);
      else to_frag<A, 2>(b, raw[j]);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t part = mma_step(ha[j], b, z);
      acc[0] += gw[j].x * part[0];
      acc[1] += gw[j].y * part[1];
      acc[2] += gw[j].z * part[2];
      acc[3] += gw[j].w * part[3];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float sum = 0.f;
    for (int w = 0; w < NW; w++) sum += red[w][i][lane];
    const int t = 4 * lg + i;
    if (t < T) {
      Y* out = y + (size_t)t * H + rg * 16 + lm;
      if constexpr (sizeof(Y) == 4) *out = sum; else *out = to_bf16(sum);
    }
  }
}

}  // namespace

void launch_decode_gateup(int act, const Item* items, const int32_t* n_items, int max_items,
                          const void* x, int T, const Tables& tb, void* h, int H, int I,
                          hipStream_t s) {
  dim3 grid(max_items * (I / 16));
  const int nbg = H / 128;
  const int nw = nbg < 16 ? nbg : 16;
  const int nc = (nbg + 15) / 16;
  dim3 block(64 * nw);
#define MOE_GU(AT, NC)                                                                       \
  MOE_LAUNCH(MOE_K_DECODE_GATEUP, (k_decode_gateup<AT, NC>), grid, block, 0, s, items, n_items, \
             (const AT*)x, T, tb, (AT*)h, H, I)
  if (act == MOE_BF16) {
    if (nc <= 1) MOE_GU(bf16_t, 1);
    else if (nc <= 2) MOE_GU(bf16_t, 2);
    else MOE_GU(bf16_t, 4);
  } else {
    if (nc <= 1) MOE_GU(float, 1);
    else if (nc <= 2) MOE_GU(float, 2);
    else MOE_GU(float, 4);
  }
#undef MOE_GU
}

void launch_decode1_gateup(int act, const double* keys, int E, int K, const int32_t* tier_map,
                           const int32_t n_slots[3], const int32_t tier_bits[3], int has_shared,
                           const void* x, const Tables& tb, void* h, int H, int I, int32_t* ids,
                           float* w, Item* items, int32_t* n_items, hipStream_t s) {
  dim3 grid((K + 1) * (I / 16));
  const int nbg = H / 128;
  const int nw = nbg < 16 ? nbg : 16;
  const int nc = (nbg + 15) / 16;
  dim3 block(64 * (nw < 2 ? 2 : nw));   // wave 0 routes, the others prefetch the tier map
  const int3 ns = make_int3(n_slots[0], n_slots[1], n_slots[2]);
  const int3 tbits = make_int3(tier_bits[0], tier_bits[1], tier_bits[2]);
#define MOE_G1(AT, NC, KPL)                                                                    \
  MOE_LAUNCH(MOE_K_DECODE_GATEUP, (k_decode1_gateup<AT, NC, KPL>), grid, block, 0, s, keys, E, K, \
             tier_map, ns, tbits, has_shared, (const AT*)x, tb, (AT*)h, H, I, ids, w, items,    \
             n_items)
#define MOE_G1_KPL(AT, NC)                                                                     \
  do {                                                                                         \
    if (E <= 64) MOE_G1(AT, NC, 1);                                                            \
    else if (E <= 128) MOE_G1(AT, NC, 2);                                                      \
    else if (E <= 256) MOE_G1(AT, NC, 4);                                                      \
    else MOE_G1(AT, NC, 8);                                                                    \
  } while (0)
  if (act == MOE_BF16) {
    if (nc <= 1) MOE_G1_KPL(bf16_t, 1);
    else if (nc <= 2) MOE_G1_KPL(bf16_t, 2);
    else MOE_G1_KPL(bf16_t, 4);
  } else {
    if (nc <= 1) MOE_G1_KPL(float, 1);
    else if (nc <= 2) MOE_G1_KPL(float, 2);
    else MOE_G1_KPL(float, 4);
  }
#undef MOE_G1_KPL
#undef MOE_G1
}

void launch_decode_down(int act, int y_dt, const Item* items, const int32_t* n_items,
                        int max_items, const void* h, int T, const Tables& tb, void* y, int H,
                        int I, hipStream_t s) {
  dim3 grid(H / 16);
  const int pairs = max_items * (I / 128);
  const int nw = pairs < 16 ? pairs : 16;
  dim3 block(64 * nw);
  if (act == MOE_BF16) {
    if (y_dt == MOE_BF16)
      MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<bf16_t, bf16_t>), grid, block, 0, s, items,
                 n_items, pairs, (const bf16_t*)h, T, tb, (bf16_t*)y, H, I);
    else
      MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<bf16_t, float>), grid, block, 0, s, items,
                 n_items, pairs, (const bf16_t*)h, T, tb, (float*)y, H, I);
  } else {
    MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<float, float>), grid, block, 0, s, items,
               n_items, pairs, (const float*)h, T, tb, (float*)y, H, I);
  }
}

}  // namespace moe
