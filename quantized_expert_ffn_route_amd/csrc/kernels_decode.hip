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
    load_field<BITS>(field_ptr<BITS>(codes, idx), w);
    SinkBf16 sink;
    dequant_block<BITS>(w, load_scale<BITS>(dm, idx), sink);
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
    load_field<BITS>(field_ptr<BITS>(codes, idx), w);
    SinkF32 sink;
    dequant_block<BITS>(w, load_scale<BITS>(dm, idx), sink);
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
// a quantised block's code field and (d, m) word (MXFP4: scale byte), or 32
// dense act values.
template <typename A>
struct Raw {
  uint32_t v[16 * sizeof(A) / 2];  // dense: 32 act values; quantised: w[0..3], dm in v[4]
};

template <typename A, int BITS>
__device__ __forceinline__ void load_raw(Raw<A>& r, const uint8_t* codes, const uint32_t* dm,
                                         size_t idx) {
  load_field<BITS>(field_ptr<BITS>(codes, idx), r.v);
  r.v[4] = load_scale<BITS>(dm, idx);
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
// Workgroup = (work item, 16-row group of gate and of up).  Wave w takes the
// 128-wide super-steps c = w, w + NW, ... (NC of them) of the contraction;
// every load of the wave is issued before the first dequantisation.  The
// grid of one decode step must be resident in a single round (the work is
// one round of loads per wave), which fixes the workgroup shape below.

// Waves per gate/up workgroup: with two super-steps per wave two workgroups
// stay resident per CU, enough for one token's 11 x I/16 workgroups.
constexpr int kGateUpWaves = 8;

template <typename A, int BITS, int NC>
__device__ __forceinline__ void gateup_tile(const A* __restrict__ x, bool arow, int H, int I, int rg,
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
    if (c < nbg) xa[j].load_act(x + (size_t)lm * H + 128 * c + 32 * lg, arow);
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

// Sum the waves' 16x16 gate and up tiles (in wave order) and store
// act(silu(gate) * up) for the tokens of this workgroup's rows: element i of
// lane l is token 4 * (l / 16) + i, weight row l % 16; route[i] names the h
// row of token 4 * (l / 16) + i (-1: token not routed here).
template <typename A>
__device__ __forceinline__ void gateup_store(float (*red)[8][64], const f32x4_t& accg,
                                             const f32x4_t& accu, int wave, int NW, int lane,
                                             const int rt[4], int T, A* __restrict__ h, int I,
                                             int rg) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    red[wave][i][lane] = accg[i];
    red[wave][4 + i][lane] = accu[i];
  }
  __syncthreads();
  if (wave != 0) return;
  const int lm = lane & 15, lg = lane >> 4;
  // all partials read first (one LDS round trip), then summed in wave order
  float pg[kGateUpWaves][4], pu[kGateUpWaves][4];
#pragma unroll
  for (int w = 0; w < kGateUpWaves; w++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      pg[w][i] = w < NW ? red[w][i][lane] : 0.f;
      pu[w][i] = w < NW ? red[w][4 + i][lane] : 0.f;
    }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = 4 * lg + i;
    if (t < T && rt[i] >= 0) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < kGateUpWaves; w++) {
        g += pg[w][i];
        u += pu[w][i];
      }
      store_act<A>(h + (size_t)rt[i] * I + rg * 16 + lm, silu_f32(g) * u);
    }
  }
}

template <typename A, int BITS, int NC>
__device__ __forceinline__ void gateup_item(float (*red)[8][64], const A* __restrict__ x, int T, bool arow,
                                            int H, int I, int rg, int tier, int slot,
                                            const Tables& tb, int wave, int NW, int lane,
                                            const int rt[4], A* __restrict__ h) {
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  gateup_tile<A, BITS, NC>(x, arow, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  gateup_store<A>(red, accg, accu, wave, NW, lane, rt, T, h, I, rg);
}

template <typename A, int NC>
__device__ __forceinline__ void gateup_dispatch(float (*red)[8][64], const A* __restrict__ x,
                                                int T, bool arow, int H, int I, int rg, int tier,
                                                int slot, int bits, const Tables& tb, int wave, int NW,
                                                int lane, const int rt[4], A* __restrict__ h) {
  if (tier == kDenseTier)
    gateup_item<A, 0, NC>(red, x, T, arow, H, I, rg, 0, 0, tb, wave, NW, lane, rt, h);
  else if (bits == 4)
    gateup_item<A, 4, NC>(red, x, T, arow, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else if (bits == kMx4)
    gateup_item<A, kMx4, NC>(red, x, T, arow, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else if (bits == 3)
    gateup_item<A, 3, NC>(red, x, T, arow, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else
    gateup_item<A, 2, NC>(red, x, T, arow, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
}

template <typename A, int NC>
__global__ __launch_bounds__(64 * kGateUpWaves) void k_decode_gateup(const Item* __restrict__ items,
                                                        const int32_t* __restrict__ n_items,
                                                        const A* __restrict__ x, int T, Tables tb,
                                                        A* __restrict__ h, int H, int I) {
  __shared__ float red[kGateUpWaves][8][64];
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  // the count and this item's header (always inside the items array) in one trip
  const int n = *n_items;
  const int tier = items[u].tier;
  const int slot = items[u].slot, bits = items[u].bits & 0xFF;   // gate / up format
  const int4 routes = *reinterpret_cast<const int4*>(&items[u].route[4 * (lane >> 4)]);
  // only the activation rows of tokens routed to this item are read (a
  // group's item takes a few of its tokens; the other rows stay zero)
  const int arow_route = items[u].route[lane & 15];
  if (u >= n || tier < 0) return;
  const int rt[4] = {routes.x, routes.y, routes.z, routes.w};
  const bool arow = (lane & 15) < T && arow_route >= 0;
  gateup_dispatch<A, NC>(red, x, T, arow, H, I, rg, tier, slot, bits, tb, wave, NW, lane, rt, h);
}

// ---- A2 + A3 + A5 for one token ----------------------------------------------
//
// Batch-1 decode.  Work item u < K is the token's rank-u expert, item K the
// shared expert; the shared-expert workgroups skip routing.  In a routed
// workgroup wave 0 selects the first u + 1 ranks (the routing workgroup all
// K) with the wave-level threshold selection while the other waves copy the
// tier map into LDS.  (A selection spread over the whole workgroup, one key
// per thread with a shared histogram, took as long: its barriers and the
// other waves' instructions cost what the shorter per-wave work saves.)
// Workgroup (K - 1, 0) publishes ids, weights and the work items for the
// down kernel.

template <typename A, int NC, int KPL>
__global__ __launch_bounds__(64 * kGateUpWaves) void k_decode1_gateup(const double* __restrict__ keys, int E, int K,
                                                         const int32_t* __restrict__ tier_map,
                                                         int3 n_slots, int3 tier_bits, int has_shared,
                                                         const A* __restrict__ x, Tables tb,
                                                         A* __restrict__ h, int H, int I,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts,
                                                         Item* __restrict__ items,
                                                         int32_t* __restrict__ n_items) {
  __shared__ float red[kGateUpWaves][8][64];
  __shared__ int32_t s_tm[4096];
  __shared__ TopkSlot s_sel[64];    // the selection's scratch, then ranks 0..u (all K)
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  int tier = kDenseTier, slot = 0, bits = 0;
  if (u < K) {
    const bool writer = u == K - 1 && rg == 0;
    if (wave == 0) {
      const int rounds = writer ? K : u + 1;
      int sid;
      uint64_t su;
      topk_threshold<KPL>(keys, E, rounds, lane, s_sel, &sid, &su);
      if (lane < rounds) {
        s_sel[lane].u = su;
        s_sel[lane].id = (uint32_t)sid;
      }
    } else {
      // tier map into LDS; four clamped loads in flight per thread per pass
      const int nt = blockDim.x - 64;
      for (int e0 = threadIdx.x - 64; e0 < E; e0 += 4 * nt) {
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int e = e0 + j * nt;
          v[j] = tier_map[e < E ? e : E - 1];
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (e0 + j * nt < E) s_tm[e0 + j * nt] = v[j];
      }
    }
    __syncthreads();
    if (writer && wave == 0) {
      // ids, weights and the down kernel's work items, after this
      // workgroup's own loads are on their way (it is one of K * I / 16)
      const int sid = lane < K ? (int)s_sel[lane].id : -1;
      const double key = lane < K ? key_of_order(s_sel[lane].u) : 0.0;
      const float g = topk_weight(key, lane, K);
      if (lane < K) {
        ids[lane] = sid;
        wts[lane] = g;
        const int tm = s_tm[sid];
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
    const int tm = s_tm[s_sel[u].id];
    const int t = tm >> 16, sl = tm & 0xFFFF;
    const int ns = t == 0 ? n_slots.x : (t == 1 ? n_slots.y : n_slots.z);
    if (t < 0 || t > 2 || sl >= ns) return;
    tier = t;
    slot = sl;
    bits = (t == 0 ? tier_bits.x : (t == 1 ? tier_bits.y : tier_bits.z)) & 0xFF;
  } else if (!has_shared) {
    return;
  }
  // token 0 sits in accumulator element 0 of lanes 0..15; its h row is u
  const int rt[4] = {lane < 16 ? u : -1, -1, -1, -1};
  gateup_dispatch<A, NC>(red, x, 1, (lane & 15) == 0, H, I, rg, tier, slot, bits, tb, wave, NW, lane, rt, h);
}

// ---- A6: down + weighted combine --------------------------------------------
//
// Workgroup = (16 output rows, row half): the MFMA tile spans 16 weight
// rows, and the lanes of the other half's rows carry zero weights, which gives
// H / 8 workgroups -- one per CU at H = 2048, so every CU streams the same
// share.  The (item, super-step) pairs are dealt to the waves round-robin and
// processed in batches of PB, all loads of a batch issued first (for one
// token's 11 items a single batch).  Each pair's 16x16 partial is scaled by
// the tokens' weights and added in a fixed order, then the waves are summed in
// wave order: the result is deterministic (no atomics).

template <typename A, int BITS>
__device__ __forceinline__ void load_down(Raw<A>& r, const Tables& tb, int t, size_t idx,
                                          const A* dense) {
  if constexpr (BITS == 0) load_raw_dense<A>(r, dense);
  else load_raw<A, BITS>(r, tb.codes[t][MOE_DOWN], tb.dm[t][MOE_DOWN], idx);
}

// The work items (and, when they fit, the group's h rows: STAGE) are first
// copied into LDS in one round trip; each wave then issues the weight loads
// of its pairs straight from the LDS headers, so only the raw weight words
// are live in registers while they are in flight.  Without STAGE the A
// operands are loaded from global memory together with the weights.
template <typename A, typename Y, int PB, bool STAGE>
__global__ __launch_bounds__(1024) void k_decode_down(const Item* __restrict__ items,
                                                      const int32_t* __restrict__ n_items,
                                                      int max_items, const A* __restrict__ h,
                                                      int h_rows, int T, Tables tb,
                                                      Y* __restrict__ y, int H, int I) {
  __shared__ float red[16][4][64];
  extern __shared__ uint4 s_dyn[];
  Item* s_items = reinterpret_cast<Item*>(s_dyn);
  const A* s_h = reinterpret_cast<const A*>(s_dyn + (size_t)max_items * (sizeof(Item) / 16));
  // the two row halves of a tile sit 8 apart in the grid, on one XCD, so its
  // lines are fetched from HBM once (the grid is a multiple of 16)
  const int rg = ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const bool mine = (lm >> 3) == half;
  const int nbg = I / 128, nrg = H / 16;
  {
    const int nh = max_items * (int)(sizeof(Item) / 16);
    const int n16 = STAGE ? h_rows * I * (int)sizeof(A) / 16 : 0;
    const uint4* si = reinterpret_cast<const uint4*>(items);
    const uint4* sh = reinterpret_cast<const uint4*>(h);
    for (int i = threadIdx.x; i < nh + n16; i += blockDim.x)
      s_dyn[i] = i < nh ? si[i] : sh[i - nh];
  }
  const int npairs = *n_items * nbg;
  __syncthreads();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = wave; p0 < npairs; p0 += NW * PB) {
    Raw<A> raw[PB];
    Frag<A> ha[STAGE ? 1 : PB];
#pragma unroll
    for (int j = 0; j < PB; j++) {
      const int p = p0 + NW * j;
      if (p >= npairs) continue;
      const Item& it = s_items[p / nbg];
      const int c = p % nbg;
      // the item is the same for the whole wave: tier, format and slot in
      // scalar registers, so the table pointers come from the kernel
      // arguments without a vector load (which would wait for every load
      // before it)
      const int t = __builtin_amdgcn_readfirstlane(it.tier);
      const int fmt = __builtin_amdgcn_readfirstlane(it.bits) >> 8;
      const int slot = __builtin_amdgcn_readfirstlane(it.slot);
      if (t >= 0) {
        // the other half's lanes load this half's rows again (their
        // columns are never stored), so no lane branches around a load
        const int ml = mine ? lane : lane ^ 8;
        const size_t idx = (((size_t)slot * nrg + rg) * nbg + c) * 64 + ml;
        const A* dense = reinterpret_cast<const A*>(tb.dense[MOE_DOWN]) +
                         (size_t)(rg * 16 + (ml & 15)) * I + 128 * c + 32 * lg;
        if (t == kDenseTier) load_down<A, 0>(raw[j], tb, t, idx, dense);
        else if (fmt == 4) load_down<A, 4>(raw[j], tb, t, idx, dense);
        else if (fmt == kMx4) load_down<A, kMx4>(raw[j], tb, t, idx, dense);
        else if (fmt == 3) load_down<A, 3>(raw[j], tb, t, idx, dense);
        else load_down<A, 2>(raw[j], tb, t, idx, dense);
      }
      if constexpr (!STAGE) {
        const int r = lm < T ? it.route[lm] : -1;
        ha[j].load_act(h + (size_t)(r < 0 ? 0 : r) * I + 128 * c + 32 * lg, r >= 0);
      }
    }
#pragma unroll
    for (int j = 0; j < PB; j++) {
      const int p = p0 + NW * j;
      if (p >= npairs) continue;
      const Item& it = s_items[p / nbg];
      const int c = p % nbg, t = __builtin_amdgcn_readfirstlane(it.tier);
      const int fmt = __builtin_amdgcn_readfirstlane(it.bits) >> 8;
      if (t < 0) continue;
      Frag<A>* hf;
      if constexpr (STAGE) {
        const int r = lm < T ? it.route[lm] : -1;
        ha[0].load_act(s_h + (size_t)(r < 0 ? 0 : r) * I + 128 * c + 32 * lg, r >= 0);
        hf = &ha[0];
      } else {
        hf = &ha[j];
      }
      Frag<A> b;
      if (t == kDenseTier) to_frag<A, 0>(b, raw[j]);
      else if (fmt == 4) to_frag<A, 4>(b, raw[j]);
      else if (fmt == kMx4) to_frag<A, kMx4>(b, raw[j]);
      else if (fmt == 3) to_frag<A, 3>(b, raw[j]);
      else to_frag<A, 2>(b, raw[j]);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t part = mma_step(*hf, b, z);
      const float4 gw = *reinterpret_cast<const float4*>(&it.gw[4 * lg]);
      acc[0] += gw.x * part[0];
      acc[1] += gw.y * part[1];
      acc[2] += gw.z * part[2];
      acc[3] += gw.w * part[3];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0 || !mine) return;
  // all partials read first (one LDS round trip), then summed in wave order
  float pr[16][4];
#pragma unroll
  for (int w = 0; w < 16; w++)
#pragma unroll
    for (int i = 0; i < 4; i++) pr[w][i] = w < NW ? red[w][i][lane] : 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = 4 * lg + i;
    if (t < T) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 16; w++) sum += pr[w][i];
      Y* out = y + (size_t)t * H + rg * 16 + lm;
      if constexpr (sizeof(Y) == 4) *out = sum; else *out = to_bf16(sum);
    }
  }
}

// One bf16 token: two work items per MFMA.  Token row 0 of the A operand
// carries item X's h row and row 1 item Y's; weight-column lanes 0-7 hold
// this workgroup's eight rows of X, lanes 8-15 the same rows of Y, so every
// lane loads and dequantises a real block (the general kernel leaves half
// the lanes at zero).  C[0][n < 8] and C[1][n >= 8] are the two items'
// partial rows; the other products are never read, so the lanes that feed
// only those (A rows 2-15, and Y's lanes of a pair without Y) load X's data
// again instead of branching around their loads.  X and Y always share a
// tier (the pairing below), so the dequantisation path is uniform per wave.
//
// Nothing is staged in LDS: each lane reads its item's 16-byte header, h row
// index and weight straight from global memory, every wave pairs the items
// itself, and the few h values a unit needs come from global memory (L2)
// next to its weights.  Wave w takes the (pair, super-step) units 2w and
// 2w + 1 of each batch of 32: with an even number of super-steps (the
// launcher's condition) both are consecutive super-steps of one pair, so one
// format branch loads, dequantises and multiplies both, and the only barrier
// is the one before the final sum over the waves.

template <int BITS>
__device__ __forceinline__ void down1_unit2(const Tables& tb, int tier, size_t idx,
                                            const bf16_t* dn, const Frag<bf16_t>& a0,
                                            const Frag<bf16_t>& a1, f32x4_t& p0, f32x4_t& p1) {
  // super-steps c and c + 1: 64 blocks, or 128 dense columns, apart
  Raw<bf16_t> r0, r1;
  if constexpr (BITS == 0) {
    load_raw_dense<bf16_t>(r0, dn);
    load_raw_dense<bf16_t>(r1, dn + 128);
  } else {
    load_raw<bf16_t, BITS>(r0, tb.codes[tier][MOE_DOWN], tb.dm[tier][MOE_DOWN], idx);
    load_raw<bf16_t, BITS>(r1, tb.codes[tier][MOE_DOWN], tb.dm[tier][MOE_DOWN], idx + 64);
  }
  // every load above this point: the scheduler would otherwise pair each
  // dense load with its MFMA, one round trip per 16 bytes
  __builtin_amdgcn_sched_barrier(0);
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  Frag<bf16_t> b;
  to_frag<bf16_t, BITS>(b, r0);
  p0 = mma_step(a0, b, z);
  to_frag<bf16_t, BITS>(b, r1);
  p1 = mma_step(a1, b, z);
}

template <typename Y>
__global__ __launch_bounds__(1024) void k_decode1_down(const Item* __restrict__ items,
                                                       const int32_t* __restrict__ n_items,
                                                       int max_items, const bf16_t* __restrict__ h,
                                                       Tables tb, Y* __restrict__ y, int H, int I) {
  __shared__ float red[16][16];
  __shared__ int8_t s_pair[16][64][2];     // one copy per wave
  // the two row halves of a tile sit 8 apart in the grid, on one XCD, so its
  // lines are fetched from HBM once (the grid is a multiple of 16)
  const int rg = ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128, nrg = H / 16;
  // count and lane i's item (clamped: every load unconditional, all in flight together)
  const int n_raw = *n_items;
  const Item* me = items + min(lane, max_items - 1);
  const int4 hd = *reinterpret_cast<const int4*>(me);   // expert, tier, slot, bits
  const int hrow = me->route[0];
  const int gwb = __float_as_int(me->gw[0]);
  const int n = min(n_raw, min(max_items, 64));
  int npairs;
  {
    // pair the items of each tier (dense last) in item order; an odd one out
    // pairs with nothing.  Lane i holds item i.
    const int t = lane < n ? hd.y : -1;
    const int cls = t == kDenseTier ? 3 : (t >= 0 && t < 3 ? t : -1);
    const uint64_t below = (1ull << lane) - 1ull;
    int base = 0, my_pair = -1, my_side = 0;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const uint64_t m = __ballot(cls == c);
      if (cls == c) {
        const int rank = __popcll(m & below);
        my_pair = base + (rank >> 1);
        my_side = rank & 1;
      }
      base += (__popcll(m) + 1) >> 1;
    }
    // one wave's stores to LDS land in program order: a partner's id
    // overwrites the -1 its pair's first item wrote
    if (my_pair >= 0 && my_side == 0) {
      s_pair[wave][my_pair][0] = (int8_t)lane;
      s_pair[wave][my_pair][1] = (int8_t)-1;
    }
    if (my_pair >= 0 && my_side == 1) s_pair[wave][my_pair][1] = (int8_t)lane;
    wave_sync_lds();
    npairs = base;
  }
  const int units = npairs * nbg;
  const int row = rg * 16 + half * 8 + (lm & 7);
  float acc = 0.f;
  for (int p0 = 2 * wave; p0 < units; p0 += 32) {
    const int q = p0 / nbg, c = p0 % nbg;
    // the pair's tier and format are X's, kept in scalar registers so the
    // table pointers come from the kernel arguments without a vector load
    const int ix = s_pair[wave][q][0] & 63, iy = s_pair[wave][q][1];
    const int tier = __builtin_amdgcn_readlane(hd.y, ix);
    const int fmt = tier == kDenseTier ? 0 : __builtin_amdgcn_readlane(hd.w, ix) >> 8;  // down format
    // weight columns: X's item for lanes 0-7, Y's (if any) for lanes 8-15
    const int it = lm < 8 || iy < 0 ? ix : iy;
    const int slot = __shfl(hd.z, it, 64);
    const size_t idx = (((size_t)slot * nrg + rg) * nbg + c) * 64 + 16 * lg + half * 8 + (lm & 7);
    const bf16_t* dn = reinterpret_cast<const bf16_t*>(tb.dense[MOE_DOWN]) + (size_t)row * I + 128 * c + 32 * lg;
    // A rows: row 1 is Y's h row when there is a Y, every other row X's
    const int hr = __shfl(hrow, lm == 1 && iy >= 0 ? iy : ix, 64);
    const uint4* ap = reinterpret_cast<const uint4*>(h + (size_t)hr * I + 128 * c + 32 * lg);
    Frag<bf16_t> a0, a1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 u0 = ap[i], u1 = ap[16 + i];    // +16 uint4 = +128 columns
      a0.v[4 * i] = u0.x; a0.v[4 * i + 1] = u0.y; a0.v[4 * i + 2] = u0.z; a0.v[4 * i + 3] = u0.w;
      a1.v[4 * i] = u1.x; a1.v[4 * i + 1] = u1.y; a1.v[4 * i + 2] = u1.z; a1.v[4 * i + 3] = u1.w;
    }
    f32x4_t pa, pb;
    if (fmt == 0) down1_unit2<0>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == 4) down1_unit2<4>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == kMx4) down1_unit2<kMx4>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == 3) down1_unit2<3>(tb, tier, idx, dn, a0, a1, pa, pb);
    else down1_unit2<2>(tb, tier, idx, dn, a0, a1, pa, pb);
    // lanes 0-7: C[0][lane] (item X); lanes 8-15: C[1][lane] (item Y)
    const float gx = __int_as_float(__builtin_amdgcn_readlane(gwb, ix));
    const float gy = __int_as_float(__builtin_amdgcn_readlane(gwb, iy & 63));
    if (lg == 0 && (lm < 8 || iy >= 0)) {
      const float g = lm < 8 ? gx : gy;
      acc += g * (lm < 8 ? pa[0] : pa[1]);
      acc += g * (lm < 8 ? pb[0] : pb[1]);
    }
  }
  if (lane < 16) red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || lane >= 8) return;
  // all sixteen waves' partials read at once, then summed in wave order
  float pr[16];
#pragma unroll
  for (int w = 0; w < 16; w++) pr[w] = red[w][lane] + red[w][lane + 8];
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < 16; w++) sum += pr[w];
  Y* out = y + rg * 16 + half * 8 + lane;
  if constexpr (sizeof(Y) == 4) *out = sum; else *out = to_bf16(sum);
}

// ---- A6 for a bf16 token group: two work items per MFMA ---------------------
//
// The one-token pairing above, for groups of up to 16 tokens.  An item's
// routed tokens (in token order) are cut into slices of at most eight; two
// slices of the same tier share an MFMA: A rows 0-7 carry slice X's tokens' h
// rows and rows 8-15 slice Y's, weight-column lanes 0-7 hold this
// workgroup's eight rows of X's expert and lanes 8-15 the same rows of Y's.
// C[r < 8][n < 8] and C[r >= 8][n >= 8] are the two slices' partial rows; the
// cross products are never read, so every lane dequantises a block that is
// used (the general kernel repeats the other half's rows).  Each wave adds
// its partials into its own LDS rows, [token][output row], X's lanes then
// Y's in two instructions (a token routed to both items never meets itself
// in one instruction), so the order of every sum is fixed; the waves' rows
// are then summed in wave order.  Deterministic, no global atomics.

constexpr int kMaxSlices = 512;      // two slices per item, up to 256 items

struct alignas(16) Slice {
  int32_t slot;
  int16_t tier;      // 0..2, kDenseTier, or -1 (no slice)
  int16_t fmt;       // down code format (0: dense)
  int32_t ntok;      // A rows used (1..8)
  int8_t tok[8];     // token of A row j
  int16_t hrow[8];   // h row of A row j
  float gw[8];       // mixing weight of A row j
};

template <typename Y>
__global__ __launch_bounds__(1024) void k_decode_down_pair(const Item* __restrict__ items,
                                                           const int32_t* __restrict__ n_items,
                                                           int max_items,
                                                           const bf16_t* __restrict__ h, int T,
                                                           Tables tb, Y* __restrict__ y, int H,
                                                           int I) {
  __shared__ Slice s_sl[kMaxSlices];
  __shared__ int16_t s_pair[kMaxSlices][2];
  __shared__ float s_acc[16][kGroup][8];
  __shared__ int s_npairs;
  // the two row halves of a tile sit 8 apart in the grid, on one XCD, so its
  // lines are fetched from HBM once (the grid is a multiple of 16)
  const int rg = ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128, nrg = H / 16;
  const int n = min(*n_items, max_items);
  for (int i = tid; i < 16 * kGroup * 8; i += blockDim.x) (&s_acc[0][0][0])[i] = 0.f;
  // slices 2u and 2u + 1 of item u: its first eight routed tokens, then the rest
  if (tid < n) {
    const Item& it = items[tid];
    const int4 hd = *reinterpret_cast<const int4*>(&it);   // expert, tier, slot, bits
    // the item's 16 routes and weights in eight loads, all in flight together
    int rt[kGroup];
    float gv[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup / 4; k++) {
      const int4 r4 = reinterpret_cast<const int4*>(it.route)[k];
      const float4 g4 = reinterpret_cast<const float4*>(it.gw)[k];
      rt[4 * k] = r4.x; rt[4 * k + 1] = r4.y; rt[4 * k + 2] = r4.z; rt[4 * k + 3] = r4.w;
      gv[4 * k] = g4.x; gv[4 * k + 1] = g4.y; gv[4 * k + 2] = g4.z; gv[4 * k + 3] = g4.w;
    }
    int m = 0;
#pragma unroll
    for (int t = 0; t < kGroup; t++) {
      if (t < T && rt[t] >= 0) {
        Slice& sl = s_sl[2 * tid + (m >> 3)];
        sl.tok[m & 7] = (int8_t)t;
        sl.hrow[m & 7] = (int16_t)rt[t];
        sl.gw[m & 7] = gv[t];
        m++;
      }
    }
    const int tier = hd.y == kDenseTier || (hd.y >= 0 && hd.y < 3) ? hd.y : -1;
#pragma unroll
    for (int k = 0; k < 2; k++) {
      Slice& sl = s_sl[2 * tid + k];
      const int nt = min(max(m - 8 * k, 0), 8);
      sl.slot = hd.z;
      sl.tier = (int16_t)(nt > 0 ? tier : -1);
      sl.fmt = (int16_t)(tier == kDenseTier ? 0 : (hd.w >> 8));
      sl.ntok = nt;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // pair the slices of each class (tiers 0..2, then dense) in slice order;
    // an odd one out pairs with nothing
    const int ns = 2 * n;
    int cnt[4] = {0, 0, 0, 0};
    for (int b = 0; b < ns; b += 64) {
      const int sidx = b + lane, t = sidx < ns ? s_sl[sidx].tier : -1;
      const int cls = t == kDenseTier ? 3 : t;
#pragma unroll
      for (int c = 0; c < 4; c++) cnt[c] += __popcll(__ballot(cls == c));
    }
    int base[4], np = 0;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      base[c] = np;
      np += (cnt[c] + 1) >> 1;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    int seen[4] = {0, 0, 0, 0};
    for (int b = 0; b < ns; b += 64) {
      const int sidx = b + lane, t = sidx < ns ? s_sl[sidx].tier : -1;
      const int cls = t == kDenseTier ? 3 : t;
      int my_pair = -1, my_side = 0;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const uint64_t msk = __ballot(cls == c);
        if (cls == c) {
          const int rank = seen[c] + __popcll(msk & below);
          my_pair = base[c] + (rank >> 1);
          my_side = rank & 1;
        }
        seen[c] += __popcll(msk);
      }
      // one wave's LDS stores land in program order: a partner's index
      // overwrites the -1 written with its pair's first slice
      if (my_pair >= 0 && my_side == 0) {
        s_pair[my_pair][0] = (int16_t)sidx;
        s_pair[my_pair][1] = (int16_t)-1;
      }
      if (my_pair >= 0 && my_side == 1) s_pair[my_pair][1] = (int16_t)sidx;
    }
    if (lane == 0) s_npairs = np;
  }
  __syncthreads();
  const int units = s_npairs * nbg;
  const int row = rg * 16 + half * 8 + (lm & 7);
  const int j = lm & 7;
  for (int p0 = 2 * wave; p0 < units; p0 += 32) {
    // super-steps c and c + 1 of pair q
    const int q = p0 / nbg, c = p0 % nbg;
    const int sx = __builtin_amdgcn_readfirstlane(s_pair[q][0]);
    const int sy = __builtin_amdgcn_readfirstlane(s_pair[q][1]);
    const Slice& X = s_sl[sx];
    const int tier = __builtin_amdgcn_readfirstlane(X.tier);
    const int fmt = __builtin_amdgcn_readfirstlane(X.fmt);
    const int xslot = __builtin_amdgcn_readfirstlane(X.slot);
    const int yslot = __builtin_amdgcn_readfirstlane(s_sl[sy < 0 ? sx : sy].slot);
    // lanes 8-15 of a pair with a Y take Y's weights and Y's token rows
    const bool useY = lm >= 8 && sy >= 0;
    const Slice& S = s_sl[useY ? sy : sx];
    const int slot = useY ? yslot : xslot;
    const size_t idx = (((size_t)slot * nrg + rg) * nbg + c) * 64 + 16 * lg + half * 8 + j;
    const bf16_t* dn = reinterpret_cast<const bf16_t*>(tb.dense[MOE_DOWN]) + (size_t)row * I +
                       128 * c + 32 * lg;
    // A row lm: row j of its slice (its first row when the slice is shorter)
    const int hr = S.hrow[j < S.ntok ? j : 0];
    const uint4* ap = reinterpret_cast<const uint4*>(h + (size_t)hr * I + 128 * c + 32 * lg);
    Frag<bf16_t> a0, a1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 u0 = ap[i], u1 = ap[16 + i];    // +16 uint4 = +128 columns
      a0.v[4 * i] = u0.x; a0.v[4 * i + 1] = u0.y; a0.v[4 * i + 2] = u0.z; a0.v[4 * i + 3] = u0.w;
      a1.v[4 * i] = u1.x; a1.v[4 * i + 1] = u1.y; a1.v[4 * i + 2] = u1.z; a1.v[4 * i + 3] = u1.w;
    }
    f32x4_t pa, pb;
    if (fmt == 0) down1_unit2<0>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == 4) down1_unit2<4>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == kMx4) down1_unit2<kMx4>(tb, tier, idx, dn, a0, a1, pa, pb);
    else if (fmt == 3) down1_unit2<3>(tb, tier, idx, dn, a0, a1, pa, pb);
    else down1_unit2<2>(tb, tier, idx, dn, a0, a1, pa, pb);
    // C rows 4 * lg + i: lanes lg < 2 of columns 0-7 hold X's rows, lanes
    // lg >= 2 of columns 8-15 Y's
    const bool xl = lg < 2 && lm < 8, yl = sy >= 0 && lg >= 2 && lm >= 8;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int jr = 4 * (lg & 1) + i;
      if (xl && jr < X.ntok) {
        const float g = X.gw[jr];
        atomicAdd(&s_acc[wave][X.tok[jr]][j], g * pa[i] + g * pb[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int jr = 4 * (lg & 1) + i;
      if (yl && jr < S.ntok) {
        const float g = S.gw[jr];
        atomicAdd(&s_acc[wave][S.tok[jr]][j], g * pa[i] + g * pb[i]);
      }
    }
  }
  __syncthreads();
  if (tid < T * 8) {
    const int t = tid >> 3, col = tid & 7;
    float pr[16];
#pragma unroll
    for (int w = 0; w < 16; w++) pr[w] = s_acc[w][t][col];
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; w++) sum += pr[w];
    Y* out = y + (size_t)t * H + rg * 16 + half * 8 + col;
    if constexpr (sizeof(Y) == 4) *out = sum; else *out = to_bf16(sum);
  }
}

}  // namespace

void launch_decode_gateup(int act, const Item* items, const int32_t* n_items, int max_items,
                          const void* x, int T, const Tables& tb, void* h, int H, int I,
                          hipStream_t s) {
  dim3 grid(max_items * (I / 16));
  const int nbg = H / 128;
  const int nw = nbg < kGateUpWaves ? nbg : kGateUpWaves;
  const int nc = (nbg + kGateUpWaves - 1) / kGateUpWaves;
  dim3 block(64 * nw);
#define MOE_GU(AT, NC)                                                                       \
  MOE_LAUNCH(MOE_K_DECODE_GATEUP, (k_decode_gateup<AT, NC>), grid, block, 0, s, items, n_items, \
             (const AT*)x, T, tb, (AT*)h, H, I)
  if (act == MOE_BF16) {
    if (nc <= 1) MOE_GU(bf16_t, 1);
    else if (nc <= 2) MOE_GU(bf16_t, 2);
    else if (nc <= 4) MOE_GU(bf16_t, 4);
    else MOE_GU(bf16_t, 8);
  } else {
    if (nc <= 1) MOE_GU(float, 1);
    else if (nc <= 2) MOE_GU(float, 2);
    else if (nc <= 4) MOE_GU(float, 4);
    else MOE_GU(float, 8);
  }
#undef MOE_GU
}

void launch_decode1_gateup(int act, const double* keys, int E, int K, const int32_t* tier_map,
                           const int32_t n_slots[3], const int32_t tier_bits[3], int has_shared,
                           const void* x, const Tables& tb, void* h, int H, int I, int32_t* ids,
                           float* w, Item* items, int32_t* n_items, hipStream_t s) {
  dim3 grid((K + 1) * (I / 16));
  const int nbg = H / 128;
  const int nw = nbg < kGateUpWaves ? nbg : kGateUpWaves;
  const int nc = (nbg + kGateUpWaves - 1) / kGateUpWaves;
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
    else if (nc <= 4) MOE_G1_KPL(bf16_t, 4);
    else MOE_G1_KPL(bf16_t, 8);
  } else {
    if (nc <= 1) MOE_G1_KPL(float, 1);
    else if (nc <= 2) MOE_G1_KPL(float, 2);
    else if (nc <= 4) MOE_G1_KPL(float, 4);
    else MOE_G1_KPL(float, 8);
  }
#undef MOE_G1_KPL
#undef MOE_G1
}

void launch_decode_down(int act, int y_dt, const Item* items, const int32_t* n_items,
                        int max_items, const void* h, int h_rows, int T, const Tables& tb, void* y,
                        int H, int I, hipStream_t s) {
  dim3 grid(H / 16 * 2);
  const int pairs = max_items * (I / 128);
  const int nw = pairs < 16 ? pairs : 16;
  const int per_wave = (pairs + nw - 1) / nw;
  dim3 block(64 * nw);
  const size_t item_bytes = (size_t)max_items * sizeof(Item);
  const size_t stage_bytes = (size_t)h_rows * I * (act == MOE_BF16 ? 2 : 4);
  const bool stage = act == MOE_BF16 && item_bytes + stage_bytes <= 48 * 1024;
  const size_t lds = item_bytes + (stage ? stage_bytes : 0);
  if (T == 1 && act == MOE_BF16 && max_items <= 64 && (I / 128) % 2 == 0) {
    // one token: two items per MFMA, no zero lanes; two super-steps per wave
    if (y_dt == MOE_BF16)
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode1_down<bf16_t>, grid, dim3(1024), 0, s, items,
                 n_items, max_items, (const bf16_t*)h, tb, (bf16_t*)y, H, I);
    else
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode1_down<float>, grid, dim3(1024), 0, s, items,
                 n_items, max_items, (const bf16_t*)h, tb, (float*)y, H, I);
    return;
  }
  if (T > 1 && T <= kGroup && act == MOE_BF16 && max_items <= kMaxSlices / 2 &&
      (I / 128) % 2 == 0) {
    // a token group: two item slices per MFMA
    if (y_dt == MOE_BF16)
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode_down_pair<bf16_t>, grid, dim3(1024), 0, s, items,
                 n_items, max_items, (const bf16_t*)h, T, tb, (bf16_t*)y, H, I);
    else
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode_down_pair<float>, grid, dim3(1024), 0, s, items,
                 n_items, max_items, (const bf16_t*)h, T, tb, (float*)y, H, I);
    return;
  }
#define MOE_DN(AT, YT, PB, ST)                                                                 \
  MOE_LAUNCH(MOE_K_DECODE_DOWN, (k_decode_down<AT, YT, PB, ST>), grid, block, lds, s, items,   \
             n_items, max_items, (const AT*)h, h_rows, T, tb, (YT*)y, H, I)
#define MOE_DN_PB(YT, ST)                                                                      \
  do {                                                                                         \
    if (per_wave <= 1) MOE_DN(bf16_t, YT, 1, ST);                                              \
    else if (per_wave <= 2) MOE_DN(bf16_t, YT, 2, ST);                                         \
    else if (per_wave <= 3 || !ST) MOE_DN(bf16_t, YT, 3, ST);                                  \
    else MOE_DN(bf16_t, YT, 4, ST);                                                            \
  } while (0)
  if (act == MOE_BF16) {
    if (y_dt == MOE_BF16) {
      if (stage) MOE_DN_PB(bf16_t, true); else MOE_DN_PB(bf16_t, false);
    } else {
      if (stage) MOE_DN_PB(float, true); else MOE_DN_PB(float, false);
    }
  } else {
    MOE_DN(float, float, 1, false);
  }
#undef MOE_DN_PB
#undef MOE_DN
}

}  // namespace moe
