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
__device__ __forceinline__ void gateup_tile(const A* __restrict__ x, int T, int H, int I, int rg,
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
__device__ __forceinline__ void gateup_item(float (*red)[8][64], const A* __restrict__ x, int T,
                                            int H, int I, int rg, int tier, int slot,
                                            const Tables& tb, int wave, int NW, int lane,
                                            const int rt[4], A* __restrict__ h) {
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  gateup_tile<A, BITS, NC>(x, T, H, I, rg, tier, slot, tb, wave, NW, lane, accg, accu);
  gateup_store<A>(red, accg, accu, wave, NW, lane, rt, T, h, I, rg);
}

template <typename A, int NC>
__device__ __forceinline__ void gateup_dispatch(float (*red)[8][64], const A* __restrict__ x,
                                                int T, int H, int I, int rg, int tier, int slot,
                                                int bits, const Tables& tb, int wave, int NW,
                                                int lane, const int rt[4], A* __restrict__ h) {
  if (tier == kDenseTier)
    gateup_item<A, 0, NC>(red, x, T, H, I, rg, 0, 0, tb, wave, NW, lane, rt, h);
  else if (bits == 4)
    gateup_item<A, 4, NC>(red, x, T, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else if (bits == kMx4)
    gateup_item<A, kMx4, NC>(red, x, T, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else if (bits == 3)
    gateup_item<A, 3, NC>(red, x, T, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
  else
    gateup_item<A, 2, NC>(red, x, T, H, I, rg, tier, slot, tb, wave, NW, lane, rt, h);
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
  if (u >= n || tier < 0) return;
  const int rt[4] = {routes.x, routes.y, routes.z, routes.w};
  gateup_dispatch<A, NC>(red, x, T, H, I, rg, tier, slot, bits, tb, wave, NW, lane, rt, h);
}

// ---- A2 + A3 + A5 for one token ----------------------------------------------
//
// Batch-1 decode.  Work item u < K is the token's rank-u expert, item K the
// shared expert; the shared-expert workgroups skip routing.  When every
// thread can hold one key (E <= threads), the workgroup selects the top-K
// together (topk_block); otherwise wave 0 selects the first u + 1 ranks while
// the other waves prefetch the tier map into LDS.  Workgroup (K - 1, 0)
// publishes ids, weights and the work items for the down kernel.

// Workgroup-wide exact top-K of one token's keys, one key per thread
// (E <= blockDim.x), with the tier map copied into LDS in the same round
// trip.  The keys are counted into 256 value bins of equal width between the
// block's smallest and largest key, computed in fp32 (rounding to fp32,
// subtracting and scaling are all monotone, so the bin index never decreases
// as the key grows); wave 0 scans the histogram from the top bin down to the
// bin holding the K-th key.  The keys in that bin and above -- each larger
// than every key outside -- are gathered in LDS and ranked exactly by (key
// desc, id asc) in wave 0.  NaN or infinite keys, or more than 64 candidates,
// hand over to the wave-level selection.  Wave 0's lanes r < K end with the
// r-th id and its order key.
struct TopkBlockLds {
  TopkSlot cand[64];
  uint32_t hist[256];
  float mx[kGateUpWaves], mn[kGateUpWaves];
  int bad[kGateUpWaves];
  int cnt, cb, nb;
};

__device__ __forceinline__ void wave_maxmin_f32(float& mx, float& mn) {
#define MOE_MM_STEP(C)                                                   \
  mx = fmaxf(mx, __uint_as_float(dpp_u32<C>(__float_as_uint(mx))));     \
  mn = fminf(mn, __uint_as_float(dpp_u32<C>(__float_as_uint(mn))));
  MOE_MM_STEP(0xB1)    // quad_perm [1,0,3,2]
  MOE_MM_STEP(0x4E)    // quad_perm [2,3,0,1]
  MOE_MM_STEP(0x124)   // row_ror:4
  MOE_MM_STEP(0x128)   // row_ror:8
#undef MOE_MM_STEP
  const auto rl = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  mx = fmaxf(fmaxf(rl(mx, 0), rl(mx, 16)), fmaxf(rl(mx, 32), rl(mx, 48)));
  mn = fminf(fminf(rl(mn, 0), rl(mn, 16)), fminf(rl(mn, 32), rl(mn, 48)));
}

__device__ __forceinline__ void topk_block(const double* __restrict__ keys, int E, int K,
                                           const int32_t* __restrict__ tier_map,
                                           int32_t* __restrict__ s_tm, TopkBlockLds& S, int lane,
                                           int wave, int NW, int* sel_id, uint64_t* sel_u) {
  const int t = threadIdx.x;
  const bool ok = t < E;
  const double k = keys[ok ? t : E - 1];
  const int tm = tier_map[ok ? t : E - 1];
  const bool bad = ok && !(fabs(k) < INFINITY);
  const float kf = (float)k;
  float mx = ok && !bad ? kf : -INFINITY, mn = ok && !bad ? kf : INFINITY;
  wave_maxmin_f32(mx, mn);
  const bool wbad = __ballot(bad) != 0;
  if (t < 256) S.hist[t] = 0u;
  if (ok) s_tm[t] = tm;
  if (lane == 0) {
    S.mx[wave] = mx;
    S.mn[wave] = mn;
    S.bad[wave] = wbad ? 1 : 0;
  }
  if (t == 0) S.cnt = 0;
  __syncthreads();
  float hi = -INFINITY, lo = INFINITY;
  int anybad = 0;
  for (int w = 0; w < NW; w++) {
    hi = fmaxf(hi, S.mx[w]);
    lo = fminf(lo, S.mn[w]);
    anybad |= S.bad[w];
  }
  // mode 0: histogram; 1: every key is a candidate; 2: wave-level selection
  int mode = anybad ? 2 : (E <= 64 ? 1 : (hi > lo ? 0 : 2));
  int bin = -1;
  if (mode == 0) {
    const float scale = 256.0f / (hi - lo);
    if (ok) {
      bin = (int)fminf(fmaxf((kf - lo) * scale, 0.0f), 255.0f);
      atomicAdd(&S.hist[bin], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      int cum = 0, cb = -1, nb = 0;
      for (int pass = 0; pass < 4 && cb < 0; pass++) {
        const int c = wave_incl_scan((int)S.hist[255 - 64 * pass - lane]) + cum;
        const uint64_t m = __ballot(c >= K);
        if (m) {
          const int l = (int)__builtin_ctzll(m);
          cb = 255 - 64 * pass - l;
          nb = __builtin_amdgcn_readlane(c, l);
        } else {
          cum = __builtin_amdgcn_readlane(c, 63);
        }
      }
      if (lane == 0) {
        S.cb = cb;
        S.nb = nb;
      }
    }
    __syncthreads();
    if (S.cb < 0 || S.nb > 64) mode = 2;
  }
  if (mode != 2) {
    if (ok && (mode == 1 || bin >= S.cb)) {
      const int pos = atomicAdd(&S.cnt, 1);
      S.cand[pos].u = order_key(k);
      S.cand[pos].id = (uint32_t)t;
    }
    __syncthreads();
  }
  if (wave != 0) return;
  if (mode == 2) {
    topk_threshold<8>(keys, E, K, lane, S.cand, sel_id, sel_u);
    return;
  }
  const int nc = S.cnt;
  uint64_t mu = 0;
  uint32_t mid_ = 0xFFFFFFFFu;
  if (lane < nc) {
    mu = S.cand[lane].u;
    mid_ = S.cand[lane].id;
  }
  wave_sync_lds();
  rank_select(mu, mid_, nc, K, lane, S.cand, sel_id, sel_u);
}

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
  __shared__ int32_t s_sel;
  __shared__ TopkBlockLds s_tk;
  const int nrg = I / 16;
  const int u = blockIdx.x / nrg, rg = blockIdx.x % nrg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  int tier = kDenseTier, slot = 0, bits = 0;
  if (u < K) {
    const bool writer = u == K - 1 && rg == 0;
    int sid = -1;
    uint64_t su = 0;
    if (E <= (int)blockDim.x) {
      topk_block(keys, E, K, tier_map, s_tm, s_tk, lane, wave, NW, &sid, &su);
    } else if (wave == 0) {
      topk_threshold<KPL>(keys, E, writer ? K : u + 1, lane, s_tk.cand, &sid, &su);
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
    if (wave == 0) {
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
    }
    __syncthreads();
    const int tm = s_tm[s_sel];
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
  gateup_dispatch<A, NC>(red, x, 1, H, I, rg, tier, slot, bits, tb, wave, NW, lane, rt, h);
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
      const int c = p % nbg, t = it.tier;
#pragma unroll
      for (int i = 0; i < (int)(16 * sizeof(A) / 2); i++) raw[j].v[i] = 0u;
      if (mine && t >= 0) {
        const size_t idx = (((size_t)it.slot * nrg + rg) * nbg + c) * 64 + lane;
        const A* dense = reinterpret_cast<const A*>(tb.dense[MOE_DOWN]) +
                         (size_t)(rg * 16 + lm) * I + 128 * c + 32 * lg;
        if (t == kDenseTier) load_down<A, 0>(raw[j], tb, t, idx, dense);
        else if ((it.bits >> 8) == 4) load_down<A, 4>(raw[j], tb, t, idx, dense);
        else if ((it.bits >> 8) == kMx4) load_down<A, kMx4>(raw[j], tb, t, idx, dense);
        else if ((it.bits >> 8) == 3) load_down<A, 3>(raw[j], tb, t, idx, dense);
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
      const int c = p % nbg, t = it.tier;
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
      else if ((it.bits >> 8) == 4) to_frag<A, 4>(b, raw[j]);
      else if ((it.bits >> 8) == kMx4) to_frag<A, kMx4>(b, raw[j]);
      else if ((it.bits >> 8) == 3) to_frag<A, 3>(b, raw[j]);
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
// partial rows; the cross terms are not used.  X and Y always share a tier
// (the pairing below), so the dequantisation path is uniform per wave.
template <typename Y>
__global__ __launch_bounds__(1024) void k_decode1_down(const Item* __restrict__ items,
                                                       const int32_t* __restrict__ n_items,
                                                       int max_items, const bf16_t* __restrict__ h,
                                                       int h_rows, Tables tb, Y* __restrict__ y,
                                                       int H, int I) {
  __shared__ float red[16][16];
  __shared__ int8_t s_pair[64][2];
  __shared__ int s_npairs;
  extern __shared__ uint4 s_dyn[];
  Item* s_items = reinterpret_cast<Item*>(s_dyn);
  const bf16_t* s_h = reinterpret_cast<const bf16_t*>(s_dyn + (size_t)max_items * (sizeof(Item) / 16));
  // the two row halves of a tile sit 8 apart in the grid, on one XCD, so its
  // lines are fetched from HBM once (the grid is a multiple of 16)
  const int rg = ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int nbg = I / 128, nrg = H / 16;
  {
    const int nh = max_items * (int)(sizeof(Item) / 16);
    const int n16 = h_rows * I * (int)sizeof(bf16_t) / 16;
    const uint4* si = reinterpret_cast<const uint4*>(items);
    const uint4* sh = reinterpret_cast<const uint4*>(h);
    for (int i = threadIdx.x; i < nh + n16; i += blockDim.x)
      s_dyn[i] = i < nh ? si[i] : sh[i - nh];
  }
  const int n = min(*n_items, 64);
  __syncthreads();
  if (wave == 0) {
    // pair the items of each tier (dense last) in item order; an odd one out
    // pairs with nothing.  Lane i holds item i (n <= 64).
    const int t = lane < n ? s_items[lane].tier : -1;
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
    if (my_pair >= 0 && my_side == 0) {
      s_pair[my_pair][0] = (int8_t)lane;
      s_pair[my_pair][1] = (int8_t)-1;
    }
    if (my_pair >= 0 && my_side == 1) s_pair[my_pair][1] = (int8_t)lane;
    if (lane == 0) s_npairs = base;
  }
  __syncthreads();
  const int units = s_npairs * nbg;
  float acc = 0.f;
  constexpr int PB = 2;
  for (int p0 = wave; p0 < units; p0 += NW * PB) {
    Raw<bf16_t> raw[PB];
#pragma unroll
    for (int j = 0; j < PB; j++) {
      const int p = p0 + NW * j;
      if (p >= units) continue;
      const int c = p % nbg;
      const int it = s_pair[p / nbg][lm >> 3];
#pragma unroll
      for (int i = 0; i < 16; i++) raw[j].v[i] = 0u;
      if (it < 0) continue;
      const Item& item = s_items[it];
      const int row = rg * 16 + half * 8 + (lm & 7);
      if (item.tier == kDenseTier) {
        load_raw_dense<bf16_t>(raw[j], reinterpret_cast<const bf16_t*>(tb.dense[MOE_DOWN]) +
                                           (size_t)row * I + 128 * c + 32 * lg);
      } else {
        const size_t idx = (((size_t)item.slot * nrg + rg) * nbg + c) * 64 + 16 * lg + half * 8 + (lm & 7);
        const int dbits = item.bits >> 8;       // down format
        if (dbits == 4) load_raw<bf16_t, 4>(raw[j], tb.codes[item.tier][MOE_DOWN], tb.dm[item.tier][MOE_DOWN], idx);
        else if (dbits == kMx4) load_raw<bf16_t, kMx4>(raw[j], tb.codes[item.tier][MOE_DOWN], tb.dm[item.tier][MOE_DOWN], idx);
        else if (dbits == 3) load_raw<bf16_t, 3>(raw[j], tb.codes[item.tier][MOE_DOWN], tb.dm[item.tier][MOE_DOWN], idx);
        else load_raw<bf16_t, 2>(raw[j], tb.codes[item.tier][MOE_DOWN], tb.dm[item.tier][MOE_DOWN], idx);
      }
    }
#pragma unroll
    for (int j = 0; j < PB; j++) {
      const int p = p0 + NW * j;
      if (p >= units) continue;
      const int c = p % nbg;
      const int ix = s_pair[p / nbg][0], iy = s_pair[p / nbg][1];
      // A: row 0 = h of X, row 1 = h of Y (lanes with lm >= 2 carry zeros)
      const int ia = lm == 0 ? ix : (lm == 1 ? iy : -1);
      Frag<bf16_t> ha;
      ha.load_act(s_h + (size_t)(ia >= 0 ? s_items[ia].route[0] : 0) * I + 128 * c + 32 * lg, ia >= 0);
      const Item& hx = s_items[ix];           // the pair's tier (X always exists)
      Frag<bf16_t> b;
      if (hx.tier == kDenseTier) to_frag<bf16_t, 0>(b, raw[j]);
      else if ((hx.bits >> 8) == 4) to_frag<bf16_t, 4>(b, raw[j]);
      else if ((hx.bits >> 8) == kMx4) to_frag<bf16_t, kMx4>(b, raw[j]);
      else if ((hx.bits >> 8) == 3) to_frag<bf16_t, 3>(b, raw[j]);
      else to_frag<bf16_t, 2>(b, raw[j]);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t part = mma_step(ha, b, z);
      // lanes 0-7: C[0][lane] (item X); lanes 8-15: C[1][lane] (item Y)
      const int mine = lm < 8 ? ix : iy;
      if (lg == 0 && mine >= 0) acc += s_items[mine].gw[0] * (lm < 8 ? part[0] : part[1]);
    }
  }
  if (lane < 16) red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || lane >= 8) return;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    if (w < NW) sum += red[w][lane] + red[w][lane + 8];
  }
  Y* out = y + rg * 16 + half * 8 + lane;
  if constexpr (sizeof(Y) == 4) *out = sum; else *out = to_bf16(sum);
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
  if (T == 1 && act == MOE_BF16 && stage && max_items <= 64) {
    // one token: two items per MFMA, no zero lanes
    if (y_dt == MOE_BF16)
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode1_down<bf16_t>, grid, dim3(1024), lds, s, items,
                 n_items, max_items, (const bf16_t*)h, h_rows, tb, (bf16_t*)y, H, I);
    else
      MOE_LAUNCH(MOE_K_DECODE_DOWN, k_decode1_down<float>, grid, dim3(1024), lds, s, items,
                 n_items, max_items, (const bf16_t*)h, h_rows, tb, (float*)y, H, I);
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
