// Router scores (A1), top-K + weights (A2), decode dispatch (A3) and the
// stable counting sort of routes by expert (A4).
#include "device_common.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// A1: router keys in float64.
//
// Each wave owns one expert row; its 64 lanes take 8-element chunks of the
// row round-robin (lane l: chunks l, l+64, ...) and accumulate x*w with
// float64 FMAs, then a butterfly sums the lanes.  The order depends only on
// H, so identical router rows give bit-identical keys (ties then resolve by
// id) and every path that scores a token (decode, prefill) agrees bit for
// bit.  Inputs are exact in float64; the result differs from the exactly
// rounded key by ~1e-16 relative, far below the gaps the selection resolves.
// ---------------------------------------------------------------------------

template <typename A>
__device__ __forceinline__ void load8_f64(const A* p, double* v);

template <>
__device__ __forceinline__ void load8_f64<bf16_t>(const bf16_t* p, double* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = (double)bf16_lo(w[i]);
    v[2 * i + 1] = (double)bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void load8_f64<float>(const float* p, double* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Same conversion from raw registers (U4 = sizeof(A)/2 uint4 per chunk).
template <typename A>
__device__ __forceinline__ void cvt8_f64(const uint4* r, double* v);

template <>
__device__ __forceinline__ void cvt8_f64<bf16_t>(const uint4* r, double* v) {
  const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = (double)bf16_lo(w[i]);
    v[2 * i + 1] = (double)bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void cvt8_f64<float>(const uint4* r, double* v) {
  v[0] = __uint_as_float(r[0].x); v[1] = __uint_as_float(r[0].y);
  v[2] = __uint_as_float(r[0].z); v[3] = __uint_as_float(r[0].w);
  v[4] = __uint_as_float(r[1].x); v[5] = __uint_as_float(r[1].y);
  v[6] = __uint_as_float(r[1].z); v[7] = __uint_as_float(r[1].w);
}

template <typename A>
__global__ __launch_bounds__(256) void k_router_keys(const A* __restrict__ x, const A* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     double* __restrict__ keys, int T, int H, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int t0 = blockIdx.y * kGroup;
  const int nt = min(kGroup, T - t0);
  const A* wr = w + (size_t)e * H;
  double acc[kGroup];
#pragma unroll
  for (int t = 0; t < kGroup; t++) acc[t] = 0.0;
  const int nchunk = H / 8;
  for (int q = lane; q < nchunk; q += 64) {
    double wv[8];
    load8_f64<A>(wr + 8 * q, wv);
#pragma unroll
    for (int t = 0; t < kGroup; t++) {
      if (t < nt) {
        double xv[8];
        load8_f64<A>(x + (size_t)(t0 + t) * H + 8 * q, xv);
#pragma unroll
        for (int j = 0; j < 8; j++) acc[t] = __builtin_fma(xv[j], wv[j], acc[t]);
      }
    }
  }
  const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
  for (int t = 0; t < kGroup; t++) {
    if (t < nt) {
      const double s = wave_sum_f64(acc[t]);
      if (lane == 0) keys[(size_t)(t0 + t) * E + e] = s + b;
    }
  }
}

// Decode variant (T <= 16, tokens fit in 64 KiB of LDS), one expert per
// wave.  A single token (ONE): two experts per workgroup, so the router rows
// spread over every CU, and each lane loads its own chunks of x next to its
// router chunks, so no barrier sits between the loads and the arithmetic.
// Several tokens: kRouterGrpWaves experts per workgroup; each lane issues all
// loads of its router row first, then the group's tokens are staged in LDS
// (both round trips overlap), its row is converted to fp64 once for all the
// tokens (up to 2048 columns), and eight tokens' partials are summed over the
// wave at once.
// Same per-lane order and the same pairing of partial sums as k_router_keys,
// so the keys are bit-identical.
constexpr int kRouterDecWaves = 2;
// Group tokens: two experts per workgroup, so that the E / 2 workgroups
// spread the fp64 arithmetic (T dot products per router row) over every CU;
// each workgroup copies the group's tokens into LDS from L2.
constexpr int kRouterGrpWaves = 2;

template <typename A, int MAXC, bool ONE>
__global__ __launch_bounds__(64 * kRouterGrpWaves) void k_router_keys_dec(const A* __restrict__ x,
                                                                          const A* __restrict__ w,
                                                                          const float* __restrict__ bias,
                                                                          double* __restrict__ keys,
                                                                          int T, int H, int E) {
  extern __shared__ uint4 s_x[];
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nchunk = H / 8;
  constexpr int U4 = (int)sizeof(A) / 2;     // uint4 per 8-element chunk
  uint4 wraw[MAXC][U4];
  const A* wr = w + (size_t)(e < E ? e : E - 1) * H;
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    const int q = lane + 64 * j;
    if (q < nchunk)
#pragma unroll
      for (int u = 0; u < U4; u++) wraw[j][u] = reinterpret_cast<const uint4*>(wr + 8 * q)[u];
  }
  if constexpr (ONE) {
    uint4 xraw[MAXC][U4];
#pragma unroll
    for (int j = 0; j < MAXC; j++) {
      const int q = lane + 64 * j;
      if (q < nchunk)
#pragma unroll
        for (int u = 0; u < U4; u++) xraw[j][u] = reinterpret_cast<const uint4*>(x + 8 * q)[u];
    }
    if (e >= E) return;
    const double b = bias ? (double)bias[e] : 0.0;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < MAXC; j++) {
      const int q = lane + 64 * j;
      if (q < nchunk) {
        double wv[8], xv[8];
        cvt8_f64<A>(wraw[j], wv);
        cvt8_f64<A>(xraw[j], xv);
#pragma unroll
        for (int k = 0; k < 8; k++) acc = __builtin_fma(xv[k], wv[k], acc);
      }
    }
    const double sum = wave_sum_f64(acc);
    if (lane == 0) keys[e] = sum + b;
    return;
  }
  const uint4* xs = reinterpret_cast<const uint4*>(x);
  copy_to_lds(s_x, T * H * (int)sizeof(A) / 16, [&](int i) { return xs + i; });
  __syncthreads();
  if (e >= E) return;
  const double b = bias ? (double)bias[e] : 0.0;
  const A* sxa = reinterpret_cast<const A*>(s_x);
  // the router row in fp64 once, for every token (64 registers at 2048
  // columns; wider rows convert per token)
  constexpr bool kHoist = MAXC <= 4;
  double wv[kHoist ? MAXC : 1][8];
  if constexpr (kHoist) {
#pragma unroll
    for (int j = 0; j < MAXC; j++) cvt8_f64<A>(wraw[j], wv[j]);
  }
  // eight tokens' partials at a time, summed over the wave together
  // (wave_sum8_f64 pairs the same partial sums as wave_sum_f64, so every key
  // is bit-identical to the one-token path's); token t0 + c ends in lanes
  // 8c .. 8c + 7
  for (int t0 = 0; t0 < T; t0 += 8) {
    double p[8];
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const int t = t0 + c;
      double acc = 0.0;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < MAXC; j++) {
          const int q = lane + 64 * j;
          if (q < nchunk) {
            double xv[8];
            uint4 xr[U4];
#pragma unroll
            for (int u = 0; u < U4; u++)
              xr[u] = reinterpret_cast<const uint4*>(sxa + (size_t)t * H + 8 * q)[u];
            cvt8_f64<A>(xr, xv);
            if constexpr (kHoist) {
#pragma unroll
              for (int k = 0; k < 8; k++) acc = __builtin_fma(xv[k], wv[j][k], acc);
            } else {
              double wt[8];
              cvt8_f64<A>(wraw[j], wt);
#pragma unroll
              for (int k = 0; k < 8; k++) acc = __builtin_fma(xv[k], wt[k], acc);
            }
          }
        }
      }
      p[c] = acc;
    }
    const double sum = wave_sum8_f64(p, lane);
    const int c = lane >> 3;
    if ((lane & 7) == 0 && t0 + c < T) keys[(size_t)(t0 + c) * E + e] = sum + b;
  }
}

// Token groups with bf16 activations and up to 2048 columns: each workgroup
// takes two experts with eight waves, wave w scoring expert w & 1 for tokens
// w / 2, w / 2 + 4, ...; so the fp64 arithmetic of the group (T dot products
// per router row) is spread over four waves per expert instead of one.  Each
// wave issues its router chunks and its tokens' x chunks (from L2, no LDS
// staging and no barrier) before any arithmetic, converts its router row to
// fp64 once, and sums its tokens' partials over the wave together.  Same
// per-lane order and the same pairing of partial sums as k_router_keys, so
// the keys are bit-identical.
constexpr int kRouterSlices = 4;
constexpr int kRouterSliceTok = kGroup / kRouterSlices;   // tokens per wave

template <int MAXC>
__global__ __launch_bounds__(64 * 2 * kRouterSlices) void k_router_keys_grp(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    double* __restrict__ keys, int T, int H, int E) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.x * 2 + (wave & 1), slice = wave >> 1;
  const int nchunk = H / 8;
  const bf16_t* wr = w + (size_t)(e < E ? e : E - 1) * H;
  // every load unconditional (clamped chunk and token), so all are in flight
  // together
  uint4 wraw[MAXC], xraw[kRouterSliceTok][MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    const int q = lane + 64 * j;
    wraw[j] = *reinterpret_cast<const uint4*>(wr + 8 * (q < nchunk ? q : nchunk - 1));
  }
#pragma unroll
  for (int i = 0; i < kRouterSliceTok; i++) {
    const int t = slice + kRouterSlices * i;
    const bf16_t* xr = x + (size_t)(t < T ? t : T - 1) * H;
#pragma unroll
    for (int j = 0; j < MAXC; j++) {
      const int q = lane + 64 * j;
      xraw[i][j] = *reinterpret_cast<const uint4*>(xr + 8 * (q < nchunk ? q : nchunk - 1));
    }
  }
  // keep every load above this point: the scheduler would otherwise move
  // each one next to its use, one round trip per token
  __builtin_amdgcn_sched_barrier(0);
  double wv[MAXC][8];
#pragma unroll
  for (int j = 0; j < MAXC; j++) cvt8_f64<bf16_t>(&wraw[j], wv[j]);
  double p[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    double acc = 0.0;
    if (i < kRouterSliceTok) {
#pragma unroll
      for (int j = 0; j < MAXC; j++) {
        double xv[8];
        cvt8_f64<bf16_t>(&xraw[i < kRouterSliceTok ? i : 0][j], xv);
        double a = acc;
#pragma unroll
        for (int k = 0; k < 8; k++) a = __builtin_fma(xv[k], wv[j][k], a);
        acc = lane + 64 * j < nchunk ? a : acc;
      }
    }
    p[i] = acc;
  }
  // token slice + 4c ends in lanes 8c .. 8c + 7
  const double sum = wave_sum8_f64(p, lane);
  const int c = lane >> 3, t = slice + kRouterSlices * c;
  // (a wave past the last expert stores nothing; it has no early exit, which
  // would let the compiler sink its loads next to their uses)
  if ((lane & 7) == 0 && c < kRouterSliceTok && t < T && e < E) {
    const double b = bias ? (double)bias[e] : 0.0;
    keys[(size_t)t * E + e] = sum + b;
  }
}

void launch_router_keys(int act, const void* x, const void* w, const float* b, double* keys,
                        int T, int H, int E, hipStream_t s) {
  const size_t xbytes = (size_t)T * H * (act == MOE_BF16 ? 2 : 4);
  if (T <= kGroup && xbytes <= 65536 && H <= 4096) {
    const int maxc = (H / 8 + 63) / 64;
    const dim3 grid1((E + kRouterDecWaves - 1) / kRouterDecWaves);
    const dim3 gridg((E + kRouterGrpWaves - 1) / kRouterGrpWaves);
    if (T > 1 && act == MOE_BF16 && maxc <= 4) {
      const dim3 grid2((E + 1) / 2), block2(64 * 2 * kRouterSlices);
      if (maxc <= 1)
        MOE_LAUNCH(MOE_K_ROUTER_KEYS, k_router_keys_grp<1>, grid2, block2, 0, s, (const bf16_t*)x,
                   (const bf16_t*)w, b, keys, T, H, E);
      else if (maxc <= 2)
        MOE_LAUNCH(MOE_K_ROUTER_KEYS, k_router_keys_grp<2>, grid2, block2, 0, s, (const bf16_t*)x,
                   (const bf16_t*)w, b, keys, T, H, E);
      else
        MOE_LAUNCH(MOE_K_ROUTER_KEYS, k_router_keys_grp<4>, grid2, block2, 0, s, (const bf16_t*)x,
                   (const bf16_t*)w, b, keys, T, H, E);
      return;
    }
#define MOE_RK(AT, MC)                                                                          \
  do {                                                                                          \
    if (T == 1)                                                                                 \
      MOE_LAUNCH(MOE_K_ROUTER_KEYS, (k_router_keys_dec<AT, MC, true>), grid1,                   \
                 dim3(64 * kRouterDecWaves), 0, s, (const AT*)x, (const AT*)w, b, keys, T, H, E); \
    else                                                                                        \
      MOE_LAUNCH(MOE_K_ROUTER_KEYS, (k_router_keys_dec<AT, MC, false>), gridg,                  \
                 dim3(64 * kRouterGrpWaves), xbytes, s, (const AT*)x, (const AT*)w, b, keys, T, \
                 H, E);                                                                         \
  } while (0)
    if (act == MOE_BF16) {
      if (maxc <= 1) MOE_RK(bf16_t, 1);
      else if (maxc <= 2) MOE_RK(bf16_t, 2);
      else if (maxc <= 4) MOE_RK(bf16_t, 4);
      else MOE_RK(bf16_t, 8);
    } else {
      if (maxc <= 1) MOE_RK(float, 1);
      else if (maxc <= 2) MOE_RK(float, 2);
      else if (maxc <= 4) MOE_RK(float, 4);
      else MOE_RK(float, 8);
    }
#undef MOE_RK
    return;
  }
  dim3 grid((E + 3) / 4, (T + kGroup - 1) / kGroup);
  if (act == MOE_BF16)
    MOE_LAUNCH(MOE_K_ROUTER_KEYS, k_router_keys<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w, b, keys, T, H, E);
  else
    MOE_LAUNCH(MOE_K_ROUTER_KEYS, k_router_keys<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)w, b, keys, T, H, E);
}

// ---------------------------------------------------------------------------
// A2: top-K by (key descending, id ascending), one wave per token.
// ---------------------------------------------------------------------------

// Selects the top K of `krow` (E keys) with one wave.  Lane r < K returns the
// r-th selected id in *sel_id and its key in *sel_key.  KPL keys per lane are
// kept in registers (E <= 64*KPL); KPL == 0 rescans memory each round.  Each
// round picks the best entry ranked after the previous pick with a DPP wave
// argmax.
template <int KPL>
__device__ void topk_wave(const double* __restrict__ krow, int E, int K, int lane, int* sel_id,
                          double* sel_key, TopkSlot* __restrict__ scratch) {
  if constexpr (KPL >= 1 && KPL <= 8) {
    uint64_t su;
    topk_threshold<KPL>(krow, E, K, lane, scratch, sel_id, &su);
    *sel_key = lane < K ? key_of_order(su) : 0.0;
    return;
  }
  uint64_t uk[KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
    double kv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; j++) {   // unconditional loads: all in flight at once
      const int e = lane + 64 * j;
      kv[j] = krow[e < E ? e : E - 1];
    }
#pragma unroll
    for (int j = 0; j < KPL; j++) {
      const int e = lane + 64 * j;
      uk[j] = e < E ? order_key(kv[j]) : 0ull;
    }
  }
  uint64_t last_u = 0, my_u = 0;
  uint32_t last_id = 0;
  int my_id = -1;
  for (int r = 0; r < K; r++) {
    uint64_t bu = 0;
    uint32_t bid = 0xFFFFFFFFu;
    // not yet selected <=> ranked after the last selected entry
    auto consider = [&](uint64_t cu, int e) {
      const bool fresh = r == 0 || cu < last_u || (cu == last_u && (uint32_t)e > last_id);
      if (fresh && ranks_before(cu, (uint32_t)e, bu, bid)) {
        bu = cu;
        bid = (uint32_t)e;
      }
    };
    if constexpr (KPL > 0) {
#pragma unroll
      for (int j = 0; j < KPL; j++) {
        const int e = lane + 64 * j;
        if (e < E) consider(uk[j], e);
      }
    } else {
      for (int e = lane; e < E; e += 64) consider(order_key(krow[e]), e);
    }
    wave_argmax(bu, bid);
    last_u = bu;
    last_id = bid;
    if (lane == r) {
      my_id = (int)bid;
      my_u = bu;
    }
  }
  *sel_id = my_id;
  *sel_key = lane < K ? key_of_order(my_u) : 0.0;
}


template <int KPL>
__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ keys, int T, int E, int K,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ TopkSlot s_scr[16][64];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (t >= T) return;
  int sid;
  double skey;
  topk_wave<KPL>(keys + (size_t)t * E, E, K, lane, &sid, &skey, s_scr[threadIdx.x >> 6]);
  const float g = topk_weight(skey, lane, K);
  if (lane < K) {
    ids[(size_t)t * K + lane] = sid;
    w[(size_t)t * K + lane] = g;
  }
}

#define MOE_TOPK_DISPATCH(KID, KERNEL, ...)                                                      \
  do {                                                                                        \
    if (E <= 64) MOE_LAUNCH(KID, KERNEL<1>, __VA_ARGS__);                                     \
    else if (E <= 128) MOE_LAUNCH(KID, KERNEL<2>, __VA_ARGS__);                               \
    else if (E <= 256) MOE_LAUNCH(KID, KERNEL<4>, __VA_ARGS__);                               \
    else if (E <= 512) MOE_LAUNCH(KID, KERNEL<8>, __VA_ARGS__);                               \
    else if (E <= 1024) MOE_LAUNCH(KID, KERNEL<16>, __VA_ARGS__);                             \
    else MOE_LAUNCH(KID, KERNEL<0>, __VA_ARGS__);                                             \
  } while (0)

void launch_topk(const double* keys, int T, int E, int K, int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + 15) / 16);
  MOE_TOPK_DISPATCH(MOE_K_TOPK, k_topk, grid, dim3(1024), 0, s, keys, T, E, K, ids, w);
}

// ---------------------------------------------------------------------------
// A1-A2 for many tokens with bf16 activations: certified selection from the
// bf16-MFMA approximate keys.
//
// The MFMA pass gives approx = fp32 sum of the exact bf16 products + bias.
// With fp32 accumulation over H terms, |approx - key| <= gamma * sum|x_i w_i|
// + (rounding of the bias add) <= delta, gamma = 1.1 (H + 64) 2^-23 (allows
// truncating adds), sum|x_i w_i| <= |x| max_e |w_e| (Cauchy-Schwarz).  An
// expert whose approx is below the K-th largest approx minus 2 delta is beaten
// exactly by at least K others, so the exact top-K lies among the candidates
// approx >= approx_K - 2 delta.  The candidates are rescored with the fp64
// dot of k_router_keys (same per-lane order and butterfly, hence the same
// keys as decode) and the top K taken by (key desc, id asc).
// ---------------------------------------------------------------------------

// Largest value over the wave (float, all 64 lanes active).
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x124>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x128>(__float_as_uint(v))));
  return fmaxf(fmaxf(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0)),
                     __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16))),
               fmaxf(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32)),
                     __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48))));
}

// The float64 key partial of this lane for a token held as raw bf16 pairs
// (canonical chunk order, identical arithmetic to k_router_keys): both
// operands are widened per use, which keeps the register footprint small.
template <int MAXC>
__device__ __forceinline__ double lane_dot_bf16(const uint4 (&xr)[MAXC], const uint4 (&wr)[MAXC],
                                                int lane, int nchunk) {
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    if (lane + 64 * j < nchunk) {
      double x8[8], w8[8];
      cvt8_f64<bf16_t>(&xr[j], x8);
      cvt8_f64<bf16_t>(&wr[j], w8);
#pragma unroll
      for (int k = 0; k < 8; k++) acc = __builtin_fma(x8[k], w8[k], acc);
    }
  }
  return acc;
}

template <int KPL, int MAXC>
__global__ __launch_bounds__(512) void k_topk_recheck(const bf16_t* __restrict__ x,
                                                       const bf16_t* __restrict__ w,
                                                       const float* __restrict__ bias,
                                                       const float* __restrict__ approx,
                                                       const float* __restrict__ wnorm2, int T,
                                                       int H, int E, int K,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ wts) {
  __shared__ int32_t s_cand[8][64];
  __shared__ TopkSlot s_scr[8][64];
  __shared__ double s_keys[8][64 * KPL];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 8 + wv;
  if (t >= T) return;
  const int nchunk = H / 8;
  // token row in fp64 registers, canonical chunk order; approximate keys
  uint4 xr[MAXC];   // token row, raw bf16 (widened per use)
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    const int q = lane + 64 * j;
    xr[j] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[q < nchunk ? q : 0];
  }
  float ap[KPL], wn[KPL];
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const int e = lane + 64 * j, ec = e < E ? e : E - 1;
    ap[j] = approx[(size_t)t * E + ec];
    wn[j] = wnorm2[ec];
  }
  double xx = 0.0;
#pragma unroll
  for (int j = 0; j < MAXC; j++)
    if (lane + 64 * j < nchunk) {
      double x8[8];
      cvt8_f64<bf16_t>(&xr[j], x8);
#pragma unroll
      for (int k = 0; k < 8; k++) xx = __builtin_fma(x8[k], x8[k], xx);
    }
  float wm = 0.0f, am = 0.0f, amx = -INFINITY, nmn = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const bool ok = lane + 64 * j < E;
    bad |= ok && !(fabsf(ap[j]) < INFINITY);
    if (ok) {
      wm = fmaxf(wm, wn[j]);
      am = fmaxf(am, fabsf(ap[j]));
      amx = fmaxf(amx, ap[j]);
      nmn = fmaxf(nmn, -ap[j]);
    } else {
      ap[j] = -INFINITY;
    }
  }
  bad = __ballot(bad) != 0;
  wm = wave_max_f32(wm);
  am = wave_max_f32(am);
  amx = wave_max_f32(amx);
  nmn = wave_max_f32(nmn);
  xx = wave_sum_f64(xx);
  const double gamma = 1.1 * (double)(H + 64) * 0x1.0p-23;
  const double delta =
      gamma * sqrt(xx) * sqrt((double)wm * 1.001) + 0x1.0p-21 * ((double)am + 1.0);
  // a value th <= the K-th largest approximate key: bisect until K or K + 1
  // keys reach it (or the interval cannot shrink; th keeps the smallest key
  // when the bisection is skipped)
  float th = -nmn;
  if (!bad && E > K + 8) {
    float lo = -nmn, hi = amx;
    for (int it = 0; it < 40; it++) {
      const float mid = lo + (hi - lo) * 0.5f;
      if (!(mid > lo && mid < hi)) break;
      int c = 0;
#pragma unroll
      for (int j = 0; j < KPL; j++) c += __popcll(__ballot(ap[j] >= mid));
      if (c < K) hi = mid;
      else if (c > K + 1) lo = mid;
      else { lo = mid; break; }
    }
    th = lo;
  }
  // candidates: approximate key within 2 delta of th (ascending id)
  const double theta = (double)th - 2.0 * delta;
  int nc = 0;
#pragma unroll
  for (int j = 0; j < KPL; j++) {
    const int e = lane + 64 * j;
    const bool c = e < E && (double)ap[j] >= theta;
    const uint64_t m = __ballot(c);
    if (c) {
      const int pos = nc + __popcll(m & ((1ull << lane) - 1ull));
      if (pos < 64) s_cand[wv][pos] = e;
    }
    nc += __popcll(m);
  }
  // an oversized candidate set, or non-finite inputs, rescore every expert
  const bool all = bad || nc > 64 || nc < K || !(theta > -INFINITY) || !(delta < INFINITY);
  const int ncand = all ? E : nc;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // rescore in rounds of 8 candidates (rows loaded CB at a time), the 8
  // wave sums taken together; candidate i's key ends in lane i (all: in s_keys)
  uint64_t mu = 0;
  uint32_t mid_ = 0xFFFFFFFFu;
  constexpr int CB = MAXC >= 8 ? 1 : 2;
  for (int r0 = 0; r0 < ncand; r0 += 8) {
    double part[8];
#pragma unroll
    for (int b = 0; b < 8; b += CB) {
      // slots past the last candidate are not computed (their sums are unused)
      if (r0 + b >= ncand) {
#pragma unroll
        for (int c = 0; c < CB; c++) part[b + c] = 0.0;
        continue;
      }
      uint4 wr[CB][MAXC];
#pragma unroll
      for (int c = 0; c < CB; c++) {
        const int i = r0 + b + c < ncand ? r0 + b + c : ncand - 1;
        const int e = all ? i : s_cand[wv][i];
        const uint4* row = reinterpret_cast<const uint4*>(w + (size_t)e * H);
#pragma unroll
        for (int j = 0; j < MAXC; j++) {
          const int q = lane + 64 * j;
          wr[c][j] = row[q < nchunk ? q : 0];
        }
      }
#pragma unroll
      for (int c = 0; c < CB; c++) part[b + c] = lane_dot_bf16<MAXC>(xr, wr[c], lane, nchunk);
    }
    const double sum = wave_sum8_f64(part, lane);   // candidate r0 + j in lanes 8j .. 8j + 7
    const int jc = lane >> 3;
    const int ic = r0 + jc < ncand ? r0 + jc : ncand - 1;
    const int ec = all ? ic : s_cand[wv][ic];
    const double key = sum + (bias ? (double)bias[ec] : 0.0);
    if (all) {
      if ((lane & 7) == 0 && r0 + jc < ncand) s_keys[wv][r0 + jc] = key;
    } else {
      // candidate i = r0 + j moves from lane 8 j to lane i
      const int src = 8 * ((lane - r0) & 7);
      const double ki = __shfl(key, src, 64);
      const int ei = __shfl(ec, src, 64);
      if (lane >= r0 && lane < r0 + 8 && lane < ncand) {
        mu = order_key(ki);
        mid_ = (uint32_t)ei;
      }
    }
  }
  int sid;
  uint64_t su;
  if (all) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    topk_threshold<KPL>(s_keys[wv], E, K, lane, s_scr[wv], &sid, &su);
  } else {
    rank_select(mu, mid_, nc, K, lane, s_scr[wv], &sid, &su);
  }
  const float g = topk_weight(lane < K ? key_of_order(su) : 0.0, lane, K);
  if (lane < K) {
    ids[(size_t)t * K + lane] = sid;
    wts[(size_t)t * K + lane] = g;
  }
}

void launch_topk_recheck(const void* x, const void* w, const float* bias, const float* approx,
                         const float* wnorm2, int T, int H, int E, int K, int32_t* ids, float* wts,
                         hipStream_t s) {
  dim3 grid((T + 7) / 8);
  const int maxc = (H / 8 + 63) / 64;
#define MOE_RC(KPL, MC)                                                                         \
  MOE_LAUNCH(MOE_K_TOPK_RECHECK, (k_topk_recheck<KPL, MC>), grid, dim3(512), 0, s,              \
             (const bf16_t*)x, (const bf16_t*)w, bias, approx, wnorm2, T, H, E, K, ids, wts)
#define MOE_RC_KPL(MC)                                                                          \
  do {                                                                                          \
    if (E <= 64) MOE_RC(1, MC);                                                                 \
    else if (E <= 128) MOE_RC(2, MC);                                                           \
    else if (E <= 256) MOE_RC(4, MC);                                                           \
    else MOE_RC(8, MC);                                                                         \
  } while (0)
  if (maxc <= 1) MOE_RC_KPL(1);
  else if (maxc <= 2) MOE_RC_KPL(2);
  else if (maxc <= 4) MOE_RC_KPL(4);
  else MOE_RC_KPL(8);
#undef MOE_RC_KPL
#undef MOE_RC
}

// ---------------------------------------------------------------------------
// A2 + A3 for a decode group (T <= 16): top-K per token, then the union of
// chosen experts as work items.  One routing decision reaches every tier:
// each item carries (tier, slot) = tier_map[expert] (P1, "step 4: three
// shelves, all on the GPU").  Items are ordered by expert id; each lists the
// h row of every token that chose it.  The shared expert, used by every token
// (P5, "What the model actually is"), is the last item.
// ---------------------------------------------------------------------------

constexpr int kMaxBitmapWords = 2048;  // E <= 65535

template <int KPL>
__global__ __launch_bounds__(1024) void k_topk_items(const double* __restrict__ keys, int T, int E,
                                                     int K, const int32_t* __restrict__ tier_map,
                                                     int3 n_slots, int3 tier_bits, int has_shared,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w, Item* __restrict__ items,
                                                     int32_t* __restrict__ n_items) {
  __shared__ uint32_t bitmap[kMaxBitmapWords];
  __shared__ int32_t wordbase[kMaxBitmapWords + 1];
  __shared__ int32_t s_id[kGroup * 64];
  __shared__ int32_t s_tm[kGroup * 64];
  __shared__ float s_w[kGroup * 64];
  __shared__ TopkSlot s_scr[kGroup][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nwords = (E + 31) / 32;
  for (int i = tid; i < nwords; i += blockDim.x) bitmap[i] = 0u;
  if (wv < T) {
    int sid;
    double skey;
    topk_wave<KPL>(keys + (size_t)wv * E, E, K, lane, &sid, &skey, s_scr[wv]);
    const int tm = lane < K ? tier_map[sid] : 0;       // in flight during the softmax
    const float g = topk_weight(skey, lane, K);
    if (lane < K) {
      ids[wv * K + lane] = sid;
      w[wv * K + lane] = g;
      s_id[wv * K + lane] = sid;
      s_w[wv * K + lane] = g;
      s_tm[wv * K + lane] = tm;
    }
  }
  __syncthreads();
  const int nroutes = T * K;
  for (int i = tid; i < nroutes; i += blockDim.x) {
    const int e = s_id[i];
    atomicOr(&bitmap[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (wv == 0) {  // exclusive prefix of per-word popcounts
    int carry = 0;
    for (int base = 0; base < nwords; base += 64) {
      const int i = base + lane;
      const int c = i < nwords ? __popc(bitmap[i]) : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      if (i < nwords) wordbase[i] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) wordbase[nwords] = carry;
  }
  __syncthreads();
  const int n_union = wordbase[nwords];
  // phase 1: clear the token slots of every item (and fill the shared one)
  for (int i = tid; i < (n_union + 1) * kGroup; i += blockDim.x) {
    const int u = i / kGroup, t = i % kGroup;
    if (u < n_union) {
      items[u].route[t] = -1;
      items[u].gw[t] = 0.0f;
    } else if (has_shared) {
      items[u].route[t] = t < T ? nroutes + t : -1;
      items[u].gw[t] = t < T ? 1.0f : 0.0f;
    }
  }
  __syncthreads();
  // phase 2: each route fills its token slot and (redundantly, same values)
  // the header of its item; items are in ascending expert id
  for (int i = tid; i < nroutes; i += blockDim.x) {
    const int e = s_id[i];
    const uint32_t word = bitmap[e >> 5];
    const int u = wordbase[e >> 5] + __popc(word & ((1u << (e & 31)) - 1u));
    const int t = i / K;
    const int tm = s_tm[i];
    const int tier = tm >> 16, slot = tm & 0xFFFF;
    const int ns = tier == 0 ? n_slots.x : (tier == 1 ? n_slots.y : n_slots.z);
    const bool ok = tier >= 0 && tier < 3 && slot < ns;
    Item& it = items[u];
    it.expert = e;
    it.tier = ok ? tier : -1;
    it.slot = ok ? slot : 0;
    it.bits = ok ? (tier == 0 ? tier_bits.x : (tier == 1 ? tier_bits.y : tier_bits.z)) : 0;
    it.route[t] = i;
    it.gw[t] = s_w[i];
  }
  if (tid == 0) {
    if (has_shared) {
      Item& it = items[n_union];
      it.expert = -1;
      it.tier = kDenseTier;
      it.slot = 0;
      it.bits = 0;
    }
    *n_items = n_union + (has_shared ? 1 : 0);
  }
}

void launch_topk_items(const double* keys, int T, int E, int K, const int32_t* tier_map,
                       const int32_t n_slots[3], const int32_t tier_bits[3], int has_shared,
                       int32_t* ids, float* w, Item* items, int32_t* n_items, hipStream_t s) {
  const int3 ns = make_int3(n_slots[0], n_slots[1], n_slots[2]);
  const int3 tb = make_int3(tier_bits[0], tier_bits[1], tier_bits[2]);
  MOE_TOPK_DISPATCH(MOE_K_TOPK_ITEMS, k_topk_items, dim3(1), dim3(1024), 0, s, keys, T, E, K, tier_map, ns, tb,
                    has_shared, ids, w, items, n_items);
}

// ---------------------------------------------------------------------------
// A4: stable counting sort of routes r = t*K + k by expert.
//
// Tokens are cut into chunks of 64 (one bit per token).  Because a token
// picks an expert at most once, "routes of expert e before route (t, k)" in
// ascending route order are exactly the earlier tokens that chose e: the
// rank of (t, k) inside its bucket is the popcount of the chunk's token mask
// of e below bit t, plus the counts of earlier chunks.  Integer only, hence
// deterministic and bit-exact.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_sort_count(const int32_t* __restrict__ ids, int T, int K,
                                                    int E, uint64_t* __restrict__ chunk_mask,
                                                    int32_t* __restrict__ chunk_cnt) {
  extern __shared__ unsigned long long s_mask[];
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();
  const int t0 = chunk * 64;
  const int nt = min(64, T - t0);
  for (int i = threadIdx.x; i < nt * K; i += blockDim.x) {
    const int t = i / K;
    const int e = ids[(size_t)t0 * K + i];
    atomicOr(&s_mask[e], 1ull << t);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const uint64_t m = s_mask[e];
    chunk_mask[(size_t)chunk * E + e] = m;
    chunk_cnt[(size_t)chunk * E + e] = __popcll(m);
  }
}

// Bucket offsets (exclusive scan of the per-expert totals), each chunk's
// base inside every bucket, and the GEMM tile list: bucket e splits into
// ceil(n_e / tile_rows) tiles, recorded as (e, first row of the tile inside
// the bucket).  Longest first: the full tiles of every bucket (expert
// order), then the ragged last tiles of more than half a tile, then the
// rest, so the short workgroups fill the end of the grouped GEMMs.
// chunk_base holds the counts on entry.  One workgroup; E <= 4096.
// Class of a bucket's ragged last tile: 1 when it holds more than half a
// tile of rows, 1 << 16 when it holds fewer, 0 when there is none.
__device__ __forceinline__ int tile_class(int n_e, int tile_rows) {
  const int r = n_e % tile_rows;
  return r == 0 ? 0 : (2 * r > tile_rows ? 1 : 1 << 16);
}

__global__ __launch_bounds__(1024) void k_sort_scan(int n_chunks, int E, int tile_rows,
                                                    int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ offsets,
                                                    int2* __restrict__ tiles,
                                                    int32_t* __restrict__ n_tiles) {
  __shared__ int32_t s_tot[4096];
  __shared__ int32_t s_til[4096];   // full tiles of the bucket, then their scan
  __shared__ int32_t s_prt[4096];   // ragged tile: 1 (long) or 1 << 16 (short), then the scan
  __shared__ int32_t s_wave[16][3];
  __shared__ int32_t s_total, s_full, s_long;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // one expert per thread and at most 64 chunks (4096 tokens): every count is
  // loaded at once and kept in registers for the second pass
  constexpr int CMAX = 64;
  const bool regs = E <= (int)blockDim.x && n_chunks <= CMAX;
  int rc[CMAX];
  if (regs) {
    const int e = tid < E ? tid : E - 1;
#pragma unroll
    for (int c = 0; c < CMAX; c++) rc[c] = chunk_base[(size_t)(c < n_chunks ? c : n_chunks - 1) * E + e];
    if (tid < E) {
      int sum = 0;
#pragma unroll
      for (int c = 0; c < CMAX; c++) sum += c < n_chunks ? rc[c] : 0;
      s_tot[tid] = sum;
      s_til[tid] = sum / tile_rows;
      s_prt[tid] = tile_class(sum, tile_rows);
    }
  }
  // otherwise: per-expert totals over the chunks, 8 loads in flight per thread
  for (int e = tid; e < E && !regs; e += blockDim.x) {
    int sum = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int c = c0 + j < n_chunks ? c0 + j : n_chunks - 1;
        v[j] = chunk_base[(size_t)c * E + e];
      }
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (c0 + j < n_chunks) sum += v[j];
    }
    s_tot[e] = sum;
    s_til[e] = sum / tile_rows;
    s_prt[e] = tile_class(sum, tile_rows);
  }
  __syncthreads();
  // exclusive scans of s_tot, s_til and s_prt (two 16-bit counts packed;
  // each stays <= E), 4 consecutive experts per thread
  int v[4], u[4], w[4];
  int local = 0, ulocal = 0, wlocal = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = tid * 4 + j;
    v[j] = e < E ? s_tot[e] : 0;
    u[j] = e < E ? s_til[e] : 0;
    w[j] = e < E ? s_prt[e] : 0;
    local += v[j];
    ulocal += u[j];
    wlocal += w[j];
  }
  int incl = local, uincl = ulocal, wincl = wlocal;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    const int uo = __shfl_up(uincl, off, 64);
    const int wo = __shfl_up(wincl, off, 64);
    if (lane >= off) {
      incl += o;
      uincl += uo;
      wincl += wo;
    }
  }
  if (lane == 63) {
    s_wave[wv][0] = incl;
    s_wave[wv][1] = uincl;
    s_wave[wv][2] = wincl;
  }
  __syncthreads();
  int wbase = 0, ubase = 0, pbase = 0;
  for (int i = 0; i < wv; i++) {
    wbase += s_wave[i][0];
    ubase += s_wave[i][1];
    pbase += s_wave[i][2];
  }
  int run = wbase + incl - local, urun = ubase + uincl - ulocal, wrun = pbase + wincl - wlocal;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = tid * 4 + j;
    if (e < E) {
      s_tot[e] = run;
      s_til[e] = urun;
      s_prt[e] = wrun;
    }
    run += v[j];
    urun += u[j];
    wrun += w[j];
  }
  if (tid == blockDim.x - 1) {
    offsets[E] = run;
    *n_tiles = urun + (wrun & 0xFFFF) + (wrun >> 16);
    s_total = run;
    s_full = urun;
    s_long = wrun & 0xFFFF;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int base0 = s_tot[e];
    offsets[e] = base0;
    const int n_e = (e + 1 < E ? s_tot[e + 1] : s_total) - base0;
    const int nf = n_e / tile_rows, r = n_e - nf * tile_rows;
    for (int p = 0; p < nf; p++) tiles[s_til[e] + p] = make_int2(e, p * tile_rows);
    if (r > 0) {
      const int pr = s_prt[e];
      const int pos = 2 * r > tile_rows ? s_full + (pr & 0xFFFF) : s_full + s_long + (pr >> 16);
      tiles[pos] = make_int2(e, nf * tile_rows);
    }
    int base = base0;
    if (regs) {
#pragma unroll
      for (int c = 0; c < CMAX; c++) {
        if (c < n_chunks) {
          chunk_base[(size_t)c * E + e] = base;
          base += rc[c];
        }
      }
      continue;
    }
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      int cnt[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int c = c0 + j < n_chunks ? c0 + j : n_chunks - 1;
        cnt[j] = chunk_base[(size_t)c * E + e];
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (c0 + j < n_chunks) {
          chunk_base[(size_t)(c0 + j) * E + e] = base;
          base += cnt[j];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t* __restrict__ ids, int T, int K,
                                                      int E, const uint64_t* __restrict__ chunk_mask,
                                                      const int32_t* __restrict__ chunk_base,
                                                      int32_t* __restrict__ sorted_routes,
                                                      int32_t* __restrict__ route_pos) {
  const int chunk = blockIdx.x;
  const int t0 = chunk * 64;
  const int nt = min(64, T - t0);
  for (int i = threadIdx.x; i < nt * K; i += blockDim.x) {
    const int t = i / K;
    const int r = t0 * K + i;
    const int e = ids[r];
    const uint64_t m = chunk_mask[(size_t)chunk * E + e];
    const uint64_t below = t == 0 ? 0ull : (m & ((1ull << t) - 1ull));
    const int pos = chunk_base[(size_t)chunk * E + e] + __popcll(below);
    sorted_routes[pos] = r;
    route_pos[r] = pos;
  }
}

void launch_sort_routes(const int32_t* ids, int T, int K, int E, uint64_t* chunk_mask,
                        int32_t* chunk_base, int32_t* offsets, int32_t* sorted_routes,
                        int32_t* route_pos, int tile_rows, int2* tiles, int32_t* n_tiles,
                        hipStream_t s) {
  const int n_chunks = (T + 63) / 64;
  MOE_LAUNCH(MOE_K_SORT_COUNT, k_sort_count, dim3(n_chunks), dim3(256), E * sizeof(uint64_t), s, ids, T, K, E,
                     chunk_mask, chunk_base);
  MOE_LAUNCH(MOE_K_SORT_SCAN, k_sort_scan, dim3(1), dim3(1024), 0, s, n_chunks, E, tile_rows,
             chunk_base, offsets, tiles, n_tiles);
  MOE_LAUNCH(MOE_K_SORT_SCATTER, k_sort_scatter, dim3(n_chunks), dim3(256), 0, s, ids, T, K, E, chunk_mask,
                     chunk_base, sorted_routes, route_pos);
}

}  // namespace moe
