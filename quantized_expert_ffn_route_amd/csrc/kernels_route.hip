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

void launch_router_keys(int act, const void* x, const void* w, const float* b, double* keys,
                        int T, int H, int E, hipStream_t s) {
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

// Monotone map of a key to uint64: larger key -> larger value; -0 == +0;
// NaN maps to 0, below every number.
__device__ __forceinline__ uint64_t order_key(double k) {
  if (k != k) return 0ull;
  if (k == 0.0) k = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(k);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ bool ranks_before(uint64_t au, uint32_t aid, uint64_t bu, uint32_t bid) {
  return au > bu || (au == bu && aid < bid);
}

// Selects the top K of `krow` (E keys) with one wave.  Lane r < K returns the
// r-th selected id in *sel_id and its key in *sel_key.  KPL keys per lane are
// kept in registers (E <= 64*KPL); KPL == 0 rescans memory each round.
template <int KPL>
__device__ void topk_wave(const double* __restrict__ krow, int E, int K, int lane, int* sel_id,
                          double* sel_key) {
  uint64_t uk[KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
#pragma unroll
    for (int j = 0; j < KPL; j++) {
      const int e = lane + 64 * j;
      uk[j] = e < E ? order_key(krow[e]) : 0ull;
    }
  }
  uint64_t last_u = 0;
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
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t ou = __shfl_xor(bu, off, 64);
      const uint32_t oid = __shfl_xor(bid, off, 64);
      if (ranks_before(ou, oid, bu, bid)) {
        bu = ou;
        bid = oid;
      }
    }
    last_u = bu;
    last_id = bid;
    if (lane == r) my_id = (int)bid;
  }
  *sel_id = my_id;
  *sel_key = (lane < K) ? krow[my_id] : 0.0;
}

// Mixing weights over the K selected keys: softmax in float64, stored fp32.
__device__ __forceinline__ float topk_weight(double key, int lane, int K) {
  const double k0 = __shfl(key, 0, 64);
  const double z = lane < K ? exp(key - k0) : 0.0;
  const double sum = wave_sum_f64(z);
  return (float)(z / sum);
}

template <int KPL>
__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ keys, int T, int E, int K,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (t >= T) return;
  int sid;
  double skey;
  topk_wave<KPL>(keys + (size_t)t * E, E, K, lane, &sid, &skey);
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
  __shared__ float s_w[kGroup * 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nwords = (E + 31) / 32;
  for (int i = tid; i < nwords; i += blockDim.x) bitmap[i] = 0u;
  if (wv < T) {
    int sid;
    double skey;
    topk_wave<KPL>(keys + (size_t)wv * E, E, K, lane, &sid, &skey);
    const float g = topk_weight(skey, lane, K);
    if (lane < K) {
      ids[wv * K + lane] = sid;
      w[wv * K + lane] = g;
      s_id[wv * K + lane] = sid;
      s_w[wv * K + lane] = g;
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
  // item headers, in ascending expert id
  for (int e = tid; e < E; e += blockDim.x) {
    const uint32_t word = bitmap[e >> 5];
    if (!((word >> (e & 31)) & 1u)) continue;
    const int u = wordbase[e >> 5] + __popc(word & ((1u << (e & 31)) - 1u));
    const int tm = tier_map[e];
    const int tier = tm >> 16, slot = tm & 0xFFFF;
    const int ns = tier == 0 ? n_slots.x : (tier == 1 ? n_slots.y : n_slots.z);
    const bool ok = tier >= 0 && tier < 3 && slot < ns;
    Item& it = items[u];
    it.expert = e;
    it.tier = ok ? tier : -1;
    it.slot = ok ? slot : 0;
    it.bits = ok ? (tier == 0 ? tier_bits.x : (tier == 1 ? tier_bits.y : tier_bits.z)) : 0;
#pragma unroll
    for (int t = 0; t < kGroup; t++) {
      it.route[t] = -1;
      it.gw[t] = 0.0f;
    }
  }
  __syncthreads();
  for (int i = tid; i < nroutes; i += blockDim.x) {
    const int e = s_id[i];
    const uint32_t word = bitmap[e >> 5];
    const int u = wordbase[e >> 5] + __popc(word & ((1u << (e & 31)) - 1u));
    const int t = i / K;
    items[u].route[t] = i;
    items[u].gw[t] = s_w[i];
  }
  if (tid == 0) {
    if (has_shared) {
      Item& it = items[n_union];
      it.expert = -1;
      it.tier = kDenseTier;
      it.slot = 0;
      it.bits = 0;
#pragma unroll
      for (int t = 0; t < kGroup; t++) {
        it.route[t] = t < T ? nroutes + t : -1;
        it.gw[t] = t < T ? 1.0f : 0.0f;
      }
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

// One block: per-expert totals over chunks, exclusive scan over experts,
// then per-chunk bases.  chunk_base holds the counts on entry.
__global__ __launch_bounds__(1024) void k_sort_scan(int n_chunks, int E, int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t s_tot[4096];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) {
    int sum = 0;
    for (int c = 0; c < n_chunks; c++) sum += chunk_base[(size_t)c * E + e];
    s_tot[e] = sum;
  }
  __syncthreads();
  // exclusive scan of s_tot[0..E) with 1024 threads, 4 consecutive per thread
  int v[4];
  int local = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = tid * 4 + j;
    v[j] = e < E ? s_tot[e] : 0;
    local += v[j];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wv] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < wv; i++) wbase += s_wave[i];
  int run = wbase + incl - local;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = tid * 4 + j;
    if (e < E) s_tot[e] = run;
    run += v[j];
  }
  if (tid == blockDim.x - 1) offsets[E] = run;
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int base = s_tot[e];
    offsets[e] = base;
    for (int c = 0; c < n_chunks; c++) {
      const int cnt = chunk_base[(size_t)c * E + e];
      chunk_base[(size_t)c * E + e] = base;
      base += cnt;
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
                        int32_t* route_pos, hipStream_t s) {
  const int n_chunks = (T + 63) / 64;
  MOE_LAUNCH(MOE_K_SORT_COUNT, k_sort_count, dim3(n_chunks), dim3(256), E * sizeof(uint64_t), s, ids, T, K, E,
                     chunk_mask, chunk_base);
  MOE_LAUNCH(MOE_K_SORT_SCAN, k_sort_scan, dim3(1), dim3(1024), 0, s, n_chunks, E, chunk_base, offsets);
  MOE_LAUNCH(MOE_K_SORT_SCATTER, k_sort_scatter, dim3(n_chunks), dim3(256), 0, s, ids, T, K, E, chunk_mask,
                     chunk_base, sorted_routes, route_pos);
}

}  // namespace moe
