// C ABI of the tiered MoE layer: argument validation, workspace layout, the
// host tier build (A0) and the launch sequences of route / decode / prefill.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "internal.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t act_bytes(int act) { return act == MOE_BF16 ? 2 : 4; }

void mat_shape(const moe_dims* d, int mat, int* rows, int* cols) {
  if (mat == MOE_DOWN) {
    *rows = d->hidden;
    *cols = d->inter;
  } else {
    *rows = d->inter;
    *cols = d->hidden;
  }
}

int check_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (d->n_experts > 65535) return MOE_EINVAL;
  if (d->top_k > d->n_experts || d->top_k > 64) return MOE_EINVAL;
  if (d->has_shared != 0 && d->has_shared != 1) return MOE_EINVAL;
  if (d->act != MOE_F32 && d->act != MOE_BF16) return MOE_EINVAL;
  if (d->hidden % 128 || d->inter % 128 || d->hidden > 8192) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_tiers(const moe_dims* d, const int32_t n_slots[3], const int32_t tier_bits[3]) {
  int64_t sum = 0;
  for (int t = 0; t < 3; t++) {
    if (n_slots[t] < 0) return MOE_EINVAL;
    sum += n_slots[t];
    if (n_slots[t] > 0 && !valid_format(tier_bits[t])) return MOE_EINVAL;
  }
  return sum == d->n_experts ? MOE_OK : MOE_EINVAL;
}

int check_layer(const moe_dims* d, const moe_layer* L) {
  if (!L) return MOE_EINVAL;
  if (!L->w_router || !aligned(L->w_router, 16) || !L->tier_map) return MOE_EINVAL;
  if (L->b_router && !aligned(L->b_router, 4)) return MOE_EINVAL;
  int rc = check_tiers(d, L->n_slots, L->tier_bits);
  if (rc) return rc;
  for (int t = 0; t < 3; t++)
    if (L->down_bits[t] != 0 && !valid_format(L->down_bits[t])) return MOE_EINVAL;
  for (int t = 0; t < 3; t++) {
    if (L->n_slots[t] == 0) continue;
    for (int m = 0; m < 3; m++)
      if (!L->codes[t][m] || !L->dm[t][m] || !aligned(L->codes[t][m], 16) || !aligned(L->dm[t][m], 16))
        return MOE_EINVAL;
  }
  if (d->has_shared)
    for (int m = 0; m < 3; m++)
      if (!L->w_shared[m] || !aligned(L->w_shared[m], 16)) return MOE_EINVAL;
  return MOE_OK;
}

Tables make_tables(const moe_dims* d, const moe_layer* L) {
  Tables tb;
  std::memset(&tb, 0, sizeof(tb));
  for (int t = 0; t < 3; t++) {
    tb.bits[t] = L->tier_bits[t];
    tb.bits_dn[t] = L->down_bits[t] ? L->down_bits[t] : L->tier_bits[t];
    tb.n_slots[t] = L->n_slots[t];
    for (int m = 0; m < 3; m++) {
      tb.codes[t][m] = L->codes[t][m];
      tb.dm[t][m] = L->dm[t][m];
    }
  }
  for (int m = 0; m < 3; m++) tb.dense[m] = d->has_shared ? L->w_shared[m] : nullptr;
  return tb;
}

// Workspace carving: every region 256-byte aligned.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

struct RouteWs {
  size_t keys, total;
};
RouteWs route_ws(const moe_dims* d, int64_t T) {
  Carve c;
  RouteWs w;
  w.keys = c.take((size_t)T * d->n_experts * sizeof(double));
  w.total = c.off;
  return w;
}

struct DecodeWs {
  size_t keys, ids, w, items, n_items, h, total;
  int max_items;
};
DecodeWs decode_ws(const moe_dims* d) {
  Carve c;
  DecodeWs w;
  const int G = kGroup, K = d->top_k;
  w.max_items = G * K + 1;
  w.keys = c.take((size_t)G * d->n_experts * sizeof(double));
  w.ids = c.take((size_t)G * K * sizeof(int32_t));
  w.w = c.take((size_t)G * K * sizeof(float));
  w.items = c.take((size_t)w.max_items * sizeof(Item));
  w.n_items = c.take(sizeof(int32_t));
  w.h = c.take((size_t)(G * K + G) * d->inter * act_bytes(d->act));
  w.total = c.off;
  return w;
}

struct PrefillWs {
  size_t keys, approx, wnorm2, ids, w, chunk_mask, chunk_base, offsets, tiles, n_tiles, sorted,
      route_pos, h, h_s, route_rows, shared_rows, total;
  int max_tiles;
};
// The bf16 prefill router: MFMA keys + exact float64 rescoring of the
// candidates (the recheck kernel holds up to 512 keys per token and H <= 4096
// in registers; the MFMA pass works on 32-row groups of the router matrix).
bool mfma_router(const moe_dims* d) {
  return d->act == MOE_BF16 && d->n_experts <= 512 && d->n_experts % 32 == 0 &&
         d->top_k <= 64 && d->hidden <= 4096;
}

PrefillWs prefill_ws(const moe_dims* d, int64_t T) {
  Carve c;
  PrefillWs w;
  const int64_t K = d->top_k, E = d->n_experts, H = d->hidden, n_chunks = (T + 63) / 64;
  const bool bf16 = mfma_router(d);
  // float64 keys for fp32 activations; bf16 takes the MFMA keys + recheck
  w.keys = c.take(bf16 ? 0 : (size_t)T * E * sizeof(double));
  w.approx = c.take(bf16 ? (size_t)T * E * sizeof(float) : 0);
  w.wnorm2 = c.take(bf16 ? (size_t)E * sizeof(float) : 0);
  w.ids = c.take((size_t)T * K * sizeof(int32_t));
  w.w = c.take((size_t)T * K * sizeof(float));
  w.chunk_mask = c.take((size_t)n_chunks * E * sizeof(uint64_t));
  w.chunk_base = c.take((size_t)n_chunks * E * sizeof(int32_t));
  w.offsets = c.take((size_t)(E + 1) * sizeof(int32_t));
  const int64_t rows = prefill_tile_rows(d->act);
  w.max_tiles = (int)(E + (T * K + rows - 1) / rows);
  w.tiles = c.take((size_t)w.max_tiles * 2 * sizeof(int32_t));
  w.n_tiles = c.take(sizeof(int32_t));
  w.sorted = c.take((size_t)T * K * sizeof(int32_t));
  w.route_pos = c.take((size_t)T * K * sizeof(int32_t));
  w.h = c.take((size_t)T * K * d->inter * act_bytes(d->act));
  w.h_s = c.take(d->has_shared ? (size_t)T * d->inter * act_bytes(d->act) : 0);
  w.route_rows = c.take((size_t)T * K * H * sizeof(float));
  w.shared_rows = c.take(d->has_shared ? (size_t)T * H * sizeof(float) : 0);
  w.total = c.off;
  return w;
}

// Common checks of the forward / route calls.  Returns MOE_OK and sets
// *size_only when the caller asked for the workspace size.
int check_ws(void* ws, size_t* ws_bytes, size_t need, bool* size_only) {
  if (!ws_bytes) return MOE_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    *size_only = true;
    return MOE_OK;
  }
  *size_only = false;
  if (!aligned(ws, kAlign)) return MOE_EINVAL;
  if (*ws_bytes < need) return MOE_ENOSPC;
  return MOE_OK;
}

// Launch errors are read from hipGetLastError(); clear_hip_error() at the
// start of a launch sequence keeps errors left by unrelated HIP calls of the
// process from being reported as this library's.
inline void clear_hip_error() { (void)hipGetLastError(); }
inline int hip_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

struct Trace {
  hipEvent_t* events = nullptr;
  int32_t* tags = nullptr;
  int32_t capacity = 0;
  int32_t* n_used = nullptr;
};
Trace g_trace;

}  // namespace

namespace moe {

void trace_slot(int kernel_id, hipStream_t s, hipEvent_t* start, hipEvent_t* stop) {
  Trace& t = g_trace;
  *start = *stop = nullptr;
  if (!t.events || *t.n_used >= t.capacity / 2) return;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();  // query unsupported on this stream: not capturing
    st = hipStreamCaptureStatusNone;
  }
  if (st != hipStreamCaptureStatusNone) return;  // no timing events inside graphs
  const int i = (*t.n_used)++;
  t.tags[i] = kernel_id;
  *start = t.events[2 * i];
  *stop = t.events[2 * i + 1];
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported shape or dtype";
    case MOE_ENOSPC: return "MOE_ENOSPC: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}

int moe_check_layer(const moe_dims* dims, const moe_layer* layer, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_layer(dims, layer))) return rc;
  const int E = dims->n_experts;
  std::vector<int32_t> tmap(E);
  clear_hip_error();
  if (hipMemcpyAsync(tmap.data(), layer->tier_map, (size_t)E * sizeof(int32_t),
                     hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_EHIP;
  // every entry names a slot of a non-empty tier, and no slot twice
  std::vector<uint8_t> used[3];
  for (int t = 0; t < 3; t++) used[t].assign((size_t)layer->n_slots[t], 0);
  for (int e = 0; e < E; e++) {
    const int t = tmap[e] >> 16, sl = tmap[e] & 0xFFFF;
    if (t < 0 || t > 2 || sl >= layer->n_slots[t] || used[t][sl]) return MOE_EINVAL;
    used[t][sl] = 1;
  }
  return MOE_OK;
}

int moe_set_trace(hipEvent_t* events, int32_t* tags, int32_t capacity, int32_t* n_used) {
  if (events && (capacity < 0 || !tags || !n_used)) return MOE_EINVAL;
  g_trace.events = events;
  g_trace.tags = events ? tags : nullptr;
  g_trace.capacity = events ? capacity : 0;
  g_trace.n_used = events ? n_used : nullptr;
  return MOE_OK;
}

size_t moe_tier_table_bytes(const moe_dims* dims, int32_t bits, int32_t n_slots, int32_t mat,
                            int32_t which) {
  if (check_dims(dims) != MOE_OK || n_slots < 0 || mat < 0 || mat > 2) return 0;
  if (!valid_format(bits)) return 0;
  int rows, cols;
  mat_shape(dims, mat, &rows, &cols);
  const size_t blocks = (size_t)n_slots * rows * (cols / 32);
  if (which == MOE_CODES) return blocks * field_bytes(bits);
  if (which == MOE_DM) return blocks * scale_bytes(bits);
  return 0;
}

// ---------------------------------------------------------------------------
// A0: tier build.
// ---------------------------------------------------------------------------

// Tier sizes for a byte budget: the popularity-band plan of least expected
// error.  Error of an expert at b bits = popularity * 11025 / (2^b - 1)^2
// (exact integers: 49, 225, 1225 for 4, 3, 2 bits).  For a given n0 the
// error is monotone in n1 (it moves ranks between tiers 1 and 2), so the
// best n1 is an end of its feasible interval: O(E log E) in all.
int moe_plan_tiers(const moe_dims* dims, const uint64_t* popularity, const int32_t tier_bits[3],
                   uint64_t budget_bytes, int32_t n_slots_out[3]) {
  return moe_plan_tiers_ladder(dims, popularity, tier_bits, nullptr, budget_bytes, n_slots_out);
}

// With a down ladder an expert of tier t stores gate and up at tier_bits[t]
// and down at its own width: bytes and error add up over the three matrices
// (equal sizes), so the band search is the same with per-tier totals.
int moe_plan_tiers_ladder(const moe_dims* dims, const uint64_t* popularity,
                          const int32_t tier_bits[3], const int32_t down_bits[3],
                          uint64_t budget_bytes, int32_t n_slots_out[3]) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!popularity || !tier_bits || !n_slots_out) return MOE_EINVAL;
  int32_t dn[3];
  for (int t = 0; t < 3; t++) {
    dn[t] = down_bits && down_bits[t] ? down_bits[t] : tier_bits[t];
    if (tier_bits[t] != 2 && tier_bits[t] != 3 && tier_bits[t] != 4) return MOE_EINVAL;
    if (dn[t] != 2 && dn[t] != 3 && dn[t] != 4) return MOE_EINVAL;
  }
  const int E = dims->n_experts;
  std::vector<int32_t> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return popularity[a] != popularity[b] ? popularity[a] > popularity[b] : a < b;
  });
  typedef unsigned __int128 u128;
  // P[r]: popularity of ranks < r
  std::vector<u128> P(E + 1, 0);
  for (int r = 0; r < E; r++) P[r + 1] = P[r] + popularity[order[r]];
  auto werr = [](int b) -> u128 { return b == 4 ? 49 : (b == 3 ? 225 : 1225); };
  // error weight and bytes of one expert of tier t (gate, up, down)
  auto wt = [&](int t) { return 2 * werr(tier_bits[t]) + werr(dn[t]); };
  const u128 w0 = wt(0), w1 = wt(1), w2 = wt(2);
  const int64_t blocks = (int64_t)dims->hidden * dims->inter / 32;   // per matrix
  auto ct = [&](int t) { return blocks * (2 * (4 * tier_bits[t] + 4) + (4 * dn[t] + 4)); };
  const int64_t c0 = ct(0), c1 = ct(1), c2 = ct(2);
  const __int128 budget = (__int128)budget_bytes;
  bool found = false;
  u128 best = 0;
  int bn0 = 0, bn1 = 0;
  for (int n0 = E; n0 >= 0; n0--) {
    const int rest = E - n0;
    // n1 * (c1 - c2) <= R
    const __int128 R = budget - (__int128)n0 * c0 - (__int128)rest * c2;
    int lo = 0, hi = rest;
    if (c1 > c2) {
      if (R < 0) continue;
      const __int128 m = R / (c1 - c2);
      hi = m < rest ? (int)m : rest;
    } else if (c1 < c2) {
      const __int128 need = R >= 0 ? 0 : (-R + (c2 - c1) - 1) / (c2 - c1);
      if (need > rest) continue;
      lo = (int)need;
    } else if (R < 0) {
      continue;
    }
    // error of (n0, n1): tier 0 on ranks < n0, tier 1 on [n0, n0 + n1), tier 2 after
    auto err = [&](int n1) {
      return w0 * P[n0] + w1 * (P[n0 + n1] - P[n0]) + w2 * (P[E] - P[n0 + n1]);
    };
    int n1;
    if (w1 <= w2) {
      n1 = hi;                                   // error never rises with n1
    } else {
      // error never falls with n1: the largest n1 as good as the smallest
      n1 = lo;
      const u128 at = P[n0 + lo];
      int a = lo, b = hi;                        // P[n0 + a] == at; find the last such
      while (a < b) {
        const int mid = a + (b - a + 1) / 2;
        if (P[n0 + mid] == at) a = mid; else b = mid - 1;
      }
      n1 = a;
    }
    const u128 e = err(n1);
    if (!found || e < best) {
      found = true;
      best = e;
      bn0 = n0;
      bn1 = n1;
    }
  }
  if (!found) return MOE_EINVAL;
  n_slots_out[0] = bn0;
  n_slots_out[1] = bn1;
  n_slots_out[2] = E - bn0 - bn1;
  return MOE_OK;
}


int moe_build_tiers(const moe_dims* dims, const uint64_t* popularity, const int32_t n_slots[3],
                    const int32_t tier_bits[3], const moe_expert_source* src,
                    int32_t* tier_map_out, int32_t* slot_expert_out, moe_layer* dst,
                    int32_t dst_on_device, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!popularity || !n_slots || !tier_bits || !tier_map_out) return MOE_EINVAL;
  rc = check_tiers(dims, n_slots, tier_bits);
  if (rc) return rc;
  const int E = dims->n_experts;
  // rank: popularity descending, lower id first on equal counts
  std::vector<int32_t> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return popularity[a] != popularity[b] ? popularity[a] > popularity[b] : a < b;
  });
  const int start[3] = {0, n_slots[0], n_slots[0] + n_slots[1]};
  std::vector<int32_t> tmap(E);
  for (int rank = 0; rank < E; rank++) {
    const int tier = rank < start[1] ? 0 : (rank < start[2] ? 1 : 2);
    tmap[order[rank]] = (tier << 16) | (rank - start[tier]);
  }
  if (!src || !dst) {
    std::memcpy(tier_map_out, tmap.data(), E * sizeof(int32_t));
    if (slot_expert_out) std::memcpy(slot_expert_out, order.data(), E * sizeof(int32_t));
    return MOE_OK;
  }
  if (src->kind != MOE_SRC_F32 && src->kind != MOE_SRC_CODES) return MOE_EINVAL;
  for (int m = 0; m < 3; m++) {
    if (src->kind == MOE_SRC_F32 && !src->w[m]) return MOE_EINVAL;
    if (src->kind == MOE_SRC_CODES && (!src->q[m] || !src->d[m])) return MOE_EINVAL;
  }
  for (int t = 0; t < 3; t++)
    if (n_slots[t] > 0)
      for (int m = 0; m < 3; m++)
        if (!dst->codes[t][m] || !dst->dm[t][m]) return MOE_EINVAL;
  if (dst_on_device && !dst->tier_map) return MOE_EINVAL;
  // code width of tier t, matrix m: the down matrices may have their own
  int32_t mbits[3][3];
  for (int t = 0; t < 3; t++) {
    const int dn = dst->down_bits[t];
    if (dn != 0 && !valid_format(dn)) return MOE_EINVAL;
    for (int m = 0; m < 3; m++) mbits[t][m] = m == MOE_DOWN && dn ? dn : tier_bits[t];
  }
  // affine blocks given as codes need their min table
  for (int t = 0; t < 3; t++)
    for (int m = 0; m < 3; m++)
      if (src->kind == MOE_SRC_CODES && n_slots[t] > 0 && mbits[t][m] != kMx4 && !src->m[m])
        return MOE_EINVAL;

  std::atomic<int> status{MOE_OK};
  // pack one (tier, matrix, slot) expert matrix into `codes`/`dm`
  auto pack_one = [&](int t, int m, int slot, uint8_t* codes, uint32_t* dm) {
    const int bits = mbits[t][m];
    const bool mx = bits == kMx4;
    const int L = mx ? 15 : (1 << bits) - 1, fb = field_bytes(bits);
    const int e = order[start[t] + slot];
    int R, C;
    mat_shape(dims, m, &R, &C);
    const int nb = C / 32;
    uint8_t q[32], field[16];
    for (int r = 0; r < R; r++) {
      for (int j = 0; j < nb; j++) {
        uint16_t db = 0, mb = 0;
        uint8_t eb = 0;
        const size_t blk = ((size_t)e * R + r) * nb + j;
        if (src->kind == MOE_SRC_F32) {
          const int rc = mx ? quantise_block_mx(src->w[m] + blk * 32, &eb, q)
                            : quantise_block(src->w[m] + blk * 32, bits, &db, &mb, q);
          if (rc != MOE_OK) {
            status = MOE_EINVAL;
            return;
          }
        } else {
          const uint8_t* qs = src->q[m] + blk * 32;
          for (int i = 0; i < 32; i++) {
            if (qs[i] > L) {
              status = MOE_EINVAL;
              return;
            }
            q[i] = qs[i];
          }
          if (mx) {
            eb = (uint8_t)src->d[m][blk];
            if (eb < 2 || eb > 252) {
              status = MOE_EINVAL;
              return;
            }
          } else {
            db = src->d[m][blk];
            mb = src->m[m][blk];
            if ((db & 0x7C00u) == 0x7C00u || (mb & 0x7C00u) == 0x7C00u) {
              status = MOE_EINVAL;
              return;
            }
          }
        }
        encode_codes(q, bits, field);
        const size_t idx = tile_block_index(slot, r, j, R, C);
        std::memcpy(codes + idx * fb, field, fb);
        if (mx) reinterpret_cast<uint8_t*>(dm)[idx] = eb;
        else dm[idx] = (uint32_t)db | ((uint32_t)mb << 16);
      }
    }
  };

  // host destination buffers (staging when the tables live on the device)
  std::vector<std::vector<uint8_t>> stage_codes(9), stage_dm(9);
  uint8_t* hc[3][3] = {};
  uint32_t* hd[3][3] = {};
  for (int t = 0; t < 3; t++) {
    if (n_slots[t] == 0) continue;
    for (int m = 0; m < 3; m++) {
      const size_t cb = moe_tier_table_bytes(dims, mbits[t][m], n_slots[t], m, MOE_CODES);
      const size_t db = moe_tier_table_bytes(dims, mbits[t][m], n_slots[t], m, MOE_DM);
      if (dst_on_device) {
        stage_codes[3 * t + m].assign(cb, 0);
        stage_dm[3 * t + m].assign(db, 0);
        hc[t][m] = stage_codes[3 * t + m].data();
        hd[t][m] = reinterpret_cast<uint32_t*>(stage_dm[3 * t + m].data());
      } else {
        hc[t][m] = dst->codes[t][m];
        hd[t][m] = dst->dm[t][m];
      }
    }
  }
  struct Job { int t, m, slot; };
  std::vector<Job> jobs;
  for (int t = 0; t < 3; t++)
    for (int m = 0; m < 3; m++)
      for (int s = 0; s < n_slots[t]; s++) jobs.push_back({t, m, s});
  std::atomic<size_t> next{0};
  const unsigned nthreads =
      std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::vector<std::thread> pool;
  for (unsigned i = 0; i < nthreads; i++)
    pool.emplace_back([&] {
      for (size_t j; (j = next++) < jobs.size() && status == MOE_OK;)
        pack_one(jobs[j].t, jobs[j].m, jobs[j].slot, hc[jobs[j].t][jobs[j].m], hd[jobs[j].t][jobs[j].m]);
    });
  for (auto& th : pool) th.join();
  if (status != MOE_OK) return status;

  if (dst_on_device) {
    // a tier's tables are device memory or pinned, device-mapped host memory
    // (a tier kept in host memory): the runtime takes the direction from the
    // destination pointer
    for (int t = 0; t < 3; t++) {
      if (n_slots[t] == 0) continue;
      for (int m = 0; m < 3; m++) {
        if (hipMemcpyAsync(dst->codes[t][m], hc[t][m], stage_codes[3 * t + m].size(),
                           hipMemcpyDefault, stream) != hipSuccess ||
            hipMemcpyAsync(dst->dm[t][m], hd[t][m], stage_dm[3 * t + m].size(),
                           hipMemcpyDefault, stream) != hipSuccess)
          return MOE_EHIP;
      }
    }
    if (hipMemcpyAsync(dst->tier_map, tmap.data(), E * sizeof(int32_t), hipMemcpyHostToDevice,
                       stream) != hipSuccess)
      return MOE_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_EHIP;
  } else if (dst->tier_map) {
    std::memcpy(dst->tier_map, tmap.data(), E * sizeof(int32_t));
  }
  std::memcpy(tier_map_out, tmap.data(), E * sizeof(int32_t));
  if (slot_expert_out) std::memcpy(slot_expert_out, order.data(), E * sizeof(int32_t));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// A1-A2: route.
// ---------------------------------------------------------------------------

int moe_route(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
              int32_t* topk_ids, float* topk_w, void* ws, size_t* ws_bytes, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_layer(dims, layer))) return rc;
  if (T < 0 || (int64_t)T * dims->top_k > INT32_MAX) return MOE_EINVAL;
  const RouteWs w = route_ws(dims, T);
  bool size_only;
  if ((rc = check_ws(ws, ws_bytes, w.total, &size_only)) || size_only) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !topk_ids || !topk_w) return MOE_EINVAL;
  clear_hip_error();
  char* base = static_cast<char*>(ws);
  const int H = dims->hidden, E = dims->n_experts, K = dims->top_k;
  if (mfma_router(dims) && T > kGroup) {
    // many tokens: MFMA keys + exact float64 rescoring of the candidates (the
    // fp32 keys and row norms fit in the space of the float64 keys)
    float* approx = reinterpret_cast<float*>(base + w.keys);
    float* wnorm2 = approx + (size_t)T * E;
    launch_dense_router(x, T, layer->w_router, layer->b_router, E, H, approx, wnorm2, stream);
    launch_topk_recheck(x, layer->w_router, layer->b_router, approx, wnorm2, T, H, E, K, topk_ids,
                        topk_w, stream);
    return hip_status();
  }
  double* keys = reinterpret_cast<double*>(base + w.keys);
  launch_router_keys(dims->act, x, layer->w_router, layer->b_router, keys, T, H, E, stream);
  launch_topk(keys, T, E, K, topk_ids, topk_w, stream);
  return hip_status();
}

// ---------------------------------------------------------------------------
// Decode: groups of up to 16 tokens, four launches per group.
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

// The decode launch sequence on a checked workspace `base` of the decode
// layout (arguments already validated).
int decode_launches(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
                    void* y, int32_t y_dt, int32_t* topk_ids, float* topk_w, char* base,
                    const DecodeWs& w, hipStream_t stream);

int check_decode_args(const moe_dims* dims, const moe_layer* layer, int32_t T, int32_t y_dt) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_layer(dims, layer))) return rc;
  if (T < 0 || (int64_t)T * dims->top_k > INT32_MAX) return MOE_EINVAL;
  if (y_dt != MOE_F32 && y_dt != dims->act) return MOE_EINVAL;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_decode(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
                       void* y, int32_t y_dt, int32_t* topk_ids, float* topk_w, void* ws,
                       size_t* ws_bytes, hipStream_t stream) {
  int rc = check_decode_args(dims, layer, T, y_dt);
  if (rc) return rc;
  const DecodeWs w = decode_ws(dims);
  bool size_only;
  if ((rc = check_ws(ws, ws_bytes, w.total, &size_only)) || size_only) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16)) return MOE_EINVAL;
  return decode_launches(dims, layer, x, T, y, y_dt, topk_ids, topk_w, static_cast<char*>(ws), w,
                         stream);
}

int moe_forward_decode_noalloc(const moe_dims* dims, const moe_layer* layer, const void* x,
                               int32_t T, void* y, int32_t y_dt, int32_t* topk_ids,
                               float* topk_w, hipStream_t stream) {
  int rc = check_decode_args(dims, layer, T, y_dt);
  if (rc) return rc;
  const DecodeWs w = decode_ws(dims);
  static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (w.total > kScratchBytes) return MOE_ENOSPC;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16)) return MOE_EINVAL;
  void* scratch = nullptr;
  if ((rc = scratch_for_current_device(&scratch))) return rc;
  return decode_launches(dims, layer, x, T, y, y_dt, topk_ids, topk_w,
                         static_cast<char*>(scratch), w, stream);
}

}  // extern "C"

namespace {

int decode_launches(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
                    void* y, int32_t y_dt, int32_t* topk_ids, float* topk_w, char* base,
                    const DecodeWs& w, hipStream_t stream) {
  clear_hip_error();
  const int H = dims->hidden, K = dims->top_k, E = dims->n_experts;
  const Tables tb = make_tables(dims, layer);
  const size_t xb = act_bytes(dims->act), yb = y_dt == MOE_BF16 ? 2 : 4;
  // the work items carry both code widths of a tier: gate/up | down << 8
  const int32_t wbits[3] = {tb.bits[0] | tb.bits_dn[0] << 8, tb.bits[1] | tb.bits_dn[1] << 8,
                            tb.bits[2] | tb.bits_dn[2] << 8};
  for (int t0 = 0; t0 < T; t0 += kGroup) {
    const int nt = std::min(kGroup, T - t0);
    const char* xg = static_cast<const char*>(x) + (size_t)t0 * H * xb;
    char* yg = static_cast<char*>(y) + (size_t)t0 * H * yb;
    double* keys = reinterpret_cast<double*>(base + w.keys);
    int32_t* ids = topk_ids ? topk_ids + (size_t)t0 * K : reinterpret_cast<int32_t*>(base + w.ids);
    float* wts = topk_w ? topk_w + (size_t)t0 * K : reinterpret_cast<float*>(base + w.w);
    Item* items = reinterpret_cast<Item*>(base + w.items);
    int32_t* n_items = reinterpret_cast<int32_t*>(base + w.n_items);
    void* h = base + w.h;
    launch_router_keys(dims->act, xg, layer->w_router, layer->b_router, keys, nt, H, E, stream);
    if (nt == 1 && E <= 512) {
      // one token: the top-K is folded into the gate/up kernel
      launch_decode1_gateup(dims->act, keys, E, K, layer->tier_map, layer->n_slots,
                            wbits, dims->has_shared, xg, tb, h, H, dims->inter, ids,
                            wts, items, n_items, stream);
    } else {
      launch_topk_items(keys, nt, E, K, layer->tier_map, layer->n_slots, wbits,
                        dims->has_shared, ids, wts, items, n_items, stream);
      launch_decode_gateup(dims->act, items, n_items, nt * K + dims->has_shared, xg, nt, tb, h,
                           H, dims->inter, stream);
    }
    launch_decode_down(dims->act, y_dt, items, n_items, nt * K + dims->has_shared, h,
                       nt * (K + dims->has_shared), nt, tb, yg, H, dims->inter, stream);
  }
  return hip_status();
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Prefill: route, counting sort, grouped GEMMs, weighted scatter-combine.
// ---------------------------------------------------------------------------

int moe_forward_prefill(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
                        void* y, int32_t y_dt, int32_t* topk_ids, float* topk_w,
                        int32_t* expert_offsets, int32_t* sorted_routes, void* ws,
                        size_t* ws_bytes, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_layer(dims, layer))) return rc;
  if (dims->n_experts > 4096) return MOE_EUNSUPPORTED;
  if (T < 0 || (int64_t)T * dims->top_k > INT32_MAX) return MOE_EINVAL;
  // the routed GEMMs gather token rows (x, and h per route) with 32-bit
  // element offsets
  if ((int64_t)T * dims->hidden > INT32_MAX ||
      (int64_t)T * dims->top_k * dims->inter > INT32_MAX)
    return MOE_EUNSUPPORTED;
  if (y_dt != MOE_F32 && y_dt != dims->act) return MOE_EINVAL;
  const PrefillWs w = prefill_ws(dims, T);
  bool size_only;
  if ((rc = check_ws(ws, ws_bytes, w.total, &size_only)) || size_only) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16)) return MOE_EINVAL;
  clear_hip_error();
  char* base = static_cast<char*>(ws);
  const int H = dims->hidden, I = dims->inter, K = dims->top_k, E = dims->n_experts;
  const Tables tb = make_tables(dims, layer);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(base + w.ids);
  float* wts = topk_w ? topk_w : reinterpret_cast<float*>(base + w.w);
  int32_t* offsets = expert_offsets ? expert_offsets : reinterpret_cast<int32_t*>(base + w.offsets);
  int32_t* sorted = sorted_routes ? sorted_routes : reinterpret_cast<int32_t*>(base + w.sorted);
  int32_t* route_pos = reinterpret_cast<int32_t*>(base + w.route_pos);
  void* h = base + w.h;
  void* h_s = base + w.h_s;
  float* route_rows = reinterpret_cast<float*>(base + w.route_rows);
  float* shared_rows = dims->has_shared ? reinterpret_cast<float*>(base + w.shared_rows) : nullptr;

  // bf16 with the MFMA router: the shared expert's gate/up rides in the
  // router's launch (same token rows)
  const bool shared_gu_done = mfma_router(dims) && dims->has_shared;
  if (mfma_router(dims)) {
    float* approx = reinterpret_cast<float*>(base + w.approx);
    float* wnorm2 = reinterpret_cast<float*>(base + w.wnorm2);
    if (shared_gu_done)
      launch_dense_router_shared_gateup(x, T, layer->w_router, layer->b_router, E, H, approx,
                                        wnorm2, tb.dense[MOE_GATE], tb.dense[MOE_UP], h_s, I,
                                        stream);
    else
      launch_dense_router(x, T, layer->w_router, layer->b_router, E, H, approx, wnorm2, stream);
    launch_topk_recheck(x, layer->w_router, layer->b_router, approx, wnorm2, T, H, E, K, ids, wts,
                        stream);
  } else {
    double* keys = reinterpret_cast<double*>(base + w.keys);
    launch_router_keys(dims->act, x, layer->w_router, layer->b_router, keys, T, H, E, stream);
    launch_topk(keys, T, E, K, ids, wts, stream);
  }
  int2* tiles = reinterpret_cast<int2*>(base + w.tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(base + w.n_tiles);
  launch_sort_routes(ids, T, K, E, reinterpret_cast<uint64_t*>(base + w.chunk_mask),
                     reinterpret_cast<int32_t*>(base + w.chunk_base), offsets, sorted, route_pos,
                     prefill_tile_rows(dims->act), tiles, n_tiles, stream);
  launch_prefill_gateup(dims->act, offsets, sorted, tiles, n_tiles, w.max_tiles, layer->tier_map,
                        E, K, x, tb, h, H, I, stream);
  // bf16 with a shared expert: its down projection runs after the routed one
  // and adds the route rows in its epilogue (no shared rows in HBM)
  const bool fused_combine = dims->has_shared && dims->act == MOE_BF16;
  if (dims->has_shared) {
    if (!shared_gu_done) launch_prefill_shared_gateup(dims->act, x, T, tb, h_s, H, I, stream);
    if (!fused_combine) launch_prefill_shared_down(dims->act, h_s, T, tb, shared_rows, H, I, stream);
  }
  launch_prefill_down(dims->act, offsets, sorted, tiles, n_tiles, w.max_tiles, layer->tier_map, E,
                      K, h, tb, route_rows, H, I, stream);
  if (fused_combine)
    launch_dense_shared_down_combine(h_s, T, tb.dense[MOE_DOWN], route_rows, route_pos, wts, K, H,
                                     I, y, y_dt, stream);
  else
    launch_combine(y_dt, shared_rows, route_rows, route_pos, wts, T, K, H, y, stream);
  return hip_status();
}

}  // extern "C"
