// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe.h"

namespace moe {

// Tokens handled together by the decode kernels: the M side of one 16x16
// MFMA tile.
constexpr int kGroup = 16;
// Tier index used for the shared expert (dense weights in the act dtype).
constexpr int kDenseTier = 3;

// Code formats of a tier table: the affine widths 2, 3, 4 and MXFP4.
constexpr int kMx4 = MOE_MXFP4;
__host__ __device__ constexpr bool valid_format(int f) {
  return f == 2 || f == 3 || f == 4 || f == kMx4;
}
// Bytes of one block's code field and of its scale entry in the dm table.
__host__ __device__ constexpr int field_bytes(int f) { return f == kMx4 ? 16 : 4 * f; }
__host__ __device__ constexpr int scale_bytes(int f) { return f == kMx4 ? 1 : 4; }

// One expert of a decode group together with the tokens that route to it.
struct Item {
  int32_t expert;          // expert id, -1 for the shared expert
  int32_t tier;            // 0..2 quantised tier, kDenseTier, or -1 (skip)
  int32_t slot;            // slot inside the tier table
  int32_t bits;            // code formats: gate/up | down << 8 (0 for dense)
  int32_t route[kGroup];   // row of h for token t of the group, or -1
  float gw[kGroup];        // mixing weight of token t (0 when not routed)
};

// Kernel-side view of the expert tables of one layer.
struct Tables {
  const uint8_t* codes[3][3];
  const uint32_t* dm[3][3];  // (d, m) words; uint8 E8M0 bytes for MXFP4
  int32_t bits[3];         // gate / up code format of each tier
  int32_t bits_dn[3];      // down code format of each tier
  int32_t n_slots[3];
  const void* dense[3];    // shared expert gate / up / down (act dtype)
};

// Bytes of the library-owned device scratch of moe_forward_decode_noalloc
// (one array per GPU, held until the process ends).
constexpr size_t kScratchBytes = (size_t)4 << 20;

// Device address of that scratch on the current device (scratch.hip): the
// symbol's address is looked up once per device and kept.  MOE_OK or
// MOE_EHIP / MOE_EUNSUPPORTED.
int scratch_for_current_device(void** out);

// ---- launch trace (moe_set_trace); defined in moe_abi.cpp ----
// Returns the start/stop events of the next trace slot for a kernel launched
// on `s`, or leaves them null (no trace installed, slots used up, or `s` is
// being captured into a graph).
void trace_slot(int kernel_id, hipStream_t s, hipEvent_t* start, hipEvent_t* stop);

// Launches a kernel; when traced, the events are attached to the dispatch
// itself (hipExtLaunchKernel), so they time the kernel's execution only.
#define MOE_LAUNCH(KID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                           \
  do {                                                                                     \
    hipEvent_t moe_e0_ = nullptr, moe_e1_ = nullptr;                                       \
    ::moe::trace_slot((KID), (STREAM), &moe_e0_, &moe_e1_);                                \
    if (moe_e0_)                                                                           \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, moe_e0_, moe_e1_, 0,       \
                            __VA_ARGS__);                                                  \
    else                                                                                   \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                 \
  } while (0)

// ---- launchers (defined in the .hip files; all enqueue on `s`) ----

// keys[t][e] = x[t] . w[e] + b[e] in float64, for t < T (any T).
void launch_router_keys(int act, const void* x, const void* w, const float* b, double* keys,
                        int T, int H, int E, hipStream_t s);

// Top-K + softmax weights for T tokens (any T): ids[t][k], w[t][k].
void launch_topk(const double* keys, int T, int E, int K, int32_t* ids, float* w, hipStream_t s);

// Decode group (T <= kGroup): top-K, weights, then the union of experts as
// work items (ascending expert id, then the shared expert).  tier_bits[t] =
// gate/up width | down width << 8, copied into the items' bits.
void launch_topk_items(const double* keys, int T, int E, int K, const int32_t* tier_map,
                       const int32_t n_slots[3], const int32_t tier_bits[3], int has_shared,
                       int32_t* ids, float* w, Item* items, int32_t* n_items, hipStream_t s);

// Decode gate/up over the work items: h[route][I] = act(silu(gate) * up).
void launch_decode_gateup(int act, const Item* items, const int32_t* n_items, int max_items,
                          const void* x, int T, const Tables& tb, void* h, int H, int I,
                          hipStream_t s);

// Batch-1 decode (one token): top-K + weights + work items fused with the
// gate/up of each item (E <= 512, K <= 64).  Items are in rank order;
// tier_bits as for launch_topk_items.
void launch_decode1_gateup(int act, const double* keys, int E, int K, const int32_t* tier_map,
                           const int32_t n_slots[3], const int32_t tier_bits[3], int has_shared,
                           const void* x, const Tables& tb, void* h, int H, int I, int32_t* ids,
                           float* w, Item* items, int32_t* n_items, hipStream_t s);

// Decode down + combine: y[t][H] = sum over items of gw * (W_d h).
// h holds rows [0, h_rows) of the group (staged in LDS when they fit).
void launch_decode_down(int act, int y_dt, const Item* items, const int32_t* n_items,
                        int max_items, const void* h, int h_rows, int T, const Tables& tb,
                        void* y, int H, int I, hipStream_t s);

// ---- prefill ----

// Stable counting sort of the routes by expert.
//   chunk_mask: [n_chunks][E] uint64, chunk_base: [n_chunks][E] int32.
// Also lists the grouped-GEMM tiles: bucket e splits into ceil(n_e /
// tile_rows) tiles (e, first row inside the bucket), *n_tiles of them
// (at most E + T * K / tile_rows).
void launch_sort_routes(const int32_t* ids, int T, int K, int E, uint64_t* chunk_mask,
                        int32_t* chunk_base, int32_t* offsets, int32_t* sorted_routes,
                        int32_t* route_pos, int tile_rows, int2* tiles, int32_t* n_tiles,
                        hipStream_t s);

// Routed gate/up grouped GEMM: for every expert bucket, h[pos][I] for the
// sorted positions pos of that bucket.
void launch_prefill_gateup(int act, const int32_t* offsets, const int32_t* sorted_routes,
                           const int2* tiles, const int32_t* n_tiles, int max_tiles,
                           const int32_t* tier_map, int E, int K, const void* x, const Tables& tb,
                           void* h, int H, int I, hipStream_t s);

// Shared expert gate/up for all T tokens: h_s[t][I].
void launch_prefill_shared_gateup(int act, const void* x, int T, const Tables& tb, void* h_s,
                                  int H, int I, hipStream_t s);

// Shared expert down: rows[t][H] = W_sd h_s[t] in fp32 (plain stores).
void launch_prefill_shared_down(int act, const void* h_s, int T, const Tables& tb, float* rows,
                                int H, int I, hipStream_t s);

// Routed down: route_rows[pos][H] = W_d h[pos] in fp32 for every sorted
// position pos (plain stores; the gate weight is applied by the combine).
void launch_prefill_down(int act, const int32_t* offsets, const int32_t* sorted_routes,
                         const int2* tiles, const int32_t* n_tiles, int max_tiles,
                         const int32_t* tier_map, int E, int K, const void* h, const Tables& tb,
                         float* route_rows, int H, int I, hipStream_t s);

// Token rows per routed GEMM tile for the activation dtype.
int prefill_tile_rows(int act);

// y[t] = shared_rows[t] (if any) + sum_k topk_w[t][k] * route_rows[route_pos[t][k]],
// summed in k order in fp32, stored in y_dt.
void launch_combine(int y_dt, const float* shared_rows, const float* route_rows,
                    const int32_t* route_pos, const float* topk_w, int T, int K, int H, void* y,
                    hipStream_t s);

// Exact top-K from approximate keys (bf16 activations): candidates within the
// rounding bound of the K-th approximate key are rescored in float64 with the
// arithmetic of launch_router_keys, then ranked (key desc, id asc).
void launch_topk_recheck(const void* x, const void* w, const float* bias, const float* approx,
                         const float* wnorm2, int T, int H, int E, int K, int32_t* ids, float* wts,
                         hipStream_t s);

// ---- dense bf16 GEMMs of the prefill (kernels_dense.hip) ----

// The dense kernels take any contraction length that is a multiple of 64
// (every H and I the entry points accept, which are multiples of 128).
// Approximate router keys with bf16 MFMA (bf16 activations only):
// keys_approx[t][e] = fp32 x[t] . w[e] + b[e]; wnorm2[e] = |w[e]|^2 (fp32).
void launch_dense_router(const void* x, int T, const void* w_router, const float* bias, int E,
                         int H, float* keys_approx, float* wnorm2, hipStream_t s);
// Both of the above in one launch (they multiply the same token rows x).
void launch_dense_router_shared_gateup(const void* x, int T, const void* w_router,
                                      const float* bias, int E, int H, float* keys_approx,
                                      float* wnorm2, const void* w_gate, const void* w_up,
                                      void* h_s, int I, hipStream_t s);
// h_s[t][i] = bf16(silu(x[t] . w_gate[i]) * (x[t] . w_up[i])).
void launch_dense_shared_gateup(const void* x, int T, const void* w_gate, const void* w_up,
                                void* h_s, int H, int I, hipStream_t s);
// rows[t][n] = fp32 h_s[t] . w_down[n].
void launch_dense_shared_down(const void* h_s, int T, const void* w_down, float* rows, int H,
                              int I, hipStream_t s);
// The shared expert's down projection with the combine in its epilogue:
// y[t] = shared row + the token's K weighted route rows, in route order.
void launch_dense_shared_down_combine(const void* h_s, int T, const void* w_down,
                                      const float* route_rows, const int32_t* route_pos,
                                      const float* topk_w, int K, int H, int I, void* y, int y_dt,
                                      hipStream_t s);

// ---- host packer (pack.cpp; no HIP calls) ----

// Quantise one block of 32 floats; returns MOE_OK or MOE_EINVAL.
int quantise_block(const float* x, int bits, uint16_t* d, uint16_t* m, uint8_t* q);
// Quantise one block of 32 floats to MXFP4: E8M0 byte and E2M1 codes.
int quantise_block_mx(const float* x, uint8_t* e, uint8_t* q);
// Pack 32 codes (each <= 2^bits - 1, or E2M1 codes for kMx4) into a
// field_bytes(bits)-byte code field.
void encode_codes(const uint8_t* q, int bits, uint8_t* field);
// Index of block (slot, row, block column) in a tier table of R x C matrices.
inline size_t tile_block_index(size_t slot, int r, int j, int R, int C) {
  size_t tile = (slot * (size_t)(R / 16) + (size_t)(r / 16)) * (size_t)(C / 128) + (size_t)(j / 4);
  return tile * 64 + (size_t)(16 * (j % 4) + (r % 16));
}

}  // namespace moe
