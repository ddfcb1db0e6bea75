// Prefill path (A7, A8): grouped GEMMs over the expert buckets produced by
// the counting sort, plus the shared expert's dense GEMMs.
//
// A workgroup owns 128 weight rows (4 waves x 2 row-groups of 16) of one
// expert and walks that expert's bucket of routes in passes of up to ROWS
// token rows.  For each 128-wide slice of the contraction axis the gathered
// token rows are staged once in LDS (rows padded to 272 bytes so the
// fragment reads are bank-conflict free) and shared by the 4 waves; every
// lane dequantises its own weight blocks straight into MFMA operand
// registers and reuses them across all token tiles of the pass, so each
// weight is dequantised once per pass.  The down projection scatters
// topk_w-weighted rows into the fp32 accumulator with atomics on top of the
// shared expert's output.  The pages' prefill path is the weak spot of the
// consumer-GPU build (P1, "speed vs context, and the 256k profile").
#include "device_common.hpp"

namespace moe {

namespace {

enum Mode { kRoutedGateUp = 0, kSharedGateUp = 1, kRoutedDown = 2, kSharedDown = 3 };

struct PArgs {
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* tier_map;
  const float* topk_w;
  int E, K, T, H, I;
  const void* src;   // x for gate/up, h for down
  void* dst;         // h for gate/up, y_acc for down
  Tables tb;
};

template <typename A> struct PTraits;
template <> struct PTraits<bf16_t> {
  static constexpr int ROWS = 128;        // token rows per pass
  static constexpr int ROW_U32 = 64 + 4;  // 128 bf16 + pad
};
template <> struct PTraits<float> {
  static constexpr int ROWS = 64;
  static constexpr int ROW_U32 = 128 + 4;
};

// B fragment of one lane for a super-step: bf16 -> 16 packed words; f32 -> 32 floats.
template <typename A> struct BFrag;
template <> struct BFrag<bf16_t> { uint32_t v[16]; };
template <> struct BFrag<float> { float v[32]; };

template <typename A, int BITS>
__device__ __forceinline__ void load_b(BFrag<A>& b, const Tables& tb, int tier, int mat, int slot,
                                       int R, int C, int rg, int c, int lane, const void* dense) {
  const int lm = lane & 15, lg = lane >> 4;
  if constexpr (BITS == 0) {
    const A* p = reinterpret_cast<const A*>(dense) + (size_t)(rg * 16 + lm) * C + 128 * c + 32 * lg;
    if constexpr (sizeof(A) == 2) {
      const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 t = q[i];
        b.v[4 * i] = t.x; b.v[4 * i + 1] = t.y; b.v[4 * i + 2] = t.z; b.v[4 * i + 3] = t.w;
      }
    } else {
      const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float4 t = q[i];
        b.v[4 * i] = t.x; b.v[4 * i + 1] = t.y; b.v[4 * i + 2] = t.z; b.v[4 * i + 3] = t.w;
      }
    }
  } else {
    const size_t idx = (((size_t)slot * (R / 16) + rg) * (C / 128) + c) * 64 + lane;
    uint32_t w[4];
    load_field<BITS>(tb.codes[tier][mat] + idx * (4 * BITS), w);
    const uint32_t dm = tb.dm[tier][mat][idx];
    if constexpr (sizeof(A) == 2) {
      SinkBf16 sink;
      dequant_block<BITS>(w, dm, sink);
#pragma unroll
      for (int i = 0; i < 16; i++) b.v[i] = sink.v[i];
    } else {
      SinkF32 sink;
      dequant_block<BITS>(w, dm, sink);
#pragma unroll
      for (int i = 0; i < 32; i++) b.v[i] = sink.v[i];
    }
  }
}

// One workgroup's work: weight rows [nt*128, nt*128 + 128) of one expert
// (or of the shared expert) against `nrows` token rows starting at `row0`.
template <typename A, int BITS, int MODE>
__device__ __forceinline__ void prefill_body(const PArgs& a, int row0, int nrows, int tier, int slot,
                                             int nt, uint32_t* __restrict__ sA) {
  constexpr bool GATEUP = MODE == kRoutedGateUp || MODE == kSharedGateUp;
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int ROWS = PTraits<A>::ROWS, RU = PTraits<A>::ROW_U32;
  constexpr int MT = ROWS / 16;
  const int Kc = GATEUP ? a.H : a.I;        // contraction length
  const int Nr = GATEUP ? a.I : a.H;        // weight rows (output features)
  const int nbg = Kc / 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const A* src = reinterpret_cast<const A*>(a.src);
  const int n0 = nt * 128 + wave * 32;      // first weight row of this wave

  for (int pass0 = 0; pass0 < nrows; pass0 += ROWS) {
    const int rows_here = min(ROWS, nrows - pass0);
    const int ntiles = (rows_here + 15) / 16;
    f32x4_t acc[2][NMAT][MT];
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int m = 0; m < NMAT; m++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[r][m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nbg; c++) {
      __syncthreads();
      // stage the pass's token rows, columns [128c, 128c + 128)
      {
        constexpr int PARTS = 256 / ROWS;           // threads per row
        constexpr int U32_PER = 128 * sizeof(A) / 4 / PARTS;
        const int row = threadIdx.x / PARTS, part = threadIdx.x % PARTS;
        uint32_t* dst = sA + row * RU + part * U32_PER;
        if (row < rows_here) {
          int srow;
          if constexpr (MODE == kRoutedGateUp) srow = a.sorted[row0 + pass0 + row] / a.K;
          else srow = row0 + pass0 + row;           // sorted h rows, or tokens
          const uint4* q = reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint32_t*>(src + (size_t)srow * Kc + 128 * c) + part * U32_PER);
#pragma unroll
          for (int i = 0; i < U32_PER / 4; i++) {
            const uint4 t = q[i];
            dst[4 * i] = t.x; dst[4 * i + 1] = t.y; dst[4 * i + 2] = t.z; dst[4 * i + 3] = t.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < U32_PER; i++) dst[i] = 0u;
        }
      }
      __syncthreads();
      // this wave's weight fragments: 2 row-groups x NMAT matrices
      BFrag<A> bf[2][NMAT];
#pragma unroll
      for (int r = 0; r < 2; r++) {
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
          const int mat = GATEUP ? m : MOE_DOWN;
          const int rg = (n0 + 16 * r) / 16;
          const void* dense = a.tb.dense[mat];
          load_b<A, BITS>(bf[r][m], a.tb, tier, mat, slot, Nr, Kc, rg, c, lane, dense);
        }
      }
#pragma unroll
      for (int t = 0; t < MT; t++) {
        if (t >= ntiles) break;
        const uint32_t* arow = sA + (16 * t + lm) * RU;
        if constexpr (sizeof(A) == 2) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * lg + 4 * i);
#pragma unroll
            for (int r = 0; r < 2; r++)
#pragma unroll
              for (int m = 0; m < NMAT; m++)
                acc[r][m][t] = mfma_bf16(av.x, av.y, av.z, av.w, bf[r][m].v[4 * i],
                                         bf[r][m].v[4 * i + 1], bf[r][m].v[4 * i + 2],
                                         bf[r][m].v[4 * i + 3], acc[r][m][t]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < 32; s++) {
            const float av = __uint_as_float(arow[32 * lg + s]);
#pragma unroll
            for (int r = 0; r < 2; r++)
#pragma unroll
              for (int m = 0; m < NMAT; m++) acc[r][m][t] = mfma_f32(av, bf[r][m].v[s], acc[r][m][t]);
          }
        }
      }
    }

    // epilogue
#pragma unroll
    for (int t = 0; t < MT; t++) {
      if (t >= ntiles) break;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int p = 16 * t + 4 * lg + i;      // row inside the pass
        if (p >= rows_here) continue;
        const int gp = row0 + pass0 + p;        // sorted position or token
#pragma unroll
        for (int r = 0; r < 2; r++) {
          const int n = n0 + 16 * r + lm;
          if constexpr (GATEUP) {
            const float v = silu_f32(acc[r][0][t][i]) * acc[r][1][t][i];
            A* out = reinterpret_cast<A*>(a.dst) + (size_t)gp * a.I + n;
            if constexpr (sizeof(A) == 2) *out = to_bf16(v); else *out = v;
          } else if constexpr (MODE == kRoutedDown) {
            const int route = a.sorted[gp];
            const int tok = route / a.K;
            atomicAdd(reinterpret_cast<float*>(a.dst) + (size_t)tok * a.H + n,
                      a.topk_w[route] * acc[r][0][t][i]);
          } else {
            reinterpret_cast<float*>(a.dst)[(size_t)gp * a.H + n] = acc[r][0][t][i];
          }
        }
      }
    }
  }
}

template <typename A, int MODE>
__global__ __launch_bounds__(256) void k_prefill(PArgs a) {
  constexpr bool GATEUP = MODE == kRoutedGateUp || MODE == kSharedGateUp;
  constexpr bool ROUTED = MODE == kRoutedGateUp || MODE == kRoutedDown;
  constexpr int ROWS = PTraits<A>::ROWS, RU = PTraits<A>::ROW_U32;
  __shared__ uint32_t sA[ROWS * RU];
  const int Nr = GATEUP ? a.I : a.H;
  const int NT = Nr / 128;
  // XCD-aware mapping: the workgroups that share one expert's (or one token
  // chunk's) rows land on the same XCD, whose L2 then serves the re-reads.
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  const int grp = (j / NT) * 8 + xcd, nt = j % NT;
  if constexpr (ROUTED) {
    if (grp >= a.E) return;
    const int row0 = a.offsets[grp];
    const int nrows = a.offsets[grp + 1] - row0;
    if (nrows == 0) return;
    const int tm = a.tier_map[grp];
    const int tier = tm >> 16, slot = tm & 0xFFFF;
    if (tier < 0 || tier > 2 || slot >= a.tb.n_slots[tier]) return;
    // the tier's code width is uniform over the workgroup
    switch (a.tb.bits[tier]) {
      case 4: prefill_body<A, 4, MODE>(a, row0, nrows, tier, slot, nt, sA); break;
      case 3: prefill_body<A, 3, MODE>(a, row0, nrows, tier, slot, nt, sA); break;
      default: prefill_body<A, 2, MODE>(a, row0, nrows, tier, slot, nt, sA); break;
    }
  } else {
    const int row0 = grp * ROWS;
    if (row0 >= a.T) return;
    prefill_body<A, 0, MODE>(a, row0, min(ROWS, a.T - row0), 0, 0, nt, sA);
  }
}

template <typename A, int MODE>
void launch_mode(const PArgs& a, int n_groups, hipStream_t s) {
  constexpr bool GATEUP = MODE == kRoutedGateUp || MODE == kSharedGateUp;
  const int Nr = GATEUP ? a.I : a.H;
  const int NT = Nr / 128;
  dim3 grid(((n_groups + 7) / 8) * 8 * NT);
  constexpr int kid = MODE == kRoutedGateUp   ? MOE_K_PREFILL_GATEUP
                      : MODE == kSharedGateUp ? MOE_K_PREFILL_SHARED_GATEUP
                      : MODE == kSharedDown   ? MOE_K_PREFILL_SHARED_DOWN
                                              : MOE_K_PREFILL_DOWN;
  MOE_LAUNCH(kid, (k_prefill<A, MODE>), grid, dim3(256), 0, s, a);
}

PArgs make_args(const int32_t* offsets, const int32_t* sorted, const int32_t* tier_map,
                const float* topk_w, int E, int K, int T, int H, int I, const void* src, void* dst,
                const Tables& tb) {
  PArgs a;
  a.offsets = offsets;
  a.sorted = sorted;
  a.tier_map = tier_map;
  a.topk_w = topk_w;
  a.E = E;
  a.K = K;
  a.T = T;
  a.H = H;
  a.I = I;
  a.src = src;
  a.dst = dst;
  a.tb = tb;
  return a;
}

__global__ void k_cast_out(const float* __restrict__ in, bf16_t* __restrict__ out, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = to_bf16(in[i]);
}

__global__ void k_zero(float* __restrict__ p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

}  // namespace

void launch_prefill_gateup(int act, const int32_t* offsets, const int32_t* sorted_routes,
                           const int32_t* tier_map, int E, int K, const void* x, const Tables& tb,
                           void* h, int H, int I, hipStream_t s) {
  const PArgs a = make_args(offsets, sorted_routes, tier_map, nullptr, E, K, 0, H, I, x, h, tb);
  if (act == MOE_BF16) launch_mode<bf16_t, kRoutedGateUp>(a, E, s);
  else launch_mode<float, kRoutedGateUp>(a, E, s);
}

void launch_prefill_shared_gateup(int act, const void* x, int T, const Tables& tb, void* h_s,
                                  int H, int I, hipStream_t s) {
  const PArgs a = make_args(nullptr, nullptr, nullptr, nullptr, 0, 0, T, H, I, x, h_s, tb);
  if (act == MOE_BF16) launch_mode<bf16_t, kSharedGateUp>(a, (T + 127) / 128, s);
  else launch_mode<float, kSharedGateUp>(a, (T + 63) / 64, s);
}

void launch_prefill_shared_down(int act, const void* h_s, int T, const Tables& tb, float* y_acc,
                                int H, int I, hipStream_t s) {
  const PArgs a = make_args(nullptr, nullptr, nullptr, nullptr, 0, 0, T, H, I, h_s, y_acc, tb);
  if (act == MOE_BF16) launch_mode<bf16_t, kSharedDown>(a, (T + 127) / 128, s);
  else launch_mode<float, kSharedDown>(a, (T + 63) / 64, s);
}

void launch_prefill_down(int act, const int32_t* offsets, const int32_t* sorted_routes,
                         const int32_t* tier_map, const float* topk_w, int E, int K, const void* h,
                         const Tables& tb, float* y_acc, int H, int I, hipStream_t s) {
  const PArgs a = make_args(offsets, sorted_routes, tier_map, topk_w, E, K, 0, H, I, h, y_acc, tb);
  if (act == MOE_BF16) launch_mode<bf16_t, kRoutedDown>(a, E, s);
  else launch_mode<float, kRoutedDown>(a, E, s);
}

void launch_cast_out(const float* y_acc, void* y, size_t n, hipStream_t s) {
  MOE_LAUNCH(MOE_K_CAST, k_cast_out, dim3(1024), dim3(256), 0, s, y_acc, (bf16_t*)y, n);
}

void launch_zero(float* p, size_t n, hipStream_t s) {
  MOE_LAUNCH(MOE_K_ZERO, k_zero, dim3(1024), dim3(256), 0, s, p, n);
}

}  // namespace moe
