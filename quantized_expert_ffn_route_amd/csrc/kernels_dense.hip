// Dense bf16 GEMMs of the prefill: the MFMA router pass (A1), the shared
// expert's gate/up with the SwiGLU activation and its down projection (A7,
// A8 for the always-on expert).  out[m][n] = sum_k a[m][k] * b[n][k] with
// both operands row-major along the contraction axis: token rows against
// weight rows.
//
// A workgroup of four waves owns a tile of (32 * MTW) token rows and 128
// weight rows; each wave owns a (16 * MTW) x 64 sub-tile, i.e. MTW x 4 MFMA
// 16x16x32 accumulators, fed by MTW + 4 LDS fragment reads per k-step.  The
// contraction axis goes in chunks of 64 (two MFMA k-steps), so each row read
// is one whole 128-byte line.  Both operands
// move from global memory straight into LDS (one 16-byte direct-to-LDS load
// per lane and piece) through a three-stage ring, two chunks ahead of the
// multiply.  A row of a stage is 8 pieces of 16 bytes; piece p of row r sits
// in slot p ^ ((r >> 1) & 7), so the 16 rows of a fragment read hit 16
// distinct bank groups.  The loads are issued from inline assembly and the
// loop waits for exactly the loads of the chunk it is about to read (vmcnt),
// then hands the stage over with a barrier: the only global loads inside the
// loop are these, so no other wait is needed.
#include "device_common.hpp"

namespace moe {

namespace {

constexpr int kDWaves = 4;
constexpr int kDThreads = 64 * kDWaves;
constexpr int kDKC = 64;                // contraction elements per chunk (two MFMA k-steps)
constexpr int kDPPR = kDKC / 8;         // 16-byte pieces per row of a stage
constexpr int kDRowsB = 128;            // weight rows per workgroup tile
constexpr int kDStages = 3;

// kDRouterGateUp: one launch over the router's column tiles followed by the
// shared expert's gate/up column tiles -- both multiply the same token rows.
// kDDownCombine: the shared expert's down projection whose epilogue adds the
// token's K weighted route rows (the combine) and stores y.
enum DenseMode { kDRouter = 0, kDGateUp = 1, kDDown = 2, kDRouterGateUp = 3, kDDownCombine = 4 };

struct DArgs {
  const bf16_t* a;    // token rows [M][K]
  const bf16_t* b0;   // weight rows [N][K] (router, down projection, gate)
  const bf16_t* b1;   // up rows [N][K] (gate/up)
  int M, N, K;        // N: router experts, hidden size (down) or intermediate size (gate/up)
  const float* bias;  // router bias or null
  float* outf;        // router keys / shared rows, [M][N] fp32
  bf16_t* outh;       // gate/up activations, [M][N] bf16
  float* wnorm2;      // router: squared row norms [N]
  // kDRouterGateUp: the gate/up part (b0/b1/outh above belong to the router
  // then, as b0 / bias / outf / wnorm2 do)
  const bf16_t* g_gate;
  const bf16_t* g_up;
  bf16_t* g_out;
  int g_N;            // intermediate size
  // kDDownCombine: route rows [T*K][N] fp32, the row of route (t, k) and its
  // mixing weight, and the output y [M][N] (bf16 when y_bf16)
  const float* route_rows;
  const int32_t* route_pos;
  const float* topk_w;
  int topK;
  void* y;
  int y_bf16;
};

template <int N>
__device__ __forceinline__ void dwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Waits until at most `ahead` chunks of DPC loads each are still in flight.
template <int DPC>
__device__ __forceinline__ void dwait_chunks(int ahead) {
  static_assert(DPC * 3 < 64, "vmcnt");
  switch (ahead) {
    case 0: dwait_vmcnt<0>(); break;
    case 1: dwait_vmcnt<DPC>(); break;
    case 2: dwait_vmcnt<2 * DPC>(); break;
    default: dwait_vmcnt<3 * DPC>(); break;
  }
}

// One 16-byte piece per lane from global memory into LDS: lane i's piece
// lands at lds + 16 i (lds wave-uniform).  No register destination.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(g)
               : "memory", "m0");
}

// LDS hand-over: this wave's LDS operations done, then the workgroup barrier
// (not __syncthreads, which would also drain the loads still in flight).
__device__ __forceinline__ void dlds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int dswz(int r) { return (r >> 1) & 7; }

template <int MODE, int MTW>
__global__ __launch_bounds__(kDThreads) void k_dense(DArgs a) {
  constexpr int MROWS = 32 * MTW;                         // token rows per workgroup
  constexpr int APIECES = MROWS * kDPPR, BPIECES = kDRowsB * kDPPR;
  constexpr int LA = APIECES / kDThreads, LB = BPIECES / kDThreads;
  constexpr int DPC = LA + LB;                            // loads per thread per chunk
  constexpr int STAGE = (APIECES + BPIECES) * 16;         // bytes
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kDStages * STAGE];

  constexpr bool COMB = MODE == kDRouterGateUp;
  // column tiles: router tiles of kDRowsB columns, then (combined mode)
  // gate/up tiles of kDRowsB / 2 columns
  const int NTr = MODE == kDGateUp ? 0 : (a.N + kDRowsB - 1) / kDRowsB;
  const int NTg = MODE == kDGateUp ? (a.N + kDRowsB / 2 - 1) / (kDRowsB / 2)
                                   : (COMB ? (a.g_N + kDRowsB / 2 - 1) / (kDRowsB / 2) : 0);
  const int NT = NTr + NTg;
  // XCD-aware order: workgroups go to the 8 XCDs round-robin, so all column
  // tiles of token tile mt run on XCD mt % 8 and share its L2 copy of the rows
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int mt = (j / NT) * 8 + xcd, nt = j % NT;
  // this workgroup's part: gate/up (gu) or router / down
  const bool gu = MODE == kDGateUp || (COMB && nt >= NTr);
  const int n0 = gu ? (nt - NTr) * (kDRowsB / 2) : nt * kDRowsB;
  const int NN = COMB && gu ? a.g_N : a.N;                  // columns of this part
  const bf16_t* bg = COMB ? a.g_gate : a.b0;
  const bf16_t* bu = COMB ? a.g_up : a.b1;
  bf16_t* outg = COMB ? a.g_out : a.outh;
  const int m0 = mt * MROWS;
  if (m0 >= a.M) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, NC = K / kDKC;

  // this thread's load sources (chunk 0) and LDS slots
  const bf16_t* asrc[LA];
  const bf16_t* bsrc[LB];
#pragma unroll
  for (int j = 0; j < LA; j++) {
    const int q = threadIdx.x + kDThreads * j;            // slot in the A part
    const int r = q / kDPPR, p = (q % kDPPR) ^ dswz(r);
    const int gm = min(m0 + r, a.M - 1);
    asrc[j] = a.a + (size_t)gm * K + 8 * p;
  }
#pragma unroll
  for (int j = 0; j < LB; j++) {
    const int q = threadIdx.x + kDThreads * j;
    const int r = q / kDPPR, p = (q % kDPPR) ^ dswz(r);
    const bf16_t* base;
    int gn;
    if (gu) {
      // rows [64 w, 64 w + 32): gate rows, [64 w + 32, 64 w + 64): up rows
      const int w = r >> 6, rr = r & 63;
      gn = min(n0 + 32 * w + (rr & 31), NN - 1);
      base = rr < 32 ? bg : bu;
    } else {
      gn = min(n0 + r, NN - 1);
      base = a.b0;
    }
    bsrc[j] = base + (size_t)gn * K + 8 * p;
  }
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)s_ring;
  auto issue = [&](int c, int st) {
    const uint32_t sb = ring + (uint32_t)(st * STAGE);
#pragma unroll
    for (int j = 0; j < LA; j++)
      dma16(asrc[j] + kDKC * c, __builtin_amdgcn_readfirstlane(sb + (uint32_t)((kDThreads * j + 64 * wave) * 16)));
#pragma unroll
    for (int j = 0; j < LB; j++)
      dma16(bsrc[j] + kDKC * c,
            __builtin_amdgcn_readfirstlane(sb + (uint32_t)((APIECES + kDThreads * j + 64 * wave) * 16)));
  };

  // fragment slots (bytes inside a stage): k-step s of a chunk reads
  // logical piece 4 s + lg of the lane's row
  constexpr int KS = kDKC / 32;
  uint32_t aoff[KS][MTW], boff[KS][4];
#pragma unroll
  for (int s = 0; s < KS; s++) {
#pragma unroll
    for (int t = 0; t < MTW; t++) {
      const int r = wm * 16 * MTW + 16 * t + lm;
      aoff[s][t] = (uint32_t)((r * kDPPR + ((4 * s + lg) ^ dswz(r))) * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int r = wn * 64 + 16 * u + lm;
      boff[s][u] = (uint32_t)((APIECES + r * kDPPR + ((4 * s + lg) ^ dswz(r))) * 16);
    }
  }

  f32x4_t acc[MTW][4];
#pragma unroll
  for (int t = 0; t < MTW; t++)
#pragma unroll
    for (int u = 0; u < 4; u++) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float wsq = 0.f;   // router: this thread's weight row norm (first token tile, threads < 128)
  const bool norms = (MODE == kDRouter || (COMB && !gu)) && mt == 0 && a.wnorm2 != nullptr &&
                     threadIdx.x < kDRowsB;

  static_assert(kDStages - 2 <= 3, "dwait_chunks covers up to three chunks ahead");
  for (int c = 0; c < kDStages - 1 && c < NC; c++) issue(c, c);
  for (int c = 0; c < NC; c++) {
    // chunks c + 1 .. c + kDStages - 2 may stay in flight
    dwait_chunks<DPC>(min(kDStages - 2, NC - 1 - c));
    dlds_barrier();
    const int st = c % kDStages;
    if (c + kDStages - 1 < NC) issue(c + kDStages - 1, (c + kDStages - 1) % kDStages);
    const uint8_t* sp = s_ring + st * STAGE;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      uint4 bf[4];
#pragma unroll
      for (int u = 0; u < 4; u++) bf[u] = *reinterpret_cast<const uint4*>(sp + boff[ks][u]);
#pragma unroll
      for (int t = 0; t < MTW; t++) {
        const uint4 af = *reinterpret_cast<const uint4*>(sp + aoff[ks][t]);
#pragma unroll
        for (int u = 0; u < 4; u++)
          acc[t][u] = mfma_bf16(af.x, af.y, af.z, af.w, bf[u].x, bf[u].y, bf[u].z, bf[u].w, acc[t][u]);
      }
    }
    if (norms) {
      const uint4* row = reinterpret_cast<const uint4*>(sp + APIECES * 16) + threadIdx.x * kDPPR;
#pragma unroll
      for (int p = 0; p < kDPPR; p++) {
        const uint4 v = row[p];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float lo = bf16_lo(w4[i]), hi = bf16_hi(w4[i]);
          wsq = __builtin_fmaf(lo, lo, wsq);
          wsq = __builtin_fmaf(hi, hi, wsq);
        }
      }
    }
  }
  if (norms && n0 + (int)threadIdx.x < NN) a.wnorm2[n0 + threadIdx.x] = wsq;

  if constexpr (MODE == kDDownCombine) {
    // the tile's shared rows go to LDS (the ring is free once every wave has
    // left the loop), then each token row of the tile gets its K weighted
    // route rows added in route order, as a float4 per thread: the same
    // arithmetic as the separate combine, with no shared row in HBM
    constexpr int TS = kDRowsB + 4;                       // padded row (floats)
    static_assert(MROWS * TS * 4 <= kDStages * STAGE, "tile fits the ring");
    float* tile = reinterpret_cast<float*>(s_ring);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MTW; t++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int u = 0; u < 4; u++)
          tile[(wm * 16 * MTW + 16 * t + 4 * lg + i) * TS + wn * 64 + 16 * u + lm] = acc[t][u][i];
    __syncthreads();
    const int c4 = threadIdx.x & 31, n = n0 + 4 * c4;
    const int K = a.topK;
    constexpr int KB = 16;
    for (int r = threadIdx.x >> 5; r < MROWS; r += kDThreads / 32) {
      const int m = m0 + r;
      if (m >= a.M || n >= a.N) continue;
      float4 v = *reinterpret_cast<const float4*>(tile + r * TS + 4 * c4);
      for (int k0 = 0; k0 < K; k0 += KB) {
        float4 rv[KB];
        float g[KB];
        // every route's position and weight first, then every row: a row
        // load issued between two position loads would make the second one's
        // wait also wait for that row (loads complete in order).  Guards, not
        // breaks, so the loops unroll and the arrays stay in registers.
        int pos[KB];
#pragma unroll
        for (int j = 0; j < KB; j++) {
          if (k0 + j < K) {
            const size_t q = (size_t)m * K + k0 + j;
            pos[j] = a.route_pos[q];
            g[j] = a.topk_w[q];
          }
        }
#pragma unroll
        for (int j = 0; j < KB; j++) {
          if (k0 + j < K) {
            // each route row is read exactly once: keep it out of the caches
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v x4 = __builtin_nontemporal_load(
                reinterpret_cast<const f4v*>(a.route_rows + (size_t)pos[j] * a.N + n));
            rv[j] = make_float4(x4.x, x4.y, x4.z, x4.w);
          }
        }
#pragma unroll
        for (int j = 0; j < KB; j++) {
          if (k0 + j >= K) continue;
          v.x = __builtin_fmaf(g[j], rv[j].x, v.x);
          v.y = __builtin_fmaf(g[j], rv[j].y, v.y);
          v.z = __builtin_fmaf(g[j], rv[j].z, v.z);
          v.w = __builtin_fmaf(g[j], rv[j].w, v.w);
        }
      }
      if (a.y_bf16) {
        bf16_t* out = reinterpret_cast<bf16_t*>(a.y) + (size_t)m * a.N + n;
        *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + (size_t)m * a.N + n) = v;
      }
    }
    return;
  }

  // epilogue: lane holds C[4 lg + i][lm] of each 16x16 tile.  The router
  // bias of the lane's four columns is read once, before any store (read
  // inside the loop it would be fetched again after every store that might
  // alias it, one round trip per output)
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == kDRouter || COMB) {
    if (!gu && a.bias) {
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int n = n0 + wn * 64 + 16 * u + lm;
        bv[u] = a.bias[n < NN ? n : NN - 1];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MTW; t++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int m = m0 + wm * 16 * MTW + 16 * t + 4 * lg + i;
      if (m >= a.M) continue;
      if (gu) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const int n = n0 + wn * 32 + 16 * u + lm;
          if (n < NN)
            outg[(size_t)m * NN + n] = to_bf16(silu_f32(acc[t][u][i]) * acc[t][u + 2][i]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int n = n0 + wn * 64 + 16 * u + lm;
          if (n < NN) {
            float v = acc[t][u][i];
            if constexpr (MODE == kDRouter || COMB) v += bv[u];
            a.outf[(size_t)m * NN + n] = v;
          }
        }
      }
    }
  }
}

template <int MODE, int MTW>
void launch_dense(const DArgs& a, int kid, hipStream_t s) {
  const int NTr = MODE == kDGateUp ? 0 : (a.N + kDRowsB - 1) / kDRowsB;
  const int NTg = MODE == kDGateUp ? (a.N + kDRowsB / 2 - 1) / (kDRowsB / 2)
                                   : (MODE == kDRouterGateUp ? (a.g_N + kDRowsB / 2 - 1) / (kDRowsB / 2) : 0);
  const int NT = NTr + NTg;
  const int MTt = (a.M + 32 * MTW - 1) / (32 * MTW);
  if (MTt <= 0 || NT <= 0) return;
  // token tiles rounded up to a multiple of 8 (one per XCD); the extra ones exit
  MOE_LAUNCH(kid, (k_dense<MODE, MTW>), dim3(((MTt + 7) / 8) * 8 * NT), dim3(kDThreads), 0, s, a);
}

DArgs dargs(const void* a, int M, int N, int K) {
  DArgs d = {};
  d.a = reinterpret_cast<const bf16_t*>(a);
  d.M = M;
  d.N = N;
  d.K = K;
  return d;
}

}  // namespace

void launch_dense_router(const void* x, int T, const void* w_router, const float* bias, int E,
                         int H, float* keys_approx, float* wnorm2, hipStream_t s) {
  DArgs d = dargs(x, T, E, H);
  d.b0 = reinterpret_cast<const bf16_t*>(w_router);
  d.bias = bias;
  d.outf = keys_approx;
  d.wnorm2 = wnorm2;
  launch_dense<kDRouter, 2>(d, MOE_K_ROUTER_APPROX, s);
}

void launch_dense_shared_gateup(const void* x, int T, const void* w_gate, const void* w_up,
                                void* h_s, int H, int I, hipStream_t s) {
  DArgs d = dargs(x, T, I, H);
  d.b0 = reinterpret_cast<const bf16_t*>(w_gate);
  d.b1 = reinterpret_cast<const bf16_t*>(w_up);
  d.outh = reinterpret_cast<bf16_t*>(h_s);
  launch_dense<kDGateUp, 2>(d, MOE_K_PREFILL_SHARED_GATEUP, s);
}

void launch_dense_router_shared_gateup(const void* x, int T, const void* w_router,
                                      const float* bias, int E, int H, float* keys_approx,
                                      float* wnorm2, const void* w_gate, const void* w_up,
                                      void* h_s, int I, hipStream_t s) {
  DArgs d = dargs(x, T, E, H);
  d.b0 = reinterpret_cast<const bf16_t*>(w_router);
  d.bias = bias;
  d.outf = keys_approx;
  d.wnorm2 = wnorm2;
  d.g_gate = reinterpret_cast<const bf16_t*>(w_gate);
  d.g_up = reinterpret_cast<const bf16_t*>(w_up);
  d.g_out = reinterpret_cast<bf16_t*>(h_s);
  d.g_N = I;
  launch_dense<kDRouterGateUp, 2>(d, MOE_K_ROUTER_APPROX, s);
}

void launch_dense_shared_down(const void* h_s, int T, const void* w_down, float* rows, int H,
                              int I, hipStream_t s) {
  DArgs d = dargs(h_s, T, H, I);
  d.b0 = reinterpret_cast<const bf16_t*>(w_down);
  d.outf = rows;
  launch_dense<kDDown, 2>(d, MOE_K_PREFILL_SHARED_DOWN, s);
}

void launch_dense_shared_down_combine(const void* h_s, int T, const void* w_down,
                                      const float* route_rows, const int32_t* route_pos,
                                      const float* topk_w, int K, int H, int I, void* y, int y_dt,
                                      hipStream_t s) {
  DArgs d = dargs(h_s, T, H, I);
  d.b0 = reinterpret_cast<const bf16_t*>(w_down);
  d.route_rows = route_rows;
  d.route_pos = route_pos;
  d.topk_w = topk_w;
  d.topK = K;
  d.y = y;
  d.y_bf16 = y_dt == MOE_BF16;
  launch_dense<kDDownCombine, 2>(d, MOE_K_COMBINE, s);
}

}  // namespace moe
