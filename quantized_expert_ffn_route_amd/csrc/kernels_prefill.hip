// Prefill path (A7, A8): grouped GEMMs over the expert buckets produced by
// the counting sort, and a deterministic combine.  The shared expert's bf16
// GEMMs and the MFMA router pass run on the dense kernels (kernels_dense.hip).
//
// A workgroup of 8 waves owns 128 weight rows (gate/up: 16 rows of gate and
// of up per wave) or 256 weight rows (down: 32 rows per wave) of one expert
// and one tile of that expert's bucket of routes.  Every lane dequantises its
// own weight blocks straight into MFMA operand registers, one MFMA k-step at
// a time, and reuses them for all token tiles of the tile.  Dequantisation
// is vector-ALU work that shares the SIMD's issue slots with the MFMAs, so a
// routed bf16 tile holds 96 token rows: about one whole bucket at the usual
// prefill load, so that each weight block is dequantised once per expert.
//
// Routed bf16 tiles: the gathered token rows of each 128-wide slice of the
// contraction axis go from global memory straight into LDS (one 16-byte
// direct-to-LDS load per lane and piece) through a three-stage ring, two
// slices ahead; weight blocks are loaded one slice ahead into registers.
// The K loop is unrolled at compile time, so every wait is an exact count of
// the loads still allowed in flight.  The other cases (fp32 activations,
// routed or shared, and contractions the unrolled loop does not cover)
// stage the token rows through registers into a
// double-buffered LDS tile (rows padded so the fragment reads are
// bank-conflict free).  The down projection writes one fp32 row per route;
// the combine kernel then sums each token's K rows in rank order on top of
// the shared expert's output -- no atomics, deterministic.  The pages'
// prefill path is the weak spot of the consumer-GPU build (P1, "speed vs
// context, and the 256k profile").
#include "device_common.hpp"

namespace moe {

namespace {

enum Mode {
  kRoutedGateUp = 0,
  kSharedGateUp = 1,
  kRoutedDown = 2,
  kSharedDown = 3
};

struct PArgs {
  const int32_t* offsets;
  const int2* tiles;         // routed modes: (expert, first row inside its bucket)
  const int32_t* n_tiles;
  const int32_t* sorted;
  const int32_t* tier_map;
  int E, K, T, H, I;
  const void* src;       // x (gate/up) or h (down)
  void* dst;             // h / fp32 route rows / fp32 shared rows
  Tables tb;
};

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <typename A> struct PT;
template <> struct PT<bf16_t> {
  static constexpr int ROWS = 64;         // token rows per pass
  static constexpr int RU = 64 + 4;       // LDS row stride in u32 (128 bf16 + pad)
};
template <> struct PT<float> {
  static constexpr int ROWS = 64;
  static constexpr int RU = 128 + 4;
};

// Token rows per pass of the register-staged body: 64 keeps a routed
// workgroup within its register budget; the fp32 shared-expert modes take 32
// rows, so that a 4096-token prefill still has 128 token tiles to spread.
template <typename A, int MODE> struct PR {
  static constexpr int ROWS = (MODE == kRoutedGateUp || MODE == kRoutedDown || sizeof(A) == 2)
                                  ? PT<A>::ROWS
                                  : PT<A>::ROWS / 2;
};

template <int MODE> struct MC {
  static constexpr bool GATEUP = MODE == kRoutedGateUp || MODE == kSharedGateUp;
  static constexpr bool ROUTED = MODE == kRoutedGateUp || MODE == kRoutedDown;
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int RGW = GATEUP ? 1 : 2;          // 16-row groups per wave
  static constexpr int NWG = kWaves * RGW * 16;       // weight rows per workgroup
};

// Raw weight data of one lane for one super-step (loaded one step ahead):
// dense, 32 act values; quantised, the code field w[0..3] and dm in v[4].
template <typename A, int BITS>
struct BRaw {
  uint32_t v[BITS == 0 ? 16 * sizeof(A) / 2 : 5];
};

// MFMA operand fragment of the weights.
template <typename A> struct BFrag;
template <> struct BFrag<bf16_t> { uint32_t v[16]; };
template <> struct BFrag<float> { float v[32]; };

template <typename A, int BITS>
__device__ __forceinline__ void load_braw(BRaw<A, BITS>& r, const Tables& tb, int tier, int mat, int slot,
                                          int R, int C, int rg, int c, int lane, const void* dense) {
  const int lm = lane & 15, lg = lane >> 4;
  if constexpr (BITS == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const A*>(dense) +
                                                    (size_t)(rg * 16 + lm) * C + 128 * c + 32 * lg);
#pragma unroll
    for (int i = 0; i < (int)(2 * sizeof(A)); i++) {
      const uint4 t = q[i];
      r.v[4 * i] = t.x; r.v[4 * i + 1] = t.y; r.v[4 * i + 2] = t.z; r.v[4 * i + 3] = t.w;
    }
  } else {
    const size_t idx = (((size_t)slot * (R / 16) + rg) * (C / 128) + c) * 64 + lane;
    load_field<BITS>(field_ptr<BITS>(tb.codes[tier][mat], idx), r.v);
    r.v[4] = load_scale<BITS>(tb.dm[tier][mat], idx);
  }
}

template <typename A, int BITS>
__device__ __forceinline__ void to_bfrag(BFrag<A>& f, const BRaw<A, BITS>& r) {
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

// One workgroup's work: weight rows [nt*NWG, nt*NWG + NWG) of one expert (or
// of the shared expert) against `nrows` token rows starting at row0.
template <typename A, int BITS, int MODE>
__device__ __forceinline__ void prefill_body(const PArgs& a, int grp, int row0, int nrows, int tier,
                                             int slot, int nt, uint32_t* __restrict__ sA) {
  using C = MC<MODE>;
  constexpr int NMAT = C::NMAT, RGW = C::RGW;
  constexpr int ROWS = PR<A, MODE>::ROWS, RU = PT<A>::RU;
  constexpr int MT = ROWS / 16;
  constexpr int PARTS = kThreads / ROWS;                 // threads staging one row
  constexpr int U4 = 128 * (int)sizeof(A) / 16 / PARTS;  // uint4 per staging thread
  const int Kc = MODE == kRoutedDown || MODE == kSharedDown ? a.I : a.H;
  const int Nr = C::GATEUP ? a.I : a.H;
  const int nbg = Kc / 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const A* src = reinterpret_cast<const A*>(a.src);
  const int n0 = nt * C::NWG + wave * RGW * 16;           // first weight row of this wave
  const bool active = n0 < Nr;                            // down: H may be < NWG
  const int srow = threadIdx.x / PARTS, spart = threadIdx.x % PARTS;

  auto load_b = [&](BRaw<A, BITS> (&r)[RGW][NMAT], int c) {
    if (!active) return;
#pragma unroll
    for (int q = 0; q < RGW; q++)
#pragma unroll
      for (int m = 0; m < NMAT; m++)
        load_braw<A, BITS>(r[q][m], a.tb, tier, C::GATEUP ? m : MOE_DOWN, slot, Nr, Kc,
                           n0 / 16 + q, c, lane, a.tb.dense[C::GATEUP ? m : MOE_DOWN]);
  };

  for (int pass0 = 0; pass0 < nrows; pass0 += ROWS) {
    const int rows_here = min(ROWS, nrows - pass0);
    const int ntiles = (rows_here + 15) / 16;
    // token row this thread stages (fixed for the pass)
    int srcrow = -1;
    if (srow < rows_here) {
      if constexpr (MODE == kRoutedGateUp) srcrow = a.sorted[row0 + pass0 + srow] / a.K;
      else srcrow = row0 + pass0 + srow;
    }
    // thread (srow, spart) moves 16-byte pieces spart, spart + PARTS, ... of
    // its row: the PARTS threads of a row cover contiguous 16 * PARTS bytes per
    // step, in global memory and in LDS (no bank conflicts on the store)
    auto load_a = [&](uint4 (&r)[U4], int c) {
      if (srcrow >= 0) {
        const uint4* q = reinterpret_cast<const uint4*>(src + (size_t)srcrow * Kc + 128 * c) + spart;
#pragma unroll
        for (int i = 0; i < U4; i++) r[i] = q[PARTS * i];
      } else {
#pragma unroll
        for (int i = 0; i < U4; i++) r[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto store_a = [&](const uint4 (&r)[U4], int buf) {
      uint32_t* d = sA + buf * ROWS * RU + srow * RU + spart * 4;
#pragma unroll
      for (int i = 0; i < U4; i++) *reinterpret_cast<uint4*>(d + 4 * PARTS * i) = r[i];
    };

    f32x4_t acc[RGW][NMAT][MT];
#pragma unroll
    for (int q = 0; q < RGW; q++)
#pragma unroll
      for (int m = 0; m < NMAT; m++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[q][m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[U4];
    BRaw<A, BITS> rb[RGW][NMAT];
    __syncthreads();                 // previous pass done with the LDS buffers
    load_a(ra, 0);
    load_b(rb, 0);
    store_a(ra, 0);
    __syncthreads();
    for (int c = 0; c < nbg; c++) {
      BRaw<A, BITS> nb[RGW][NMAT];
      const bool more = c + 1 < nbg;
      if (more) {
        load_a(ra, c + 1);
        load_b(nb, c + 1);
      }
      if (active) {
        BFrag<A> bf[RGW][NMAT];
#pragma unroll
        for (int q = 0; q < RGW; q++)
#pragma unroll
          for (int m = 0; m < NMAT; m++) to_bfrag<A, BITS>(bf[q][m], rb[q][m]);
        const uint32_t* buf = sA + (c & 1) * ROWS * RU;
#pragma unroll
        for (int t = 0; t < MT; t++) {
          if (t >= ntiles) break;
          const uint32_t* arow = buf + (16 * t + lm) * RU;
          if constexpr (sizeof(A) == 2) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * lg + 4 * i);
#pragma unroll
              for (int q = 0; q < RGW; q++)
#pragma unroll
                for (int m = 0; m < NMAT; m++)
                  acc[q][m][t] = mfma_bf16(av.x, av.y, av.z, av.w, bf[q][m].v[4 * i],
                                           bf[q][m].v[4 * i + 1], bf[q][m].v[4 * i + 2],
                                           bf[q][m].v[4 * i + 3], acc[q][m][t]);
            }
          } else {
#pragma unroll
            for (int s = 0; s < 32; s++) {
              const float av = __uint_as_float(arow[32 * lg + s]);
#pragma unroll
              for (int q = 0; q < RGW; q++)
#pragma unroll
                for (int m = 0; m < NMAT; m++) acc[q][m][t] = mfma_f32(av, bf[q][m].v[s], acc[q][m][t]);
            }
          }
        }
      }
      if (more) {
        store_a(ra, (c + 1) & 1);
#pragma unroll
        for (int q = 0; q < RGW; q++)
#pragma unroll
          for (int m = 0; m < NMAT; m++) rb[q][m] = nb[q][m];
      }
      __syncthreads();
    }

    if (!active) continue;
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
        for (int q = 0; q < RGW; q++) {
          const int n = n0 + 16 * q + lm;
          if (n >= Nr) continue;
          if constexpr (C::GATEUP) {
            const float v = silu_f32(acc[q][0][t][i]) * acc[q][1][t][i];
            A* out = reinterpret_cast<A*>(a.dst) + (size_t)gp * a.I + n;
            if constexpr (sizeof(A) == 2) *out = to_bf16(v); else *out = v;
          } else {
            reinterpret_cast<float*>(a.dst)[(size_t)gp * a.H + n] = acc[q][0][t][i];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 routed grouped GEMM with a deeper pipeline.  The 96 x 128 token tile
// of a chunk goes from global memory straight into LDS (global_load_lds_dwordx4:
// every lane gathers one 16-byte piece of a token row, the wave's 64 pieces
// land contiguously), through a ring of three stages; in LDS, piece p of row
// r sits at position p ^ pswz(r) (below), which keeps the fragment reads free
// of bank conflicts.  Weight blocks are prefetched one chunk ahead in two
// register slots (the chunk loop is unrolled, so the slots rotate without
// copies).  Per chunk: wait for the chunk's own loads, one barrier, issue the
// weight loads one chunk ahead and the token loads two chunks ahead, then
// dequantise and multiply.
// ---------------------------------------------------------------------------

constexpr int kStages = 3;
// Consecutive tiles (or token chunks) that one XCD takes together.
constexpr int kXcdRun = 4;
// Routed bf16 tiles: 96 token rows, so that one tile holds a whole expert
// bucket at the usual prefill load (about 80 routes per expert at 4096 tokens,
// top-10 of 512) and each weight block is dequantised once per expert.
constexpr int kTileRows = 96;
constexpr int kPieces = kTileRows * 16;           // 16-byte pieces per stage
constexpr int kStagePieces = kPieces;

// Swizzle of the 16 pieces of a 256-byte token row in LDS.  A fragment read
// takes piece 4 * (lane / 16) + i of row lane % 16.  The piece is XORed with
// the row's two 2-bit halves swapped, so rows 0-3 start at pieces 0, 4, 8,
// 12, rows 4-7 at 1, 5, 9, 13, and so on.  Measured on gfx950 with all waves
// of a CU reading: 2.2 ns per wave-wide 16-byte read against 4.2 ns with the
// plain row XOR and 13.6 ns with no swizzle.
__device__ __forceinline__ int pswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// s_waitcnt with vmcnt(n) (expcnt, lgkmcnt left at their maxima), n < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One 16-byte piece per lane from global memory straight into LDS: lane i's
// piece lands at lds + 16 i (lds is wave-uniform).  The ring stages are
// distinct LDS objects, so the compiler's wait tracking tells them apart and
// adds no drain before LDS reads; completion of a stage is awaited explicitly
// (vmcnt, then a barrier) before any wave reads it.
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Barrier for LDS hand-over only: waits for this wave's LDS operations, not
// for its outstanding global loads (which __syncthreads would drain).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The whole K loop is unrolled at compile time (NBG chunks), so the stage,
// the weight register slot and the exact wait of every step are constants and
// the code is straight-line (the compiler's own waits then stay precise too).
template <int BITS, int MODE, int NBG>
__device__ __forceinline__ void prefill_body_lds(const PArgs& a, int grp, int row0, int nrows,
                                                 int tier, int slot, int nt,
                                                 uint4* __restrict__ s0, uint4* __restrict__ s1,
                                                 uint4* __restrict__ s2) {
  using A = bf16_t;
  using C = MC<MODE>;
  constexpr int NMAT = C::NMAT, RGW = C::RGW;
  constexpr int MT = kTileRows / 16;
  constexpr int LA = kPieces / kThreads;                          // A loads per wave per chunk
  constexpr int LB = RGW * NMAT * (BITS == 0 ? 2 * (int)sizeof(A) : 2);  // B loads per wave per chunk
  const int Kc = MODE == kRoutedDown || MODE == kSharedDown ? a.I : a.H;
  const int Nr = C::GATEUP ? a.I : a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const A* src = reinterpret_cast<const A*>(a.src);
  const int n0 = nt * C::NWG + wave * RGW * 16;
  // routed modes: the weight rows are a multiple of the workgroup's rows, so
  // every wave is active (a compile-time fact keeps the loads unconditional)
  const bool active = C::ROUTED || n0 < Nr;
  const int rows_here = min(kTileRows, nrows);
  const int ntiles = (rows_here + 15) / 16;

  // this lane's pieces: LA of them, LDS slot (LA * wave + j) * 64 + lane;
  // element offsets from src (32 bits: the activations hold < 2^31 elements)
  uint32_t aoff[LA];
#pragma unroll
  for (int j = 0; j < LA; j++) {
    const int sidx = (LA * wave + j) * 64 + lane;
    const int r = sidx >> 4, p = sidx & 15;
    const int lp = p ^ pswz(r);                                   // logical piece
    const int rr = r < rows_here ? r : 0;                         // rows past the tile: any valid row
    int srcrow;
    if constexpr (MODE == kRoutedGateUp) srcrow = a.sorted[row0 + rr] / a.K;
    else srcrow = row0 + rr;
    aoff[j] = (uint32_t)srcrow * (uint32_t)Kc + 8u * (uint32_t)lp;
  }
  auto load_a = [&](int c, uint4* __restrict__ st) {
#pragma unroll
    for (int j = 0; j < LA; j++) lds_dma16(src + aoff[j] + 128 * c, st + (LA * wave + j) * 64);
  };
  auto load_b = [&](BRaw<A, BITS> (&r)[RGW][NMAT], int c) {
#pragma unroll
    for (int q = 0; q < RGW; q++)
#pragma unroll
      for (int m = 0; m < NMAT; m++) {
        if (C::ROUTED || active)
          load_braw<A, BITS>(r[q][m], a.tb, tier, C::GATEUP ? m : MOE_DOWN, slot, Nr, Kc,
                             n0 / 16 + q, c, lane, nullptr);
      }
  };

  f32x4_t acc[RGW][NMAT][MT];
#pragma unroll
  for (int q = 0; q < RGW; q++)
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
      for (int t = 0; t < MT; t++) acc[q][m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one MFMA k-step at a time: dequantise its 8 codes of every weight block,
  // then multiply all token tiles (8 operand registers live instead of 32)
  auto compute = [&](const uint4* __restrict__ st, const BRaw<A, BITS> (&rb)[RGW][NMAT]) {
    static_assert(BITS != 0 && C::ROUTED, "quantised routed weights");
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t bq[RGW][NMAT][4];
#pragma unroll
      for (int q = 0; q < RGW; q++)
#pragma unroll
        for (int m = 0; m < NMAT; m++) dequant_kstep<BITS>(i, rb[q][m].v, rb[q][m].v[4], bq[q][m]);
#pragma unroll
      for (int t = 0; t < MT; t++) {
        if (t >= ntiles) break;
        const uint4 av = st[(16 * t + lm) * 16 + ((4 * lg + i) ^ pswz(lm))];
#pragma unroll
        for (int q = 0; q < RGW; q++)
#pragma unroll
          for (int m = 0; m < NMAT; m++)
            acc[q][m][t] = mfma_bf16(av.x, av.y, av.z, av.w, bq[q][m][0], bq[q][m][1],
                                     bq[q][m][2], bq[q][m][3], acc[q][m][t]);
      }
    }
  };

  // token rows run two chunks ahead (three LDS stages), weight blocks one
  // chunk ahead (two register slots); step c issues B(c + 1) before A(c + 2),
  // so at the start of step c the newest loads are B(c) then A(c + 1)
  BRaw<A, BITS> b0[RGW][NMAT], b1[RGW][NMAT];
  load_a(0, s0);
  load_b(b0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NBG > 1) load_a(1, s1);
  auto step = [&](int c, const uint4* __restrict__ st, uint4* __restrict__ st2,
                  const BRaw<A, BITS> (&cur)[RGW][NMAT], BRaw<A, BITS> (&nxt)[RGW][NMAT]) {
    if (c + 1 < NBG) wait_vmcnt<LA>();   // A(c + 1) may stay in flight
    else wait_vmcnt<0>();
    lds_barrier();
    if (c + 1 < NBG) load_b(nxt, c + 1);
    // keep the issue order: the waits above count on the A pieces being the
    // newest loads in flight
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < NBG) load_a(c + 2, st2);
    compute(st, cur);
  };
#pragma unroll
  for (int c = 0; c < NBG; c += 6) {
    step(c, s0, s2, b0, b1);
    if (c + 1 < NBG) step(c + 1, s1, s0, b1, b0);
    if (c + 2 < NBG) step(c + 2, s2, s1, b0, b1);
    if (c + 3 < NBG) step(c + 3, s0, s2, b1, b0);
    if (c + 4 < NBG) step(c + 4, s1, s0, b0, b1);
    if (c + 5 < NBG) step(c + 5, s2, s1, b1, b0);
  }

  if (!C::ROUTED && !active) return;
#pragma unroll
  for (int t = 0; t < MT; t++) {
    if (t >= ntiles) break;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int p = 16 * t + 4 * lg + i;
      if (p >= rows_here) continue;
      const int gp = row0 + p;
#pragma unroll
      for (int q = 0; q < RGW; q++) {
        const int n = n0 + 16 * q + lm;
        if (n >= Nr) continue;
        if constexpr (C::GATEUP) {
          const float v = silu_f32(acc[q][0][t][i]) * acc[q][1][t][i];
          reinterpret_cast<A*>(a.dst)[(size_t)gp * a.I + n] = to_bf16(v);
        } else {
          reinterpret_cast<float*>(a.dst)[(size_t)gp * a.H + n] = acc[q][0][t][i];
        }
      }
    }
  }
}

// NBG > 0 (bf16 routed modes): the unrolled pipeline for NBG chunks; the
// launcher picks it when the contraction has NBG chunks and the workgroup
// rows divide the weight rows.  NBG == 0: the register-staged body.
// FAM selects the table formats a kernel handles: 0 the affine widths, 1
// MXFP4, -1 all.  Every body inlined into one kernel adds to the register
// pressure of the others (at the bf16 kernels' 128-register budget the four
// together spill, each family alone does not), so the bf16 launcher runs one
// kernel per family present and a workgroup whose tier is of the other
// family leaves at once.
template <typename A, int MODE, int NBG, int FAM>
__device__ __forceinline__ void prefill_wg(const PArgs& a) {
  using C = MC<MODE>;
  constexpr int ROWS = PR<A, MODE>::ROWS;
  // routed modes: rows per tile of the sorted routes (the register-staged
  // body walks a tile in passes of ROWS)
  constexpr int TILE = sizeof(A) == 2 ? kTileRows : ROWS;
  const int Nr = C::GATEUP ? a.I : a.H;
  const int NT = (Nr + C::NWG - 1) / C::NWG;
  // XCD-aware mapping: the workgroups that share one expert's (or one token
  // chunk's) rows land on the same XCD, whose L2 then serves the re-reads.
  // Groups of kXcdRun consecutive tiles go to one XCD: the sort lists an
  // expert's full tiles next to each other, so they share that XCD's L2 and
  // its table lines are fetched once (the grid covers whole groups).
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3, g8 = j / NT;
  const int grp = ((g8 / kXcdRun) * 8 + xcd) * kXcdRun + g8 % kXcdRun, nt = j % NT;
  if constexpr (C::ROUTED) {
    if (grp >= *a.n_tiles) return;
    const int2 tile = a.tiles[grp];
    const int e = tile.x;
    const int row0 = a.offsets[e] + tile.y;
    const int nrows = min(TILE, a.offsets[e + 1] - row0);
    if (nrows <= 0) return;
    const int tm = a.tier_map[e];
    const int tier = tm >> 16, slot = tm & 0xFFFF;
    if (tier < 0 || tier > 2 || slot >= a.tb.n_slots[tier]) return;
    // the tier's code format (of this matrix) is uniform over the workgroup
    const int wbits = MODE == kRoutedDown ? a.tb.bits_dn[tier] : a.tb.bits[tier];
    if constexpr (FAM >= 0) {
      if ((wbits == kMx4) != (FAM == 1)) return;
    }
    if constexpr (sizeof(A) == 2 && NBG > 0) {
      __shared__ uint4 sL0[kStagePieces], sL1[kStagePieces], sL2[kStagePieces];
      if constexpr (FAM == 1) {
        prefill_body_lds<kMx4, MODE, NBG>(a, grp, row0, nrows, tier, slot, nt, sL0, sL1, sL2);
      } else {
        switch (wbits) {
          case 4: prefill_body_lds<4, MODE, NBG>(a, grp, row0, nrows, tier, slot, nt, sL0, sL1, sL2); break;
          case 3: prefill_body_lds<3, MODE, NBG>(a, grp, row0, nrows, tier, slot, nt, sL0, sL1, sL2); break;
          case 2: prefill_body_lds<2, MODE, NBG>(a, grp, row0, nrows, tier, slot, nt, sL0, sL1, sL2); break;
          default:
            if constexpr (FAM < 0)
              prefill_body_lds<kMx4, MODE, NBG>(a, grp, row0, nrows, tier, slot, nt, sL0, sL1, sL2);
            break;
        }
      }
    } else {
      __shared__ uint32_t sA[2 * ROWS * PT<A>::RU];
      if constexpr (FAM == 1) {
        prefill_body<A, kMx4, MODE>(a, grp, row0, nrows, tier, slot, nt, sA);
      } else {
        switch (wbits) {
          case 4: prefill_body<A, 4, MODE>(a, grp, row0, nrows, tier, slot, nt, sA); break;
          case 3: prefill_body<A, 3, MODE>(a, grp, row0, nrows, tier, slot, nt, sA); break;
          case 2: prefill_body<A, 2, MODE>(a, grp, row0, nrows, tier, slot, nt, sA); break;
          default:
            if constexpr (FAM < 0) prefill_body<A, kMx4, MODE>(a, grp, row0, nrows, tier, slot, nt, sA);
            break;
        }
      }
    }
  } else {
    const int row0 = grp * ROWS;
    if (row0 >= a.T) return;
    // shared expert with fp32 activations: dense weights, register-staged
    __shared__ uint32_t sA[2 * ROWS * PT<A>::RU];
    prefill_body<A, 0, MODE>(a, grp, row0, min(ROWS, a.T - row0), 0, 0, nt, sA);
  }
}

// bf16: four waves per SIMD (two workgroups per CU); the fp32 variants keep
// their registers (no spills) at lower occupancy.
template <int MODE, int NBG, int FAM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_prefill_bf16(PArgs a) {
  prefill_wg<bf16_t, MODE, NBG, FAM>(a);
}
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_prefill_f32(PArgs a) {
  prefill_wg<float, MODE, 0, -1>(a);
}

template <typename A, int MODE>
void launch_mode(const PArgs& a, int n_groups, hipStream_t s) {
  using C = MC<MODE>;
  const int Nr = C::GATEUP ? a.I : a.H;
  const int NT = (Nr + C::NWG - 1) / C::NWG;
  dim3 grid(((n_groups + 8 * kXcdRun - 1) / (8 * kXcdRun)) * 8 * kXcdRun * NT);
  constexpr int kid = MODE == kRoutedGateUp   ? MOE_K_PREFILL_GATEUP
                      : MODE == kSharedGateUp ? MOE_K_PREFILL_SHARED_GATEUP
                      : MODE == kSharedDown   ? MOE_K_PREFILL_SHARED_DOWN
                                              : MOE_K_PREFILL_DOWN;
  static_assert(sizeof(A) == 4 || C::ROUTED, "bf16 shared GEMMs run on the dense kernels");
  if constexpr (sizeof(A) == 2) {
    int nbg = 0;
    const int k = (MODE == kRoutedDown ? a.I : a.H) / 128;
    if (Nr % C::NWG == 0 && (k & (k - 1)) == 0 && k <= 32) nbg = k;
    // one launch per format family present in this matrix's tier tables
    bool fam[2] = {false, false};
    for (int t = 0; t < 3; t++) {
      if (a.tb.n_slots[t] == 0) continue;
      const int f = MODE == kRoutedDown ? a.tb.bits_dn[t] : a.tb.bits[t];
      fam[f == kMx4] = true;
    }
#define MOE_PREFILL_FAMILY(F)                                                                         \
  switch (nbg) {                                                                                      \
    case 1: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 1, F>), grid, dim3(kThreads), 0, s, a); break;   \
    case 2: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 2, F>), grid, dim3(kThreads), 0, s, a); break;   \
    case 4: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 4, F>), grid, dim3(kThreads), 0, s, a); break;   \
    case 8: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 8, F>), grid, dim3(kThreads), 0, s, a); break;   \
    case 16: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 16, F>), grid, dim3(kThreads), 0, s, a); break; \
    case 32: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 32, F>), grid, dim3(kThreads), 0, s, a); break; \
    default: MOE_LAUNCH(kid, (k_prefill_bf16<MODE, 0, F>), grid, dim3(kThreads), 0, s, a); break;  \
  }
    if (fam[0]) MOE_PREFILL_FAMILY(0)
    if (fam[1]) MOE_PREFILL_FAMILY(1)
#undef MOE_PREFILL_FAMILY
  } else {
    MOE_LAUNCH(kid, (k_prefill_f32<MODE>), grid, dim3(kThreads), 0, s, a);
  }
}

PArgs make_args(const int32_t* offsets, const int32_t* sorted, const int32_t* tier_map, int E,
                int K, int T, int H, int I, const void* src, void* dst, const Tables& tb) {
  PArgs a;
  a.offsets = offsets;
  a.tiles = nullptr;
  a.n_tiles = nullptr;
  a.sorted = sorted;
  a.tier_map = tier_map;
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

// y[t] = shared[t] + sum_k w[t][k] * rows[pos[t*K + k]], k in rank order.
// The rows of up to KB routes are loaded before any is added, so they are in
// flight together; the sum itself runs in rank order.
template <typename Y, int KB>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ shared_rows,
                                                 const float* __restrict__ route_rows,
                                                 const int32_t* __restrict__ route_pos,
                                                 const float* __restrict__ topk_w, int K, int H,
                                                 int nb, Y* __restrict__ y) {
  const int t = blockIdx.x / nb;
  const int c = ((blockIdx.x % nb) * blockDim.x + threadIdx.x) * 4;
  if (c >= H) return;
  float4 acc = shared_rows ? *reinterpret_cast<const float4*>(shared_rows + (size_t)t * H + c)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < K; k0 += KB) {
    float4 v[KB];
    float g[KB];
#pragma unroll
    for (int j = 0; j < KB; j++) {
      if (k0 + j >= K) break;
      const int k = k0 + j;
      const int pos = route_pos[(size_t)t * K + k];
      g[j] = topk_w[(size_t)t * K + k];
      // each route row is read exactly once: keep it out of the caches
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v r = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(route_rows + (size_t)pos * H + c));
      v[j] = make_float4(r.x, r.y, r.z, r.w);
    }
#pragma unroll
    for (int j = 0; j < KB; j++) {
      if (k0 + j >= K) continue;
      acc.x = __builtin_fmaf(g[j], v[j].x, acc.x);
      acc.y = __builtin_fmaf(g[j], v[j].y, acc.y);
      acc.z = __builtin_fmaf(g[j], v[j].z, acc.z);
      acc.w = __builtin_fmaf(g[j], v[j].w, acc.w);
    }
  }
  Y* out = y + (size_t)t * H + c;
  if constexpr (sizeof(Y) == 4) {
    *reinterpret_cast<float4*>(out) = acc;
  } else {
    const uint32_t lo = pack_bf16(acc.x, acc.y), hi = pack_bf16(acc.z, acc.w);
    *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
  }
}

}  // namespace

int prefill_tile_rows(int act) {
  return act == MOE_BF16 ? kTileRows : PR<float, kRoutedGateUp>::ROWS;
}

void launch_prefill_gateup(int act, const int32_t* offsets, const int32_t* sorted_routes,
                           const int2* tiles, const int32_t* n_tiles, int max_tiles,
                           const int32_t* tier_map, int E, int K, const void* x, const Tables& tb,
                           void* h, int H, int I, hipStream_t s) {
  PArgs a = make_args(offsets, sorted_routes, tier_map, E, K, 0, H, I, x, h, tb);
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  if (act == MOE_BF16) launch_mode<bf16_t, kRoutedGateUp>(a, max_tiles, s);
  else launch_mode<float, kRoutedGateUp>(a, max_tiles, s);
}

// The shared expert's bf16 GEMMs run on the dense kernels (kernels_dense.hip);
// fp32 activations take the register-staged body with dense weights.
void launch_prefill_shared_gateup(int act, const void* x, int T, const Tables& tb, void* h_s,
                                  int H, int I, hipStream_t s) {
  if (act == MOE_BF16) {
    launch_dense_shared_gateup(x, T, tb.dense[MOE_GATE], tb.dense[MOE_UP], h_s, H, I, s);
    return;
  }
  const PArgs a = make_args(nullptr, nullptr, nullptr, 0, 0, T, H, I, x, h_s, tb);
  constexpr int R = PR<float, kSharedGateUp>::ROWS;
  launch_mode<float, kSharedGateUp>(a, (T + R - 1) / R, s);
}

void launch_prefill_shared_down(int act, const void* h_s, int T, const Tables& tb, float* rows,
                                int H, int I, hipStream_t s) {
  if (act == MOE_BF16) {
    launch_dense_shared_down(h_s, T, tb.dense[MOE_DOWN], rows, H, I, s);
    return;
  }
  const PArgs a = make_args(nullptr, nullptr, nullptr, 0, 0, T, H, I, h_s, rows, tb);
  constexpr int R = PR<float, kSharedDown>::ROWS;
  launch_mode<float, kSharedDown>(a, (T + R - 1) / R, s);
}


void launch_prefill_down(int act, const int32_t* offsets, const int32_t* sorted_routes,
                         const int2* tiles, const int32_t* n_tiles, int max_tiles,
                         const int32_t* tier_map, int E, int K, const void* h, const Tables& tb,
                         float* route_rows, int H, int I, hipStream_t s) {
  PArgs a = make_args(offsets, sorted_routes, tier_map, E, K, 0, H, I, h, route_rows, tb);
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  if (act == MOE_BF16) launch_mode<bf16_t, kRoutedDown>(a, max_tiles, s);
  else launch_mode<float, kRoutedDown>(a, max_tiles, s);
}

void launch_combine(int y_dt, const float* shared_rows, const float* route_rows,
                    const int32_t* route_pos, const float* topk_w, int T, int K, int H, void* y,
                    hipStream_t s) {
  const int nb = (H / 4 + 255) / 256;
  dim3 grid((unsigned)((size_t)T * nb));
  if (y_dt == MOE_BF16)
    MOE_LAUNCH(MOE_K_COMBINE, (k_combine<bf16_t, 16>), grid, dim3(256), 0, s, shared_rows, route_rows,
               route_pos, topk_w, K, H, nb, (bf16_t*)y);
  else
    MOE_LAUNCH(MOE_K_COMBINE, (k_combine<float, 16>), grid, dim3(256), 0, s, shared_rows, route_rows,
               route_pos, topk_w, K, H, nb, (float*)y);
}

}  // namespace moe
