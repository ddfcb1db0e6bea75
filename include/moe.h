/*
 * moe.h -- C ABI of the routed, popularity-tiered, dequantised MoE FFN layer
 * on AMD Instinct MI355X (gfx950).
 *
 * One layer = a router over E experts that keeps the top K per token, E
 * SwiGLU experts whose weights live in three precision tiers, and optionally
 * one shared expert that every token uses.  Pages cited by title and section:
 *
 *   [P1] "I ran a 125B model on three RTX 3090s at 80 tokens/s by teaching
 *        llama.cpp which experts matter" (dev.to)
 *   [P2] "Running Qwen3.8-Flash-Next 125B on Three RTX 3090s at 80 Tokens per
 *        Second" (explore.n1n.ai)
 *   [P5] "Qwen3.8-Flash-Next hits 39 tok/s on a 24GB GPU, provided you bring
 *        96GB of system RAM" (deniz.in)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer named "device" is device memory owned by the caller; the
 *   library never allocates device memory and keeps no global state apart
 *   from the optional launch trace of moe_set_trace.
 * - Forward calls and moe_route only enqueue work on `stream` and return;
 *   they never synchronise, print or abort.  They may be captured into a HIP
 *   graph (they issue kernels only; no memset or memcpy nodes).
 * - Workspace: pass ws == NULL to get the required size in *ws_bytes (nothing
 *   is launched, MOE_OK is returned).  Otherwise ws must be device memory,
 *   256-byte aligned, of at least *ws_bytes bytes (else MOE_ENOSPC).  The
 *   workspace needs no initial contents.  Calls that share one workspace
 *   must be ordered on one stream.
 * - All arguments are validated on the host before any launch; an invalid
 *   argument returns MOE_EINVAL (or MOE_EUNSUPPORTED for a valid but
 *   unsupported shape) and launches nothing.  A failed launch returns
 *   MOE_EHIP.  No call ever falls back to another algorithm, changes the
 *   batch, or uses managed memory.
 * - Expert ids are int32 in [0, E); "no expert" is never encoded in an id
 *   ([P1] "the four bugs, briefly": a -1 sentinel promoted to unsigned read
 *   four billion rows past a buffer).
 *
 * Steps of the layer (the labels the comments of this library use)
 * ----------------------------------------------------------------
 *   A0  tier build: rank experts by popularity, assign (tier, slot), pack.
 *   A1  router scores: key[t][e] = x[t] . W_r[e] + b[e].
 *   A2  top-K by (key desc, id asc) and softmax weights over the K kept.
 *   A3  tier dispatch of a decode group: the union of its experts.
 *   A4  stable counting sort of the routes t*K + k by expert (prefill).
 *   A5  decode gate/up: dequantise and multiply, h = silu(gate) * up.
 *   A6  decode down projection and weighted combine (+ shared expert).
 *   A7  prefill gate/up as grouped GEMMs over the expert buckets.
 *   A8  prefill down projection, shared expert and weighted combine.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* invalid argument (null, misaligned, out of range) */
  MOE_EUNSUPPORTED = -2, /* valid but unsupported shape or dtype              */
  MOE_ENOSPC = -3,       /* workspace smaller than required                  */
  MOE_EHIP = -4          /* a HIP runtime call or kernel launch failed        */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

enum { MOE_GATE = 0, MOE_UP = 1, MOE_DOWN = 2 };
enum { MOE_CODES = 0, MOE_DM = 1 };
enum { MOE_SRC_F32 = 0, MOE_SRC_CODES = 1 };

/* Format code of an MXFP4 table, accepted wherever a code width is (a code,
 * not a bit count): 4-bit E2M1 elements sharing one E8M0 power-of-two scale
 * per block of 32, as in the OCP Microscaling (MX) v1.0 definition.  The
 * pages give MXFP4 as the low tier of the down matrices ([P1] "step 4: three
 * shelves, all on the GPU"; [P2] "Lever 2"). */
#define MOE_MXFP4 0x14

/* Shape of one layer.
 *   hidden (H), inter (I): multiples of 128, H <= 8192 (MOE_EUNSUPPORTED
 *   otherwise).  E in [1, 65535].
 *   top_k (K) in [1, min(E, 64)].  has_shared: 0 or 1.
 *   act: moe_dtype of the activations x, the router weights, the shared
 *   expert's weights and the intermediate h (bf16 for the full-size layer,
 *   f32 for small parity layers). */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t has_shared;
  int32_t act;
} moe_dims;

/* Device tables of one layer.  Forward calls only read them.
 *
 * w_router  device [E][H], act dtype, row-major.
 * b_router  device [E] fp32, or NULL for no bias.
 * tier_map  device [E] int32: tier_map[e] = tier << 16 | slot.  Built by
 *           moe_build_tiers: experts ranked busiest first, the busiest in
 *           tier 0 ([P1] "step 2: the experts are not equal", "step 4: three
 *           shelves, all on the GPU"; [P2] "Lever 2").
 * n_slots   experts per tier; they sum to E.
 * tier_bits code width of each tier, each in {2, 3, 4} (4/3/2 by default),
 *           or MOE_MXFP4.
 * codes, dm [tier][matrix] device tables of the quantised experts of that
 *           tier, matrix = MOE_GATE ([I][H]), MOE_UP ([I][H]), MOE_DOWN
 *           ([H][I]).  Blocks are 32 consecutive weights along the
 *           contraction axis of one row with an fp16 scale d and fp16 min m;
 *           the weight is the float32 value d*q + m (bf16-rounded for bf16
 *           activations).  A tier table holds n_slots[tier] experts in slot
 *           order; within an expert matrix of R rows and C columns, 16-row by
 *           4-block tiles are stored row-group major: the block (slot s, row
 *           r, block column j) has index
 *             ((s*(R/16) + r/16)*(C/128) + j/4)*64 + 16*(j%4) + r%16
 *           and its code field is codes[index*4*bits .. +4*bits) (bit layout
 *           below), dm[index] = bits(d) | bits(m) << 16.  May be NULL for a
 *           tier with n_slots == 0.  A tier's codes and dm may instead live
 *           in pinned host memory mapped into the device's address space
 *           (hipHostMalloc; pass the address hipHostGetDevicePointer
 *           returns): the kernels then read that tier over the host link,
 *           the cold tier of [P1] "step 3: split every layer into hot and
 *           cold" kept in system RAM.  Results are unchanged.
 *           Code field of a b-bit block: b little-endian 32-bit words; each
 *           word's low half holds even-numbered codes and its high half the
 *           following odd codes at the same offsets, packed from bit 0:
 *             b=4: code 8i+2p+s at bit 32i + 16s + 4p
 *             b=2: code 16i+2p+s at bit 32i + 16s + 2p
 *             b=3: code 10i+2p+s at bit 32i + 16s + 3p (i < 3, p < 5); code
 *                  30+s has its bit r at bit 32r + 16s + 15.
 *           An MXFP4 table uses the same tile order with a 16-byte code
 *           field per block (code k at bits 4k..4k+3: byte j holds codes 2j
 *           in its low nibble and 2j+1 in its high nibble; E2M1 code = sign
 *           << 3 | exponent << 1 | mantissa) and one scale byte per block:
 *           dm then addresses uint8 E8M0 bytes, ((uint8_t*)dm)[index] = X +
 *           127, weight = E2M1(q) * 2^X.  X must lie in [-125, 125], which
 *           keeps every weight a normal bf16 (exact in bf16 and fp32).
 * w_shared  device, act dtype: gate [I][H], up [I][H], down [H][I]
 *           (row-major); NULL when has_shared == 0.
 * down_bits code width of each tier's down matrices, in {2, 3, 4} or
 *           MOE_MXFP4, or 0 to
 *           use tier_bits[t]: the down projection's own precision ladder
 *           ([P1] "step 4: three shelves, all on the GPU" and [P2] "Lever 2":
 *           gate/up and down take different formats per tier).  codes[t][2]
 *           and dm[t][2] are then sized and packed at that width; routing,
 *           the tier map and gate/up are unchanged.  A zeroed struct keeps
 *           one width per tier. */
typedef struct {
  void* w_router;
  float* b_router;
  int32_t* tier_map;
  int32_t n_slots[3];
  int32_t tier_bits[3];
  uint8_t* codes[3][3];
  uint32_t* dm[3][3];
  void* w_shared[3];
  int32_t down_bits[3];
} moe_layer;

/* Host-side source of the expert weights for moe_build_tiers, indexed by
 * expert id (not by slot).
 *   kind = MOE_SRC_F32:   w[mat] host fp32 [E][rows][cols]; the library
 *                         quantises every block (see moe_build_tiers).
 *   kind = MOE_SRC_CODES: already-quantised blocks: q[mat] host uint8
 *                         [E][rows][cols] (one code per weight, each <= the
 *                         largest code of the expert's tier), d[mat], m[mat]
 *                         host fp16 bit patterns [E][rows][cols/32].  For a
 *                         matrix whose table is MXFP4, q holds E2M1 codes
 *                         (0..15), the low byte of each d entry the block's
 *                         E8M0 byte (in [2, 252]) and m is not read.
 * rows x cols is I x H for MOE_GATE and MOE_UP, H x I for MOE_DOWN. */
typedef struct {
  int32_t kind;
  const float* w[3];
  const uint8_t* q[3];
  const uint16_t* d[3];
  const uint16_t* m[3];
} moe_expert_source;

/* Size in bytes of one tier table: `which` = MOE_CODES or MOE_DM, for
 * `n_slots` experts at `bits` bits (or MOE_MXFP4) of matrix `mat`.  Returns 0
 * for invalid arguments. */
size_t moe_tier_table_bytes(const moe_dims* dims, int32_t bits, int32_t n_slots,
                            int32_t mat, int32_t which);

/* A0 -- build the popularity tiers and (optionally) pack the expert tables.
 *
 * Ranks experts by popularity[e] (descending; equal counts -> lower id first)
 * and assigns ranks [0, n_slots[0]) to tier 0, the next n_slots[1] to tier 1,
 * the rest to tier 2; slot = rank - first rank of the tier, so each table is
 * stored hottest-first ([P1] "step 4: three shelves, all on the GPU": experts
 * reordered hottest-first, more bits for the busiest; [P2] "Lever 2").
 *
 *   popularity      host [E] usage counts.
 *   n_slots, tier_bits  as in moe_layer.  The down matrices are packed at
 *                   dst->down_bits[t] where dst is given and that is non-zero.
 *   src             host expert weights, or NULL to compute only the map.
 *   tier_map_out    host [E] int32: tier << 16 | slot.
 *   slot_expert_out host [E] int32: expert id at each rank, or NULL.
 *   dst             tables to fill, or NULL.  If dst_on_device != 0, dst's
 *                   codes/dm pointers and dst->tier_map are device buffers of
 *                   moe_tier_table_bytes() / E*4 bytes (a tier's codes/dm may
 *                   instead be pinned host memory mapped into the device's
 *                   address space, see moe_layer); the call packs on the
 *                   host, copies on `stream` and synchronises it.  If
 *                   dst_on_device == 0 they are host buffers and no HIP call
 *                   is made (dst->tier_map may then be NULL).
 *
 * Quantiser (MOE_SRC_F32), per block of 32 weights, each step one IEEE
 * rounding to nearest-even: lo/hi = min/max; m = f16(lo);
 * d = f16(f32(f32(hi - lo) / L)); q = clamp(rint(f32(f32(x - m) / d)), 0, L),
 * q = 0 when d == 0; L = 2^bits - 1.  MXFP4 blocks: X = floor(log2(max|x|))
 * - 2 clamped to [-125, 125] (X = -125 for an all-zero block), each q the
 * E2M1 code nearest to x / 2^X (exact), ties to the even mantissa, magnitudes
 * above 6 saturating to 6, zero stored as code 0.  Non-finite weights, a
 * scale or min that overflows fp16, or (MOE_SRC_CODES) a code above L or an
 * E8M0 byte outside [2, 252] return MOE_EINVAL.
 * Synchronous; not capturable. */
int moe_build_tiers(const moe_dims* dims, const uint64_t* popularity,
                    const int32_t n_slots[3], const int32_t tier_bits[3],
                    const moe_expert_source* src, int32_t* tier_map_out,
                    int32_t* slot_expert_out, moe_layer* dst, int32_t dst_on_device,
                    hipStream_t stream);

/* Tier sizes for a memory budget ([P1] "step 4: three shelves, all on the
 * GPU": the re-packer's planner fills a memory budget, each byte going where
 * it removes the most expected error; "reproduce it" passes the budget).
 *
 * Chooses n_slots (sum E) for moe_build_tiers: experts in popularity rank
 * order (as moe_build_tiers ranks them) fill tier 0, then tier 1, then tier
 * 2.  The expert tables (three matrices per expert, 3*H*I/32 blocks of
 * 4*bits + 4 bytes) must take at most budget_bytes.  Among such plans the one
 * of least expected error is returned, the error of an expert at b bits
 * being popularity * (2^b - 1)^-2 (a uniform b-bit quantiser's mean square
 * error over a block's range, up to a common factor); on equal error, more
 * experts in tier 0, then in tier 1.  With tier widths that do not increase
 * from tier 0 to tier 2, no assignment of widths to experts does better.
 * Host only, exact integer arithmetic.
 *
 *   popularity   host [E] usage counts.   tier_bits  each in {2, 3, 4}
 *                (MOE_MXFP4 is rejected: its error is not a function of a
 *                width, so the model above does not cover it).
 *   n_slots_out  host [3] (out).
 * Returns MOE_EINVAL for invalid arguments or when no plan fits the budget.
 * The plan sizes every matrix at its tier's width (no down ladder). */
int moe_plan_tiers(const moe_dims* dims, const uint64_t* popularity,
                   const int32_t tier_bits[3], uint64_t budget_bytes,
                   int32_t n_slots_out[3]);

/* moe_plan_tiers with the down matrices on their own ladder, as the pages'
 * re-packer plans with separate gate/up and down format lists ([P1] "step 4:
 * three shelves, all on the GPU" and its command line).  down_bits[t] in
 * {2, 3, 4}, or 0 for tier_bits[t]; NULL: no ladder (moe_plan_tiers).  An
 * expert of tier t costs two matrices at tier_bits[t] and one at its down
 * width (each H*I/32 blocks of 4*bits + 4 bytes), and its error is the sum
 * of the three matrices' errors under the model above.  Same ranking, search,
 * tie rule and errors as moe_plan_tiers; MOE_MXFP4 is rejected in either
 * list. */
int moe_plan_tiers_ladder(const moe_dims* dims, const uint64_t* popularity,
                          const int32_t tier_bits[3], const int32_t down_bits[3],
                          uint64_t budget_bytes, int32_t n_slots_out[3]);

/* A1-A2 -- router scores, top-K and mixing weights for T tokens.
 *
 * key[t][e] = x[t] . w_router[e] + b[e] accumulated in float64 (all inputs
 * are exact in float64); the K best experts per token in rank order
 * (key descending, lower id first on equal keys, NaN last, -0 == +0) go to
 * topk_ids[t][k], and topk_w[t][k] = exp(key_k - key_0) / sum_j exp(key_j -
 * key_0) over the K selected keys (float64, stored fp32).  The router picks
 * the best 10 of 512 experts per token ([P1] "a small dictionary before we
 * start"; [P2] "The Bottleneck").
 *
 *   x         device [T][H] act dtype.
 *   topk_ids  device [T][K] int32 (out).   topk_w device [T][K] fp32 (out).
 * T == 0 is a no-op.  For bf16 and more than 16 tokens the keys are first
 * formed in fp32 with MFMA and only the candidates within the fp32 error
 * bound of the K-th key are rescored in float64; the result is identical. */
int moe_route(const moe_dims* dims, const moe_layer* layer, const void* x, int32_t T,
              int32_t* topk_ids, float* topk_w, void* ws, size_t* ws_bytes,
              hipStream_t stream);

/* A1-A3, A5-A6 -- the layer for a few tokens (decode, speculative verify).
 *
 * y[t] = sum_k topk_w[t][k] * FFN_{ids[t][k]}(x[t]) + FFN_shared(x[t]),
 * FFN(x) = W_d h, h = act(silu(W_g x) * (W_u x)) -- the chosen experts'
 * results add up ([P1] "step 4: three shelves, all on the GPU") with one
 * always-on shared expert ([P5] "What the model actually is").  The
 * contractions accumulate in fp32 on dequantised weights; h is rounded to the
 * act dtype.  One routing decision reaches every tier through tier_map.
 * Tokens are processed in groups of up to 16; each group streams the union
 * of its experts once.  Deterministic (no atomics).
 *
 *   x         device [T][H] act dtype.
 *   y         device [T][H], dtype y_dt (MOE_F32 or the act dtype).
 *   topk_ids, topk_w  optional device outputs [T][K] (may be NULL).
 * T == 0 is a no-op. */
int moe_forward_decode(const moe_dims* dims, const moe_layer* layer, const void* x,
                       int32_t T, void* y, int32_t y_dt, int32_t* topk_ids,
                       float* topk_w, void* ws, size_t* ws_bytes, hipStream_t stream);

/* moe_forward_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result and launches as
 * moe_forward_decode, which it shares its kernels with; the workspace is a
 * library-owned device array of MOE_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * created with the library's code object on each GPU it runs on and held
 * until the process ends.  The call itself allocates nothing.
 *
 * Returns MOE_ENOSPC (nothing launched) when the layer's decode workspace
 * (moe_forward_decode with ws == NULL reports its size) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES; about 0.27 MB for the full-size layer of 512
 * experts, top-10, intermediate 512.  Every call on one GPU uses the same
 * array and leaves its contents behind (no call needs them cleared): calls
 * that may overlap on one GPU -- concurrent streams, or host threads -- race
 * and must be ordered by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int moe_forward_decode_noalloc(const moe_dims* dims, const moe_layer* layer, const void* x,
                               int32_t T, void* y, int32_t y_dt, int32_t* topk_ids,
                               float* topk_w, hipStream_t stream);

/* A1-A2, A4, A7-A8 -- the layer for many tokens (prefill).
 *
 * Same function as moe_forward_decode.  T * H and T * K * I must each stay
 * below 2^31 (the routed GEMMs gather token rows with 32-bit element
 * offsets): MOE_EUNSUPPORTED otherwise, before any launch or workspace
 * query.  Routes r = t*K + k are grouped by
 * expert with a stable counting sort (expert_offsets[E+1] exclusive prefix
 * of per-expert counts; sorted_routes[T*K] the routes of expert e at
 * offsets[e]..offsets[e+1] in ascending r), the grouping the batched path
 * needs ([P1] "the four bugs, briefly").  Each expert's bucket then runs a
 * grouped GEMM on bf16 MFMA (fp32 MFMA for f32 activations) with weights
 * dequantised on the fly; the down projection writes one fp32 row per route,
 * and each token's K rows are then added in rank order, weighted by topk_w,
 * on top of the shared expert's output.  Deterministic (no atomics).
 *
 *   topk_ids, topk_w, expert_offsets, sorted_routes: optional device outputs
 *   (may be NULL).
 * T == 0 is a no-op. */
int moe_forward_prefill(const moe_dims* dims, const moe_layer* layer, const void* x,
                        int32_t T, void* y, int32_t y_dt, int32_t* topk_ids,
                        float* topk_w, int32_t* expert_offsets, int32_t* sorted_routes,
                        void* ws, size_t* ws_bytes, hipStream_t stream);

/* Checks a layer before use: the arguments as the forward calls check them,
 * then the device tier map (copied on `stream`, which is synchronised): every
 * entry must name a slot of its tier (tier in 0..2, slot < n_slots[tier]) and
 * no slot may be named twice.  The forward calls read the tier map on the
 * device and cannot report a bad entry: an expert whose entry is out of range
 * contributes nothing to the output (it is skipped; no table is read out of
 * bounds).  moe_build_tiers always writes a valid map; callers that fill
 * tier_map themselves run this check once after loading.  Returns MOE_OK,
 * MOE_EINVAL (bad map or argument) or MOE_EHIP.  Synchronous; not
 * capturable. */
int moe_check_layer(const moe_dims* dims, const moe_layer* layer, hipStream_t stream);

/* Kernels of the library, as reported by the launch trace. */
typedef enum {
  MOE_K_ROUTER_KEYS = 1,           /* A1: float64 router GEMV                   */
  MOE_K_TOPK = 2,                  /* A2: top-K + weights, many tokens          */
  MOE_K_TOPK_ITEMS = 3,            /* A2+A3: top-K + decode work items          */
  MOE_K_DECODE_GATEUP = 4,         /* A5: decode gate/up + SwiGLU               */
  MOE_K_DECODE_DOWN = 5,           /* A6: decode down + combine                 */
  MOE_K_SORT_COUNT = 6,            /* A4: per-chunk expert masks                */
  MOE_K_SORT_SCAN = 7,             /* A4: bucket offsets                        */
  MOE_K_SORT_SCATTER = 8,          /* A4: stable scatter                        */
  MOE_K_PREFILL_GATEUP = 9,        /* A7: routed grouped gate/up GEMM           */
  MOE_K_PREFILL_SHARED_GATEUP = 10,/* A7: shared expert gate/up GEMM            */
  MOE_K_PREFILL_SHARED_DOWN = 11,  /* A8: shared expert down GEMM (initialises) */
  MOE_K_PREFILL_DOWN = 12,         /* A8: routed down GEMM, fp32 row per route  */
  MOE_K_ROUTER_APPROX = 13,        /* A1: bf16 MFMA router keys (approximate)   */
  MOE_K_TOPK_RECHECK = 14,         /* A1+A2: float64 rescoring + exact top-K    */
  MOE_K_COMBINE = 15               /* A8: shared + weighted routed rows -> y    */
} moe_kernel_id;

/* Launch trace, for measurement harnesses (not part of the computation).
 * While installed, every kernel this library launches on a stream that is
 * not being captured into a graph carries events[2i] and events[2i+1] as the
 * start and stop events of its dispatch (hipExtLaunchKernel: they time the
 * kernel's own execution), with i = (*n_used)++ and tags[i] set to its
 * moe_kernel_id, for the first capacity/2 launches.  Launches captured into
 * a graph are not traced: event-record nodes inside graphs are not available
 * on ROCm.  Events must be created without hipEventDisableTiming.
 * events == NULL removes the trace.  Process-wide, not thread-safe.  Returns
 * MOE_EINVAL for a negative capacity or missing tags / n_used when
 * events != NULL. */
int moe_set_trace(hipEvent_t* events, int32_t* tags, int32_t capacity, int32_t* n_used);

/* Human-readable name of a moe_status value (static string). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
