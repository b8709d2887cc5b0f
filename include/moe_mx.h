/*
 * moe_mx.h -- C ABI of the fused microscaling (MX) mixture-of-experts layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (mxfp6-sm120 page, table of paths, "Routed MoE" row, and its
 * "Execution model" figure; TokenSpeed SiTU page, sections "Activation
 * precision (w4a16 vs w4a8)" and "Supported contract"):
 *   1. softmax/top-k routing of fp32 router logits (or a precomputed top-k);
 *   2. permutation of the T*k (token, slot) assignments by expert;
 *   3. for MXFP8 activations: per-token E4M3 quantization of x with one E8M0
 *      scale per 32 hidden values;
 *   4. FC1: gathered rows times W1 = [gate; up] (MXFP4 E2M1 or MXFP6 E3M2,
 *      one E8M0 scale per 32 along K), fp32 accumulation;
 *   5. h = SiLU(gate) * up (or another gated activation, act_fn) in fp32,
 *      stored as bf16 (bf16 activations) or requantized to MXFP8 along I
 *      (MXFP8 activations);
 *   6. FC2: h times W2, fp32 accumulation;
 *   7. y[t] = sum_j w[t,j] * FC2 output of (t, j), plus an optional shared
 *      expert with its own weight: each weighted expert row is rounded to
 *      bf16, the rows are summed in fp32 and the sum is rounded to bf16
 *      (two roundings; see moe_fused below).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer (inputs, outputs and workspace).  The library
 *     never allocates, frees, synchronizes or reads device memory on the host,
 *     so a call can be captured in a HIP graph.
 *   - Work is enqueued asynchronously on `stream`; results are ready when the
 *     stream reaches that point.
 *   - Errors are returned as moe_status_t; nothing else crosses the ABI.
 *     Arguments are validated on the host before any HIP call: an invalid
 *     argument returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED /
 *     MOE_ERR_WORKSPACE without touching the device.  A device that is not
 *     gfx950 (or no device) gives MOE_ERR_ARCH.  A failed launch gives
 *     MOE_ERR_HIP.
 *   - Device trust boundary: contents of device buffers are not inspected on
 *     the host.  Expert ids outside [0, E), non-finite inputs and NaN scale
 *     codes (255) give unspecified results (but no out-of-bounds access for
 *     ids: ids outside the local shard are skipped).  The k expert ids of one
 *     token must be distinct (moe_route always produces distinct ids); a
 *     precomputed top-k that repeats an id for a token gives an unspecified
 *     output row for that token (still no out-of-bounds access).
 *
 * Canonical MX layouts (element codes along the contraction axis K):
 *   E2M1: two codes per byte, element 2j in bits 0-3, element 2j+1 in bits 4-7;
 *   E3M2: four codes in three bytes, element 4j+i in bits 6i..6i+5 of the
 *         little-endian 24-bit word;
 *   E4M3: one code per byte (OCP E4M3: no infinities, S.1111.111 is NaN);
 *   scales: E8M0 codes 2**(c-127), one per 32 consecutive K elements, stored
 *         row-major [rows, K/32].
 */
#ifndef MOE_MX_H
#define MOE_MX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, k > E, bad enum, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (tile multiples, format combination) */
  MOE_ERR_WORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes() */
  MOE_ERR_ARCH = 4,         /* no device, or the current device is not gfx950 */
  MOE_ERR_HIP = 5           /* a HIP launch or runtime call failed */
} moe_status_t;

/* MX element formats; the scale is always E8M0, one per 32 elements along K. */
typedef enum { MX_E2M1 = 1, MX_E3M2 = 2, MX_E4M3 = 3 } mx_elem_t;

/* Source dtype for mx_quantize. */
typedef enum { MOE_SRC_BF16 = 0, MOE_SRC_FP32 = 1 } moe_src_t;

/* Activation precision of the layer (TokenSpeed SiTU page, "Activation
 * precision"): bf16 activations (w4a16) or MXFP8 E4M3 activations (w4a8 /
 * w6a8) quantized on the device. */
typedef enum { MOE_ACT_BF16 = 0, MOE_ACT_MXFP8 = 1 } moe_act_t;

/* Gated activation applied to FC1's gate half g and up half u (b12x page,
 * "What's in here", MoE: SiLU, ReLU2 and SwiGLU-OAI activations), in fp32:
 *   MOE_FN_SILU        SiLU(g) * u = g / (1 + exp(-g)) * u   (default)
 *   MOE_FN_RELU2       max(g, 0)^2 * u
 *   MOE_FN_SWIGLU_OAI  (clamp(u, -7, 7) + 1) * g' / (1 + exp(-1.702 g')),
 *                      g' = min(g, 7)  (the gpt-oss form) */
typedef enum { MOE_FN_SILU = 0, MOE_FN_RELU2 = 1, MOE_FN_SWIGLU_OAI = 2 } moe_act_fn_t;

/*
 * mx_quantize -- block quantization of a row-major matrix to MX codes.
 *
 * Defines the MX conversion named on the mxfp6-sm120 page ("Execution model":
 * dynamic E4M3 quantization with a UE8M0 scale per 32 K values; packed E3M2
 * weights) and the MXFP4 weights of the TokenSpeed SiTU page.  Per block of 32
 * consecutive elements of a row (OCP MX v1.0 rule):
 *   amax = max|v|; scale code = clamp(floor(log2 amax) - emax, -127, 127) + 127
 *   (emax = 2 for E2M1, 4 for E3M2, 8 for E4M3; amax == 0 gives code 0);
 *   element = v / 2**(code-127) rounded to the nearest element value, ties to
 *   the even code, magnitudes beyond the largest finite one saturate to it;
 *   the sign of v is kept (-0 gives the negative-zero code).
 *
 * src      [rows, cols] elements of `src_dtype`, row stride `src_ld` elements
 *          (src_ld >= cols); values must be finite.
 * codes    [rows, cols*bits/8] bytes (bits = 4, 6, 8), packed as above,
 *          rows contiguous.
 * scales   [rows, cols/32] E8M0 codes, rows contiguous.
 * Requires rows >= 0, cols % 32 == 0, cols > 0.  rows == 0 is a no-op.
 * Output is bit-identical to the reference rule for every finite input.
 */
moe_status_t mx_quantize(const void* src, moe_src_t src_dtype, int64_t rows, int64_t cols,
                         int64_t src_ld, mx_elem_t fmt, uint8_t* codes, uint8_t* scales,
                         hipStream_t stream);

/*
 * moe_route -- softmax/top-k routing and the permutation of assignments by
 * expert (mxfp6-sm120 page, "Execution model": indirect routing; TokenSpeed
 * SiTU page, "Supported contract": global top-k expert ids; fusedtok page:
 * selection ties resolve to the earliest index).
 *
 * logits          [T, E] fp32 router logits (finite or -inf; no NaN).
 * topk_ids        [T, k] int32 out: for each token the k experts with the
 *                 largest logits, larger first, equal logits -> lower id first.
 * topk_w          [T, k] fp32 out: softmax of the k chosen logits (= the full
 *                 softmax renormalised over the chosen experts).
 * expert_offsets  [E+1] int32 out: exclusive prefix sum of per-expert counts.
 * sorted_assign   [T*k] int32 out: assignment ids a = t*k + j ordered by
 *                 (expert, token); segment e is
 *                 sorted_assign[expert_offsets[e] .. expert_offsets[e+1]).
 * workspace       device scratch of at least moe_route_workspace_bytes(T,E,k).
 * Requires 0 <= T, 1 <= k <= E <= 1024.  ids, offsets and sorted_assign are
 * deterministic (no dependence on scheduling).
 */
size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k);
moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_gemm -- dense MX GEMM with bf16 output (mxfp6-sm120 page, table of
 * paths, "Dense" row; "Execution model" figure: bf16 activations quantized
 * on the device to E4M3 with one UE8M0 scale per 32 K values, packed MX
 * weights with one UE8M0 scale per 32 K values, FP32 accumulation, bf16
 * output; "Validated scope": M > 0, N % 8 == 0, K % 128 == 0).
 *
 *   C[m, n] = bf16_RNE(alpha * sum_k A'[m, k] * W'[n, k])   (fp32 accumulation)
 *
 * a        act == MOE_ACT_BF16: [M, K] bf16, rows contiguous; multiplied as
 *          given (W4A16 / W6A16).
 *          act == MOE_ACT_MXFP8 and a_scale == NULL: [M, K] bf16, quantized
 *          on the device to E4M3 + E8M0 per 32 along K into the workspace
 *          (W4A8 / W6A8), exactly as mx_quantize does.
 *          act == MOE_ACT_MXFP8 and a_scale != NULL: [M, K] E4M3 codes with
 *          scales a_scale [M, K/32] (e.g. from mx_quantize); no workspace.
 * w, w_scale  [N, K*b/8] packed codes and [N, K/32] E8M0 scales of w_fmt
 *          (MX_E2M1 or MX_E3M2), the canonical layout above.
 * c        [M, N] bf16 out, rows contiguous.
 * workspace   mx_gemm_workspace_bytes(M, N, K, act, w_fmt) bytes, 256-byte
 *          aligned; contents need not be set.  It holds the quantized A
 *          (MXFP8 from bf16; required), or, for few rows of bf16 A against
 *          E2M1 weights (M < 32), the fp32 partial sums of a K split over
 *          more workgroups (optional: with less workspace the GEMM runs
 *          unsplit, with the same result up to the fp32 summation order).
 *          The split's partial sums are added in a fixed order, so the
 *          result stays deterministic.
 * Requires M >= 0 (0: no-op), K % 32 == 0, 16-byte aligned a, c, w (and
 * a_scale if given); N % 8 != 0, K % 128 != 0 or E4M3 weights give
 * MOE_ERR_UNSUPPORTED.  Deterministic.
 */
size_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, moe_act_t act, mx_elem_t w_fmt);
moe_status_t mx_gemm(const void* a, const uint8_t* a_scale, int64_t M, int64_t N, int64_t K, moe_act_t act,
                     const uint8_t* w, const uint8_t* w_scale, mx_elem_t w_fmt, float alpha, void* c,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Problem description of one fused MoE layer call. */
typedef struct {
  int32_t T;                   /* tokens (>= 0)                                      */
  int32_t H;                   /* hidden size, K of FC1 and N of FC2 (% 128 == 0)    */
  int32_t I;                   /* expert intermediate size (% 128 == 0)              */
  int32_t E;                   /* global number of experts (1 <= E <= 1024)          */
  int32_t k;                   /* experts per token (1 <= k <= E)                    */
  mx_elem_t w_fmt;             /* MX_E2M1 or MX_E3M2 (weights, routed and shared)   */
  moe_act_t act;               /* MOE_ACT_BF16 or MOE_ACT_MXFP8                      */
  int32_t I_shared;            /* shared-expert intermediate size, 0 = none (% 128)  */
  float shared_weight;         /* weight of the shared expert's output (e.g. 1.0)    */
  int32_t local_expert_offset; /* first expert held by this call (TokenSpeed SiTU    */
  int32_t local_num_experts;   /* page, "Supported contract"); 0 means all E         */
  moe_act_fn_t act_fn;         /* gated activation of every expert (0 = SiLU)       */
  uint32_t flags;              /* MOE_FLAG_* (0: defaults)                           */
} moe_problem_t;

/* Flags of moe_problem_t.
 * MOE_FLAG_FUSED_SMALL_BATCH: run the two-launch small-batch path (the
 *   mxfp6-sm120 page, "Execution model", gives small batches a path of their
 *   own with allocation-free routing and a fused W2 routed/shared
 *   reduction): every FC1 workgroup routes the batch itself (no routing
 *   launch) and FC2 adds the routed and shared outputs per token in fp32, so
 *   y is ONE bf16 rounding of the whole sum (the default path rounds each
 *   weighted expert row first).  Requires bf16 activations, E2M1 weights,
 *   T <= 8, T*k <= 64, H % 512 == 0, I and I_shared multiples of 256 and
 *   T*(2H+16) + 24 KiB of LDS <= 160 KiB; otherwise MOE_ERR_UNSUPPORTED.
 *   Its kernels load the weights straight into registers; on MI355X they
 *   stream them more slowly than the default path's LDS rings, so this is an
 *   option, not the default. */
#define MOE_FLAG_FUSED_SMALL_BATCH 1u

/* Tensors of one call.  W1/W2 hold only the local experts: expert index
 * local_expert_offset + i is stored at position i. */
typedef struct {
  const void* x;                 /* [T, H] bf16                                          */
  const float* router_logits;    /* [T, E] fp32, or NULL when topk_*_in are given        */
  const int32_t* topk_ids_in;    /* [T, k] optional precomputed global expert ids        */
  const float* topk_w_in;        /* [T, k] optional precomputed routing weights          */
  const uint8_t* w1;             /* [L, 2I, H*b/8]: rows [0, I) gate, [I, 2I) up         */
  const uint8_t* w1_scale;       /* [L, 2I, H/32]                                        */
  const uint8_t* w2;             /* [L, H, I*b/8]                                        */
  const uint8_t* w2_scale;       /* [L, H, I/32]                                         */
  const uint8_t* ws1;            /* shared expert [2*I_shared, H*b/8] (NULL if none)     */
  const uint8_t* ws1_scale;      /* [2*I_shared, H/32]                                   */
  const uint8_t* ws2;            /* [H, I_shared*b/8]                                    */
  const uint8_t* ws2_scale;      /* [H, I_shared/32]                                     */
  void* y;                       /* [T, H] bf16 out, overwritten                         */
  int32_t* topk_ids_out;         /* [T, k] optional: routing ids used                    */
  float* topk_w_out;             /* [T, k] optional: routing weights used                */
  const hipEvent_t* stage_events;/* optional [MOE_NUM_STAGES + 1] caller-created events:  */
                                 /* event i is recorded on `stream` when stage i starts, */
                                 /* the last one after the final stage (NULL: none)      */
} moe_tensors_t;

/* Stages of moe_fused, in launch order, for stage_events.  A stage that a
 * problem does not need (x quantization with bf16 activations, the shared
 * expert without one) still records its event and takes no time.  A batch of
 * at most 16 tokens and 128 assignments (k <= 64) with bf16 activations (E2M1
 * weights, router logits given) is routed and permuted inside FC1: the route and
 * permute stages then take no time and FC1's includes them. */
enum {
  MOE_STAGE_ROUTE = 0,     /* top-k routing (or copy of the given top-k)                        */
  MOE_STAGE_PERMUTE = 1,   /* histogram, scan, permutation and tile list                        */
  MOE_STAGE_QUANT_X = 2,   /* MXFP8 quantization of x                                           */
  MOE_STAGE_FC1 = 3,       /* FC1 grouped GEMM + SiLU(gate)*up (+ MXFP8 requantization)         */
  MOE_STAGE_FC2 = 4,       /* FC2 grouped GEMM, routing weight applied, rows in token order     */
  MOE_STAGE_SHARED = 5,    /* shared expert FC1 + FC2                                           */
  MOE_STAGE_FINALIZE = 6,  /* unpermute-combine: sum over slots (+ shared) -> bf16 y            */
  MOE_NUM_STAGES = 7
};

/*
 * moe_fused -- the whole layer (steps 1-7 above) on `stream`.
 *
 * With local_num_experts < E only assignments to experts in
 * [local_expert_offset, local_expert_offset + local_num_experts) contribute
 * and y is that shard's partial output (the caller sums shards); the shared
 * expert, if any, is added by every call.
 * Precision: FC products accumulate in fp32; each expert's output row is
 * scaled by its routing weight in fp32 and rounded to bf16 (RNE); y is one
 * bf16 rounding of the fp32 sum of those rows taken in slot order
 * j = 0..k-1, then the shared expert's row (scaled and rounded the same way);
 * results are deterministic from run to run.
 * Workspace: at least moe_fused_workspace_bytes(p) bytes, 256-byte aligned.
 * Its contents need not be initialised; nothing in it is read before this
 * call writes it.
 */
size_t moe_fused_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_fused(const moe_problem_t* p, const moe_tensors_t* t, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * moe_fused_workspace_offset -- where moe_fused leaves an intermediate result
 * in its workspace, for inspection after the stream has reached the end of
 * the call (housekeeping: testing and debugging; the layer's steps are those
 * listed at the top of this file).  Returns the byte offset from the start of
 * the workspace, or (size_t)-1 for an invalid problem or a part the problem
 * does not have.  Parts (L = local experts, A = T*k):
 *   MOE_WS_EXPERT_OFFSETS  int32 [L+1]: exclusive prefix sum of the per-local-
 *                          expert assignment counts (step 2);
 *   MOE_WS_SORTED_ASSIGN   int32 [A]: assignment ids t*k + j of the local
 *                          experts ordered by (expert, token); entries from
 *                          offsets[L] on are unused;
 *   MOE_WS_H               the FC2 input of permuted row p (step 5), rows of I
 *                          values: bf16 (bf16 activations) or E4M3 codes
 *                          (MXFP8 activations), [A, I] row-major;
 *   MOE_WS_H_SCALE         E8M0 scales of MOE_WS_H, [A, I/32] (MXFP8 only).
 */
typedef enum {
  MOE_WS_EXPERT_OFFSETS = 0,
  MOE_WS_SORTED_ASSIGN = 1,
  MOE_WS_H = 2,
  MOE_WS_H_SCALE = 3
} moe_ws_part_t;
size_t moe_fused_workspace_offset(const moe_problem_t* p, moe_ws_part_t part);

/*
 * moe_fused_noalloc -- moe_fused for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same problem, tensors and results as moe_fused,
 * without a workspace argument.  Its workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that every device using the library holds until
 * the process ends; the call itself allocates nothing.
 *   - A problem whose moe_fused_workspace_bytes() exceeds the array returns
 *     MOE_ERR_WORKSPACE (e.g. T = 64 at H = 7168, I = 2048, k = 8 needs about
 *     10 MiB).
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents (nothing in it needs to start at zero): calls that
 *     overlap on one device (other streams, other threads) race and must be
 *     serialised by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status_t moe_fused_noalloc(const moe_problem_t* p, const moe_tensors_t* t, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* moe_status_str(moe_status_t s);

/* Library version, "major.minor.patch". */
const char* moe_mx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MX_H */
