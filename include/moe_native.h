/*
 * moe_native.h -- C ABI of the capacity-padded, permute-free MoE FFN forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The forward runs in four calls, in this order, on one HIP stream:
 *
 *   moe_route_capacity   top-K softmax routing + fixed-capacity slot selection
 *   moe_align            expert-sorted, block-padded route list and its inverse
 *   moe_grouped_ffn_fwd  gather-in-GEMM FC1 -> SwiGLU*prob -> FC2 (bf16 MFMA)
 *   moe_gather_combine   each token sums its own kept, already-weighted routes
 *
 * moe_route_capacity_align does the first two calls' work in two kernels
 * instead of three (same outputs, bit for bit).
 *
 * The dropless variant ([PF]'s own form: no capacity, every route kept,
 * real extents as device scalars) runs moe_route_dropless,
 * moe_grouped_ffn_fwd_dropless and moe_gather_combine;
 * moe_route_dropless_live in place of the first serves a variable number of
 * tokens from one static shape.  The backward of the fixed-capacity layer is
 * declared at the end.
 *
 * Pages defining the operations (cited by title and section):
 *   [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution"
 *        (NVIDIA-NeMo Automodel pull request 2932), Design notes.
 *   [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)"
 *        (ROCm TransformerEngine pull request 694), sections 2-6.
 *   [BK] "[4/5] feat: capture the FFN experts at bucketed padded shapes"
 *        (vllm-project afd-plugin pull request 335), What this adds.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer, owned by the caller, row-major
 *   and contiguous, 16-byte aligned (MOE_ERR_MISALIGNED otherwise).  The
 *   library keeps no pointer after a call returns.
 * - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 * - A call only enqueues kernels on `stream` (0 = the null stream).  It never
 *   allocates, never synchronises and never reads device memory on the host,
 *   so the four calls can be captured into one hipGraph and replayed.
 * - Arguments are validated on the host from scalars only.  Anything outside
 *   the supported envelope fails closed (no fallback path):
 *       1 <= K <= min(E, 32),  1 <= E <= 1024,  0 <= N <= 16384,
 *       H and I multiples of 64 in [64, 16384],
 *       (the grouped FFN calls of step 4 take any N their 32-bit offsets
 *       allow, (N + 1) * H * 2 < 2^31: after an expert-parallel exchange a
 *       rank's received rows exceed the routing envelope),
 *       C = the value moe_source_capacity returns for (N, K, E, F).
 *   N == 0 is a no-op that returns MOE_OK.
 * - After launching, the call maps hipGetLastError() != hipSuccess to
 *   MOE_ERR_LAUNCH.
 * - The layout block BM is a library constant (moe_layout_block_m()); each
 *   expert owns Cp = moe_padded_capacity(C) consecutive slots, and the route
 *   list has R = E*Cp slots in total.
 */
#ifndef MOE_NATIVE_H
#define MOE_NATIVE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* null pointer, negative size, K > E, F <= 0, ... */
    MOE_ERR_UNSUPPORTED = -2,  /* valid, but outside the supported envelope    */
    MOE_ERR_MISALIGNED = -3,   /* a tensor pointer is not 16-byte aligned      */
    MOE_ERR_LAUNCH = -4        /* a kernel launch reported an error            */
} moe_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* [FC] Design notes: source capacity C = ceil(N*K*F/E) slots per expert,
 * evaluated exactly on the binary value of the double F (128-bit integer
 * arithmetic, no float rounding decides the ceiling).
 * Returns C >= 0, or MOE_ERR_INVALID_ARG (< 0) when N < 0, K < 1, E < 1,
 * K > E, or F is not finite and positive; MOE_ERR_UNSUPPORTED when C would
 * exceed 2^31 - 1.  Host-only, no device work. */
int64_t moe_source_capacity(int64_t N, int32_t K, int32_t E, double F);

/* Layout block BM: the number of slots in one route-list block ([PF]
 * section 4, block_size_m).  Constant 32 (one 32x32 MFMA M-extent). */
int32_t moe_layout_block_m(void);

/* Per-expert segment length Cp = C rounded up to a multiple of BM
 * (< 0 if C < 0).  Host-only. */
int64_t moe_padded_capacity(int64_t C);

/* Dropless variant ([PF] section 4): slots of the route list when every
 * route is kept, N*min(K,E) + E*(BM-1) rounded up to a whole block -- the
 * static length of sorted_slot_ids, slot_probs, act and route_out; the
 * dropless expert_ids has (this)/BM entries.  <0 on bad arguments. */
int64_t moe_dropless_bound(int64_t N, int32_t K, int32_t E);

/* Workspace of the routing calls (moe_route_capacity, moe_route_capacity_align,
 * moe_route_dropless, moe_route_dropless_live): the routing map ([PF]
 * section 4 builds the layout from the routing map), expert-major with rows
 * of Np = N rounded up to a multiple of 16 tokens -- first E*Np bytes, byte
 * [e*Np + t] = k+1 when token t's pick k is expert e, else 0; then E*Np
 * float32 words holding each pick's probability at the same position.
 * Returns 5*E*Np, or 0 when the arguments fall outside the routing envelope.
 * Host-only.  The workspace is a device buffer of at least this many bytes,
 * 16-byte aligned, owned by the caller; each call overwrites it (its
 * contents between calls mean nothing), so calls that share one workspace
 * must not overlap. */
size_t moe_route_capacity_workspace_bytes(int64_t N, int32_t E, int32_t K);

/* Steps 1-2: top-K softmax routing and fixed-capacity drop-and-pad
 * selection ([FC] Design notes; [PF] section 4, route_counts/route_within).
 *
 *   logits       in   float32 [N, E]  router logits
 *   topk_ids     out  int32   [N, K]  chosen experts, descending logit;
 *                                     equal logits -> lower expert first
 *   topk_probs   out  float32 [N, K]  softmax over the K chosen logits:
 *                                     float64 exp(l_k - l_0), summed in k
 *                                     order, divided, rounded once to fp32
 *   route_slot   out  int32   [N, K]  slot of route (t,k) inside its expert's
 *                                     segment, or -1 if the route is dropped
 *   expert_count out  int32   [E]     kept routes per expert = min(C, load)
 *   workspace    scratch               moe_route_capacity_workspace_bytes(N, E, K)
 *                                     bytes (MOE_ERR_INVALID_ARG if null or
 *                                     smaller, MOE_ERR_MISALIGNED if not
 *                                     16-byte aligned)
 *
 * Per expert, the min(C, load) routes with the largest topk_probs are kept
 * (equal probabilities: lower token first); kept routes take slots
 * 0..count-1 in ascending token order. */
int moe_route_capacity(const float* logits, int64_t N, int32_t E, int32_t K, int64_t C,
                       int32_t* topk_ids, float* topk_probs, int32_t* route_slot,
                       int32_t* expert_count, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Step 3: sync-free align ([PF] section 4, Data structures; section 5,
 * route_list_align), fixed-capacity form: expert e owns slots
 * [e*Cp, (e+1)*Cp).
 *
 *   topk_ids, topk_probs, route_slot [N, K], expert_count [E]   in (step 1-2)
 *   sorted_slot_ids        out int32   [E*Cp]  slot -> token row to gather;
 *                                              N (sentinel) for pad slots
 *   slot_probs             out float32 [E*Cp]  routing probability; +0.0 at pads
 *   expert_ids             out int32   [E*Cp/BM]  expert owning each block
 *   block_start            out int32   [E]     first block of each expert
 *   token_routes           out int32   [N, K]  slot of route (t,k), -1 if dropped
 *   token_route_count      out int32   [N]     kept routes of each token
 *   num_tokens_post_padded out int32   [1]     E*Cp, written as a device scalar
 */
int moe_align(const int32_t* topk_ids, const float* topk_probs, const int32_t* route_slot,
              const int32_t* expert_count, int64_t N, int32_t E, int32_t K, int64_t C,
              int32_t* sorted_slot_ids, float* slot_probs, int32_t* expert_ids,
              int32_t* block_start, int32_t* token_routes, int32_t* token_route_count,
              int32_t* num_tokens_post_padded, hipStream_t stream);

/* Steps 1-3 in one call: moe_route_capacity followed by moe_align, with the
 * selection workgroup of each expert writing its own segment of the route
 * list and the token_routes entries of its routes (sources as above).  Same
 * arguments as the two calls together (with moe_route_capacity's
 * workspace), same outputs bit for bit; the
 * per-token kept counts are accumulated with integer atomics (order-free),
 * so the result is deterministic. */
int moe_route_capacity_align(const float* logits, int64_t N, int32_t E, int32_t K, int64_t C,
                             int32_t* topk_ids, float* topk_probs, int32_t* route_slot,
                             int32_t* expert_count, int32_t* sorted_slot_ids, float* slot_probs,
                             int32_t* expert_ids, int32_t* block_start, int32_t* token_routes,
                             int32_t* token_route_count, int32_t* num_tokens_post_padded,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_route_capacity_align without a workspace argument, for callers that
 * cannot allocate device memory (code under hipGraph capture, tight serving
 * loops, harnesses that forbid allocation): the routing map lives in a
 * scratch array the library holds on each device it runs on, 16 MiB, until
 * the process ends.  Same arguments (minus the workspace), same outputs bit
 * for bit.  MOE_ERR_UNSUPPORTED when the map would not fit the array, i.e.
 * moe_route_capacity_workspace_bytes(N, E, K) > 16 MiB (the DeepSeek-style
 * layer, N=8192 and E=256, needs 10 MiB); MOE_ERR_LAUNCH if the array's
 * address cannot be resolved on the current device.  Every call on one
 * device shares that device's array: calls that overlap on one device (two
 * streams, two host threads) race and must be ordered by the caller.  Calls
 * no allocating routine. */
int moe_route_capacity_align_noalloc(const float* logits, int64_t N, int32_t E, int32_t K,
                                     int64_t C, int32_t* topk_ids, float* topk_probs,
                                     int32_t* route_slot, int32_t* expert_count,
                                     int32_t* sorted_slot_ids, float* slot_probs,
                                     int32_t* expert_ids, int32_t* block_start,
                                     int32_t* token_routes, int32_t* token_route_count,
                                     int32_t* num_tokens_post_padded, hipStream_t stream);

/* Dropless variant of steps 1-3 ([PF] sections 4-5: route_list_scan and
 * route_list_align over the routing map, with no capacity): top-K routing as
 * in moe_route_capacity, then every route is kept.
 *
 *   logits               in   float32 [N, E]
 *   topk_ids, topk_probs out  [N, K]   as in moe_route_capacity
 *   route_within         out  int32   [N, K]  rank of route (t,k) among its
 *                                     expert's routes, in token order
 *   route_counts         out  int32   [E]     routes per expert
 *   sorted_slot_ids      out  int32   [Rd]    Rd = moe_dropless_bound(N, K, E).
 *                                     Expert e's routes fill slots
 *                                     block_start[e]*BM + rank; each expert's
 *                                     segment is padded to a multiple of BM;
 *                                     segments follow in expert order; pad
 *                                     slots and the tail past the extent hold
 *                                     the sentinel N
 *   slot_probs           out  float32 [Rd]    probability; +0.0 at pads and tail
 *   expert_ids           out  int32   [Rd/BM] owning expert of each block up
 *                                     to the extent, -1 past it
 *   block_start          out  int32   [E]     first block of each expert
 *   token_routes         out  int32   [N, K]  slot of route (t,k) (never -1)
 *   token_route_count    out  int32   [N]     K
 *   num_tokens_post_padded out int32  [1]     the real extent (sum of the
 *                                     padded segments), a device scalar
 *
 * Within-expert order (token order) and the pad contents follow the
 * fixed-capacity form.  Same validation and workspace as moe_route_capacity
 * (no C). */
int moe_route_dropless(const float* logits, int64_t N, int32_t E, int32_t K, int32_t* topk_ids,
                       float* topk_probs, int32_t* route_within, int32_t* route_counts,
                       int32_t* sorted_slot_ids, float* slot_probs, int32_t* expert_ids,
                       int32_t* block_start, int32_t* token_routes, int32_t* token_route_count,
                       int32_t* num_tokens_post_padded, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* moe_route_dropless for a variable number of live tokens, read on the
 * device: [BK] "What this adds" (one shape is captured and every smaller
 * work item runs in it, its grouping taken from device-side counts).
 *
 *   n_live  in  int32 [1]  device scalar, clamped to [0, N]: tokens
 *                          t < n_live are routed exactly as
 *                          moe_route_dropless routes the first n_live rows
 *                          alone; tokens t >= n_live route nowhere
 *                          (topk_ids -1, topk_probs 0, token_routes -1,
 *                          token_route_count 0; route_within unspecified) and
 *                          their logits are not read.
 *
 * Every other argument, output and bound is moe_route_dropless's with N the
 * capacity of the buffers (the static shape a captured graph was built at;
 * pad slots hold that N as their sentinel row, since rows n_live..N-1 of
 * the caller's x are real rows with stale contents):
 * the route list, block map and extent then describe the live tokens only,
 * so the dropless FFN and the combine do work for them alone and write zero
 * rows of y for the rest.  A null n_live is MOE_ERR_INVALID_ARG. */
int moe_route_dropless_live(const float* logits, int64_t N, int32_t E, int32_t K,
                            const int32_t* n_live, int32_t* topk_ids, float* topk_probs,
                            int32_t* route_within, int32_t* route_counts,
                            int32_t* sorted_slot_ids, float* slot_probs, int32_t* expert_ids,
                            int32_t* block_start, int32_t* token_routes,
                            int32_t* token_route_count, int32_t* num_tokens_post_padded,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step 4 over the dropless route list: the same FC1 -> SwiGLU*prob -> FC2
 * as moe_grouped_ffn_fwd, with expert e's rows the slots
 * [block_start[e]*BM, block_start[e+1]*BM) (the last expert's end is
 * num_tokens_post_padded); the tile count is taken from these device values,
 * so nothing is read back to the host.  act [Rd, I] and route_out [Rd, H]
 * (Rd = moe_dropless_bound(N, K, E)); rows past the extent are left
 * unwritten and are never read by the combine.  Inputs as in
 * moe_grouped_ffn_fwd; K only sizes Rd. */
int moe_grouped_ffn_fwd_dropless(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                                 const int32_t* sorted_slot_ids, const float* slot_probs,
                                 const int32_t* block_start, const int32_t* num_tokens_post_padded,
                                 int64_t N, int32_t H, int32_t I, int32_t E, int32_t K,
                                 uint16_t* act, uint16_t* route_out, hipStream_t stream);

/* moe_grouped_ffn_fwd_dropless as its two GEMM launches (for callers that
 * schedule or time them separately); same arguments, same results. */
int moe_grouped_fc1_swiglu_dropless(const uint16_t* x, const uint16_t* w1,
                                    const int32_t* sorted_slot_ids, const float* slot_probs,
                                    const int32_t* block_start,
                                    const int32_t* num_tokens_post_padded, int64_t N, int32_t H,
                                    int32_t I, int32_t E, int32_t K, uint16_t* act,
                                    hipStream_t stream);
int moe_grouped_fc2_dropless(const uint16_t* act, const uint16_t* w2, const int32_t* block_start,
                             const int32_t* num_tokens_post_padded, int64_t N, int32_t H,
                             int32_t I, int32_t E, int32_t K, uint16_t* route_out,
                             hipStream_t stream);

/* Step 4: permute-free grouped FFN ([PF] sections 2-3 and 6).
 *
 *   x          in  bf16 [N, H]      token-order activations, never permuted
 *   w1         in  bf16 [E, 2I, H]  FC1; rows 0..I-1 gate, rows I..2I-1 up
 *   w2         in  bf16 [E, H, I]   FC2
 *   sorted_slot_ids, slot_probs [E*Cp]   in (step 3)
 *   act        out bf16 [E*Cp, I]   silu(x_r W1g^T) * (x_r W1u^T) * prob,
 *                                   r = sorted_slot_ids[s]; a transient that
 *                                   FC2 consumes
 *   route_out  out bf16 [E*Cp, H]   act W2^T per slot (already weighted)
 *
 * FC1 gathers its A rows through sorted_slot_ids inside the tile loads (the
 * sentinel row N reads as zeros); FC2 reads act by route position.  bf16
 * MFMA with float32 accumulation; the SwiGLU and the probability are applied
 * in FC1's epilogue.  Pad-slot rows of act and route_out come out as zeros. */
int moe_grouped_ffn_fwd(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                        const int32_t* sorted_slot_ids, const float* slot_probs,
                        int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                        uint16_t* act, uint16_t* route_out, hipStream_t stream);

/* Step 4 as its two GEMM launches, for callers that schedule or time them
 * separately ([PF] section 3: one align drives FC1 and FC2, a direction flag
 * selects how A is read).  moe_grouped_ffn_fwd == moe_grouped_fc1_swiglu
 * followed by moe_grouped_fc2 on the same stream, bit for bit.  Arguments,
 * layouts and checks as in moe_grouped_ffn_fwd. */
int moe_grouped_fc1_swiglu(const uint16_t* x, const uint16_t* w1, const int32_t* sorted_slot_ids,
                           const float* slot_probs, int64_t N, int32_t H, int32_t I, int32_t E,
                           int64_t C, uint16_t* act, hipStream_t stream);
int moe_grouped_fc2(const uint16_t* act, const uint16_t* w2, int64_t N, int32_t H, int32_t I,
                    int32_t E, int64_t C, uint16_t* route_out, hipStream_t stream);

/* FC2 with a row map: slot s's output row goes to route_out[out_rows[s]]
 * instead of route_out[s] (same products, same bits).  For an
 * expert-parallel rank: with out_rows the inverse of the receive-order route
 * list, route_out leaves FC2 already in the source-major chunks the return
 * all-to-all sends ([FC] Design notes: every chunk C rows per expert), with
 * no reorder pass.
 *   out_rows  in int32 [E*Cp]; an entry outside [0, E*Cp) drops that row.
 *             Entries should name distinct rows (a repeated row receives one
 *             of its slots' results); rows no entry names are left as they were.
 * Other arguments as moe_grouped_fc2; additionally E*Cp*H*2 must stay below
 * 2^31 bytes (MOE_ERR_UNSUPPORTED otherwise). */
int moe_grouped_fc2_rows(const uint16_t* act, const uint16_t* w2, const int32_t* out_rows, int64_t N,
                         int32_t H, int32_t I, int32_t E, int64_t C, uint16_t* route_out,
                         hipStream_t stream);

/* Step 5: contention-free gather-combine ([PF] sections 2 and 5,
 * route_gather_combine): y[t] = bf16( float32 sum over k = 0..K-1 with
 * token_routes[t,k] >= 0 of route_out[token_routes[t,k]] ), summed in k order
 * from +0.0; no atomics, each output row has one writer.
 *
 *   route_out     in  bf16  [R, H] with R = E*Cp (rows indexed by slot)
 *   token_routes  in  int32 [N, K]
 *   y             out bf16  [N, H]
 * R is needed to validate that no route index can fall outside route_out. */
int moe_gather_combine(const uint16_t* route_out, const int32_t* token_routes, int64_t N,
                       int32_t K, int32_t H, int64_t R, uint16_t* y, hipStream_t stream);

/* Dispatch rows for an expert-parallel exchange: the send buffer of a
 * uniform all-to-all, each slot's token row in route order,
 *   rows[s] = x[sorted_slot_ids[s]]   (a zero row where the entry is not a
 *                                      token index in [0, N): the pads)
 * [FC] Design notes: with a fixed capacity every source rank sends exactly
 * C rows per expert, so expert e's segment [e*Cp, (e+1)*Cp) goes whole to
 * the rank that owns e; [PF] section 4: pad slots name the sentinel row N,
 * which carries zeros.  Received rows are already grouped by expert, so a
 * rank runs the grouped FFN on them with the identity route list
 * (sorted_slot_ids[s] = s), and route_out comes back in this same order for
 * moe_gather_combine.  On one GPU this is the whole dispatch side of that
 * exchange except the transfer itself.
 *
 *   x                in  bf16  [N, H] (token order)
 *   sorted_slot_ids  in  int32 [R]    (R = E*Cp; entries range-checked)
 *   rows             out bf16  [R, H], every row written
 * N may exceed the routing envelope (up to INT32_MAX); H a multiple of 64 up
 * to 16384.  R == 0 returns MOE_OK without launching. */
int moe_dispatch_rows(const uint16_t* x, const int32_t* sorted_slot_ids, int64_t N, int32_t H,
                      int64_t R, uint16_t* rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward (training) of the fixed-capacity layer
 *
 * [PF] sections 3, 5 and 6: the forward keeps only the 2I pre-activation;
 * the backward gathers dy through the same route list (FC2 dgrad), recomputes
 * the gated activation and differentiates it together with the route
 * probability, contracts against the transposed weights (FC1 dgrad), reduces
 * the per-route input gradients to token rows with moe_gather_combine, and
 * forms the weight gradients by contracting over each expert's slots (one
 * owner per dW tile, no atomics).  Order, on one stream:
 *
 *   moe_grouped_fc1_swiglu_save   (forward FC1, also storing the pre-activation)
 *   moe_grouped_fc2 + moe_gather_combine   (rest of the forward)
 *   moe_grouped_fc2_dgrad   d_act  = dy[row(s)] @ W2[e]
 *   moe_swiglu_bwd          act (recomputed), d_preact, d_prob
 *   moe_grouped_fc1_dgrad   d_a    = d_preact[s] @ W1[e]
 *   moe_gather_combine      dx[t]  = sum over t's kept routes of d_a
 *   moe_grouped_fc2_wgrad   dW2[e] = sum_s dy[row(s)]^T act[s]
 *   moe_grouped_fc1_wgrad   dW1[e] = sum_s d_preact[s]^T x[row(s)]
 *   moe_route_bwd           d_logits through the top-K softmax
 *
 * row(s) = sorted_slot_ids[s]; pad slots (row N) contribute nothing.  All
 * bf16 results are rounded once (nearest-even) from float32 accumulators.
 * The sizes and envelope are the forward's (N, H, I, E, C as there, R = E*Cp);
 * outputs are fully overwritten (dW included; the _accum forms below add
 * into float32 main gradients instead),
 * except that N == 0 or C == 0 is a no-op that leaves every output as it was.
 * ------------------------------------------------------------------------ */

/* moe_grouped_fc1_swiglu that also stores the raw FC1 product
 * h = x[row(s)] @ W1[e]^T as bf16:  preact  out bf16 [R, 2I], row s =
 * [gate (I) | up (I)].  act is the same as moe_grouped_fc1_swiglu's. */
int moe_grouped_fc1_swiglu_save(const uint16_t* x, const uint16_t* w1,
                                const int32_t* sorted_slot_ids, const float* slot_probs,
                                int64_t N, int32_t H, int32_t I, int32_t E, int64_t C,
                                uint16_t* act, uint16_t* preact, hipStream_t stream);

/* FC2 data gradient:  d_act[s] = bf16( dy[row(s)] @ W2[e] ), e = s / Cp.
 *   dy      in  bf16 [N, H]  gradient of y, token order (never permuted)
 *   w2      in  bf16 [E, H, I]
 *   d_act   out bf16 [R, I]  (pad slots: zeros) */
int moe_grouped_fc2_dgrad(const uint16_t* dy, const uint16_t* w2, const int32_t* sorted_slot_ids,
                          int64_t N, int32_t H, int32_t I, int32_t E, int64_t C, uint16_t* d_act,
                          hipStream_t stream);

/* Gated-activation recompute + backward, one pass over R slot rows ([PF]
 * section 6), with g = preact[s, :I], u = preact[s, I:], p = slot_probs[s],
 * sig = sigmoid(g):
 *   act[s]          = bf16( silu(g) * u * p )
 *   d_preact[s, :I] = bf16( d_act * p * u * sig * (1 + g * (1 - sig)) )
 *   d_preact[s, I:] = bf16( d_act * p * silu(g) )
 *   d_prob[s]       = float32 sum over the row of d_act * silu(g) * u
 *   preact in bf16 [R, 2I], d_act in bf16 [R, I], slot_probs in f32 [R];
 *   act out bf16 [R, I], d_preact out bf16 [R, 2I], d_prob out f32 [R]. */
int moe_swiglu_bwd(const uint16_t* preact, const uint16_t* d_act, const float* slot_probs,
                   int64_t R, int32_t I, uint16_t* act, uint16_t* d_preact, float* d_prob,
                   hipStream_t stream);

/* FC1 data gradient, per route:  d_a[s] = bf16( d_preact[s] @ W1[e] ).
 *   d_preact in bf16 [R, 2I], w1 in bf16 [E, 2I, H], d_a out bf16 [R, H].
 * dx follows as moe_gather_combine(d_a, token_routes, ...). */
int moe_grouped_fc1_dgrad(const uint16_t* d_preact, const uint16_t* w1, int64_t N, int32_t H,
                          int32_t I, int32_t E, int64_t C, uint16_t* d_a, hipStream_t stream);

/* FC2 weight gradient:  dW2[e] = bf16( sum over e's slots s of dy[row(s)]^T act[s] ).
 *   dy in bf16 [N, H], act in bf16 [R, I] (moe_swiglu_bwd's recompute),
 *   dw2 out bf16 [E, H, I]. */
int moe_grouped_fc2_wgrad(const uint16_t* dy, const uint16_t* act, const int32_t* sorted_slot_ids,
                          int64_t N, int32_t H, int32_t I, int32_t E, int64_t C, uint16_t* dw2,
                          hipStream_t stream);

/* FC1 weight gradient:  dW1[e] = bf16( sum over e's slots s of d_preact[s]^T x[row(s)] ).
 *   d_preact in bf16 [R, 2I], x in bf16 [N, H], dw1 out bf16 [E, 2I, H]. */
int moe_grouped_fc1_wgrad(const uint16_t* d_preact, const uint16_t* x,
                          const int32_t* sorted_slot_ids, int64_t N, int32_t H, int32_t I,
                          int32_t E, int64_t C, uint16_t* dw1, hipStream_t stream);

/* Weight gradients added into float32 main gradients, for gradient
 * accumulation over micro-batches ([PF] section 5: the weight-gradient GEMM
 * writes bf16 or accumulates into a float32 main gradient inside the kernel):
 *   moe_grouped_fc2_wgrad_accum  main_dw2[e] += sum_s dy[row(s)]^T act[s]
 *   moe_grouped_fc1_wgrad_accum  main_dw1[e] += sum_s d_preact[s]^T x[row(s)]
 * with the same inputs as moe_grouped_fc2_wgrad / moe_grouped_fc1_wgrad;
 * main_dw2 in/out float32 [E, H, I], main_dw1 in/out float32 [E, 2I, H],
 * 16-byte aligned, owned by the caller.  Each element becomes
 * float32(old + sum), sum being the float32 accumulation the bf16 entry
 * points round (so rounding the result of an accumulation into zeros gives
 * their output bit for bit); every element has one writer, no atomics, so
 * the result does not depend on the schedule.  N == 0 or C == 0 leaves
 * main_dw as it is (the sums are zero).  MOE_ERR_UNSUPPORTED also when one
 * expert's float32 gradient (2*I*H*4 bytes) reaches 2 GiB. */
int moe_grouped_fc2_wgrad_accum(const uint16_t* dy, const uint16_t* act,
                                const int32_t* sorted_slot_ids, int64_t N, int32_t H, int32_t I,
                                int32_t E, int64_t C, float* main_dw2, hipStream_t stream);
int moe_grouped_fc1_wgrad_accum(const uint16_t* d_preact, const uint16_t* x,
                                const int32_t* sorted_slot_ids, int64_t N, int32_t H, int32_t I,
                                int32_t E, int64_t C, float* main_dw1, hipStream_t stream);

/* Router-logit gradient through the softmax over each token's top K.  Route
 * (t, k) takes dp = d_prob[token_routes[t, k]] (0 if dropped, or if the index
 * is outside [0, R)); with p = topk_probs[t]:
 *   d_logits[t, topk_ids[t, k]] = p_k * (dp_k - sum_j p_j dp_j), 0 elsewhere.
 *   topk_ids in int32 [N, K], topk_probs in f32 [N, K], token_routes in
 *   int32 [N, K], d_prob in f32 [R]; d_logits out f32 [N, E] (every entry
 *   written). */
int moe_route_bwd(const int32_t* topk_ids, const float* topk_probs, const int32_t* token_routes,
                  const float* d_prob, int64_t N, int32_t E, int32_t K, int64_t R,
                  float* d_logits, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NATIVE_H */
