/*
 * libmoe - one Mixture-of-Experts layer's expert path on one AMD Instinct
 * MI355X (gfx950): softmax top-k gate, dispatch permutation, grouped SwiGLU
 * expert FFN, gate-weighted combine, and the expert-activation statistics.
 *
 * Where the operations come from (three web summaries of 2026 MoE-serving
 * papers):
 *   ELDR page ("Expert-Locality-Aware Decode Routing for PD-Disaggregated MoE
 *   Serving"), section "What it solves": a decode step reads the weights of
 *   every distinct expert that any token of the batch selected; section "Core
 *   idea / structure / operation": the gate is standard top-k gating, left
 *   unchanged, and each request is summarised by its per-expert top-k
 *   activation counts reweighted by IDF over a subset of layers.
 *   GRACE-MoE page, section 1: every MoE layer dispatches tokens to their
 *   experts and combines the results back; sections 3-4: expert co-activation
 *   (affinity) and per-expert load are read off recorded top-k selections.
 *   ExpertPlex page, "Instance vs module disaggregation": the expert FFN is the
 *   bulk (~95 %) of a MoE layer; "Adaptive Persistent Kernels": expert work is
 *   cut into tiles served from a device-side queue, decode tiles first.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer to a dense, row-major,
 *     contiguous array, 16-byte aligned.  The caller owns all memory; the
 *     library never allocates or frees device memory and keeps no pointer after
 *     the work it enqueued has completed.  Outputs must not alias inputs.
 *   - Each call checks its arguments on the host, enqueues kernels on `stream`
 *     and returns.  No call synchronises, copies device->host or reads device
 *     data on the host; device faults surface at the caller's next sync.
 *   - Errors are returned synchronously as moe_status and nothing is enqueued:
 *       MOE_ERR_INVALID_ARG  negative sizes, k < 1, k > E, n_priority > T,
 *                            NULL required pointer, misaligned pointer
 *       MOE_ERR_UNSUPPORTED  E > 512, n_shared > 256, d or I not a multiple of 8,
 *                            unknown dtype,
 *                            sizes whose element counts overflow int32
 *       MOE_ERR_WORKSPACE    workspace smaller than the queried size
 *       MOE_ERR_HIP          a HIP launch reported an error (after enqueueing)
 *   - T = 0 (no tokens) is valid: outputs with zero elements are untouched;
 *     fixed-size outputs (group offsets, counts, ...) receive their empty-batch
 *     values.
 *   - Workspace query: when `workspace` is NULL, the call stores the number of
 *     bytes it needs in *workspace_bytes, returns MOE_OK and enqueues nothing.
 *     The size depends only on the scalar arguments.  Otherwise
 *     *workspace_bytes is the size of the caller's buffer.
 *   - Calls are reentrant; apart from moe_grouped_ffn_noalloc's per-device
 *     scratch array the library holds no mutable global state.  Two calls that
 *     share a workspace must not overlap in time.
 *   - Expert ids outside [0, E) in an input id array are a precondition
 *     violation: kernels clamp them into range to stay memory safe, the
 *     results are then unspecified.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Largest routed-expert and shared-expert counts the kernels accept. */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_SHARED 256

/*
 * moe_router - router projection in front of the gate: one fp32 score per
 * routed expert and token, logits[t][e] = sum_i x[t][i] * w_router[e][i].
 * (ELDR page, "Core idea / structure / operation": the gate is standard
 * top-k gating over per-expert router scores; the pages do not spell the
 * router out, and it is read as a bias-free linear map of the hidden state.)
 *
 *   x         [T][d] in dtype (bf16 or fp32), read only.
 *   w_router  [E][d] in dtype, read only ([out][in] layout, like the experts).
 *   logits    [T][E] fp32, written; the input of moe_gate.
 *   Accumulation is fp32 in an unspecified order.  bf16 products are exact in
 *   fp32, so an element is within d * 2^-24 * sum_i |x[t][i] w_router[e][i]|
 *   of the exact dot product (fp32 inputs: (d + 1) * 2^-24 * the same sum).
 *   Requires T >= 0, 1 <= E <= 512, d a positive multiple of 8; x, w_router
 *   and logits 16-byte aligned.
 */
moe_status moe_router(const void* x, const void* w_router, int32_t T, int32_t d, int32_t E,
                      moe_dtype dtype, float* logits, hipStream_t stream);

/*
 * moe_gate - softmax top-k gate over fp32 router logits.
 * (ELDR page, "Core idea / structure / operation": standard top-k gating.)
 *
 *   logits   [T][E] fp32, read only.
 *   topk_ids [T][k] int32, written: the k largest logits of each row in
 *            descending order; equal logits go to the lower expert id; -0.0
 *            equals +0.0; NaN ranks as -inf.
 *   topk_w   [T][k] fp32, written: renormalize = 1 -> softmax over the k chosen
 *            logits (the full softmax renormalised over the chosen experts);
 *            renormalize = 0 -> the full-E softmax probability of each chosen
 *            expert.  Weights are computed in double and rounded once.
 *   Requires 1 <= k <= E <= 512, T >= 0.
 */
moe_status moe_gate(const float* logits, int32_t T, int32_t E, int32_t k,
                    int32_t renormalize, int32_t* topk_ids, float* topk_w,
                    hipStream_t stream);

/*
 * moe_gate_record - moe_gate that also records the batch's expert activations
 * per KV block for one layer of a recorded layer stack.
 * (ELDR page, "Core idea / structure / operation": during prefill the expert
 * activations are recorded at KV-block granularity, and a request's signature
 * is built from its blocks' counts.)
 *
 *   logits, T, E, k, renormalize, topk_ids, topk_w: as moe_gate, with the
 *                same results bit for bit.
 *   block_tokens tokens per KV block (>= 1): block b holds tokens
 *                [b * block_tokens, min(T, (b + 1) * block_tokens)); there are
 *                nb = ceil(T / block_tokens) blocks.
 *   layer, L     0 <= layer < L: the row of the record this call fills.
 *   block_counts [nb][L][E] int32: row (b, layer) is written in full, zeros
 *                included: entry e = number of top-k slots of the block's
 *                tokens that chose expert e (moe_stats' req_counts for block
 *                offsets).  Rows of other layers are not touched, so L calls
 *                with layer = 0 .. L-1 fill the whole record; nothing needs
 *                clearing first.
 *   Errors: MOE_ERR_INVALID_ARG for block_tokens < 1, L < 1, layer outside
 *   [0, L), a NULL or misaligned block_counts (T > 0), and moe_gate's
 *   argument errors; otherwise as moe_gate.
 */
moe_status moe_gate_record(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                           int32_t* topk_ids, float* topk_w, int32_t block_tokens, int32_t layer, int32_t L,
                           int32_t* block_counts, hipStream_t stream);

/*
 * moe_stage_to_host - enqueue the copy of `bytes` bytes of device memory into
 * pinned host memory on `stream` (ELDR page, "Core idea / structure /
 * operation" and its overhead measurements: the recorded signatures are
 * staged from the GPU to the host).
 *
 *   src       device memory (for example moe_gate_record's block_counts or
 *             moe_stats' signature), read by the copy.
 *   dst_host  page-locked host memory the caller allocated (hipHostMalloc, or
 *             a pinned torch tensor); written when the copy runs, so the caller
 *             waits on the stream (or an event recorded after the call) before
 *             reading it.  Nothing is allocated.
 *   Errors: MOE_ERR_INVALID_ARG for a NULL pointer with bytes > 0, a
 *   destination that is not page-locked host memory (a pageable buffer would
 *   turn the copy synchronous), or a source that is not device memory;
 *   MOE_ERR_HIP if the copy cannot be enqueued.  bytes = 0 enqueues nothing.
 */
moe_status moe_stage_to_host(const void* src, void* dst_host, size_t bytes, hipStream_t stream);

/*
 * moe_permute - dispatch as a stable counting sort of token->expert
 * assignments into contiguous per-expert groups (histogram, prefix scan,
 * scatter, row gather).  (GRACE-MoE page, section 1: the dispatch exchange.)
 *
 *   Assignments: routed f = t*k + j (expert topk_ids[t][j]) and, for the
 *   n_shared always-on experts, f = T*k + s*T + t (expert E + s).
 *   Group of an assignment: routed g = seg(t)*E + e with seg(t) = 1 when
 *   n_priority > 0 and t >= n_priority, else 0 (the first n_priority tokens form
 *   a priority segment whose groups come first: ExpertPlex page, "Adaptive
 *   Persistent Kernels"); shared g = nseg*E + s with nseg = (n_priority > 0 ? 2
 *   : 1).  G = nseg*E + n_shared groups, N = T*(k + n_shared) assignments.
 *   Assignments are ordered by (g, f).
 *
 *   topk_ids       [T][k] int32, read only, ids in [0, E).
 *   x              [T][d] of `dtype`, or NULL (then no row gather; x_sorted
 *                  is ignored and may be NULL).
 *   group_offsets  [G+1] int32, written: exclusive scan of the group sizes.
 *   sorted_to_flat [N] int32, written: f of the assignment at sorted row n.
 *   flat_to_sorted [N] int32, written: its inverse.
 *   sorted_token   [N] int32 or NULL, written: the token of sorted row n
 *                  (f / k for routed f, (f - T*k) mod T for shared); the row
 *                  index list that lets moe_grouped_ffn read x directly.
 *   x_sorted       [N][d] of `dtype`, written: x_sorted[n] = x[token(f)]
 *                  bit for bit.
 *   workspace      device scratch of the queried size.
 *   Requires 0 <= n_priority <= T, 1 <= k <= E <= 512, n_shared >= 0, d % 8 == 0
 *   when x is given.
 */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                       int32_t n_shared, int32_t n_priority,
                       const void* x, moe_dtype dtype, int32_t d,
                       int32_t* group_offsets, int32_t* sorted_to_flat,
                       int32_t* flat_to_sorted, int32_t* sorted_token, void* x_sorted,
                       void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn - grouped SwiGLU expert FFN over the sorted rows.
 * (ExpertPlex page, "Instance vs module disaggregation": the expert FFN;
 * "Adaptive Persistent Kernels": tiles served from a device-side queue with
 * the priority segment's tiles ahead of the rest.)
 *
 *   For sorted row n of group g (expert e = g mod E for g < nseg*E, else
 *   E + g - nseg*E):
 *     h[n] = W_down[e] . ( silu(W_gate[e] . xs[n]) * (W_up[e] . xs[n]) ).
 *   x_sorted       [n_rows][d] of `dtype` when x_rows is NULL.  Otherwise the
 *                  token matrix [n_x][d] and x_rows [n_rows] int32 names the
 *                  row of it that sorted row n reads (moe_permute's
 *                  sorted_token), so the permutation's row gather is folded
 *                  into the FFN's loads; entries are clamped to [0, n_x).
 *   n_x            rows of x_sorted when x_rows is given (ignored otherwise).
 *   group_offsets  [G+1] int32 with G = nseg*E + n_shared, non-decreasing,
 *                  group_offsets[G] == n_rows (device data: never read on the
 *                  host; the tile list is built on the device).
 *   w_gate, w_up   [E+n_shared][I][d] of `dtype` (nn.Linear [out][in] layout).
 *   w_down         [E+n_shared][d][I] of `dtype`.
 *   h_sorted       [n_rows][d] of `dtype`, written.
 *   Only experts with at least one row are read.  bf16: bf16 operands, fp32
 *   accumulation, the SwiGLU product rounded to bf16 (round to nearest even)
 *   before the down projection.  f32: fp32 throughout.
 *   Requires d % 8 == 0, I % 8 == 0, nseg in {1, 2}, 1 <= E <= 512.
 *   bf16 batches with a priority segment (nseg == 2) whose groups average
 *   more than 48 rows and whose d and I are multiples of 32 run both phases
 *   in one launch of persistent workers that take tiles from device-side
 *   queues, the priority segment's tiles first ("Adaptive Persistent
 *   Kernels (APK)"); other batches run two launches (gate/up, then down).
 *   The 4 bytes at offset (queried workspace size - 4) hold a diagnostic
 *   word once the call has completed: 0, or nonzero if a wait of the
 *   persistent tile queue for a phase-1 tile gave up after its bound (20 ms);
 *   the outputs are then not to be trusted.
 */
moe_status moe_grouped_ffn(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                           const int32_t* group_offsets,
                           int32_t n_rows, int32_t E, int32_t n_shared, int32_t nseg,
                           int32_t d, int32_t I,
                           const void* w_gate, const void* w_up, const void* w_down,
                           moe_dtype dtype, void* h_sorted,
                           void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn_traced - moe_grouped_ffn with a per-tile timeline of the
 * persistent tile queue.
 * (ExpertPlex page, "Adaptive Persistent Kernels (APK)": a decode tile waits at
 * most for the tiles already running; the timeline shows when the priority
 * segment's tiles ran and finished.)
 *
 *   Arguments, results and workspace as moe_grouped_ffn, plus
 *   trace           device buffer of trace_capacity records, 4 uint64 each,
 *                   16-byte aligned; the caller zero-fills it.
 *   trace_capacity  records (>= 0; 0: no trace, exactly moe_grouped_ffn or
 *                   moe_grouped_ffn_packed).
 *   weights_packed  0: w_gate, w_up, w_down in moe_grouped_ffn's layout and
 *                   `dtype`; 1: in moe_grouped_ffn_packed's layout (dtype must
 *                   be MOE_BF16, d and I multiples of 32).
 *   Records are written only on the persistent-queue path, which has nq = 8
 *   queues (block b takes its tiles from queue b mod 8).  Queue q owns records
 *   [q * (trace_capacity / nq), (q + 1) * (trace_capacity / nq)); its tile
 *   popped at position t writes record q * (trace_capacity / nq) + t if
 *   t < trace_capacity / nq:
 *     [0] start and [1] end of the tile, s_memrealtime ticks (100 MHz);
 *     [2] unit << 32 | column chunk << 8 | priority << 1 | (phase - 1)
 *         (a unit is 128 sorted rows of one expert);
 *     [3] queue << 32 | block index.
 *   A record whose end is 0 was not written.  Tracing adds a wait for the
 *   tile's stores before its end stamp.
 *   Errors: MOE_ERR_INVALID_ARG for trace_capacity < 0, a NULL or misaligned
 *   trace with trace_capacity > 0, or weights_packed not 0 or 1;
 *   MOE_ERR_UNSUPPORTED for packed weights with another dtype or with d or I
 *   not multiples of 32; otherwise as moe_grouped_ffn.
 */
moe_status moe_grouped_ffn_traced(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                  const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                  int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                  const void* w_down, moe_dtype dtype, void* h_sorted, void* workspace,
                                  size_t* workspace_bytes, uint64_t* trace, int32_t trace_capacity,
                                  int32_t weights_packed, hipStream_t stream);

/*
 * moe_grouped_ffn_combine - moe_grouped_ffn followed by moe_combine, with the
 * combine folded into the down projection's epilogue: no h_sorted round trip
 * and no separate combine launch.  (GRACE-MoE page, section 1: every MoE layer
 * dispatches tokens to their experts and gathers the results back;
 * ExpertPlex page, "Adaptive Persistent Kernels (APK)": per-batch launch cost.)
 *
 *   x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I,
 *   w_gate, w_up, w_down: as moe_grouped_ffn with dtype MOE_BF16, or as
 *                  moe_grouped_ffn_packed when weights_packed = 1.
 *   sorted_to_flat [n_rows] int32 and topk_w [T][k] fp32: moe_permute's and
 *                  moe_gate's outputs for the same batch; n_rows must equal
 *                  T * (k + n_shared).
 *   y              [T][d] bf16, written: y[t] = sum over t's routed slots j of
 *                  topk_w[t][j] * h[row of (t, j)] + sum over shared experts
 *                  of h[row of (s, t)], where h is the FFN output rounded to
 *                  bf16 (as moe_grouped_ffn stores it).  The terms are added
 *                  in fp32 with atomic adds, in no fixed order, and rounded to
 *                  bf16 once; so y can differ from moe_combine's in the last
 *                  bits and from one call to the next.
 *   workspace      [T][d] fp32 sums (rounded up to 256 bytes), then
 *                  moe_grouped_ffn's workspace; the diagnostic word is its
 *                  last 4 bytes as for moe_grouped_ffn.
 *   Only batches that run on the decode-shaped kernels are supported (groups
 *   averaging at most 48 rows; see moe_grouped_ffn), where the launch and the
 *   h round trip weigh most; others get MOE_ERR_UNSUPPORTED.
 *   Errors: MOE_ERR_INVALID_ARG for n_rows != T * (k + n_shared), k < 1,
 *   weights_packed not 0 or 1, NULL or misaligned pointers (y and workspace
 *   16-byte aligned); MOE_ERR_UNSUPPORTED for the shapes above and
 *   moe_grouped_ffn's unsupported cases; MOE_ERR_WORKSPACE as usual.
 */
moe_status moe_grouped_ffn_combine(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                   const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                   int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                   const void* w_down, int32_t weights_packed, const int32_t* sorted_to_flat,
                                   const float* topk_w, int32_t T, int32_t k, void* y, void* workspace,
                                   size_t* workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn_noalloc - moe_grouped_ffn with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 *   Arguments and results as moe_grouped_ffn without `workspace` and
 *   `workspace_bytes`.  The workspace lives in a device array of
 *   MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 *   until the process ends; its device address is looked up on the first call
 *   on each device.  All calls on one GPU share that array and it keeps the
 *   last call's contents (every call writes what it reads first): calls that
 *   overlap in time on one GPU (for example on two streams) race, so the
 *   caller orders them.  The diagnostic word of moe_grouped_ffn stays inside
 *   the array and is not visible to the caller.
 *   Errors: as moe_grouped_ffn; MOE_ERR_WORKSPACE when the call needs more
 *   than MOE_NOALLOC_SCRATCH_BYTES of workspace (the SwiGLU intermediate
 *   n_rows * I values plus a little; decode-sized batches fit), MOE_ERR_HIP
 *   when the array's address cannot be looked up.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_grouped_ffn_noalloc(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                   const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                   int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                   const void* w_down, moe_dtype dtype, void* h_sorted, hipStream_t stream);

/*
 * moe_grouped_ffn_packed - moe_grouped_ffn (bf16) on expert weights pre-packed
 * so that each weight load instruction reads 1 KiB of contiguous memory: the
 * weight-streaming kernels load it into MFMA registers, the GEMM kernels copy
 * it into LDS as is.
 * (ExpertPlex page, "Instance vs module disaggregation": the expert FFN; the
 * packing is a one-time weight layout, not a change of the computation.)
 *
 *   Arguments, results, numerics, kernels chosen and the diagnostic word as
 *   moe_grouped_ffn with dtype MOE_BF16, except the weight layout.  A weight
 *   matrix W [R][K] (gate and up: R = I, K = d; down: R = d, K = I) of expert
 *   e is stored as blocks of 16 rows x 32 K values, block (r / 16, k / 32) at
 *   element offset ((r / 16) * (K / 32) + k / 32) * 512 of the expert's
 *   matrix, and inside a block W[r][k] at (((k % 32) / 8) * 16 + r % 16) * 8 +
 *   k % 8.  Each expert's matrix keeps its R * K elements at the same place as
 *   in the unpacked [E+S][R][K] array.  The results equal moe_grouped_ffn's
 *   on the unpacked weights bit for bit.
 *   Requires d and I multiples of 32.
 *   Errors: MOE_ERR_UNSUPPORTED when d or I is not a multiple of 32 or
 *   E > 512; otherwise as moe_grouped_ffn.  The workspace size is
 *   moe_grouped_ffn's.
 */
moe_status moe_grouped_ffn_packed(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                  const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                  int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                  const void* w_down, void* h_sorted, void* workspace, size_t* workspace_bytes,
                                  hipStream_t stream);

/*
 * moe_grouped_ffn_fp8w - the grouped SwiGLU expert FFN with FP8 expert weights.
 * (ExpertPlex page, "Experimental results", models table: GLM-5.1-FP8 serves
 * its experts in FP8.  The page does not give the format; it is read as OCP
 * E4M3 codes with one fp32 scale per weight row.)
 *
 *   As moe_grouped_ffn with dtype MOE_BF16 (x_sorted / x_rows, group offsets,
 *   h_sorted and the bf16 SwiGLU intermediate), except the weights:
 *   w_gate, w_up   [E+S][I][d] uint8 E4M3 codes; s_gate, s_up [E+S][I] fp32.
 *   w_down         [E+S][d][I] uint8 E4M3 codes; s_down [E+S][d] fp32.
 *   Weight row r of expert e is fp8(w[e][r][:]) * s[e][r].  E4M3 values are
 *   exact in bf16; products accumulate in fp32 and the scale multiplies the
 *   accumulated row product.  Runs on the decode-shaped kernel (any group
 *   sizes; meant for decode-sized groups; moe_grouped_ffn_fp8w_packed runs
 *   prefill-sized batches on a GEMM).
 *   Requires d and I multiples of 16; every pointer 16-byte aligned.
 *   Errors: MOE_ERR_UNSUPPORTED when d or I is not a multiple of 16 or
 *   E > 512;
 *   MOE_ERR_INVALID_ARG for nseg outside {1, 2}, a NULL required
 *   pointer (the three scale arrays included) or a misaligned one;
 *   MOE_ERR_WORKSPACE for a workspace below the queried size.  The workspace
 *   holds the bf16 SwiGLU intermediate [n_rows][I]; its last 4 bytes are
 *   written 0 by every call with n_rows > 0 (this call has no bounded waits).
 */
moe_status moe_grouped_ffn_fp8w(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                const int32_t* group_offsets, int32_t n_rows, int32_t E,
                                int32_t n_shared, int32_t nseg, int32_t d, int32_t I,
                                const void* w_gate, const float* s_gate,
                                const void* w_up, const float* s_up,
                                const void* w_down, const float* s_down,
                                void* h_sorted, void* workspace, size_t* workspace_bytes,
                                hipStream_t stream);

/*
 * moe_grouped_ffn_fp8w_packed - moe_grouped_ffn_fp8w on pre-packed codes.
 * (ExpertPlex page, "Experimental results", models table, as above; the
 * packing is a one-time weight layout, not a change of the computation.)
 *
 *   As moe_grouped_ffn_fp8w, except that each code matrix C [R][K] of an
 *   expert is stored as blocks of 16 rows x 64 codes (1 KiB): block
 *   (r / 16, k / 64) at byte offset ((r / 16) * (K / 64) + k / 64) * 1024 of
 *   the expert's matrix, and C[r][k] at (((k % 64) / 16) * 16 + r % 16) * 16 +
 *   k % 16 inside it.  Each expert's matrix keeps its R * K bytes at the same
 *   place as in the unpacked array; the scales are unchanged.
 *   Batches whose groups average at most 48 rows run on the decode-shaped
 *   kernel and equal moe_grouped_ffn_fp8w's results on the unpacked codes bit
 *   for bit.  Larger groups, with d and I at least 128 and 16-byte aligned
 *   scale arrays, run both phases on an LDS-tiled GEMM (256 x 256 tiles for
 *   groups of 256 rows or more on average, 128 x 256 below) that converts the
 *   codes to bf16 as it reads them (exact) and applies the row scales to the
 *   fp32 sums; its results differ from the decode-shaped kernel's only in the
 *   order of the fp32 sums.  On the 128 x 256 tiles a batch with a priority
 *   segment (nseg == 2) runs both phases in the persistent tile queues of
 *   moe_grouped_ffn (priority tiles first), and the workspace's last 4 bytes
 *   are its diagnostic word as for moe_grouped_ffn.  The queried workspace
 *   size depends on the batch shape (n_rows, E, n_shared, nseg, d, I).
 *   Requires d and I multiples of 64 (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status moe_grouped_ffn_fp8w_packed(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                const int32_t* group_offsets, int32_t n_rows, int32_t E,
                                int32_t n_shared, int32_t nseg, int32_t d, int32_t I,
                                const void* w_gate, const float* s_gate,
                                const void* w_up, const float* s_up,
                                const void* w_down, const float* s_down,
                                void* h_sorted, void* workspace, size_t* workspace_bytes,
                                hipStream_t stream);

/*
 * moe_combine - gate-weighted combine back to token order.
 * (GRACE-MoE page, section 1: the combine exchange.)
 *
 *   y[t] = sum_{j<k} topk_w[t][j] * h[flat_to_sorted[t*k+j]]
 *        + sum_{s<n_shared} h[flat_to_sorted[T*k+s*T+t]],
 *   accumulated in fp32 in that order and rounded once to `dtype`.
 *   h_sorted       [T*(k+n_shared)][d] of `dtype`.
 *   flat_to_sorted [T*(k+n_shared)] int32.
 *   topk_w         [T][k] fp32.
 *   y              [T][d] of `dtype`, written.
 *   Requires k >= 1, n_shared >= 0, d % 8 == 0.
 */
moe_status moe_combine(const void* h_sorted, const int32_t* flat_to_sorted,
                       const float* topk_w, int32_t T, int32_t k, int32_t n_shared,
                       int32_t d, moe_dtype dtype, void* y, hipStream_t stream);

/*
 * moe_stats - per-batch expert-activation statistics over a stack of L layers.
 * (ELDR page, "What it solves": the distinct-expert union; "Core idea /
 * structure / operation": count x IDF request signatures over a layer subset;
 * GRACE-MoE page, sections 3-4: co-activation (affinity) and load.)
 *
 *   topk_ids    [L][T][k] int32 routed ids (no shared experts).
 *   With M_l[t][e] = number of slots j with ids[l][t][j] == e:
 *   counts      [L][E] int32, written: column sums of M_l.
 *   union_size  [L] int32, written: number of experts with a nonzero count.
 *   union_mask  [L][E] uint8 or NULL, written: 1 where the count is nonzero.
 *   affinity    [L][E][E] int32 or NULL, written: M_l^T M_l (symmetric, the
 *               diagonal equals counts for distinct ids per token).
 *   req_offsets [R+1] int32 or NULL: request r owns tokens
 *               [req_offsets[r], req_offsets[r+1]) (0 <= ... <= T, non
 *               decreasing; a request may be a KV block).
 *   req_counts  [R][L][E] int32 or NULL, written: column sums of M_l over the
 *               request's tokens.
 *   idf         [L][E] fp32 or NULL.  NULL: idf = ln(R / df) from this batch,
 *               df = number of requests with a nonzero count, idf = 0 where
 *               df = 0 (computed in double).
 *   signature   [R][L][E] fp32 or NULL, written: req_counts * idf (double,
 *               rounded once).
 *   req_counts and signature need req_offsets.  R >= 0.
 */
moe_status moe_stats(const int32_t* topk_ids, int32_t L, int32_t T, int32_t k, int32_t E,
                     const int32_t* req_offsets, int32_t R, const float* idf,
                     int32_t* counts, int32_t* union_size, uint8_t* union_mask,
                     int32_t* affinity, int32_t* req_counts, float* signature,
                     void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * moe_prob_signature - continuous request signature: for request r, layer l
 * and expert e, the sum over the request's tokens of the full-E softmax
 * probability of e.  (ELDR page, "Core idea / structure / operation": the
 * paper compares its count x IDF signature against continuous alternatives
 * such as the softmax gate probability; this is that alternative, read as the
 * plain per-request sum, without IDF.)
 *
 *   logits      [L][T][E] fp32 router logits of the recorded layers, read only.
 *               NaN counts as -inf; a token whose logits are all -inf adds
 *               nothing; +inf logits are a precondition violation.
 *   req_offsets [R+1] int32: request r owns tokens [req_offsets[r],
 *               req_offsets[r+1]), clamped to [0, T] (as in moe_stats).
 *   signature   [R][L][E] fp32, written.  Probabilities and sums in double
 *               (token order), rounded to fp32 once (deterministic).
 *   Requires L >= 1, T >= 0, 1 <= E <= 512, R >= 0; R = 0 enqueues nothing.
 */
moe_status moe_prob_signature(const float* logits, int32_t L, int32_t T, int32_t E,
                              const int32_t* req_offsets, int32_t R, float* signature,
                              hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
