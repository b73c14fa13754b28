/*
 * moe_route.h - C ABI of the MI355X (gfx950) MoE top-k route / dispatch /
 * combine library (libmoe_route.so).
 *
 * The operations follow the pages' statement of the problem:
 *   - "Efficient and portable mixture-of-experts communication":
 *     sections "Introduction" (router, top-K, weighted average),
 *     "Dispatch" (per-expert token counts, packing, routing metadata kept
 *     for combine) and "Combine" (receiver-side weighted sum into tensors
 *     the caller allocated).
 *   - "Enabling trillion-parameter models on AWS EFA": sections "Send and
 *     Receive Buffers" (prefix sum of counts gives per-peer contiguous
 *     offsets; buffers sized for the worst case) and "Dispatch and Combine"
 *     (per-expert counts accumulated in one block; send and receive halves
 *     as separate kernels so other work can overlap them).
 *   - "Lower latency and higher throughput with multi-node DeepSeek
 *     deployment": section "MoE Router" (top-K indices and scores per token;
 *     dense dispatch needs routing aggregated per expert) and "CUDA Graph"
 *     (no host-side knowledge of routed counts, so launches can be captured).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller (for
 *    instance a torch tensor's data_ptr()).  The library allocates and frees
 *    nothing and is reentrant.  Its only global state is the per-device
 *    scratch array of moe_dispatch_noalloc (for callers that cannot
 *    allocate); every other entry point uses caller memory only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work on it; none synchronises the device or copies
 *    device -> host.  Stream order is the only synchronisation: results are
 *    valid once the stream reaches the end of the enqueued work.
 *  - bf16 crosses the ABI as raw 16-bit storage (IEEE bfloat16 bit patterns).
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  On any error
 *    nothing has been enqueued and no output has been touched, except
 *    MOE_ERR_HIP, which reports a failed kernel launch (work enqueued before
 *    the failing launch in the same call may have run).
 *  - T == 0 is valid: the call returns MOE_OK and enqueues nothing (the
 *    output pointers may then be NULL).
 *  - Checked on the host: null pointers (when T > 0), sizes and limits,
 *    16-byte alignment of bf16 row pointers, capacity >= T*k, workspace size.
 *    NOT checked (undefined behaviour if violated): that pointers are device
 *    memory of the stated size and that logits are finite.  Out-of-range
 *    expert indices and row indices are handled on the device as documented
 *    per entry point (never an out-of-bounds access).
 *
 * Limits: 1 <= E <= 1024; 1 <= k <= min(E, 32); T*k < 2^31;
 *         H % 8 == 0 and 8 <= H <= 2^20 for bf16 rows (rows move in 16-byte chunks).
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, size or limit out of range     */
  MOE_ERR_ALIGNMENT = -2,   /* H % 8 != 0 or a bf16 row pointer not 16-B aligned */
  MOE_ERR_CAPACITY = -3,    /* capacity < T*k: tokens are never dropped      */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required       */
  MOE_ERR_HIP = -5          /* a kernel launch failed (hipLaunchKernel error) */
};

/* ABI version of the loaded library (== MOE_ABI_VERSION it was built with). */
int moe_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* moe_strerror(int status);

/*
 * moe_route_topk - top-k routing of every token (the router of "Efficient and
 * portable mixture-of-experts communication", section "Introduction"; the
 * Mixtral special case of "Lower latency and higher throughput with
 * multi-node DeepSeek deployment", section "MoE Router").
 *
 *   logits   [T, E] fp32, row-major: router logits of each token.
 *   topk_idx [T, k] int32 (out): the k experts with the largest logits,
 *            in descending order; equal logits go to the lower expert index
 *            (+0.0 and -0.0 are equal).  Selecting on the logits equals
 *            selecting on the softmax probabilities, which are strictly
 *            increasing in the logits.
 *   topk_w   [T, k] fp32 (out): the softmax probabilities of the k
 *            selected experts divided by their sum (sum to 1 up to fp32
 *            rounding); topk_w[t, j] belongs to topk_idx[t, j].  The E-term
 *            softmax denominator cancels in that quotient, so it is computed
 *            as exp(l_j - l_max) over the sum of the k such terms, within
 *            2^-20 relative of the exact value.
 *   Logits may be any finite values; the difference of two is not needed
 *   to fit in fp32.
 * Errors: MOE_ERR_INVALID_ARG for T < 0, E or k out of range, null pointers.
 */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                   int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_route_topk_grouped - group-limited top-k routing.  The Mixtral router
 * is the special case of the DeepSeek router in which the top-K group is the
 * group of all experts ("Lower latency and higher throughput with multi-node
 * DeepSeek deployment", section "MoE Router"); the group rule is this
 * library's reading, as the page does not state it:
 *   - experts form n_group contiguous groups of E / n_group;
 *   - a group's score is its largest logit;
 *   - the topk_group best groups are kept (equal scores: the lower group);
 *   - top-k, ties and weights are as in moe_route_topk, over the kept
 *     experts only; the weights are the full-E softmax probabilities
 *     renormalised over the k chosen, as there.
 * topk_group == n_group is exactly moe_route_topk.
 * Errors: MOE_ERR_INVALID_ARG as moe_route_topk, and for n_group < 1,
 *         n_group > 64, E % n_group != 0, topk_group outside [1, n_group],
 *         or topk_group * (E / n_group) < k.
 */
int moe_route_topk_grouped(const float* logits, int64_t T, int32_t E, int32_t k,
                           int32_t n_group, int32_t topk_group,
                           int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_dispatch_workspace_bytes - device scratch moe_dispatch_send needs for
 * (T, E, k): per-block per-expert counts for the multi-block scan, at most
 * 64 KiB.  0 means no workspace is needed (T*k <= 4096; workspace may then
 * be NULL).  Returns 0 as well for arguments moe_dispatch_send would reject.
 */
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_dispatch_send - the "send" half of dispatch: per-expert token counts,
 * their exclusive scan into offsets, and a destination row for every
 * (token, j) pair ("Enabling trillion-parameter models on AWS EFA", sections
 * "Send and Receive Buffers" and "Dispatch and Combine"; "Efficient and
 * portable mixture-of-experts communication", section "Dispatch").
 *
 * The dispatch buffer is expert-major and packed: expert e owns rows
 * [expert_offsets[e], expert_offsets[e+1]); expert e = r*L + le belongs to
 * virtual rank r = e / L (L = E / num_vranks), so the buffer reads as
 * [virtual_rank][local_expert][slot] and rank r's rows are the contiguous
 * segment [rank_offsets[r], rank_offsets[r+1]).  Inside one expert, rows
 * follow the ascending flat pair index p = t*k + j (a stable counting sort).
 *
 *   topk_idx       [T, k] int32: expert of each pair.  A pair whose index is
 *                  outside [0, E) is dropped: it is not counted and its
 *                  pair_row entry is -1 (indices from moe_route_topk are
 *                  always in range).
 *   num_vranks     R >= 1 with E % R == 0.
 *   expert_counts  [E]   int32 (out): pairs routed to each expert.
 *   expert_offsets [E+1] int32 (out): exclusive scan; [E] = number of
 *                  counted pairs (T*k when every index is in range).
 *   pair_row       [T, k] int32 (out): row of pair (t, j) in the buffer.
 *   row_token      [T*k] int32 (out): token held by each row (entries past
 *                  expert_offsets[E] are left untouched).
 *   rank_offsets   [R+1] int32 (out) or NULL.
 *   workspace      device scratch of >= moe_dispatch_workspace_bytes(T,E,k)
 *                  bytes (any contents; overwritten); NULL if that is 0.
 * Errors: MOE_ERR_INVALID_ARG (limits, E % R != 0, null outputs),
 *         MOE_ERR_WORKSPACE (workspace missing or too small).
 */
int moe_dispatch_send(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k,
                      int32_t num_vranks, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* pair_row,
                      int32_t* row_token, int32_t* rank_offsets,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_recv - the "receive" half of dispatch: copy each token row
 * into its k rows of the expert-major buffer, so each expert's tokens are
 * contiguous for the grouped GEMM ("Efficient and portable
 * mixture-of-experts communication", section "Dispatch"; "Enabling
 * trillion-parameter models on AWS EFA", section "Dispatch and Combine").
 *
 *   x        [T, H] bf16 (16-byte aligned): token activations.
 *   pair_row [T, k] int32: from moe_dispatch_send.  Entries outside
 *            [0, capacity) (the -1 of a dropped pair) are skipped.
 *   buf      [capacity, H] bf16 (out, 16-byte aligned): buf[pair_row[t,j]]
 *            becomes a bit copy of x[t]; rows no pair maps to are untouched.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_ALIGNMENT, MOE_ERR_CAPACITY
 *         (capacity < T*k).
 */
int moe_dispatch_recv(const void* x, const int32_t* pair_row, int64_t T,
                      int32_t H, int32_t k, void* buf, int64_t capacity,
                      void* stream);

/*
 * moe_dispatch - moe_dispatch_send followed by moe_dispatch_recv on one
 * stream; arguments are the union of theirs, with the same meaning.  All
 * arguments of both halves are checked before anything is enqueued.  With
 * T*k <= 2048 and k <= 8 both halves run in one launch (the copies find
 * their rows from topk_idx themselves; the results are identical), and the
 * workspace is not used.
 */
int moe_dispatch(const int32_t* topk_idx, const void* x, int64_t T, int32_t E,
                 int32_t k, int32_t H, int32_t num_vranks,
                 int32_t* expert_counts, int32_t* expert_offsets,
                 int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets,
                 void* buf, int64_t capacity, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results.  The multi-block send keeps its
 * [blocks][E] count matrix in a device array the library owns instead:
 * 64 KiB per device, held on each device the library runs on until the
 * process ends (the send plan never needs more; a larger need would return
 * MOE_ERR_WORKSPACE).  Nothing is allocated; the first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress) once.
 * Every call on one device shares that device's array and the kernels
 * overwrite the part they use, so nothing needs clearing, but calls that
 * overlap on one device (different streams, or different threads without
 * ordering) race on it and must not be made.
 * Errors: as moe_dispatch, plus MOE_ERR_HIP if the device or its array
 *         cannot be looked up.
 */
int moe_dispatch_noalloc(const int32_t* topk_idx, const void* x, int64_t T,
                         int32_t E, int32_t k, int32_t H, int32_t num_vranks,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* pair_row, int32_t* row_token,
                         int32_t* rank_offsets, void* buf, int64_t capacity,
                         void* stream);

/*
 * moe_route_dispatch - moe_route_topk, moe_dispatch_send and
 * moe_dispatch_recv on one stream, in one call: the router's top-K output
 * goes straight into dispatch ("Efficient and portable mixture-of-experts
 * communication", sections "Introduction" and "Dispatch"; "Lower latency and
 * higher throughput with multi-node DeepSeek deployment", section "MoE
 * Router").  Arguments are the union of the three calls', with the same
 * meaning; topk_idx and topk_w are outputs.  n_group and topk_group select
 * group-limited routing as in moe_route_topk_grouped (n_group = topk_group =
 * 1 is plain moe_route_topk).  All arguments are checked before anything is
 * enqueued.  The outputs are identical to the separate calls.
 *
 * Launches, by size: with T*k <= 2048 and k <= 8, routing and then one
 * launch for send and recv (as moe_dispatch).  Otherwise, with T <= 2048 and
 * T*k <= 4096, route and send share one launch: the last routing block to
 * finish runs the single-block send, found with an arrival counter at the
 * start of the workspace.  Larger batches with E >= 128 skip the histogram
 * launch: the routing kernel counts every pair into the send histogram in
 * the workspace, and the last block of the rank kernel zeroes it again.
 *
 *   workspace  moe_route_dispatch_workspace_bytes(T, E, k) bytes (4-byte
 *              aligned).  All of it must be zero before the first call that
 *              uses it (e.g. hipMemset, torch.zeros); every call that
 *              returns MOE_OK leaves it zero again once its work has run, so
 *              it can serve the next call of any size it is large enough
 *              for.  After MOE_ERR_HIP, zero it again.  Calls that share a
 *              workspace must be ordered on one stream, and it must not be
 *              passed to the other dispatch calls, which leave counts in
 *              theirs.
 * Errors: as the three calls; MOE_ERR_WORKSPACE for a NULL or short
 *         workspace (T > 0).
 */
int moe_route_dispatch(const float* logits, const void* x, int64_t T, int32_t E,
                       int32_t k, int32_t n_group, int32_t topk_group,
                       int32_t H, int32_t num_vranks,
                       int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets,
                       void* buf, int64_t capacity, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_route_dispatch_workspace_bytes - the workspace moe_route_dispatch
 * needs for (T, E, k): a 256-byte block of arrival counters followed by the
 * moe_dispatch_send workspace.  Returns 0 for arguments moe_route_topk would
 * reject.
 */
size_t moe_route_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_dispatch_recv_fp8 - moe_dispatch_recv with block-scaled fp8 payloads:
 * each token row is quantised on the fly with one scale per 128-element block
 * and the fp8 row plus its scales are written to the token's k rows
 * ("Lower latency and higher throughput with multi-node DeepSeek
 * deployment", section "Quantization"; "Efficient and portable
 * mixture-of-experts communication", section "Dispatch": tokens travel with
 * their block scale factors; combine stays 16-bit).
 *
 *   x         [T, H] bf16 (16-byte aligned), H % 128 == 0, finite values.
 *   pair_row  [T, k] int32: as for moe_dispatch_recv (out-of-range skipped).
 *   buf_q     [capacity, H] uint8 (out, 16-byte aligned): OCP E4M3 codes
 *             (4 exponent bits, bias 7, 3 mantissa bits, no infinities).
 *   buf_scale [capacity, H/128] fp32 (out, 4-byte aligned).
 * For block b of token t: amax = max |x[t, 128b : 128b+128]|;
 * scale = amax / 448 in fp32 (1.0 when amax == 0); every code is the nearest
 * E4M3 value to fp32(x / scale), ties to the even code, saturating at +-448.
 * Dequantised value = E4M3(code) * scale.
 * Errors: as moe_dispatch_recv, plus MOE_ERR_ALIGNMENT when H % 128 != 0,
 *         MOE_ERR_INVALID_ARG for a NULL buf_scale.
 */
int moe_dispatch_recv_fp8(const void* x, const int32_t* pair_row, int64_t T,
                          int32_t H, int32_t k, void* buf_q, float* buf_scale,
                          int64_t capacity, void* stream);

/*
 * moe_dispatch_fp8 - moe_dispatch_send followed by moe_dispatch_recv_fp8 on
 * one stream; arguments as theirs, all checked before anything is enqueued.
 * As in moe_dispatch, T*k <= 2048 and k <= 8 run both halves in one launch
 * (identical results) without the workspace.
 */
int moe_dispatch_fp8(const int32_t* topk_idx, const void* x, int64_t T,
                     int32_t E, int32_t k, int32_t H, int32_t num_vranks,
                     int32_t* expert_counts, int32_t* expert_offsets,
                     int32_t* pair_row, int32_t* row_token,
                     int32_t* rank_offsets, void* buf_q, float* buf_scale,
                     int64_t capacity, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * moe_route_dispatch_fp8 - moe_route_dispatch with the block-scaled fp8
 * receive of moe_dispatch_recv_fp8: the router's top-K output goes straight
 * into dispatch, and the rows travel as E4M3 codes plus one fp32 scale per
 * 128 elements ("Lower latency and higher throughput with multi-node
 * DeepSeek deployment", sections "MoE Router" and "Quantization").
 * Arguments are moe_route_dispatch's, with buf_q / buf_scale as in
 * moe_dispatch_recv_fp8 in place of buf; the same workspace rules apply
 * (moe_route_dispatch_workspace_bytes, zeroed once, left zeroed).  All
 * arguments are checked before anything is enqueued.  The outputs equal
 * moe_route_topk_grouped followed by moe_dispatch_fp8, and the launches by
 * size are moe_route_dispatch's with the fp8 receive in place of the copy.
 * Errors: as moe_route_dispatch and moe_dispatch_recv_fp8.
 */
int moe_route_dispatch_fp8(const float* logits, const void* x, int64_t T, int32_t E,
                           int32_t k, int32_t n_group, int32_t topk_group,
                           int32_t H, int32_t num_vranks,
                           int32_t* topk_idx, float* topk_w,
                           int32_t* expert_counts, int32_t* expert_offsets,
                           int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets,
                           void* buf_q, float* buf_scale, int64_t capacity,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_combine - receiver-side weighted sum of each token's k expert-output
 * rows ("Efficient and portable mixture-of-experts communication", section
 * "Combine"; accumulation at the receiver as in "Enabling trillion-parameter
 * models on AWS EFA", section "Evaluation").
 *
 *   y        [capacity, H] bf16 (16-byte aligned): expert outputs, one row per
 *            dispatched row (same order as the dispatch buffer).
 *   pair_row [T, k] int32: from moe_dispatch_send.  A term whose entry is
 *            outside [0, capacity) is skipped (acc is left unchanged).
 *   topk_w   [T, k] fp32: weights from moe_route_topk.
 *   out      [T, H] bf16 (out, 16-byte aligned, caller-allocated):
 *            out[t] = bf16_rne(acc), acc = +0.0f, then for j = 0..k-1
 *            acc = fmaf(topk_w[t,j], y[pair_row[t,j]], acc) in fp32.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_ALIGNMENT, MOE_ERR_CAPACITY.
 */
int moe_combine(const void* y, const int32_t* pair_row, const float* topk_w,
                int64_t T, int32_t H, int32_t k, int64_t capacity, void* out,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
