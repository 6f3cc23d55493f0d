/*
 * libulysses: one GPU's share of Ulysses sequence parallelism on MI355X (gfx950).
 *
 * Ulysses splits a sequence of N tokens over P GPUs. Each GPU projects Q, K, V
 * for its own N/P tokens and all heads; an all-to-all switches the split from
 * tokens to heads, so each GPU then holds all N tokens of H/P heads and runs
 * ordinary attention over the full sequence; a second all-to-all switches back
 * to the token split ("Ulysses sequence parallelism", HF Transformers docs,
 * intro and its two-GPU diagram; "Ulysses Sequence Parallelism for
 * Million-Token Context Training", "How Ulysses Sequence Parallelism Works").
 *
 * This library provides the per-GPU work around and between the two
 * exchanges: the local pack/unpack that turns the token-split tensor into the
 * P per-destination chunks of the all-to-all (and back), and causal
 * grouped-query attention forward and backward over the full sequence for the
 * local heads, dense or over packed documents (cu_seqlens).
 *
 * Conventions for every call:
 *  - Tensors are bfloat16 bit patterns (uint16_t), LSE and D are float32.
 *  - All tensor pointers are device pointers; the caller allocates and owns
 *    all memory. The library allocates nothing and keeps no mutable global
 *    state apart from a per-thread error message (and, once TiledMLP has run
 *    on a device, that device's hipBLASLt handle).
 *  - Tensor pointers must be 16-byte aligned and token strides must be
 *    multiples of 8 elements (16 bytes); otherwise ULY_E_ALIGN.
 *  - Strides are in elements. Within a token row, heads are d elements apart.
 *  - Calls are asynchronous on `stream` (0 = the null stream). Arguments are
 *    validated on the host before anything is launched; on any error nothing
 *    is launched and no output is touched.
 *  - Return value: ULY_OK (0) or a negative ULY_E_* code.
 *  - No C++ exception crosses this interface.
 *  - Batch size is 1; several sequences are expressed as packed documents.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ULY_OK 0
#define ULY_E_NULL (-1)      /* a required pointer is NULL */
#define ULY_E_SHAPE (-2)     /* a size is non-positive or too large */
#define ULY_E_DIV_P (-3)     /* N or a head count is not divisible by P */
#define ULY_E_GQA (-4)       /* hq is not a multiple of hkv */
#define ULY_E_HEADDIM (-5)   /* d is not 64 or 128 */
#define ULY_E_STRIDE (-6)    /* a token stride is smaller than the row it holds */
#define ULY_E_WORKSPACE (-7) /* workspace missing or too small */
#define ULY_E_ALIAS (-8)     /* an output overlaps an input where that is not allowed */
#define ULY_E_HIP (-9)       /* a HIP launch failed; see uly_last_error() */
#define ULY_E_SEQLENS (-10)  /* cu_seqlens is not 0 = c0 < c1 < ... < c_n = N */
#define ULY_E_ALIGN (-11)    /* pointer not 16-byte aligned or stride not a multiple of 8 */
#define ULY_E_SCRATCH (-12)  /* attn_fwd_noalloc: problem needs more than its static scratch */

/* Bytes of the static per-GPU scratch buffer attn_fwd_noalloc works in. */
#define ULY_NOALLOC_SCRATCH_BYTES (80u << 20)

/* Text for a status code. Never NULL. */
const char *uly_status_string(int status);

/* Detail of the last ULY_E_HIP on the calling thread ("" if none). */
const char *uly_last_error(void);

/*
 * Tokens per rank for a sequence of N tokens on P ranks: *n_local = N / P.
 * Sequences must be padded to a multiple of the SP degree ("Ulysses sequence
 * parallelism", Configure, on sp_size): returns ULY_E_DIV_P when N % P != 0,
 * ULY_E_SHAPE when N <= 0 or P <= 0, ULY_E_NULL when n_local is NULL.
 * Host-only.
 */
int ulysses_shard_len(int64_t N, int32_t P, int64_t *n_local);

/*
 * Host-side check of a packed-document offset table (host memory):
 * cu[0] = 0, strictly increasing, cu[n_seqs] = N. Returns ULY_OK or
 * ULY_E_SEQLENS (ULY_E_NULL / ULY_E_SHAPE for a NULL table or n_seqs <= 0).
 * The attention kernels trust their device copy of the table, so callers run
 * this once when they build it. Packed samples must not attend across their
 * boundaries ("Ulysses sequence parallelism", Configure, on
 * sp_attn_implementation).
 */
int ulysses_check_cu_seqlens(const int32_t *cu, int32_t n_seqs, int64_t N);

/*
 * Sequence-to-head pack: the local half of the first all-to-all.
 *
 * x_seq  [n_local][H][d]     this rank's tokens with all H = sum(seg_heads)
 *                            heads, contiguous.
 * x_send [P][n_local][H/P][d] contiguous; chunk p is what goes to rank p:
 *                            for every local token, rank p's contiguous block
 *                            [p*s/P, (p+1)*s/P) of each segment s in order.
 *                            With seg_heads = {Hq, Hkv, Hkv} (fused q|k|v) a
 *                            chunk row is [q heads | k heads | v heads] of
 *                            rank p; with {Hq} it is rank p's query heads.
 * seg_heads: host array of n_seg (1..8) head counts, each divisible by P
 *            (the head count must divide by the SP degree: "Ulysses sequence
 *            parallelism", Configure, the warning on attention heads).
 * d: head dim, a multiple of 8 (any such value, not only 64/128).
 * Errors: ULY_E_NULL, ULY_E_SHAPE (n_local, P, d, n_seg out of range, or a
 * tensor of 2^31 16-byte vectors or more: n_local*H*d >= 2^34),
 * ULY_E_DIV_P, ULY_E_ALIGN, ULY_E_ALIAS (x_seq and x_send overlap), ULY_E_HIP.
 * Receiving a chunk from every rank in rank order gives the head shard
 * [N][H/P][d] with tokens in sequence order (intro diagram: GPU 0 holds the
 * first tokens).
 */
int ulysses_seq_to_head(const uint16_t *x_seq, uint16_t *x_send, int64_t n_local, int32_t P,
                        int32_t n_seg, const int32_t *seg_heads, int32_t d, hipStream_t stream);

/*
 * Head-to-sequence unpack: the local half of the second all-to-all, the exact
 * inverse of ulysses_seq_to_head with the same arguments:
 * x_recv [P][n_local][H/P][d] (chunk p came from rank p) -> x_seq [n_local][H][d].
 * In the backward pass the two calls swap roles (the adjoint of a permutation
 * is its inverse).
 */
int ulysses_head_to_seq(const uint16_t *x_recv, uint16_t *x_seq, int64_t n_local, int32_t P,
                        int32_t n_seg, const int32_t *seg_heads, int32_t d, hipStream_t stream);

/*
 * Attention forward over the full sequence for the local heads: the local
 * step between the two exchanges ("How Ulysses Sequence Parallelism Works",
 * step 4). Exact softmax attention, computed in tiles without an N x N buffer
 * ("The Challenge of Long Sequence Training": O(n) memory, O(n^2) compute).
 *
 * q  [N] rows of hq heads x d, token stride q_stride (elements)
 * k, v [N] rows of hkv heads x d, token strides k_stride, v_stride
 *        (q, k, v may be views into one fused [N][hq+2hkv][d] buffer)
 * o  [N] rows of hq heads x d, token stride o_stride (output, bf16)
 * lse [hq][N] float32, natural-log log-sum-exp of each row's scaled scores
 *        (output; kept for the backward pass)
 * Query head h uses KV head h / (hq / hkv) (contiguous GQA groups).
 * scale: score multiplier (1/sqrt(d) usually); must be finite and > 0.
 * causal != 0: key j is visible to query i iff j <= i.
 * ws: device workspace of at least attn_fwd_workspace_bytes(N, hq, hkv, d)
 *        bytes, 256-byte aligned, not overlapping any tensor argument; its
 *        contents on entry do not matter (it receives a transposed copy of V).
 * Errors: ULY_E_NULL, ULY_E_SHAPE, ULY_E_GQA, ULY_E_HEADDIM (d not 64/128),
 * ULY_E_STRIDE (a stride < heads*d), ULY_E_ALIGN, ULY_E_WORKSPACE,
 * ULY_E_ALIAS (o overlaps q, k or v, or ws overlaps a tensor), ULY_E_HIP.
 */
int attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o, float *lse,
             int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride,
             int64_t v_stride, int64_t o_stride, float scale, int32_t causal, void *ws,
             size_t ws_bytes, hipStream_t stream);

/*
 * attn_fwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not allocate, harnesses that forbid it). Same
 * arguments, result bits and errors as attn_fwd, except that the workspace
 * is a static buffer of ULY_NOALLOC_SCRATCH_BYTES (80 MiB) that the library
 * holds on every GPU it runs on until the process ends. Problems whose
 * attn_fwd_workspace_bytes(N, hq, hkv, d) exceed that return ULY_E_SCRATCH
 * (before anything is launched). At d = 128 that allows up to 327,552
 * tokens with one KV head or 163,776 with two; every head shard of the
 * 8K, 64K, packed 64K and 256K workloads fits.
 * The device is the stream's (the current device for stream 0). The first
 * call on a device looks up the buffer's address there; that lookup can
 * fail with ULY_E_HIP. Every call on a GPU shares that GPU's buffer and
 * leaves its contents behind: calls that may overlap on one GPU (different
 * streams, or threads) race on it and must be serialised by the caller.
 */
int attn_fwd_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o,
                     float *lse, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride,
                     int64_t k_stride, int64_t v_stride, int64_t o_stride, float scale,
                     int32_t causal, hipStream_t stream);

/* Workspace attn_fwd and attn_fwd_varlen need: hkv * d * roundup(N, 64) * 2
 * bytes (the transposed V), rounded up to 256, and, when there are fewer than
 * 512 (query block of 256 / hpw rows, group of hpw query heads) pairs, hpw
 * the largest of 4, 2, 1 dividing hq / hkv, s * N * hq * (d + 2) * 4 bytes
 * more, s = min(4, ceil(512 / pairs)), rounded up to 256: float32 partial
 * softmax states of the s workgroups that then share each pair's keys; then
 * roundup(N, 64) / 64 int32 entries, rounded up to 256 bytes (the order of
 * the query blocks over packed documents). */
size_t attn_fwd_workspace_bytes(int64_t N, int32_t hq, int32_t hkv, int32_t d);

/*
 * attn_fwd over packed documents: key j is visible to query i iff both lie in
 * the same document [cu[b], cu[b+1]) and (causal == 0 or j <= i). Several
 * samples packed into one sequence must not attend across their boundaries
 * ("Ulysses sequence parallelism", Configure, on sp_attn_implementation:
 * packed samples need an attention that respects sample boundaries;
 * "Ulysses Sequence Parallelism for Million-Token Context Training",
 * Ecosystem Integration, TRL SFTTrainer: packing several samples into one
 * sequence).
 * cu_seqlens: DEVICE int32 [n_seqs + 1], checked by ulysses_check_cu_seqlens
 * on its host copy (the kernels trust it; a table that fails the check
 * gives wrong values, but every range the kernels derive from it is cut to
 * [0, N), so no access leaves the tensors). max_seqlen: longest document,
 * used only for validation (must be in [1, N]).
 */
int attn_fwd_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o,
                    float *lse, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride,
                    int64_t k_stride, int64_t v_stride, int64_t o_stride, float scale,
                    int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs,
                    int32_t max_seqlen, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace the backward pass needs: float32 -D, D = rowsum(dO * O), and
 * LSE*log2(e), [hq][roundup(N, 64)] each, then transposed copies of K, Q and
 * dO (hkv, hq and hq heads of d * roundup(N, 64) bf16), then two int32
 * arrays of roundup(N, 64) / 64 entries (the workgroup orders of the dK/dV
 * and dq passes over packed documents), and, when there are fewer than 512
 * (128-key block, KV head) pairs,
 * float32 partial dK/dV of s * N * hkv * 2 * d values, s = min(4,
 * ceil(512 / pairs)) (the dK/dV pass then splits each pair's queries over s
 * workgroups), and, when there are fewer than 512 (query block of 256 / hpw
 * rows, group of hpw query heads) pairs, hpw the largest of 4, 2, 1 dividing
 * hq / hkv, float32 partial dQ of s' * N * hq * d values, s' = min(4,
 * ceil(512 / pairs)); each region rounded up to 256 bytes. */
size_t attn_bwd_workspace_bytes(int64_t N, int32_t hq, int32_t hkv, int32_t d, int32_t n_seqs);

/*
 * Attention backward: gradients of L = sum(dout * o) for the attn_fwd call
 * with the same arguments, i.e. the backward pass of the local attention of
 * "How Ulysses Sequence Parallelism Works", step 4, which training through
 * it needs (Ecosystem Integration, Transformers Trainer: the gradients must
 * come out correct). The scores are recomputed tile by tile from the saved
 * lse instead of being stored ("The Challenge of Long Sequence Training":
 * tiled attention keeps O(n) memory for O(n^2) work):
 *   D_i = dout_i . o_i,  p_ij = exp(s_ij - lse_i),  ds_ij = p_ij (dout_i . v_j - D_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij dout_i.
 * o and lse are that call's outputs.
 * dq [N] x hq x d, dk, dv [N] x hkv x d with their own token strides; they
 * are overwritten (not accumulated). dk and dv sum over the query heads of
 * each GQA group. dq, dk and dv may be views into one fused
 * [N][hq+2hkv][d] buffer; none may overlap an input.
 * ws: device workspace of at least attn_bwd_workspace_bytes(...) bytes,
 * 256-byte aligned; its contents on entry do not matter.
 * The result is deterministic (no atomics): the same inputs give the same bits.
 * Errors: as attn_fwd, plus ULY_E_WORKSPACE.
 */
int attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
             const float *lse, const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
             int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride,
             int64_t v_stride, int64_t o_stride, int64_t do_stride, int64_t dq_stride,
             int64_t dk_stride, int64_t dv_stride, float scale, int32_t causal, void *ws,
             size_t ws_bytes, hipStream_t stream);

/* attn_bwd over packed documents: the gradients of attn_fwd_varlen with the
 * same arguments (mask, cu_seqlens and max_seqlen as there: "Ulysses
 * sequence parallelism", Configure, packed samples must not attend across
 * their boundaries). */
int attn_bwd_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
                    const float *lse, const uint16_t *dout, uint16_t *dq, uint16_t *dk,
                    uint16_t *dv, int64_t N, int32_t hq, int32_t hkv, int32_t d,
                    int64_t q_stride, int64_t k_stride, int64_t v_stride, int64_t o_stride,
                    int64_t do_stride, int64_t dq_stride, int64_t dk_stride, int64_t dv_stride,
                    float scale, int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs,
                    int32_t max_seqlen, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The two steps of attn_bwd as separate calls, for callers that schedule them
 * on their own (e.g. to overlap the second with other work). attn_bwd is
 * exactly attn_bwd_dq followed by attn_bwd_dkdv on the same stream. The
 * split follows the gradient's definition (attn_bwd above; "The Challenge of
 * Long Sequence Training"): dq sums over keys, dk and dv over queries, so
 * each step is one pass that recomputes the scores it needs.
 *
 * attn_bwd_dq: fills ws (-D, LSE*log2(e), at d = 64 the transposed copies of
 *   K, Q and dO, over packed documents the block orders of both steps) and
 *   writes dq.
 * attn_bwd_dkdv: dk and dv. It reads -D, LSE*log2(e), (d = 64) the
 *   transposed copies of Q and dO and (packed documents) its key-block order
 *   from ws as left by attn_bwd_dq with the same arguments (not to be
 *   modified in between), and writes another region of ws: its float32
 *   partial dK/dV (when it splits its query ranges, see
 *   attn_bwd_workspace_bytes). Calls that may run at the same time therefore
 *   need workspaces of their own.
 * cu_seqlens: device table as in attn_fwd_varlen, or NULL for one document
 * (n_seqs is then ignored). Errors as attn_bwd.
 */
int attn_bwd_dq(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
                const float *lse, const uint16_t *dout, uint16_t *dq, int64_t N, int32_t hq,
                int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                int64_t o_stride, int64_t do_stride, int64_t dq_stride, float scale,
                int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs, void *ws,
                size_t ws_bytes, hipStream_t stream);

int attn_bwd_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *lse,
                  const uint16_t *dout, uint16_t *dk, uint16_t *dv, int64_t N, int32_t hq,
                  int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                  int64_t do_stride, int64_t dk_stride, int64_t dv_stride, float scale,
                  int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs, void *ws,
                  size_t ws_bytes, hipStream_t stream);

/*
 * Ring attention, the variant the pages set against Ulysses ("Sequence
 * Parallelism for Long-Context AI Training", "Advanced Scaling: Ring
 * Attention and Ulysses": each GPU keeps the queries of its S/P tokens and
 * computes local attention against the key/value block it holds while the
 * blocks travel around a ring; "Ulysses Sequence Parallelism for
 * Million-Token Context Training", "Comparing Ulysses and Ring Attention").
 *
 * One ring step on rank r is attn_fwd of its queries against the block of
 * rank b, with causal != 0 for b == r and causal == 0 for b < r (blocks of
 * later ranks are all masked and skipped). Each step's (o_j, lse_j) is the
 * softmax over that block's keys only; attn_lse_merge combines them into
 * attention over all keys:
 *   lse = log sum_j exp(lse_j),  o = sum_j exp(lse_j - lse) o_j.
 *
 * o_parts:   host array of n_parts device pointers, each [N] rows of h heads
 *            x d bf16 with token stride part_stride (elements).
 * lse_parts: host array of n_parts device pointers, each [h][N] float32
 *            (natural log, as attn_fwd writes it).
 * o_out [N] rows of h x d bf16 (token stride out_stride), lse_out [h][N].
 * n_parts: 1..16. A part whose lse is -inf for a row adds nothing to it; a
 * row that is -inf in every part gets o = 0 and lse = -inf.
 * d: a multiple of 8. Outputs may not overlap any part (no in-place merge).
 * Errors: ULY_E_NULL, ULY_E_SHAPE (n_parts, N, h or d out of range),
 * ULY_E_STRIDE, ULY_E_ALIGN (o pointers, strides or d; lse pointers need 4
 * bytes), ULY_E_ALIAS, ULY_E_HIP.
 */
int attn_lse_merge(int32_t n_parts, const uint16_t *const *o_parts, const float *const *lse_parts,
                   uint16_t *o_out, float *lse_out, int64_t N, int32_t h, int32_t d,
                   int64_t part_stride, int64_t out_stride, hipStream_t stream);

/*
 * Backward of the ring: each step's attn_bwd, run with the merged o and lse
 * (so that p and D are those of attention over all keys) and the step's
 * causal flag, gives the block's share of dQ for the local queries and of dK
 * and dV for the block's owner. ring_grad_sum adds such shares:
 *   out = sum_j parts[j], accumulated in float32 and rounded to bf16 once.
 * parts: host array of n_parts (1..16) device pointers, each [rows] x width
 * bf16 with token stride part_stride; out [rows] x width, stride out_stride.
 * width: a multiple of 8. out may not overlap any part.
 * Errors: ULY_E_NULL, ULY_E_SHAPE, ULY_E_STRIDE, ULY_E_ALIGN, ULY_E_ALIAS,
 * ULY_E_HIP.
 */
int ring_grad_sum(int32_t n_parts, const uint16_t *const *parts, uint16_t *out, int64_t rows,
                  int32_t width, int64_t part_stride, int64_t out_stride, hipStream_t stream);

/*
 * Loss of an SP step from pre-shifted labels ("Deepspeed Ulysses/ALST
 * integration", opening post, step 2; "Ulysses sequence parallelism",
 * Configure: the Trainer shifts labels and aggregates the loss across SP
 * ranks). Each rank holds the logits of its own n tokens and their
 * shift_labels (the label of token i is token i+1 of the full sequence; -100
 * marks tokens without a loss, e.g. prompt tokens or the last token).
 *
 * shifted_ce_fwd, per rank: for every row r with a good label y_r (in
 * [0, V)): row_loss[r] = lse_r - logit_{r,y_r} with lse_r = log sum_v
 * exp(logit_rv) (natural log); row_loss = 0 for other labels. Then
 * *loss_out = mean of row_loss over good rows (0 if there are none) and
 * *good_out = their count, summed in a fixed order (deterministic).
 *   logits [n] rows of V bf16, row stride `stride` elements (finite values);
 *   labels [n] int32, device; row_loss, row_lse [n] float32 (outputs;
 *   row_lse is kept for shifted_ce_bwd); loss_out, good_out: device scalars.
 *   V: a multiple of 8.
 *
 * sp_loss_aggregate: the differentiable weighted aggregation across ranks,
 *   *total_out = sum_r loss_r * good_r / max(sum_r good_r, 1),
 * from n_ranks (1..16) device scalars (host arrays of device pointers), and
 * *row_grad_scale_out = 1 / max(sum_r good_r, 1), the factor every good
 * row's gradient carries.
 *
 * shifted_ce_bwd, per rank: the gradient of the aggregate with respect to
 * the rank's logits: dlogits[r] = (softmax(logits[r]) - onehot(y_r)) *
 * (*row_grad_scale) for good rows, 0 for the others. dlogits may be the
 * logits buffer itself (same pointer and stride: each element is read before
 * it is overwritten); any other overlap is ULY_E_ALIAS.
 *
 * Errors: ULY_E_NULL, ULY_E_SHAPE (n, V or n_ranks out of range), ULY_E_STRIDE,
 * ULY_E_ALIGN (logits/dlogits 16-byte aligned, strides and V multiples of 8),
 * ULY_E_ALIAS, ULY_E_HIP.
 */
int shifted_ce_fwd(const uint16_t *logits, const int32_t *labels, int64_t n, int64_t V,
                   int64_t stride, float *row_loss, float *row_lse, float *loss_out,
                   int32_t *good_out, hipStream_t stream);
int sp_loss_aggregate(int32_t n_ranks, const float *const *rank_loss,
                      const int32_t *const *rank_good, float *total_out, float *row_grad_scale_out,
                      hipStream_t stream);
int shifted_ce_bwd(const uint16_t *logits, const int32_t *labels, const float *row_lse,
                   const float *row_grad_scale, int64_t n, int64_t V, int64_t stride,
                   uint16_t *dlogits, int64_t dstride, hipStream_t stream);

/*
 * TiledMLP: the model's SwiGLU MLP run over the sequence in token tiles, the
 * second memory component of ALST next to Ulysses ("Ulysses sequence
 * parallelism", intro note on ALST; "Ulysses Sequence Parallelism for
 * Million-Token Context Training", Additional Kernels; the pages give only
 * the name). Per token:
 *   gu = x W_gu^T (gate | up, 2I values),  a = silu(gate) * up,  y = a W_down^T.
 * Only one tile's gu and a exist at a time (in ws); the backward pass
 * recomputes them tile by tile. The GEMMs (bf16 inputs, float32
 * accumulation) run in hipBLASLt; the SwiGLU steps are HIP kernels.
 *
 * x, y, dy, dx [n][H] bf16, contiguous; w_gu [2I][H] (gate rows, then up
 * rows; nn.Linear's [out][in]); w_down [H][I]; dw_gu [2I][H] and dw_down
 * [H][I] float32. H and I multiples of 8; all pointers 16-byte aligned.
 * tile: tokens per tile (>= 1; the last tile may be shorter).
 * ws: at least tiled_mlp_workspace_bytes(tile, H, I) bytes, 256-byte aligned
 * (two [tile][2I] and two [tile][I] bf16 buffers plus 64 MiB for hipBLASLt).
 * tiled_mlp_bwd writes dx and, with accumulate == 0, overwrites dw_gu and
 * dw_down (accumulate != 0 adds to them).
 * On first use on a device the library creates one hipBLASLt handle for it
 * and keeps it until the process ends.
 * Errors: ULY_E_NULL, ULY_E_SHAPE, ULY_E_ALIGN, ULY_E_WORKSPACE, ULY_E_ALIAS
 * (an output overlaps an input, another output or ws), ULY_E_HIP (a launch or
 * hipBLASLt call failed; see uly_last_error()).
 */
size_t tiled_mlp_workspace_bytes(int64_t tile, int32_t H, int32_t I);
int tiled_mlp_fwd(const uint16_t *x, const uint16_t *w_gu, const uint16_t *w_down, uint16_t *y,
                  int64_t n, int32_t H, int32_t I, int64_t tile, void *ws, size_t ws_bytes,
                  hipStream_t stream);
int tiled_mlp_bwd(const uint16_t *x, const uint16_t *w_gu, const uint16_t *w_down,
                  const uint16_t *dy, uint16_t *dx, float *dw_gu, float *dw_down, int64_t n,
                  int32_t H, int32_t I, int64_t tile, int32_t accumulate, void *ws,
                  size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
