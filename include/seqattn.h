/*
 * seqattn.h -- C ABI of the segmented exact-attention library (libseqattn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The library computes, on one GPU, the per-device step of sequence-parallel
 * attention: exact softmax attention of a block of local queries against one
 * key/value segment at a time, the log-sum-exp merge of such partial results,
 * LongNet-style dilated attention built from the same segment kernel, and the
 * backward of a segment.
 *
 * Conventions common to every call
 * --------------------------------
 *  - Tensors are described by seqattn_tensor: a device pointer, an element
 *    type, the logical shape [b, h, n, d] and element strides for b, h and n.
 *    The innermost dimension d is always contiguous (stride 1).  Rows
 *    (d elements) must start on 16-byte boundaries: the data pointer and
 *    every stride times the element size must be multiples of 16 bytes
 *    (LSE tensors, d = 1, are exempt and may have any stride).
 *  - All pointers in tensor descriptors are DEVICE pointers owned by the
 *    caller.  Descriptor structs themselves, and the segment_lengths /
 *    dilations arrays, are HOST memory read during the call only.
 *  - Every compute call is asynchronous on `hip_stream` (a hipStream_t; NULL
 *    means the default stream).  Buffers must stay alive until the queued
 *    work completes.  The library never allocates or frees device memory;
 *    calls that need scratch take a caller-owned workspace.
 *  - Arguments are validated before any HIP call, so every error return can
 *    be produced without a GPU.  Calls return an int status (seqattn_status);
 *    no exception or abort crosses the ABI.  On a non-OK return nothing has
 *    been launched, except SEQATTN_ERR_HIP, which reports a failed launch
 *    (details in seqattn_last_error()).
 *  - Visibility ("causal offset"): key j of the segment is visible to query i
 *    of the block iff j <= i + causal_offset, where causal_offset is the
 *    global position of the block's first query minus that of the segment's
 *    first key.  SEQATTN_NONCAUSAL makes every key visible.
 *  - Softmax scale: softmax_scale <= 0 selects 1/sqrt(d).
 *  - Grouped KV heads: k->h must divide q->h; query head hq reads KV head
 *    floor(hq * k->h / q->h) (contiguous groups).
 *  - LSE is the natural-log log-sum-exp of the scaled scores of the keys a
 *    row saw, fp32; a row that saw no key has O = 0 and LSE = -inf.
 *
 * Supported: d in {64, 128}; Q/K/V all bf16 (MFMA path) or all fp32.
 */
#ifndef SEQATTN_H
#define SEQATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEQATTN_VERSION 110 /* 1.1.0: adds seqattn_attn_segment_fwd_ws */

typedef enum {
    SEQATTN_OK = 0,
    SEQATTN_ERR_NULL = -1,        /* a required pointer is NULL */
    SEQATTN_ERR_DTYPE = -2,       /* element type not allowed for this operand */
    SEQATTN_ERR_SHAPE = -3,       /* shapes inconsistent or out of range */
    SEQATTN_ERR_STRIDE = -4,      /* stride/alignment rule broken */
    SEQATTN_ERR_ALIAS = -5,       /* an output overlaps an input */
    SEQATTN_ERR_UNSUPPORTED = -6, /* valid request the library does not serve */
    SEQATTN_ERR_WORKSPACE = -7,   /* workspace missing or too small */
    SEQATTN_ERR_HIP = -8          /* HIP launch/runtime error */
} seqattn_status;

typedef enum { SEQATTN_BF16 = 1, SEQATTN_F32 = 2 } seqattn_dtype;

typedef struct {
    void *data;                 /* device pointer */
    int32_t dtype;              /* seqattn_dtype */
    int64_t b, h, n, d;         /* logical shape; LSE tensors use d = 1 */
    int64_t stride_b, stride_h, stride_n; /* in elements; stride_d is 1 */
} seqattn_tensor;

#define SEQATTN_NONCAUSAL INT64_MAX

/* flags */
#define SEQATTN_ACCUMULATE 1u /* (o, lse) hold a running partial on entry:
                                 the new partial is merged into them */
#define SEQATTN_CAUSAL 2u     /* dilated attention only: causal in original
                                 positions */
#define SEQATTN_HEAD_SHIFT 4u /* dilated attention only: query head h selects
                                 offset h mod r_i inside each segment */

/* op ids for seqattn_workspace_size */
#define SEQATTN_OP_SEGMENT_FWD 0
#define SEQATTN_OP_LSE_MERGE 1
#define SEQATTN_OP_DILATED_FWD 2
#define SEQATTN_OP_SEGMENT_BWD 3
#define SEQATTN_OP_DILATED_BWD 4

/*
 * seqattn_attn_segment_fwd -- partial attention of a query block against one
 * KV segment.
 *
 * Passage: "Ultra-Long Sequence Distributed Transformer", Abstract (each GPU
 * computes a partial self-attention for its segment); "Boosting Spec Eagle:
 * USP For Long-Context Training", The Solution (ring devices each hold a
 * slice and exchange only with their neighbours); "DeepSpeed-Ulysses"
 * article, Wie DeepSpeed-Ulysses funktioniert (after the all-to-all a GPU
 * sees the whole sequence for its share, read here as a head subset).
 *
 * q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d]; same dtype (bf16 or fp32).
 * o: [B, Hq, Nq, d], bf16 or fp32 (fp32 required with SEQATTN_ACCUMULATE;
 *    fp32 when q is fp32).  lse: [B, Hq, Nq, 1] fp32.
 * flags: 0 -> o, lse are overwritten with this segment's partial;
 *        SEQATTN_ACCUMULATE -> o, lse hold a running partial (fp32, natural
 *        log; (0, -inf) is the empty partial) and receive the log-sum-exp
 *        merge of it with this segment's partial (fused epilogue).
 * Nq = 0 or Nk = 0 is allowed (an empty segment leaves an accumulator
 * unchanged and writes (0, -inf) otherwise).
 * Errors: NULL, DTYPE, SHAPE (d not 64/128, batch mismatch, Hq % Hkv != 0,
 * lse shape), STRIDE (misalignment, overlapping rows, a tensor spanning 2^56
 * bytes), ALIAS (o or lse overlapping q/k/v), UNSUPPORTED (bf16: one head of
 * q, k or v spanning 2 GiB or more, since the kernels address a head's rows
 * with 32-bit byte offsets; unknown flags), HIP.
 */
int seqattn_attn_segment_fwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, int64_t causal_offset,
                             float softmax_scale, uint32_t flags,
                             seqattn_tensor *o, seqattn_tensor *lse,
                             void *hip_stream);

/*
 * seqattn_attn_segment_fwd_ws -- seqattn_attn_segment_fwd with a caller-owned
 * workspace, for calls too short to fill the GPU (bf16, d = 128, at least
 * 1024 keys, no SEQATTN_ACCUMULATE): when the query block's 256-row tiles
 * are fewer than two per compute unit (causal) or than one (non-causal),
 * each tile's visible keys are cut into 2-8 equal parts (at least 512
 * keys), computed by separate workgroups, whose fp32 partials (O, LSE) go
 * to the workspace and are then merged by their log-sum-exp into o and lse
 * ("Ultra-Long Sequence Distributed Transformer", Abstract: partial
 * attention per segment, combined exactly).  The result equals the unsplit
 * call's up to rounding order; a call the rule does not split runs exactly
 * as seqattn_attn_segment_fwd.
 *
 * workspace: seqattn_workspace_size(SEQATTN_OP_SEGMENT_FWD, q, k, 0) bytes,
 * 16-byte aligned device memory overlapping no tensor of the call (NULL when
 * that size is 0).  Errors: as seqattn_attn_segment_fwd, plus WORKSPACE
 * (missing, too small or misaligned when the call is split) and ALIAS (the
 * workspace overlaps a tensor).
 */
int seqattn_attn_segment_fwd_ws(const seqattn_tensor *q, const seqattn_tensor *k,
                                const seqattn_tensor *v, int64_t causal_offset,
                                float softmax_scale, uint32_t flags, seqattn_tensor *o,
                                seqattn_tensor *lse, void *workspace, size_t workspace_bytes,
                                void *hip_stream);

/*
 * seqattn_lse_merge -- in place acc <- merge(acc, b), row by row:
 *   M = max(La, Lb), wa = exp(La - M), wb = exp(Lb - M),
 *   O = (wa Oa + wb Ob) / (wa + wb), L = M + log(wa + wb);
 *   two empty partials (-inf, -inf) give (0, -inf).
 *
 * Passage: the exactness of segment-by-segment attention ("Ultra-Long
 * Sequence Distributed Transformer", Abstract: partial self-attention per
 * segment; ring attention's per-device slices) requires combining partials
 * by their softmax normalisers; no page prints the formula.
 *
 * o_acc: [B, H, N, d] fp32 (in/out), d a positive multiple of 8;
 * lse_acc: [B, H, N, 1] fp32 (in/out); o_b: same shape, fp32 or bf16;
 * lse_b: fp32.  b must not overlap acc.
 * Errors: NULL, DTYPE, SHAPE, STRIDE, ALIAS, HIP.
 */
int seqattn_lse_merge(seqattn_tensor *o_acc, seqattn_tensor *lse_acc,
                      const seqattn_tensor *o_b, const seqattn_tensor *lse_b,
                      void *hip_stream);

/*
 * seqattn_dilated_attn_fwd -- LongNet dilated attention.
 *
 * Passage: "LongNet: Scaling Transformers to 1,000,000,000 Tokens",
 * Abstract (dilated attention takes the place of dense attention with the
 * same interface) and Results (a mixture of segment lengths w and dilation
 * ratios r).  The page's formula is not legible; the reading implemented:
 * for branch i the sequence is cut into segments of w_i tokens (the last one
 * may be shorter); a position is selected when its offset inside its segment
 * is a multiple of r_i; selected queries attend to the selected keys of the
 * same segment (SEQATTN_CAUSAL: only keys at original positions <= the
 * query's); unselected positions get the empty partial; the branch partials
 * are merged by log-sum-exp.  With SEQATTN_HEAD_SHIFT the offset is h mod
 * r_i for query head h instead of 0 (positions at offset s, s + r_i, ...;
 * its keys use the same offset), so the heads of a branch together cover
 * more positions; LongNet's multi-head variant, which the page's stripped
 * formulas do not show.  The kernels apply the offset per head; only the
 * backward with grouped KV heads takes one launch per query head.
 *
 * q: [B, Hq, N, d] bf16; k, v: [B, Hkv, N, d] bf16; o: [B, Hq, N, d] fp32
 * or bf16; lse: [B, Hq, N, 1] fp32.  segment_lengths[i] >= 1 and
 * dilations[i] >= 1 (host arrays of n_branches >= 1 entries).
 * workspace: when o is bf16, seqattn_workspace_size(SEQATTN_OP_DILATED_FWD)
 * bytes of device memory (an fp32 accumulator); may be NULL when o is fp32.
 * Errors: NULL, DTYPE, SHAPE, STRIDE, ALIAS, WORKSPACE, UNSUPPORTED (a head
 * of q, k or v spanning about 2 GiB, unknown flags), HIP.
 */
int seqattn_dilated_attn_fwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v,
                             const int64_t *segment_lengths,
                             const int64_t *dilations, int32_t n_branches,
                             float softmax_scale, uint32_t flags,
                             seqattn_tensor *o, seqattn_tensor *lse,
                             void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * seqattn_attn_segment_bwd -- gradients of one (query block, KV segment)
 * pair given the GLOBAL forward statistics.
 *
 * Passage: "LongNet: Scaling Transformers to 1,000,000,000 Tokens",
 * Distributed Trainer (in the backward the all-gather of keys/values becomes
 * a reduce-scatter, i.e. each device forms gradients for the keys/values it
 * attended to); "Ultra-Long Sequence Distributed Transformer", Abstract
 * (training over segments).
 *
 * With P_ij = exp(s_ij - LSE_i) (LSE the merged, all-segment value) and
 * D_i = sum_c dO_ic O_ic (O the merged output):
 *   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . v_j - D_i),
 *   dQ_i += sigma sum_j dS_ij k_j,  dK_j = sigma sum_i dS_ij q_i,
 * with dK, dV summed over the query heads sharing a KV head.
 * q, d_o: [B, Hq, Nq, d] bf16; k, v: [B, Hkv, Nk, d] bf16; o: [B, Hq, Nq, d]
 * bf16 or fp32; lse: [B, Hq, Nq, 1] fp32.
 * dq: [B, Hq, Nq, d] fp32, ACCUMULATED (dq += ...), so a sweep over
 * segments sums into it; dk, dv: [B, Hkv, Nk, d] fp32 or bf16, OVERWRITTEN
 * (flags 0) or, with SEQATTN_ACCUMULATE, fp32 and ACCUMULATED.
 * workspace: seqattn_workspace_size(SEQATTN_OP_SEGMENT_BWD) bytes.
 * Errors: NULL, DTYPE, SHAPE, STRIDE, ALIAS, WORKSPACE, UNSUPPORTED (fp32
 * inputs, unknown flags, one head of q, k, v or d_o spanning 2 GiB or more),
 * HIP.
 */
int seqattn_attn_segment_bwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, const seqattn_tensor *o,
                             const seqattn_tensor *lse,
                             const seqattn_tensor *d_o, int64_t causal_offset,
                             float softmax_scale, uint32_t flags,
                             seqattn_tensor *dq, seqattn_tensor *dk,
                             seqattn_tensor *dv, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

/*
 * seqattn_attn_segment_bwd_noalloc -- seqattn_attn_segment_bwd without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.
 *
 * Same arguments, semantics, kernels and results as seqattn_attn_segment_bwd
 * (bit-identical).  The per-row D vector goes to a fixed 16 MiB device array
 * inside the library instead of a workspace, so B * Hq * Nq must not exceed
 * 4,194,304 query rows (else SEQATTN_ERR_WORKSPACE, before any HIP call).
 * Each GPU holds its own copy of that array from the first call on that GPU
 * until the process ends; the call itself allocates nothing.  Every call on
 * one GPU shares the array: calls that may overlap on one GPU (on streams
 * not ordered with each other) race, so order them.  The array keeps the
 * last call's contents; nothing in it needs clearing between calls.
 * Errors: as seqattn_attn_segment_bwd.
 */
int seqattn_attn_segment_bwd_noalloc(const seqattn_tensor *q,
                                     const seqattn_tensor *k,
                                     const seqattn_tensor *v,
                                     const seqattn_tensor *o,
                                     const seqattn_tensor *lse,
                                     const seqattn_tensor *d_o,
                                     int64_t causal_offset,
                                     float softmax_scale, uint32_t flags,
                                     seqattn_tensor *dq, seqattn_tensor *dk,
                                     seqattn_tensor *dv, void *hip_stream);

/*
 * seqattn_dilated_attn_bwd -- gradients of seqattn_dilated_attn_fwd.
 *
 * Passage: "LongNet: Scaling Transformers to 1,000,000,000 Tokens",
 * Abstract and Results (dilated attention, the mixture of (w, r) branches)
 * and Distributed Trainer (training through it; the backward forms the
 * gradients of exactly the keys/values each query attended to).
 *
 * The merged output is one softmax over the union of every branch's keys,
 * each key counted once per branch that lists it, so with the merged LSE and
 * D_i = sum_c dO_ic O_ic, each branch's selected (query, key) pairs take the
 * segment backward above, and the gradients of all branches add up.
 * q, d_o: [B, Hq, N, d] bf16; k, v: [B, Hkv, N, d] bf16; o: [B, Hq, N, d]
 * bf16 or fp32 and lse: [B, Hq, N, 1] fp32, both from the forward with the
 * same (segment_lengths, dilations, flags).  flags: SEQATTN_CAUSAL and/or
 * SEQATTN_HEAD_SHIFT, as in the forward.
 * dq: fp32, ACCUMULATED; dk, dv: [B, Hkv, N, d] fp32, OVERWRITTEN (rows no
 * branch selects get 0).
 * workspace: seqattn_workspace_size(SEQATTN_OP_DILATED_BWD) bytes.
 * Errors: NULL, DTYPE, SHAPE, STRIDE, ALIAS, WORKSPACE, UNSUPPORTED, HIP.
 */
int seqattn_dilated_attn_bwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, const seqattn_tensor *o,
                             const seqattn_tensor *lse,
                             const seqattn_tensor *d_o,
                             const int64_t *segment_lengths,
                             const int64_t *dilations, int32_t n_branches,
                             float softmax_scale, uint32_t flags,
                             seqattn_tensor *dq, seqattn_tensor *dk,
                             seqattn_tensor *dv, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

/*
 * seqattn_head_relayout -- copy every (head, row) vector of src into dst,
 * where the two describe the same heads in different strided layouts.
 *
 * Passage: "DeepSpeed-Ulysses" article, Wie DeepSpeed-Ulysses funktioniert
 * (the sequence is split across GPUs; an all-to-all before attention gives
 * each GPU the whole sequence, and after attention the results are gathered
 * and re-organised).  The re-layouts on either side of that all-to-all are
 * this copy: a rank's [Ns, H, d] shard, seen as b = 1, h = H, n = Ns, goes
 * to its [P][Ns][H/P][d] send buffer, seen as b = P, h = H/P, n = Ns, and
 * back after attention.
 *
 * Flat heads f = b * h + h_index enumerate both sides (src->b * src->h ==
 * dst->b * dst->h); n, d and dtype match; dst[f][row] = src[f][row].
 * d * element size must be a multiple of 16 bytes, dst rows must not
 * overlap each other or src, and one call moves fewer than 2^31 16-byte units.
 * Errors: NULL, DTYPE, SHAPE, STRIDE, ALIAS, UNSUPPORTED, HIP.
 */
int seqattn_head_relayout(const seqattn_tensor *src, seqattn_tensor *dst,
                          void *hip_stream);

/* Bytes of device workspace an op needs for these operands (0 if none).
 * For SEQATTN_OP_DILATED_FWD pass o's descriptor as `k`. */
size_t seqattn_workspace_size(int op, const seqattn_tensor *q,
                              const seqattn_tensor *k, int32_t n_branches);

/* Static description of a status code. */
const char *seqattn_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *seqattn_last_error(void);

int seqattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEQATTN_H */
