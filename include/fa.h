/*
 * fa.h - C ABI of the MI355X (gfx950) attention forward library libfa.so.
 *
 * What every entry point computes, per output row r with key set K_r:
 *
 *   s_j   = scale * <q_r, k_j>                          for j in K_r
 *   O_r   = sum_j softmax(s)_j * v_j                     (stored in q's dtype)
 *   LSE_r = ln sum_j exp(s_j)                            (fp32)
 *
 * evaluated tile by tile with an online softmax: a running row reference
 * maximum m, a running row sum l of exp(s - m) and an output accumulator
 * rescaled by exp(m_old - m_new) whenever m moves. This is the
 * standard-vs-tiled attention equivalence and the loop invariant of the
 * "FlashAttention correctness verification" page (sections on the tiled
 * computation and on formal verification). When m moves is set by a rescale
 * threshold t in log2 units, as on the flash-attention SM100 sparse-MLA page
 * (background and threshold-branch sections): m moves to a tile's row max
 * when that exceeds m by more than t. t = 0 is the exact running maximum
 * (every growth rescales; the largest weight of a row is exactly 1 before the
 * P.V product); t > 0 is the lazy rescale (weights up to 2^t, fewer
 * rescales). Both give the same O and LSE up to rounding. Rows whose key set
 * is empty produce O_r = 0 and LSE_r = -inf.
 *
 * Numerics: Q.K^T and P.V run on MFMA with fp32 accumulation; for fp16/bf16
 * inputs P is rounded to the input dtype (round to nearest even) before P.V
 * while the row sum l accumulates the unrounded fp32 p; O = acc / l is rounded
 * to the output dtype. fp32 inputs keep P in fp32.
 *
 * Conventions shared by all entry points
 *  - Tensors are described by fa_tensor: a device pointer, dtype, rank,
 *    shape and strides in ELEMENTS. The last dimension must be contiguous
 *    (stride 1). Row strides of Q/K/V/O must keep every row 16-byte aligned
 *    (multiples of 8 elements for 16-bit types, 4 for fp32) and the data
 *    pointers must be 16-byte aligned.
 *  - The caller owns every buffer. The library allocates nothing, keeps no
 *    pointer after returning and has no global mutable state except a
 *    thread-local error string.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without waiting. The caller synchronises.
 *  - Arguments are validated on the host before anything is launched. On any
 *    error nothing is launched, the status is returned and fa_last_error()
 *    describes it. No C++ exception crosses this interface.
 *  - A problem with no output rows (B, Hq, Sq or T equal to 0) returns FA_OK
 *    and launches nothing.
 *  - Unchecked preconditions (documented, not validated because they live in
 *    device memory): indices inside their range or negative; valid indices
 *    distinct within one row / list; seqlens[b] <= the sequence length.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
  FA_F32 = 0,
  FA_F16 = 1,
  FA_BF16 = 2,
  FA_U8 = 3,
  FA_I32 = 4
} fa_dtype;

typedef struct fa_tensor {
  void* data;        /* device pointer (may be NULL only when the tensor is empty) */
  int32_t dtype;     /* an fa_dtype value */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];  /* shape[0..ndim) */
  int64_t stride[4]; /* strides in elements; the last one must be 1 */
} fa_tensor;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_DTYPE = 2,       /* wrong or mismatched dtype */
  FA_ERR_SHAPE = 3,       /* rank or extents do not fit together */
  FA_ERR_STRIDE = 4,      /* non-contiguous last dim, misaligned pointer or row */
  FA_ERR_UNSUPPORTED = 5, /* valid request outside what this build implements */
  FA_ERR_VALUE = 6,       /* non-finite scale, bad flag, bad block size value */
  FA_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} fa_status;

/*
 * Dense attention forward, with optional causal mask, boolean mask, GQA head
 * broadcast and per-batch sequence lengths.
 *
 *  q    [B, Hq, Sq, D]   fp32 / fp16 / bf16 (BNSD, strided)
 *  k    [B, Hkv, Skv, D] same dtype as q; Hq % Hkv == 0; query head h reads
 *                        KV head h / (Hq / Hkv) (the GQA layout of the
 *                        ops-transformer pytest page, section 5.1)
 *  v    [B, Hkv, Skv, Dv] same dtype; Dv == D
 *  mask NULL, or uint8 [Sq, Skv] shared by every batch and head, or
 *       uint8 [B|1, Hq|1, Sq, Skv] (size-1 dims broadcast; their stride is
 *       ignored). Non-zero = the position is excluded (the atten_mask
 *       convention of the Ascend FlashAttentionScore README, parameter table).
 *  seqlens_q, seqlens_k  NULL or int32 [B]: rows i >= seqlens_q[b] have no
 *       keys (O = 0, LSE = -inf); keys j >= seqlens_k[b] are excluded (the
 *       per-batch actual_seq_lengths of the PyPTO BSA README, section 1).
 *  causal  0 or 1. Key j is excluded when j > i + (Lk - Lq), Lq/Lk being the
 *       (sequence-length-cut) query/key lengths: bottom-right alignment.
 *  scale   finite float > 0 multiplying q.k (the scale of the attention
 *       formula); scale * log2(e) must be a normal float.
 *  rescale_threshold  in [0, 10], log2 units: 0 = exact running max (the
 *       contract path); the sparse-MLA page's lazy value for the forward
 *       is 8 (its threshold-selection section).
 *  o    [B, Hq, Sq, Dv] in q's dtype (BNSD, strided)
 *  o_lo NULL, or fp32 [B, Hq, Sq, Dv] (strided, rows 16-byte aligned): on
 *       return it holds fp32(O) - rounded(O) per element, the rounding
 *       residual of the output, so that o + o_lo is the unrounded fp32 result
 *       (the o_lo output and its use for a precise dpsum on the sparse-MLA
 *       page, order-invariance-test and impact-on-backward sections). Only
 *       for fp16 / bf16 outputs.
 *  lse  fp32 [B, Hq, Sq], contiguous; natural-log LSE of the scaled scores.
 *
 * Supported: D == Dv in {64, 128}; K/V row strides up to 2^22 elements.
 * Masked/excluded keys are never read
 * into the P.V product with a non-zero weight.
 */
fa_status fa_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                 const fa_tensor* mask, const fa_tensor* seqlens_q,
                 const fa_tensor* seqlens_k, int causal, float scale,
                 float rescale_threshold, const fa_tensor* o, const fa_tensor* o_lo,
                 const fa_tensor* lse, void* stream);

/*
 * Block-sparse attention forward (the Mask2Idx block lists of the PyPTO BSA
 * README, sections 1 and 3.2, read here directly by the kernel instead of
 * being compacted into new K/V tensors).
 *
 *  q, k, v, o, lse as in fa_fwd (same dtypes, GQA rule and layouts).
 *  block_idx  int32 [nQB, maxSel] shared by every batch and KV head, or
 *       int32 [B|1, Hkv|1, nQB, maxSel]; nQB >= ceil(Sq / block_q).
 *       Row qb lists the KV blocks that query block qb attends to; a slot
 *       holding a negative value is unused and contributes nothing (it may
 *       sit anywhere in the list). Valid entries must lie in
 *       [0, ceil(Skv / block_k)) and be distinct within a row (unchecked).
 *  block_q, block_k  must both be 128.
 *  seqlens  NULL or int32 [B], applied to queries and keys alike: rows
 *       i >= seqlens[b] produce O = 0 and LSE = -inf, keys j >= seqlens[b]
 *       are excluded.
 *  rescale_threshold as in fa_fwd.
 *  maxSel must be <= 256.
 */
fa_status fa_fwd_blocksparse(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                             const fa_tensor* block_idx, int block_q, int block_k,
                             const fa_tensor* seqlens, float scale,
                             float rescale_threshold, const fa_tensor* o,
                             const fa_tensor* lse, void* stream);

/*
 * Top-k gathered sparse attention forward with one shared KV head (the
 * sparse-MLA forward of the flash-attention SM100 page, background section:
 * every row attends only to its W indexer-chosen keys). The running maximum
 * is always exact (rescale threshold 0), so the largest weight of a row is
 * exactly 1 before the P.V product.
 *
 *  q   [T, Hq, Dqk] fp16 / bf16 (strided; last dim contiguous)
 *  k   [S, Dqk] same dtype (the latent+rope key rows)
 *  v   [S, Dv] same dtype; may alias k (v.data == k.data with the same row
 *      stride, i.e. V = the first Dv columns of K, the MLA latent)
 *  idx int32 [T, W], last dim contiguous; idx[t, s] in [0, S) names a key,
 *      negative = unused slot (anywhere in the row). An index >= S is not
 *      detected; it reads key row S - 1 (never memory outside k or v).
 *  o   [T, Hq, Dv] in q's dtype (strided)
 *  o_lo NULL, or fp32 [T, Hq, Dv] (strided, rows 16-byte aligned): the
 *      output's rounding residual fp32(O) - rounded(O), as in fa_fwd
 *  lse fp32 [T, Hq], contiguous
 *
 * Supported: Dqk == 576, Dv == 512, any Hq >= 1 (query heads are processed
 * 32 per wave; a partial last group is padded, as the sparse-MLA page's
 * background section pads query heads to the tile, and its padding heads
 * store nothing), W <= 4096, and k and v each spanning less than 4 GiB
 * ((S - 1) * row stride + row length, in bytes: the gathers use 32-bit byte
 * offsets). Rows with no valid index give O = 0 and LSE = -inf.
 */
fa_status fa_fwd_topk_gather(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                             const fa_tensor* idx, float scale, const fa_tensor* o,
                             const fa_tensor* o_lo, const fa_tensor* lse, void* stream);

/*
 * Attention backward (dense, optional causal and boolean masks, GQA): the gradients of the
 * dense forward's O with respect to q, k and v, given dO. Defined by the
 * backward formulas of the ops-transformer FlashAttentionScoreGrad pytest page
 * (section 5.2: dV = P^T dO, dS = P * (dP - rowsum(dP * P)), dQ = scale dS K,
 * dK = scale dS^T Q) with P recomputed from the forward's LSE as in the PyPTO
 * BSA README (section 3); dK and dV are summed over the query heads of each KV
 * head (BSA README, section 1).
 *
 *  q, k, v     as fa_fwd (f16 or bf16, D == Dv, 64 or 128)
 *  mask        NULL or a boolean mask in one of fa_fwd's forms (non-zero =
 *              excluded); P is 0 at excluded positions, so they receive no
 *              gradient (the atten_mask input of the FlashAttentionScoreGrad
 *              page, section 5.2)
 *  seqlens_q, seqlens_k  NULL or int32 [B], as fa_fwd: rows i >= seqlens_q[b]
 *              and keys j >= seqlens_k[b] take part in nothing, and their
 *              gradients dq / dk / dv are written as zeros (the per-batch
 *              boundary mask of the PyPTO BSA README, section 3.2)
 *  o           the forward output for these q, k, v, mask, lengths, causal,
 *              scale
 *  o_lo        NULL, or the forward's fp32 rounding residual of o (fa_fwd's
 *              o_lo): Delta = dO . (o + o_lo), the precise dpsum of the
 *              sparse-MLA page (order-invariance-test section)
 *  lse         fp32 [B, Hq, Sq], contiguous: the forward's LSE
 *  dout        [B, Hq, Sq, Dv], q's dtype: the gradient of the output
 *  causal      0 or 1, as fa_fwd (bottom-right aligned)
 *  scale       as fa_fwd
 *  delta       fp32 [B, Hq, Sq], contiguous, caller-owned workspace; on
 *              return it holds Delta = dO . O per row (dO . (O + o_lo) with
 *              o_lo)
 *  dq, dk, dv  outputs shaped like q, k, v in q's dtype (written, not
 *              accumulated into)
 *  ds_workspace  NULL, or a caller-owned rank-1 tensor in q's dtype, 16-byte
 *              aligned, of at least fa_bwd_ds_workspace_elems(B, Hq, Sq, Skv)
 *              elements (contents on return unspecified). With it the dK/dV
 *              kernel stores dS (rounded to q's dtype, as it enters the dK
 *              product) and dQ = scale dS K is a product over that stored
 *              dS; without it the dQ kernel recomputes S and dP. The results
 *              agree up to rounding (dV is identical).
 *
 * Every tensor's rows must start 16-byte aligned (as fa_fwd). Rows without
 * keys (LSE = -inf) contribute nothing. Returns FA_ERR_UNSUPPORTED for other
 * head dims or fp32; the library allocates nothing. It enqueues on `stream`
 * two kernels without ds_workspace (dQ with Delta, then dK and dV), three
 * with it (Delta, dK and dV storing dS, then dQ).
 */
fa_status fa_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* mask,
                 const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, const fa_tensor* o,
                 const fa_tensor* o_lo, const fa_tensor* lse, const fa_tensor* dout, int causal, float scale,
                 const fa_tensor* delta, const fa_tensor* dq, const fa_tensor* dk,
                 const fa_tensor* dv, const fa_tensor* ds_workspace, void* stream);

/*
 * Elements of fa_bwd's optional dS workspace for these sizes (for
 * fa_bwd_varlen: B = number of sequences, Sq / Skv = max_seqlen_q /
 * max_seqlen_k): B * Hq * (Sq256 * Skv32 + 4 * Sq32), with SqN and Skv32 the
 * lengths rounded up to a multiple of N and 32: dS of every query head in
 * contiguous 32 x 32 blocks, then two fp32 values per row (the dK/dV
 * kernel's start values of S and dP). -1 for negative sizes.
 */
int64_t fa_bwd_ds_workspace_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv);

/*
 * Attention backward over a batch of packed variable-length sequences (the
 * TND layout in which the ops-transformer FlashAttentionScoreGrad pytest page,
 * section 5.4, runs the gradient operator: unpad_input packs the sequences
 * and cu_seqlens marks their bounds). Per sequence exactly fa_bwd on its own
 * rows and keys, with the formulas of that page's section 5.2; the causal
 * mask is bottom-right aligned per sequence.
 *
 *  q, k, v     [Tq, Hq, D], [Tk, Hkv, D], [Tk, Hkv, Dv] as fa_fwd_varlen
 *              (f16 or bf16, D == Dv, 64 or 128)
 *  cu_seqlens_q, cu_seqlens_k  device int32 [B + 1], as fa_fwd_varlen
 *              (non-decreasing, first entry 0, last entry <= Tq / Tk;
 *              unchecked, they live in device memory; offsets past the
 *              tensors are clamped to their last row, so no memory outside
 *              them is touched)
 *  max_seqlen_q, max_seqlen_k  >= the longest query and key sequence
 *              (rows or keys of a longer sequence past them are treated as
 *              absent)
 *  o, o_lo, lse  the forward's outputs for these inputs (fa_fwd_varlen's
 *              o [Tq, Hq, Dv] and lse fp32 [Tq, Hq], contiguous; o_lo NULL
 *              or fp32 shaped like o, for the precise Delta as fa_bwd)
 *  dout        [Tq, Hq, Dv], q's dtype
 *  causal, scale  as fa_fwd_varlen
 *  delta       fp32 [Tq, Hq], contiguous, caller-owned workspace (holds
 *              Delta per row on return)
 *  dq, dk, dv  outputs shaped like q, k, v in q's dtype (written, not
 *              accumulated into)
 *  ds_workspace  NULL, or as fa_bwd's, sized by fa_bwd_ds_workspace_elems(B,
 *              Hq, max_seqlen_q, max_seqlen_k) (each sequence's dS is stored
 *              padded to the longest lengths)
 *
 * Rows and keys outside every sequence are not written. A sequence without
 * keys gets dq = 0 for its rows, one without rows dk = dv = 0 for its keys.
 * No boolean mask in this form. The library allocates nothing and enqueues
 * two kernels on `stream` (three with ds_workspace, as fa_bwd).
 */
fa_status fa_bwd_varlen(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                        const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k, int max_seqlen_q,
                        int max_seqlen_k, const fa_tensor* o, const fa_tensor* o_lo, const fa_tensor* lse,
                        const fa_tensor* dout, int causal, float scale, const fa_tensor* delta,
                        const fa_tensor* dq, const fa_tensor* dk, const fa_tensor* dv,
                        const fa_tensor* ds_workspace, void* stream);

/*
 * Dense attention forward over a batch of packed variable-length sequences
 * (the TND layout of the ops-transformer FlashAttentionScoreGrad pytest page,
 * section 5.4, where unpad_input packs the sequences and cu_seqlens marks
 * their bounds; the Ascend FlashAttentionScore README lists TND among the
 * input layouts). Batch b's queries are rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 of q and attend to rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1 of k and v: per sequence exactly fa_fwd on its own
 * rows and keys (causal bottom-right aligned per sequence).
 *
 *  q    [Tq, Hq, D]  fp16 / bf16 (strided, last dim contiguous)
 *  k    [Tk, Hkv, D] same dtype; Hq % Hkv == 0 (GQA as fa_fwd)
 *  v    [Tk, Hkv, Dv] same dtype; Dv == D in {64, 128}
 *  cu_seqlens_q, cu_seqlens_k  device int32 [B + 1], non-decreasing, first
 *       entry 0, last entry <= Tq / Tk (unchecked: they live in device
 *       memory)
 *  max_seqlen_q  >= the longest query sequence; rows of a longer sequence
 *       past it are not computed (their o and lse are left as they were)
 *  causal, scale, rescale_threshold  as fa_fwd
 *  o    [Tq, Hq, Dv] in q's dtype; lse fp32 [Tq, Hq], contiguous
 *
 * Query rows outside every sequence are not written. A sequence with no
 * keys gives O = 0 and LSE = -inf.
 */
fa_status fa_fwd_varlen(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                        const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k,
                        int max_seqlen_q, int causal, float scale, float rescale_threshold,
                        const fa_tensor* o, const fa_tensor* lse, void* stream);

/*
 * Split-KV dense attention forward, for few query rows over many keys (the
 * grid of fa_fwd then has too few workgroups to fill the GPU). The keys are
 * cut into ranges; every (range, row block, head) computes the online
 * softmax over its range alone and leaves a normalised fp32 partial output
 * O_s and its LSE_s in `workspace`; a second kernel combines the ranges as
 * partial softmax states (the merge of the "FlashAttention correctness
 * verification" page, standard-vs-tiled section):
 *   LSE = logsumexp_s LSE_s,   O = sum_s exp(LSE_s - LSE) O_s.
 * Results equal fa_fwd's up to rounding.
 *
 *  q, k, v, seqlens_q, seqlens_k, causal, scale, rescale_threshold, o, lse
 *       as fa_fwd (fp16 / bf16 only; no boolean mask)
 *  num_splits  0 = chosen by the library (fa_fwd_splitkv_splits), else the
 *       requested number of key ranges, <= 64; each range is a multiple of
 *       192 keys, so fewer ranges may result
 *  workspace   fp32, rank 1, 16-byte aligned, caller-owned, with at least
 *       fa_fwd_splitkv_workspace_elems(...) elements; its contents on return
 *       are unspecified. Not read when a single range results (then the call
 *       is fa_fwd and workspace may be NULL).
 */
fa_status fa_fwd_splitkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                         const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, int causal,
                         float scale, float rescale_threshold, int num_splits,
                         const fa_tensor* workspace, const fa_tensor* o, const fa_tensor* lse,
                         void* stream);

/*
 * fa_fwd_splitkv without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The partial results go to a static
 * device array of the library, 64 MiB (16M fp32) per GPU, held from the
 * first call on that GPU until the process ends; its address is looked up
 * once per device. Arguments and results as fa_fwd_splitkv. A problem whose
 * partial results exceed the array (num_splits * B * Hq * Sq * (Dv + 1)
 * floats, with num_splits as fa_fwd_splitkv_splits resolves it) returns
 * FA_ERR_UNSUPPORTED and launches nothing. Every call on one GPU shares the
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller. Nothing in the array needs to start
 * at zero (every partial result a merge reads is written by the same call).
 */
fa_status fa_fwd_splitkv_noalloc(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                                 const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, int causal,
                                 float scale, float rescale_threshold, int num_splits,
                                 const fa_tensor* o, const fa_tensor* lse, void* stream);

/* Number of key ranges fa_fwd_splitkv uses for these sizes and num_splits
 * (-1 for negative sizes). With num_splits = 0: ceil(256 / W) ranges, W =
 * ceil(Sq / 256) * B * Hq the workgroups of one range, so that each of the
 * 256 compute units gets one workgroup; at most max(1, Skv / 384) and 64.
 * Ranges are then rounded up to multiples of 192 keys and those past the
 * keys dropped. */
int fa_fwd_splitkv_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int num_splits);

/* fp32 elements of the workspace fa_fwd_splitkv needs (0 when a single key
 * range results; -1 for invalid sizes). */
int64_t fa_fwd_splitkv_workspace_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int64_t Dv,
                                       int num_splits);

/* Static, human-readable name of a status code. */
const char* fa_status_str(fa_status s);

/* Detail of the last error returned on this thread ("" if none). Valid until
 * the next call into the library on the same thread. */
const char* fa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
