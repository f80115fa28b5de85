/*
 * fia.h - fused inference attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfia.so.  Plain pointers and sizes only.
 *
 * The operator computes, per batch b, query head h and query row i,
 *
 *     out[b,i,h,:] = softmax_j( scale * q[b,i,h,:] . k[b,j,g,:] + bias(h,i,j) ) v[b,j,g,:]
 *
 * over the keys j that the mask mode leaves visible, with g = h / (Q_N / KV_N)
 * (aclnnFusedInferAttentionScoreV5 and V2, "Formula"; V4 "Formula" adds the
 * ALiBi full mask after scaling; V2 "numKeyValueHeads" restrictions for GQA).
 * A query length of 1 is the incremental-decode branch, anything else the
 * prompt branch (V2 function description).  The optional softmax LSE output is
 * max + ln(sum exp(s - max)) per row (V2, softmaxLse restrictions).
 *
 * The call is two-phase, as on the pages (V5 / V2 "function prototype"):
 *   1. fia_get_workspace_size() validates every argument, classifies the call,
 *      plans the work and returns the workspace size and an executor;
 *   2. fia_run() enqueues the kernels on a HIP stream.
 *
 * Conventions shared by every entry point
 *   - Tensor data pointers are DEVICE pointers; the caller owns them and keeps
 *     them valid until the enqueued work completes.  Host arrays (lengths) are
 *     copied into the executor during phase 1.
 *   - fia_tensor strides are in elements; the innermost dimension must be
 *     contiguous (stride 1).  Any other strides are honoured.
 *   - Phase 1 never touches the GPU.  It returns FIA_ERR_PARAM_INVALID for an
 *     argument that breaks a rule stated on the pages, FIA_ERR_UNSUPPORTED for
 *     a legal feature this library does not implement, FIA_ERR_NULLPTR for a
 *     missing required pointer.  fia_last_error() describes the failure.
 *   - fia_run() returns FIA_ERR_WORKSPACE when the workspace is NULL with a
 *     non-zero required size or smaller than the required size, and
 *     FIA_ERR_HIP when a HIP call fails.
 *   - Block ids in block tables are not validated, as on the pages (V2 page
 *     attention scenario); an id outside [0, n_blocks) is clamped into range,
 *     so it yields unspecified values but never an out-of-bounds access.
 *   - Results are deterministic: repeated calls give bitwise-identical output,
 *     and the output of one batch entry does not depend on the other entries
 *     (V4 / V2 deterministic computation; sparse_flash_mla batch invariance).
 *   - An executor may be run any number of times, from one thread at a time,
 *     until fia_executor_destroy().
 */
#ifndef FIA_H_
#define FIA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FIA_SUCCESS = 0,
  FIA_ERR_NULLPTR = 1,
  FIA_ERR_PARAM_INVALID = 2,
  FIA_ERR_UNSUPPORTED = 3,
  FIA_ERR_WORKSPACE = 4,
  FIA_ERR_HIP = 5
} fia_status;

typedef enum {
  FIA_DT_BF16 = 0,
  FIA_DT_FP16 = 1,
  FIA_DT_FP32 = 2,
  FIA_DT_FP8_E4M3FN = 3,
  FIA_DT_INT32 = 4,
  FIA_DT_INT64 = 5,
  FIA_DT_UINT8 = 6,
  FIA_DT_INT8 = 7,
  FIA_DT_BOOL = 8
} fia_dtype;

/* A strided view of device memory.  Unused trailing shape/stride slots are
 * ignored.  data may be NULL only when the tensor holds zero elements. */
typedef struct {
  void* data;
  int32_t dtype;      /* fia_dtype */
  int32_t ndim;       /* 1..5 */
  int64_t shape[5];
  int64_t stride[5];  /* in elements */
} fia_tensor;

typedef struct fia_executor fia_executor;

/* Attributes of the dense / paged operator (aclnnFusedInferAttentionScoreV5
 * and V2 parameter lists, restricted to the supported feature groups). */
typedef struct {
  /* Layout of query and attention_out, and of key/value when not paged:
   * "BSND" [B,S,N,D], "BSH" [B,S,N*D], "BNSD" [B,N,S,D] or "TND" [T,N,D].
   * With TND the actual lengths are cumulative (V5 ActualSeqLen group). */
  const char* input_layout;
  int32_t num_heads;            /* Q_N, 1..256 */
  int32_t num_key_value_heads;  /* KV_N; 0 means Q_N.  Q_N % KV_N == 0, Q_N/KV_N <= 64 */
  double scale_value;           /* softmax scale, typically 1/sqrt(D) */
  /* Mask mode (V5 Attention Mask group; V2 sparseMode rules):
   *   0 all keys visible (no mask tensor)      2 left-up causal   j <= i
   *   3 right-down causal j <= i + (Lk - Lq)    4 band:
   *     i + (Lk-Lq) - pre_tokens <= j <= i + (Lk-Lq) + next_tokens
   * Modes 0 and 1 with an atten_mask tensor: key j of query row i is kept
   * only when mask[b or 0][i][j] == 0 (1 = masked out); mode 1 requires the
   * tensor, mode 0 without it keeps every key j < Lk.  For modes 2-4 the mask
   * is generated from its definition; an atten_mask tensor, if passed, must
   * be the 2048x2048 lower-triangular form and is not read. */
  int32_t sparse_mode;
  int64_t pre_tokens;           /* default 2147483647 */
  int64_t next_tokens;          /* default 2147483647; -next_tokens <= pre_tokens */
  /* pse_type 0: no positional bias, or, with a pse_shift tensor, that
   * tensor added element-wise to the scaled scores (V5 PSE group; see
   * pse_shift below).  pse_type 2: ALiBi, pse_shift is fp32 [Q_N]
   * slopes and bias(h,i,j) = slope[h] * ((kv_start_idx + j) - (q_start_idx + i)),
   * which requires S1 == S2 and equal per-batch lengths (V5 PSE group).
   * pse_type 3 is unsupported (no formula on the pages); 1 is training-only. */
  int32_t pse_type;
  int64_t q_start_idx;          /* |kv_start_idx - q_start_idx| <= 1048576 */
  int64_t kv_start_idx;
  int32_t block_size;           /* paged KV only: > 0, multiple of 16, <= 1024 (<= 512 when S1 == 1 and D is not 64/128) */
  int32_t inner_precise;        /* 0..3 accepted; softmax always runs in fp32 with invalid-row correction */
  int32_t softmax_lse_flag;     /* 1: write softmax_lse */
  /* Host arrays, copied during phase 1 (V2 actualSeqLengths / Kv).  NULL
   * means every batch uses the tensor's S.  Length 1 broadcasts, length >= B
   * uses the first B entries; TND requires exactly B cumulative entries. */
  const int64_t* actual_seq_lengths;
  int64_t actual_seq_lengths_len;
  const int64_t* actual_seq_lengths_kv;
  int64_t actual_seq_lengths_kv_len;
  /* Memory order of the paged key / value pools (V5 Paged Attention group,
   * KV cache layouts); ignored without block_table.  NULL or "PA_ND" (also
   * "BnBsH"): [n_blocks, block_size, KV_N, D] or [n_blocks, block_size,
   * KV_N*D].  "BnNBsD": [n_blocks, KV_N, block_size, D], each KV head's rows
   * of a block contiguous. */
  const char* kv_layout;
  /* NULL, or the learnable sink (V5 LearnableSink group): one logit per
   * query head, bf16 [Q_N] like the query, contiguous.  It joins every
   * row's softmax as one more term with a zero value vector and is not
   * multiplied by the scale: out = sum_j e^(s_j) v_j / (sum_j e^(s_j) +
   * e^(sink[h])), and the LSE includes it (a live row with no visible key
   * then gives 0 and LSE sink[h]; an empty key / value tensor still gives 0
   * and +inf).  Requires inner_precise 0 and no pse (pse_type 0 without a
   * pse_shift tensor).  Device memory, read during phase 2. */
  const fia_tensor* learnable_sink;
  /* Fake-quantised key / value (V5 quantisation parameter group, fake-quant
   * scenario): key and value hold int8 or float8 e4m3fn codes (both the
   * same), the query bf16; a code c is used as scale * (c + offset).
   * Supported for query length 1 (the decode branch), D 64 / 128, without
   * pse, explicit mask or learnable sink.  Modes (key, value): (0, 0) per
   * channel, (1, 1) per token, (0, 1) key per channel and value per token;
   * modes 2-6 are FIA_ERR_UNSUPPORTED.
   *   per channel: scale bf16 (fp32 in mode (0, 1)) of shape (1, N, 1, D),
   *     (1, N, D), (1, H), (N, 1, D), (N, D) or (H) with N = KV_N, H = KV_N*D,
   *     contiguous; or (1): one scale for the whole tensor (int8 only).
   *   per token: scale fp32 (B, >= S2) or (1, B, >= S2), S2 the key length
   *     (block_table cols * block_size when paged), shared by the KV heads;
   *     the last dim contiguous, the batch stride and the last extent
   *     multiples of 4 and the data 16-byte aligned (else UNSUPPORTED).
   * Offsets: NULL or the scale's dtype and shape, both key and value or
   * neither, int8 only.  Paged: block_size a multiple of 32, <= 512. */
  int32_t key_antiquant_mode;
  int32_t value_antiquant_mode;
  const fia_tensor* key_antiquant_scale;
  const fia_tensor* value_antiquant_scale;
  const fia_tensor* key_antiquant_offset;
  const fia_tensor* value_antiquant_offset;
  /* KV lengths resident on the device (the SharedKV and sparse_flash_mla
   * metadata operators likewise balance the work on the device before the
   * main kernels): int32 [B], contiguous, device memory.  Decode (query
   * length 1): read at run time by a partitioner kernel that writes the
   * per-batch records and the split-KV chunk list into the workspace.
   * Prompt (query length > 1, e.g. a chunk of prompt against a paged
   * cache): the work items are planned for the bound and each reads its
   * entry's length on the device.  A caller whose
   * lengths live on the GPU then needs no host copy and no synchronisation
   * per step, and one executor serves any lengths up to the bound (also
   * under HIP graph replay).  Each length is clamped into
   * [0, max_actual_seq_length_kv]; the bound (host, >= 0) sizes the grid and
   * the workspace and must fit the key extent (KV_S, or block_table cols *
   * block_size).  Requires actual_seq_lengths_kv == NULL, BSND / BSH /
   * BNSD (no TND), a bf16 query with bf16 key / value (or, in decode,
   * fake-quantised int8 / e4m3fn key / value), no ALiBi and no atten_mask or
   * pse_shift tensor (PARAM_INVALID / UNSUPPORTED otherwise).
   * Results equal those of the host-planned executor for the same lengths,
   * bit for bit.  NULL: lengths from actual_seq_lengths_kv as above. */
  const fia_tensor* actual_seq_lengths_kv_device;
  int64_t max_actual_seq_length_kv;
} fia_params;

/* Phase 1 of the dense / paged operator.
 *   query           [B,S1,Q_N,D] (per input_layout), bf16 or fp32.
 *   key, value      same layout [B,S2,KV_N,D]; or, when block_table is given,
 *                   pools in params->kv_layout: PA_ND [n_blocks, block_size,
 *                   KV_N, D] (also accepted as [n_blocks, block_size,
 *                   KV_N*D]) or BnNBsD [n_blocks, KV_N, block_size, D]; same
 *                   dtype as query.
 *                   key and value may be the same tensor.
 *   pse_shift       NULL, or fp32 [Q_N] slopes when pse_type == 2, or, when
 *                   pse_type == 0, a bias [B or 1, Q_N, P_S1, >= KV_S] in
 *                   the query's dtype with P_S1 >= Q_S or P_S1 == 1 (one row
 *                   for every query row); score(b,h,i,j) = scale * q.k +
 *                   pse[b or 0][h][i or 0][j], indexed by the position inside
 *                   the actual lengths.  Last dim contiguous; batch, head and
 *                   row strides, the last extent and the base (in elements)
 *                   multiples of 4, else FIA_ERR_UNSUPPORTED; not with TND.
 *                   Needs scale_value > 0 (the prefill kernel carries the
 *                   bias as bias / scale in its fp32 score accumulators).
 *   atten_mask      modes 0 / 1: NULL or int8 / uint8 / bool [B or 1, >= Q_S,
 *                   >= KV_S], [B or 1, 1, >= Q_S, >= KV_S] or [>= Q_S, >= KV_S]
 *                   (KV_S = block_table cols * block_size when paged), rows
 *                   contiguous and 4-byte aligned (KV extent padded to a
 *                   multiple of 4); not with TND.  Modes 2-4: NULL or the
 *                   2048x2048 causal mask (unread).
 *   block_table     NULL, or int32 [B, >= ceil(max Lk / block_size)]; requires
 *                   actual_seq_lengths_kv (V5 Paged Attention group).
 *   attention_out   same shape and layout as query, same dtype.
 *   softmax_lse     fp32 [B,Q_N,S1,1] (TND: [T,Q_N,1]) when softmax_lse_flag,
 *                   otherwise ignored (may be NULL).
 * Rows past a batch's actual query length, and rows with no visible key, are
 * written as 0 with LSE +inf (V4 empty-tensor rules; V2 invalid-row
 * correction).  On success *executor must later be destroyed. */
fia_status fia_get_workspace_size(const fia_params* params,
                                  const fia_tensor* query, const fia_tensor* key,
                                  const fia_tensor* value, const fia_tensor* pse_shift,
                                  const fia_tensor* atten_mask, const fia_tensor* block_table,
                                  const fia_tensor* attention_out, const fia_tensor* softmax_lse,
                                  size_t* workspace_size, fia_executor** executor);

/* Attributes of the shared-KV sparse decode operator (KvQuantSparseAttnSharedkv
 * parameter table; sparse_flash_mla SWA / CSA / HCA modes). */
typedef struct {
  double softmax_scale;
  int32_t kv_quant_mode;   /* 1: per-tile quantised nope (the only mode) */
  int32_t tile_size;       /* 64 */
  int32_t rope_head_dim;   /* 64 */
  int32_t cmp_ratio;       /* 4: compressed-sparse (cmp_kv + cmp_sparse_indices);
                            * 128: heavily compressed (cmp_kv, no indices);
                            * 1: sliding window only (no cmp_kv) */
  int32_t ori_mask_mode;   /* 4 (band) */
  int32_t cmp_mask_mode;   /* 3 (right-down causal) */
  int32_t ori_win_left;    /* 127 */
  int32_t ori_win_right;   /* 0 */
  const char* layout_q;    /* "BSND" (default) or "TND" */
  const char* layout_kv;   /* "PA_ND" */
  int32_t return_softmax_lse; /* must be 0 (reserved on the page) */
} fia_sparse_params;

/* Phase 1 of the shared-KV sparse attention: attention over the sliding
 * window of ori_kv (SWA), plus the top-k selected rows of cmp_kv (CSA), or
 * plus every row of the compressed sequence (HCA).  The S1 query tokens of a
 * batch entry are the last S1 positions of its KV sequence (token t at
 * p = Lk - S1 + t): its window is rows max(0, p - 127) .. p, and it sees the
 * compressed rows c < floor(Lk / cmp_ratio) - (S1 - 1 - t) (right-down
 * causal over the compressed sequence).  With layout_q "TND" the query
 * tokens of all entries are packed into T1 rows and entry b owns rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 (its S1 is their count).
 *   q                  bf16 [B,S1,N1,512] (BSND, B * S1 <= 65535) or
 *                      [T1,N1,512] (TND, T1 <= 65535), N1 in {64,128};
 *                      logical dim order [rope(64) | nope(448)].
 *   ori_kv, cmp_kv     uint8 (or fp8_e4m3fn) PA_ND pools [n_blk, bs, 1, 640]:
 *                      per row bf16 rope x64 | e4m3fn nope x448 | fp32 scale x7
 *                      (one per 64-wide tile) | zero pad to 640 bytes.
 *   ori_sparse_indices must be NULL (reserved on the page).
 *   cmp_sparse_indices int32 [B,S1,1,K2] (BSND) or [T1,1,K2] (TND), K2 in
 *                      {512,1024}, rows contiguous;
 *                      entry c of token t is used iff 0 <= c and c is visible
 *                      to t (above).  NULL with cmp_kv: heavily compressed
 *                      mode, every compressed row visible to t is used
 *                      (max_seqused_kv / 128 + 128 <= 4096).
 *   ori_block_table    int32 [B, >= ceil(max Lk / bs1)].
 *   cmp_block_table    int32 [B, >= ceil(floor(max Lk / cmp_ratio) / bs2)].
 *   cu_seqlens_q       TND only (NULL with BSND): int32 [B+1] device,
 *                      cumulative query-token counts, non-decreasing, first
 *                      0 and last T1 (SharedKV cu_seqlens_q).  Read on the
 *                      device only; a row outside every entry (inconsistent
 *                      counts) is written as 0.
 *   seqused_kv         int32 [B] device, KV length per batch (Lk).
 *   max_seqused_kv     host upper bound of seqused_kv, for table validation.
 *   sinks              fp32 [N1]: one extra logit per head with a zero value.
 *   metadata           ignored (the plan is built here), may be NULL.
 *   attention_out      bf16, the shape of q.
 * K~ = V~ = window rows of ori_kv followed by the used cmp_kv rows. */
fia_status fia_sparse_get_workspace_size(const fia_sparse_params* params,
                                         const fia_tensor* q, const fia_tensor* ori_kv,
                                         const fia_tensor* cmp_kv,
                                         const fia_tensor* ori_sparse_indices,
                                         const fia_tensor* cmp_sparse_indices,
                                         const fia_tensor* ori_block_table,
                                         const fia_tensor* cmp_block_table,
                                         const fia_tensor* cu_seqlens_q,
                                         const fia_tensor* seqused_kv, int64_t max_seqused_kv,
                                         const fia_tensor* sinks, const fia_tensor* metadata,
                                         const fia_tensor* attention_out,
                                         size_t* workspace_size, fia_executor** executor);

/* Attributes of sparse_flash_mla (sparse_flash_mla parameter list: the same
 * shared-KV sparse attention over unquantised fp16 / bf16 rows). */
typedef struct {
  double softmax_scale;
  /* Mode (sparse_flash_mla function description and SWA / CSA / HCA
   * constraints):
   *   1: SWA, sliding window over ori_kv only (no cmp_kv, cmp_mask_mode 0);
   *   4: CSA, plus the cmp_sparse_indices rows of cmp_kv;
   *   128: HCA, plus every row of cmp_kv (no indices).
   * With cmp_kv, cmp_mask_mode must be 3 (right-down causal). */
  int32_t cmp_ratio;
  int32_t ori_mask_mode;   /* 4 (band) */
  int32_t cmp_mask_mode;   /* 3 with cmp_kv, 0 without */
  int32_t ori_win_left;    /* 127 */
  int32_t ori_win_right;   /* 0 */
  const char* layout_q;    /* "BSND" (default) or "TND" */
  /* "PA_BBND" (default): paged pools [n_blocks, block_size, 1, 512],
   * block_size 1..1024, through ori_block_table / cmp_block_table; or equal
   * to layout_q: "BSND" [B, S2, 1, 512] / "TND" [T2, 1, 512] with entry b's
   * rows starting at cu_seqlens_ori_kv[b] / cu_seqlens_cmp_kv[b]. */
  const char* layout_kv;
  int32_t return_softmax_lse;   /* 1: write softmax_lse */
} fia_sfmla_params;

/* Phase 1 of sparse_flash_mla: the operator of fia_sparse_get_workspace_size
 * (same row sets, same S1 / TND rules) over unquantised rows.
 *   q                  fp16 or bf16 [B,S1,N1,512] (BSND, B * S1 <= 65535) or
 *                      [T1,N1,512] (TND, T1 <= 65535), N1 a power of two in
 *                      1..128.
 *   ori_kv, cmp_kv     the dtype of q, rows of 512 values (KV_N = 1) in
 *                      params->layout_kv; cmp_kv NULL in the SWA mode.
 *   ori_sparse_indices, seqused_q   must be NULL (reserved on the page).
 *   cmp_sparse_indices CSA only: int32 [B,S1,1,K2] or [T1,1,K2], K2 >= 1,
 *                      rows contiguous; entry c of token t is used iff
 *                      0 <= c and c is visible to t.
 *   ori_block_table, cmp_block_table   PA_BBND only: int32 [B, >= ceil(max
 *                      Lk / bs1)] and [B, >= ceil(floor(max Lk / cmp_ratio)
 *                      / bs2)].
 *   cu_seqlens_q       TND query only: int32 [B+1] device (as above).
 *   cu_seqlens_ori_kv, cu_seqlens_cmp_kv   TND KV only: int32 [B+1] device,
 *                      first packed row of each entry (non-decreasing).
 *   seqused_kv         int32 [B] device, KV length per batch (Lk).
 *   max_seqused_kv     host upper bound of seqused_kv.
 *   sinks              NULL, or fp32 [N1]: one extra logit per head with a
 *                      zero value vector (the shared-KV reading).
 *   metadata           ignored, may be NULL.
 *   attention_out      the dtype and shape of q.
 *   softmax_lse        with return_softmax_lse: fp32 [B,1,S1,N1] (BSND) or
 *                      [1,T1,N1] (TND), natural-log LSE of each (token, head)
 *                      row including the sink; a row with no key row and no
 *                      sink gives 0 and +inf.  Otherwise ignored.
 * The window plus the K2 (or compressed) slots must not exceed 8192 per
 * query token (FIA_ERR_UNSUPPORTED). */
fia_status fia_sparse_flash_mla_get_workspace_size(
    const fia_sfmla_params* params, const fia_tensor* q, const fia_tensor* ori_kv,
    const fia_tensor* cmp_kv, const fia_tensor* ori_sparse_indices,
    const fia_tensor* cmp_sparse_indices, const fia_tensor* ori_block_table,
    const fia_tensor* cmp_block_table, const fia_tensor* cu_seqlens_q,
    const fia_tensor* cu_seqlens_ori_kv, const fia_tensor* cu_seqlens_cmp_kv,
    const fia_tensor* seqused_q, const fia_tensor* seqused_kv, int64_t max_seqused_kv,
    const fia_tensor* sinks, const fia_tensor* metadata, const fia_tensor* attention_out,
    const fia_tensor* softmax_lse, size_t* workspace_size, fia_executor** executor);

/* Phase 2: enqueue the planned work on `stream` (a hipStream_t; NULL is the
 * default stream).  `workspace` is device memory of at least the size phase 1
 * returned (may be NULL when that size is 0); it is scratch and its contents
 * need not survive between calls.  Asynchronous: returns after enqueueing.
 * The first run of an executor on a device allocates a small device copy of
 * the plan (per-batch lengths and the work list) and uploads it
 * synchronously; later runs on that device only launch kernels, so a run
 * can be captured into a HIP graph once the executor has run once outside
 * the capture.  The copy is freed by fia_executor_destroy(). */
fia_status fia_run(void* workspace, size_t workspace_size, fia_executor* executor,
                   void* stream);

/* Phase 2 for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Runs `executor` exactly as fia_run does (same kernels, bitwise-identical
 * results), but takes no workspace: the executor's plan (copied there on
 * `stream` with hipMemcpyAsync) and its workspace live in a static device
 * array of 64 MiB that the library holds on every GPU it runs on until the
 * process ends (1 MiB for the plan, 63 MiB for the workspace).  Allocates
 * nothing (no hipMalloc / hipFree, no allocating library call).
 *   - FIA_ERR_UNSUPPORTED when the executor's plan exceeds 1 MiB or the
 *     workspace size phase 1 returned exceeds 63 MiB (fia_last_error()
 *     names the sizes); fia_run has no such limit.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; calls that overlap on one GPU (other streams, other
 *     threads) race and must be serialised by the caller.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress, with that device current); FIA_ERR_HIP if that
 *     fails. */
fia_status fia_run_no_alloc(fia_executor* executor, void* stream);

/* Release an executor (NULL is ignored). */
void fia_executor_destroy(fia_executor* executor);

/* Message describing the last non-success status returned on this thread. */
const char* fia_last_error(void);

/* Which kernel path an executor takes: 0 fill-only (empty input),
 * 1 prompt (prefill), 2 incremental decode (split-KV), 3 shared-KV sparse
 * (both sparse operators), 4 fp32 reference-precision path. */
int32_t fia_executor_kind(const fia_executor* executor);

/* Test support: gather through the same device address function the decode
 * and prefill kernels use.  Writes key (which = 0) or value (which = 1) rows
 * 0..Lk_b-1 of every batch into dst, a dense [B, S2max, KV_N, D] buffer of
 * the key dtype (S2max = max Lk); rows past Lk_b are left untouched. */
fia_status fia_debug_gather_kv(fia_executor* executor, void* workspace, size_t workspace_size,
                               int32_t which, void* dst, void* stream);

/* Measurement support: the read-rate ceiling of a split-KV decode plan's
 * access pattern.  Reads every visible key and value row of the plan's
 * chunks once, as the decode kernels would (16-byte non-temporal loads, the
 * same block-table lookups), computes nothing but an XOR of the words read,
 * and writes one uint32 per workgroup to out.
 *   order 0: a workgroup per (chunk, KV head), one head's row (D * element
 *            size bytes, 128 or 256) per request: the decode kernels' order.
 *   order 1: a workgroup per (chunk, 128 keys), a token's whole row of KV_N
 *            heads (1024 or 2048 contiguous bytes) per request; pools whose
 *            heads of one token are adjacent (PA_ND, dense BSND).
 * *out_len: in, the capacity of out (words); out, the number written.  With
 * out == NULL only *out_len is set (to the number the call would write).
 * PARAM_INVALID for executors other than a host-planned split-KV decode,
 * UNSUPPORTED for shapes outside the two orders' sizes. */
fia_status fia_debug_read_kv(fia_executor* executor, void* workspace, size_t workspace_size,
                             int32_t order, uint32_t* out, int64_t* out_len, void* stream);

/* Machine-peak probes, the measured roofline denominators beside the
 * published peaks (each returns after enqueueing on `stream`):
 *   fia_peak_mfma_bf16: n_workgroups x 4 waves, each running `iters`
 *     iterations of 8 independent v_mfma_f32_32x32x16_bf16 on register
 *     operands (n_workgroups * 4 * iters * 8 * 32768 flops, no memory
 *     traffic); writes one float per thread to out[n_workgroups * 256].
 *   fia_peak_hbm_read: streams `bytes` (a multiple of 16, 16-byte aligned
 *     device memory) once with 16-byte non-temporal loads, n_workgroups x 256
 *     threads taking contiguous 32 KiB blocks in turn; writes one uint32 per
 *     thread to out[n_workgroups * 256].
 * PARAM_INVALID for non-positive counts or misaligned sizes. */
fia_status fia_peak_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, void* stream);
fia_status fia_peak_hbm_read(const void* buf, size_t bytes, int32_t n_workgroups, uint32_t* out,
                             void* stream);

/* Test support for the sparse executors: for every query row (BSND: batch
 * entry b, token t; TND: packed token r), the row list the kernel attends
 * to, as fixed slots [B, S1, n_slots] or [T1, n_slots]: ids_out[.., s] = j
 * for window row j of ori_kv, (1 << 30) | c for row c of cmp_kv, -1 for an
 * unused slot; rows_out[.., s, :] = the raw bytes of that row (640 per
 * packed row, 1024 per fp16 / bf16 row; zero when unused).  n_slots is
 * returned through *n_slots_out (ids_out may be NULL to query it). */
fia_status fia_debug_sparse_rows(fia_executor* executor, void* workspace, size_t workspace_size,
                                 int32_t* ids_out, uint8_t* rows_out, int32_t* n_slots_out,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FIA_H_ */
