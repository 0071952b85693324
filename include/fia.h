/*
 * fia.h - C ABI of the MI355X (gfx950) fused inference attention forward.
 *
 * The operation (page "torch_npu.npu_prompt_flash_attention", function
 * description formula; page "torch_npu.npu_fused_infer_attention_score_v2",
 * function description formula):
 *
 *     attention_out = softmax(scale_value * Q K^T + atten_mask) V
 *     softmax_lse   = log(sum exp(scale_value * Q K^T + atten_mask))   (optional)
 *
 * in three forms:
 *   - prefill (query S > 1, or TND): causal / band / explicit-mask sparse modes,
 *     per-batch actual lengths, BNSD / BSND / BSH / TND layouts, GQA, against
 *     a contiguous or (outside TND) paged KV cache;
 *   - decode (query S == 1 outside TND) against a contiguous or paged KV cache,
 *     with an optional per-(batch, kv token) mask; multi-token decode (query
 *     S up to 16, sparse_mode 3 or 0 without a mask) takes the same split-KV
 *     path while the G * S (head, token) rows of a kv head number at most 16,
 *     the prefill path beyond that;
 *   - block-sparse prefill (page "aclnnBlockSparseAttentionV2"), where a
 *     block mask selects the KV blocks each Q block attends to.
 *
 * Both operators use the two-phase pattern of the aclnn pages
 * ("aclnnFusedInferAttentionScoreV5" and "aclnnBlockSparseAttentionV2",
 * interface description): phase 1 validates every input, plans the launch
 * and returns the workspace size plus an opaque plan (the pages' executor);
 * phase 2 runs the plan on a stream with a caller-owned workspace.
 *
 * Conventions for every entry point:
 *   - Tensor data pointers are DEVICE pointers; tensors are dense row-major
 *     (non-contiguous tensors are not supported, as on the pages).
 *   - Length arrays (actual_seq_*) are HOST pointers, copied in phase 1.
 *   - The plan keeps the tensor pointers: the tensors must stay allocated
 *     until the stream work of the last *_run on that plan has completed.
 *   - Phase 1 launches no kernel.  It uploads the plan's schedule tables
 *     (per-batch offsets and the tile / split order, tens of bytes per tile)
 *     into device memory the plan owns, on the current device, with a
 *     synchronous copy; fia_plan_destroy frees them.  Its host temporaries
 *     live in per-thread buffers that keep their capacity between calls (a
 *     buffer past 64 MB is released after the call), so phase-1 calls on
 *     different threads may run at the same time.  Where no device is
 *     visible, phase 1 still validates and sizes, but the plan cannot run:
 *     phase 2 then returns FIA_ERR_HIP (it never uploads or allocates).
 *   - Phase 2 only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream): it allocates nothing, copies nothing and does not
 *     synchronize.  The workspace holds scratch of one run (decode partial
 *     results, the compacted block-sparse schedule), so two runs in flight
 *     at the same time must not share a workspace.
 *   - Results are deterministic: no atomics, fixed reduction order; two runs
 *     of one plan give bitwise identical outputs ("aclnnFusedInferAttention
 *     ScoreV5", constraints: deterministic computation).
 *   - Every descriptor passed, required or optional, has rank 1..8, dims in
 *     [0, 2^31) and at most 2^48 elements over its non-zero dims;
 *     otherwise phase 1 returns FIA_ERR_SHAPE.
 *   - A phase-1 call that fails sets *plan to NULL and *workspace_size to 0
 *     (where those pointers are given) and owns nothing afterwards.
 *   - Errors are returned as fia_status; nothing is printed.
 */
#ifndef FIA_H_
#define FIA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fia_status {
    FIA_OK = 0,
    FIA_ERR_NULLPTR = 1,     /* a required tensor, pointer or output is missing   */
    FIA_ERR_DTYPE = 2,       /* dtype not allowed or q/k/v dtypes differ          */
    FIA_ERR_SHAPE = 3,       /* rank / dims inconsistent with layout and heads    */
    FIA_ERR_LAYOUT = 4,      /* unknown layout string, or layouts that must match */
    FIA_ERR_PARAM = 5,       /* a scalar parameter outside its allowed range      */
    FIA_ERR_UNSUPPORTED = 6, /* legal on the pages but not provided here          */
    FIA_ERR_WORKSPACE = 7,   /* workspace smaller than planned, or NULL           */
    FIA_ERR_HIP = 8          /* a HIP call failed (launch or copy)                */
} fia_status;

typedef enum fia_dtype {
    FIA_F16 = 0, FIA_BF16 = 1, FIA_F32 = 2, FIA_I8 = 3,
    FIA_U8 = 4, FIA_BOOL = 5, FIA_I32 = 6, FIA_I64 = 7,
    FIA_F8E4M3 = 8           /* FLOAT8_E4M3FN (block-sparse FP8 inputs) */
} fia_dtype;

/* A dense row-major tensor: dims[0] is the slowest axis. */
typedef struct fia_tensor {
    void*   data;        /* device pointer */
    int32_t dtype;       /* fia_dtype */
    int32_t ndim;        /* 1..8 */
    int64_t dims[8];
} fia_tensor;

typedef struct fia_plan fia_plan;   /* opaque; owned by the library */

/*
 * Parameters of the fused inference attention (names and defaults of the
 * parameter description of "torch_npu.npu_fused_infer_attention_score_v2").
 */
typedef struct fia_params {
    /* "BSH" (default), "BSND", "BNSD" or "TND" (input_layout).  BSH is
     * [B, S, N*D]; BSND [B, S, N, D]; BNSD [B, N, S, D]; TND [T, N, D]. */
    const char* input_layout;
    int64_t num_heads;            /* Q_N; must match the query's N axis          */
    int64_t num_key_value_heads;  /* KV_N; 0 = Q_N.  Q_N % KV_N == 0 and
                                     Q_N / KV_N <= 64 (GQA: query head h uses kv
                                     head h / (Q_N / KV_N))                        */
    double  scale_value;          /* softmax_scale, default 1.0                   */
    int64_t pre_tokens;           /* default 2147483647; band width before i     */
    int64_t next_tokens;          /* default 2147483647; band width after i      */
    /* sparse_mode (default 0), with delta_b = Lkv_b - Lq_b:
     *   0  no mask, or full mask + top-left band -pre <= j-i <= next
     *   1  full mask only
     *   2  top-left causal        j <= i
     *   3  bottom-right causal    j <= i + delta_b
     *   4  bottom-right band      -pre <= j - i - delta_b <= next
     * Modes 5-8 are unsupported on the pages and rejected (FIA_ERR_PARAM).
     * Ignored when the query S is 1 outside TND (decode). */
    int64_t sparse_mode;
    /* PageAttention block size (block_size); 0 = contiguous KV.  With a
     * block_table and query S == 1 it must be a positive multiple of 16
     * (int8 key/value: of 32); with query S > 1 a multiple of 128 in
     * [128, 512]; with a TND query 128, 512 or 1024 (page attention scenario
     * and TND constraints of the v2 page). */
    int64_t block_size;
    /* inner_precise 0..3 (bit0 precision/performance, bit1 row-invalid
     * correction).  Accepted; softmax is always computed in fp32 and rows
     * with no allowed key always give out = 0, lse = +inf. */
    int64_t inner_precise;
    int32_t return_softmax_lse;   /* 0 / 1 (default 0)                          */
    /* actual_seq_qlen / actual_seq_kvlen: host int64 arrays.  NULL = the
     * tensor's S.  Count 1 broadcasts to every batch; a count >= B takes the
     * first B.  For TND they are required and cumulative (non-decreasing, the
     * count is the batch).  Paged KV requires actual_seq_kvlen. */
    const int64_t* actual_seq_qlen;
    int64_t        n_actual_seq_qlen;
    const int64_t* actual_seq_kvlen;
    int64_t        n_actual_seq_kvlen;
    /* KV pseudo-quantization (kv pseudo-quant parameters and their
     * constraints, v2 page): int8 key and value with a bf16 query and output
     * and query S <= 16 (S > 1: sparse_mode 3, or 0 without a mask, with
     * G * S <= 16, contiguous KV only).  At query S 1 the cache may also be
     * paged (block_table, block_size a multiple of 32, either pool layout;
     * page attention scenario of the query S 1 constraints).  A cached value
     * x stands for scale * (x + offset).  key_quant_mode / value_quant_mode:
     *   0  per channel: scale / offset bf16 [KV_N, D] or [KV_N * D];
     *   1  per token:   scale / offset fp32 [B, KV_S'], indexed by the
     *      logical kv position, KV_S' >= the key's S (paged: >= the longest
     *      actual_seq_kvlen); both per token: one shape for key and value.
     * The two modes must be equal, except key 0 with value 1 at query S 1
     * (FIA_ERR_PARAM otherwise); modes 2..5 (per tensor / per head, and the
     * scales managed by page attention) are legal at query S 1 and return
     * FIA_ERR_UNSUPPORTED; at query S > 1 only 0 and 1 are legal.
     * Offsets are optional (NULL = 0) and take their scale's shape and dtype.
     * Both scales are required for int8 key/value and must be NULL for
     * fp16/bf16 key/value (FIA_ERR_PARAM).  The plan keeps the pointers. */
    const fia_tensor* dequant_scale_key;
    const fia_tensor* dequant_scale_value;
    const fia_tensor* dequant_offset_key;
    const fia_tensor* dequant_offset_value;
    int64_t key_quant_mode;
    int64_t value_quant_mode;
    /* MLA (query_rope / key_rope parameters of the v2 page and their
     * constraints for a query D of 512): both given or both NULL
     * (FIA_ERR_PARAM for one alone).  The score of query row i and key j
     * becomes scale * (q_i . k_j + q_rope_i . k_rope_j); value and output
     * keep D = 512.  Provided here: query D 512 and rope D 64, fp16 or bf16
     * (the rope inputs take the query's dtype), layouts BSH / BSND / BNSD
     * (query_rope the query's layout with D = 64), query S 1..16 (S > 1:
     * sparse_mode 3 or 4, S == 1: sparse_mode 0 without a mask or 4; mode 4
     * is the bottom-right band pre_tokens / next_tokens, also at S == 1, with
     * the 2048 template or NULL as atten_mask), or TND with
     * cumulative actual_seq_qlen (1..16 tokens per batch), actual_seq_kvlen
     * holding each batch's own length and sparse_mode 0 (no mask) or 3, Q_N in
     * {1, 2, 4, ..., 128}, KV_N 1, a paged cache (block_table required) with
     * block_size 16, 64 or 128 and key_rope a pool of the key's layout with D 64.
     * value is its own pool of the key's shape, or the key tensor itself
     * (same pointer: then the value bytes are not read a second time).
     * softmax_lse is computed as for any other call.  Errors: a rope dtype
     * other than the query's FIA_ERR_DTYPE; rope shapes that do not match
     * FIA_ERR_SHAPE; another block_size, or Q_N / KV_N above 128,
     * FIA_ERR_PARAM; other head dims, KV_N, Q_N, S, layouts, modes, masks,
     * int8 key/value or a contiguous cache FIA_ERR_UNSUPPORTED. */
    const fia_tensor* query_rope;
    const fia_tensor* key_rope;
} fia_params;

/* Fill `p` with the defaults listed above (layout "BSH", scale 1.0,
 * pre/next 2147483647, everything else 0). */
void fia_params_init(fia_params* p);

/*
 * Phase 1 of the fused inference attention (pages "aclnnFusedInferAttention
 * ScoreV5" and "torch_npu.npu_fused_infer_attention_score_v2").
 *
 *   query        [B,S,H] / [B,S,N,D] / [B,N,S,D] / [T,N,D], fp16 or bf16.
 *   key, value   same layout and dtype as query with KV_N heads; D of value
 *                may differ from D of key (TND: (192,192,128)).  With a
 *                block_table they are the paged pool, either
 *                [blocknum, KV_N, block_size, D] or [blocknum, block_size, KV_N*D].
 *   atten_mask   optional, bool/int8/uint8, nonzero = masked.  Modes 0/1:
 *                [Q_S,KV_S], [B|1,Q_S,KV_S] or [B|1,1,Q_S,KV_S] (the last axis may
 *                be padded past KV_S).  Modes 2/3/4: the 2048x2048 lower-
 *                triangular template ([2048,2048], [1,2048,2048] or
 *                [1,1,2048,2048]) or NULL; its contents are not read (the mask
 *                follows from the indices).  Query S == 1 (decode): one
 *                value per (batch, kv token), [B|1,KV_S], [B|1,1,KV_S] or
 *                [B|1,1,1,KV_S] (v2 atten_mask description); sparse_mode and
 *                pre/next do not apply there.  With a paged cache KV_S must
 *                cover maxBlockNumPerSeq * block_size.
 *   block_table  optional int32 [B, >= max blocks per sequence]: PageAttention
 *                block ids (page attention scenario of the v2 page): kv token
 *                j of batch b is row j % block_size of pool block
 *                block_table[b][j / block_size].  Any query S; with a TND
 *                query the table has one row per sequence (the count of
 *                actual_seq_qlen) and actual_seq_kvlen stays cumulative
 *                (except for MLA: see query_rope in fia_params).
 *                Ids are not checked: each referenced id must be in
 *                [0, blocknum), as the page requires; entries past
 *                ceil(Lkv_b / block_size) are never read.
 *   attention_out same shape as query with D = value's D, same dtype.
 *   softmax_lse  fp32 [B, Q_N, Q_S, 1] (TND: [T, Q_N, 1]); required when
 *                return_softmax_lse, else ignored.
 *   workspace_size, plan: outputs.  *plan must later go to fia_plan_destroy.
 *
 * An empty query, or an empty attention_out, returns FIA_OK with
 * *workspace_size = 0 and a plan whose run does nothing.  A batch whose kv
 * length is 0 gets out = 0 and lse = +inf.
 */
fia_status fia_get_workspace_size(const fia_tensor* query, const fia_tensor* key,
                                  const fia_tensor* value, const fia_tensor* atten_mask,
                                  const fia_tensor* block_table, const fia_params* params,
                                  const fia_tensor* attention_out,
                                  const fia_tensor* softmax_lse,
                                  uint64_t* workspace_size, fia_plan** plan);

/*
 * Phase 2: run `plan` on `stream` (a hipStream_t, NULL = default) with a
 * device workspace of at least the planned size (may be NULL when that size
 * is 0).  Returns FIA_ERR_WORKSPACE if it is too small, FIA_ERR_HIP if a
 * launch fails or phase 1 ran where no device was visible.  The plan may be
 * run any number of times.
 */
fia_status fia_run(void* workspace, uint64_t workspace_size, fia_plan* plan, void* stream);

/*
 * Block-sparse attention parameters (page "aclnnBlockSparseAttentionV2",
 * constraints).
 */
typedef struct bsa_params {
    const char* q_input_layout;    /* "TND" | "BNSD" | "BSND"                     */
    const char* kv_input_layout;   /* must equal q_input_layout                   */
    int64_t num_heads;             /* N1 (query heads)                            */
    int64_t num_key_value_heads;   /* N2; N1 >= N2, N1 % N2 == 0; 0 = N1          */
    double  scale_value;           /* default 1.0                                 */
    int64_t block_shape[2];        /* [X, Y]: 0 < X, Y < 2^31 and Y % 128 == 0    */
    /* Host int64 arrays, both or neither; required for TND (cumulative). */
    const int64_t* actual_seq_lengths;
    int64_t        n_actual_seq_lengths;
    const int64_t* actual_seq_lengths_kv;
    int64_t        n_actual_seq_lengths_kv;
    int64_t mask_type;             /* must be 0                                   */
    int64_t block_size;            /* must be 0 (no paged cache)                  */
    int64_t inner_precise;         /* must be 4 (mixed precision)                 */
    int64_t pre_tokens;            /* must be 2147483647                          */
    int64_t next_tokens;           /* must be 2147483647                          */
    int32_t softmax_lse_flag;      /* 0 / 1                                       */
    /* FP8 inputs (FP8 feature of the block-sparse page): query, key and value
     * all FLOAT8_E4M3FN, each element standing for value * its block's scale.
     * Scales fp32, required for FP8 inputs and NULL otherwise (FIA_ERR_PARAM):
     *   query  [B, N1, ceil(maxQS / 128), 1]   (block_shape[0] must be 128)
     *   key / value  [B, N2, ceil(maxKVS / Y), 1], Y = block_shape[1] = 256 or 512.
     * The output is bf16; D must be 128. */
    const fia_tensor* dequant_scale_query;
    const fia_tensor* dequant_scale_key;
    const fia_tensor* dequant_scale_value;
} bsa_params;

/* Defaults: layouts "BNSD", scale 1.0, block_shape [128,128], inner_precise 4,
 * pre/next 2147483647, everything else 0. */
void bsa_params_init(bsa_params* p);

/*
 * Phase 1 of block-sparse attention ("aclnnBlockSparseAttentionV2").
 *
 *   query, key, value  same layout (BNSD / BSND / TND) and dtype (fp16 / bf16,
 *                      or FLOAT8_E4M3FN with the dequant scales of bsa_params),
 *                      D of 64 or 128 (FP8: 128), equal for q, k and v.
 *   block_sparse_mask  required, uint8 or bool [B, N1, ceil(maxQS / X),
 *                      ceil(maxKVS / Y)]; nonzero = the kv block is selected for
 *                      that query head and q block.  Device tensor.
 *   atten_mask, block_table  must be NULL.
 *   attention_out      same shape as query; its dtype (bf16 for FP8 inputs).
 *   softmax_lse        fp32 [B, N1, Sq, 1] (TND [T, N1, 1]) when softmax_lse_flag.
 *
 * Attention inside the selected blocks is full (no causal mask); rows past
 * the q length and keys past the kv length are masked; the sequence lengths
 * need not be multiples of the block shape.
 */
fia_status bsa_get_workspace_size(const fia_tensor* query, const fia_tensor* key,
                                  const fia_tensor* value, const fia_tensor* block_sparse_mask,
                                  const fia_tensor* atten_mask, const fia_tensor* block_table,
                                  const bsa_params* params, const fia_tensor* attention_out,
                                  const fia_tensor* softmax_lse,
                                  uint64_t* workspace_size, fia_plan** plan);

/* Phase 2 of block-sparse attention; same contract as fia_run. */
fia_status bsa_run(void* workspace, uint64_t workspace_size, fia_plan* plan, void* stream);

/*
 * Allocation-free phase 2, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): runs a plan from either phase-1 call, like fia_run / bsa_run,
 * with the library's own static device scratch of
 * FIA_NOALLOC_MAX_WORKSPACE bytes as the workspace.  That array exists once
 * per GPU (each GPU the library runs on holds it until the process ends);
 * its device address is looked up once per device, with that device
 * current: by the first phase-1 call that uploads a plan there, else by the
 * first call of this function there.  The call allocates nothing, copies nothing and does
 * not synchronize; the caller still owns every input and output the plan
 * names.
 *   - Plans whose workspace size exceeds FIA_NOALLOC_MAX_WORKSPACE return
 *     FIA_ERR_WORKSPACE (nothing is launched).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents: calls that overlap on one GPU (different streams, or
 *     work not yet complete on another stream) race and must be ordered by
 *     the caller.  No kernel needs the scratch cleared: each run writes every
 *     scratch byte it reads.
 *   - FIA_ERR_HIP if the scratch address cannot be resolved or a launch
 *     fails.
 * bsa_schedule_layout offsets then refer to this scratch, which the caller
 * cannot address; use bsa_run with an own workspace to inspect a schedule.
 */
#define FIA_NOALLOC_MAX_WORKSPACE ((uint64_t)32 << 20)
fia_status fia_run_noalloc(fia_plan* plan, void* stream);

/*
 * Where bsa_run leaves the compacted block schedule inside the workspace
 * after it has run: int32 cnt[B, N1, nqb] at *cnt_offset and int32
 * idx[B, N1, nqb, nkb] at *idx_offset (byte offsets).  idx lists, per
 * (batch, query head, q block), the selected kv blocks below
 * ceil(Lkv_b / Y) in ascending order, followed by -1.  For inspection only.
 */
fia_status bsa_schedule_layout(const fia_plan* plan, uint64_t* cnt_offset,
                               uint64_t* idx_offset, int64_t* nqb, int64_t* nkb);

/* Release a plan from either phase-1 call.  NULL is a no-op. */
void fia_plan_destroy(fia_plan* plan);

/* Static, human-readable name of a status code. */
const char* fia_status_string(fia_status s);

#ifdef __cplusplus
}
#endif

#endif /* FIA_H_ */
