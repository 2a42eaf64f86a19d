/*
 * si_indexer.h -- C ABI of the MI355X (gfx950) lightning-indexer top-k library.
 *
 * The operation (StreamIndex abstract, quoted on the aisoku.com page "StreamIndex：
 * ストリーミングTop-kによるメモリ制限付き圧縮スパースアテンション", Abstract): a lightning
 * indexer scores every compressed key for every query and the top-k keys per query are
 * kept, without ever building the [B, S, H_I, T] FP32 score tensor; the selection is a
 * chunked partition-merge top-k (skillsdirectory.com "Streamindex Csa Topk", Core
 * Technique 1 and Implementation Steps 1-4; geoz.com.cn page FAQ: local top-k per block,
 * then a merge of the blocks' lists, no global sort).
 *
 * Score (the pages print no formula; the DeepSeek lightning-indexer form is used):
 *     I[b,t,s] = sum_h w[b,t,h] * max(0, scale[b,s] * sum_d q[b,t,h,d] * kc[b,s,d])
 * with scale = 1 for bf16 keys.  Rounding order on the GPU, identical in every entry
 * point and for every tuning knob: bf16 x bf16 products accumulated in fp32 by one
 * fixed MFMA sequence per head, then acc = fmaf(w_h, max(z_h, 0), acc) for h = 0..H-1
 * starting from +0, then (E4M3 keys) acc * scale[s]; a -0 result is reported as +0.
 * Causal mask: key s is visible to query row r iff (s + 1) * m <= q_pos0 + r + 1.
 * Order: by (score descending, key index ascending), so the top-k is unique.
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE memory owned by the caller, contiguous row-major,
 *    on the device current for the calling thread.  The library never allocates device
 *    memory and never frees caller memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay alive until the stream has passed the call.
 *  - Arguments are validated synchronously, before anything is enqueued.  On an error
 *    status nothing has been enqueued and outputs are untouched; si_last_error()
 *    returns a message for the calling thread.  A launch failure returns SI_ERR_HIP.
 *  - Non-finite inputs (NaN, inf, E4M3 NaN bytes) are outside the contract.
 *  - Thread-safe: the library keeps no mutable global state besides the per-thread
 *    error message.
 */
#ifndef SI_INDEXER_H
#define SI_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SI_ABI_VERSION 1

typedef enum si_status {
    SI_OK = 0,
    SI_ERR_INVALID_ARG = 1,   /* null pointer, negative size, k < 1, m < 1, ...   */
    SI_ERR_UNSUPPORTED = 2,   /* valid but not built: D != 128, H_I > 128, k > 2048, dtype, knob */
    SI_ERR_WORKSPACE = 3,     /* workspace (or score buffer) missing or too small */
    SI_ERR_HIP = 4            /* a HIP launch or runtime call failed              */
} si_status;

typedef enum si_dtype {
    SI_BF16 = 1,              /* bfloat16                                          */
    SI_FP8_E4M3FN = 2         /* OCP FP8 E4M3 (bias 7, no inf, max 448): keys only */
} si_dtype;

/* Tuning knobs; 0 selects the automatic value.  No knob changes any output bit
 * (the pages sweep chunk size, key-tile size and top-k: StreamIndex abstract; the
 * chunk size needs tuning per GPU: "Streamindex Csa Topk", Pitfalls). */
typedef struct si_config {
    int32_t key_tile;       /* keys scored before the running top-k is updated:
                               64, 128, 256, 512, 768 or 1024 (0 = auto)           */
    int32_t query_chunk;    /* query rows per driver step (bounds the workspace);
                               rounded up to a multiple of 32                       */
    int32_t key_partition;  /* keys per partition whose local top-k lists are merged;
                               a multiple of key_tile                               */
    int32_t reserved;       /* must be 0                                            */
} si_config;

/* The plan the driver follows for one problem (all values effective, never 0). */
typedef struct si_plan {
    int32_t key_tile;
    int32_t query_chunk;
    int32_t key_partition;
    int32_t n_partitions;     /* partitions of the widest query row                */
    int32_t n_chunks;         /* driver steps: ceil(S / query_chunk)               */
    int32_t cand_capacity;    /* candidate slots per (query, partition)            */
    int64_t workspace_bytes;  /* bytes si_indexer_topk needs                       */
} si_plan;

/* ABI version (SI_ABI_VERSION of the build). */
int32_t si_abi_version(void);

/* Static description of a status code. */
const char* si_status_str(si_status status);

/* Detail of the last error status returned on the calling thread ("" if none). */
const char* si_last_error(void);

/*
 * si_indexer_plan -- validate the problem shape and knobs and return the plan.
 * Host only: touches no device and enqueues nothing.  Shapes as in si_indexer_topk.
 * out: filled on SI_OK.  cfg may be NULL (all automatic).
 */
si_status si_indexer_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                          int32_t m, int32_t k, int64_t q_pos0, si_dtype kc_dtype,
                          const si_config* cfg, si_plan* out);

/*
 * si_indexer_topk -- streaming top-k of the indexer scores (the hot path).
 *
 *  q         [B, S, H, D] bf16 query rows; row r is absolute position q_pos0 + r
 *  kc        [B, T, D]    compressed keys, bf16 or E4M3 bytes (kc_dtype)
 *  kc_scale  [B, T] fp32  per-key scale for E4M3 keys (> 0); must be NULL for bf16
 *  w         [B, S, H]    fp32 head weights
 *  m         compression ratio (>= 1), used only by the causal mask
 *  k         keys kept per query, 1..2048
 *  q_pos0    absolute position of q row 0 (>= 0): lets a caller stream q in slices
 *  out_idx   [B, S, k] int32  key indices, row sorted by (score desc, index asc);
 *            slots past min(k, n_t) hold -1, where n_t = min(T, (q_pos0+r+1) / m)
 *  out_score [B, S, k] fp32   the matching scores; padded slots hold -inf
 *  workspace device scratch of at least plan.workspace_bytes bytes (see
 *            si_indexer_plan), 256-byte aligned; its contents are clobbered
 *
 * Supported: D = 128, 1 <= H <= 128, 1 <= k <= 2048, q bf16, keys bf16 or E4M3,
 * 0 <= T < 2^31 - 1.  S = 0 or B = 0 is a no-op.
 * Enqueues, per query chunk, the fused score + select kernel and the merge kernel.
 */
si_status si_indexer_topk(const void* q, si_dtype q_dtype,
                          const void* kc, si_dtype kc_dtype, const float* kc_scale,
                          const float* w,
                          int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                          int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                          int32_t* out_idx, float* out_score,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages si_indexer_topk runs for query chunk `chunk` (0 <= chunk <
 * plan.n_chunks), exposed so a caller can time them apart.  Same arguments and
 * validation as si_indexer_topk; si_indexer_topk is exactly select(c) then merge(c)
 * for c = 0 .. n_chunks - 1, on the same stream and workspace.
 *
 * select: scores the chunk's query rows against their visible keys (bf16 MFMA, ReLU,
 *   head-weighted sum, mask) and keeps, per (query, key partition), the exact local
 *   top-k in the workspace (running threshold + candidate buffer, compacted by an
 *   exact radix select): the per-chunk candidates of the pages' data flow
 *   (jeff.news page, sequence diagram).
 * merge: merges each query's partition lists into the final sorted top-k rows of
 *   out_idx / out_score (the merge-topk step of the same diagram).
 */
si_status si_indexer_select_chunk(const void* q, si_dtype q_dtype,
                                  const void* kc, si_dtype kc_dtype, const float* kc_scale,
                                  const float* w,
                                  int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                  int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                                  int32_t chunk, void* workspace, size_t workspace_bytes,
                                  void* stream);

si_status si_indexer_merge_chunk(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                 int32_t m, int32_t k, int64_t q_pos0, si_dtype kc_dtype,
                                 const si_config* cfg, int32_t chunk,
                                 int32_t* out_idx, float* out_score,
                                 const void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * si_materialize_scores -- reference path, score write-out.  Writes the head-summed
 * scores of query rows [row0, row0 + rows) for every batch entry into
 * scores [B, rows, T] fp32, -inf where the key is masked.  Same arithmetic, bit for
 * bit, as the streaming path.  (This is one [rows, T] slice of the head-summed score
 * tensor that public CSA implementations build in full before their top-k: StreamIndex
 * abstract.)  0 <= row0, row0 + rows <= S.
 */
si_status si_materialize_scores(const void* q, si_dtype q_dtype,
                                const void* kc, si_dtype kc_dtype, const float* kc_scale,
                                const float* w,
                                int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                int32_t m, int64_t q_pos0, int64_t row0, int64_t rows,
                                float* scores, void* stream);

/*
 * si_materialize_topk -- reference path: materialise-then-select, row block by row
 * block.  For each block of `row_block` rows: si_materialize_scores into scores_ws,
 * then a per-row exact selection (radix select on the scores, lowest index first among
 * equal scores, rank sort) into out_idx / out_score.  Outputs have the same contract
 * as si_indexer_topk and must be bit-identical to it.
 * scores_ws: device buffer of at least B * row_block * T * 4 bytes.
 */
si_status si_materialize_topk(const void* q, si_dtype q_dtype,
                              const void* kc, si_dtype kc_dtype, const float* kc_scale,
                              const float* w,
                              int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                              int32_t m, int32_t k, int64_t q_pos0,
                              int32_t* out_idx, float* out_score,
                              float* scores_ws, size_t scores_ws_bytes, int64_t row_block,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SI_INDEXER_H */
