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
 * with scale = 1 for bf16 keys, the per-row fp32 scale for E4M3 keys, and for MXFP4
 * keys kc[b,s,d] = E2M1 * 2^(E8M0 of d's block - 127) with scale = 1.  Operands:
 *   q bf16 x keys bf16 or E4M3 (E4M3 widened exactly to bf16): bf16 MFMA;
 *   q E4M3 x keys E4M3 or MXFP4: the f8f6f4 MFMA (lower indexer precision: jeff.news
 *   page, 기술 맥락; MXFP4 indexer keys: chengshu page, 部署视角).  E4M3 q is q
 *   quantised per (row, head) with its scale folded into w (si_quantize_q_e4m3), so
 *   w is then the effective weight w * q_scale.
 * Rounding order on the GPU, identical in every entry point and for every tuning knob
 * of one operand pair: the products (exact in fp32) accumulated by one fixed MFMA
 * sequence per head, then acc = fmaf(w_h, max(z_h, 0), acc) for h = 0..H-1 starting
 * from +0, then (E4M3 keys) acc * scale[s]; a -0 result is reported as +0.
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
 *    error message and the per-device address of si_indexer_topk_noalloc's scratch
 *    (looked up once, under a lock).
 */
#ifndef SI_INDEXER_H
#define SI_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SI_ABI_VERSION 2

typedef enum si_status {
    SI_OK = 0,
    SI_ERR_INVALID_ARG = 1,   /* null pointer, negative size, k < 1, m < 1, ...   */
    SI_ERR_UNSUPPORTED = 2,   /* valid but not built: D != 128, H_I > 128, k > 2048, dtype, knob */
    SI_ERR_WORKSPACE = 3,     /* workspace (or score buffer) missing or too small */
    SI_ERR_HIP = 4            /* a HIP launch or runtime call failed              */
} si_status;

typedef enum si_dtype {
    SI_BF16 = 1,              /* bfloat16                                          */
    SI_FP8_E4M3FN = 2,        /* OCP FP8 E4M3 (bias 7, no inf, max 448): q or keys */
    SI_MXFP4_E2M1 = 3         /* OCP MXFP4: E2M1 elements, two per byte (element 2i
                                 in the low nibble of byte i), one E8M0 scale byte
                                 per 32 elements: keys only, with E4M3 q           */
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
 * si_indexer_topk_workspace_bytes -- bytes of workspace si_indexer_topk needs for a
 * problem whose first q row is absolute position 0 (q_pos0 = 0) with the knobs cfg
 * (NULL = all automatic): the same value as si_indexer_plan(...).workspace_bytes.
 * The workspace holds one query chunk's candidate lists (plan.cand_capacity + 64 keys
 * of 8 bytes per query and partition, a 4-byte count and a 16-byte keep rule), so its
 * size is bounded by
 * the chunk, not by S (chunked partition-merge: skillsdirectory.com "Streamindex Csa
 * Topk", Implementation Steps 1-3).  A caller streaming q in slices with q_pos0 > 0
 * uses si_indexer_plan, whose plan depends on q_pos0.  Host only.
 * Returns SIZE_MAX when the arguments are invalid or not built (si_last_error()
 * explains); 0 when there is nothing to do (B = 0 or S = 0).
 */
size_t si_indexer_topk_workspace_bytes(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                       int32_t m, int32_t k, const si_config* cfg);

/*
 * si_indexer_topk -- streaming top-k of the indexer scores (the hot path).
 *
 *  q         [B, S, H, D] query rows, bf16 or E4M3 bytes (q_dtype); row r is absolute
 *            position q_pos0 + r
 *  kc        [B, T, D]    compressed keys, bf16 or E4M3 bytes (kc_dtype), or
 *            [B, T, D/2]  MXFP4 packed E2M1 codes
 *  kc_scale  E4M3 keys: [B, T] fp32 per-key scale (> 0); MXFP4 keys: [B, T, D/32]
 *            E8M0 bytes (4-byte aligned); must be NULL for bf16 keys
 *  w         [B, S, H]    fp32 head weights (E4M3 q: the effective w * q_scale)
 *  m         compression ratio (>= 1), used only by the causal mask
 *  k         keys kept per query, 1..2048
 *  q_pos0    absolute position of q row 0 (>= 0): lets a caller stream q in slices
 *  out_idx   [B, S, k] int32  key indices, row sorted by (score desc, index asc);
 *            slots past min(k, n_t) hold -1, where n_t = min(T, (q_pos0+r+1) / m)
 *  out_score [B, S, k] fp32   the matching scores; padded slots hold -inf
 *  workspace device scratch of at least plan.workspace_bytes bytes (see
 *            si_indexer_plan), 256-byte aligned; its contents are clobbered
 *
 * Supported: D = 128, 1 <= H <= 128, 1 <= k <= 2048, 0 <= T < 2^31 - 1, and the
 * operand pairs (q, keys): (bf16, bf16), (bf16, E4M3), (E4M3, E4M3), (E4M3, MXFP4).
 * S = 0 or B = 0 is a no-op.
 * Enqueues, per query chunk, the fused score + select kernel and the merge kernel.
 */
si_status si_indexer_topk(const void* q, si_dtype q_dtype,
                          const void* kc, si_dtype kc_dtype, const void* kc_scale,
                          const float* w,
                          int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                          int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                          int32_t* out_idx, float* out_score,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * si_indexer_topk_noalloc -- si_indexer_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and outputs, bit for bit, with the workspace taken
 * from a static device array of SI_NOALLOC_SCRATCH_BYTES bytes inside the library
 * instead of a caller buffer.  No call here allocates or frees memory.
 *
 *  - The array exists once per device and is held until the process ends; its device
 *    address is looked up on the first call on each device.
 *  - The automatic query chunk (cfg NULL or query_chunk 0) is the largest whose
 *    workspace fits the array.  A problem that does not fit even at 32 query rows per
 *    chunk, or an explicit query_chunk that does not fit, returns SI_ERR_WORKSPACE
 *    with the sizes in si_last_error().
 *  - Every call on a device shares that device's array and leaves its contents behind:
 *    calls that overlap on one device (different streams or threads, with no ordering
 *    between them) race and give undefined results.  Calls ordered on one stream are
 *    safe.  Nothing in the array needs to start at zero.
 */
#define SI_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

si_status si_indexer_topk_noalloc(const void* q, si_dtype q_dtype,
                                  const void* kc, si_dtype kc_dtype, const void* kc_scale,
                                  const float* w,
                                  int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                  int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                                  int32_t* out_idx, float* out_score, void* stream);

/*
 * The two stages si_indexer_topk runs for query chunk `chunk` (0 <= chunk <
 * plan.n_chunks), exposed so a caller can time them apart.  Same arguments and
 * validation as si_indexer_topk; si_indexer_topk is exactly select(c) then merge(c)
 * for c = 0 .. n_chunks - 1, on the same stream and workspace.
 *
 * select: scores the chunk's query rows against their visible keys (MFMA, ReLU,
 *   head-weighted sum, mask) and keeps, per (query, key partition), a candidate list
 *   in the workspace that holds the exact local top-k: a running threshold, raised
 *   after every key tile from a per-query score histogram, filters the scores, and a
 *   compaction by exact radix select cuts a list that would overflow.  With one key
 *   partition and k <= 512 the list is left holding its top k among at most
 *   plan.cand_capacity keys, with a keep rule read off the histogram; otherwise each
 *   list ends cut to exactly its top k.  These are the per-chunk candidates of the
 *   pages' data flow (jeff.news page, sequence diagram).
 * merge: cuts and merges each query's lists into the final sorted top-k rows of
 *   out_idx / out_score (the merge-topk step of the same diagram).
 */
si_status si_indexer_select_chunk(const void* q, si_dtype q_dtype,
                                  const void* kc, si_dtype kc_dtype, const void* kc_scale,
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
 * si_quantize_q_e4m3 -- the operand preparation of the fp8 path: quantises each
 * (row, head) vector of bf16 q to OCP E4M3 with its own fp32 scale and folds the scale
 * into the head weight (lower indexer precision: jeff.news page, 기술 맥락):
 *     scale    = max_d |q[r,h,d]| / 448  (1 for an all-zero vector)
 *     q8[r,h,:] = E4M3(clamp(q[r,h,:] / scale, -448, 448)), round to nearest even
 *     w_eff[r,h] = w[r,h] * scale
 * each step one correctly rounded fp32 operation.  q8 and w_eff are then the q (q_dtype
 * SI_FP8_E4M3FN) and w of si_indexer_topk: since the scale is positive,
 * w * ReLU(scale * z) = w_eff * ReLU(z).
 *
 *  q       [rows, H, D] bf16 (rows = B * S), 16-byte aligned
 *  w       [rows, H]    fp32
 *  q8      [rows, H, D] E4M3 bytes out, 8-byte aligned
 *  w_eff   [rows, H]    fp32 out
 *  q_scale [rows, H]    fp32 out, or NULL
 * D = 128, 1 <= H <= 128.  rows = 0 is a no-op.  Asynchronous on stream.
 */
si_status si_quantize_q_e4m3(const void* q, const float* w, int64_t rows, int32_t H, int32_t D,
                             void* q8, float* w_eff, float* q_scale, void* stream);

/*
 * si_sparse_attention -- the attention consumer of the indexer's selection (StreamIndex
 * abstract, aisoku.com page: a sparse attention kernel reads only the selected keys;
 * jeff.news page, sequence diagram: merge-topk hands the key indices to the sparse
 * attention).  The pages give no formula; reading used: per query row t and head h,
 *     out[b,t,h,:] = sum_j softmax_j(scale * <qa[b,t,h,:], kv[b,s_j,:]>) * kv[b,s_j,:]
 * over the row's selected entries s_j = idx[b,t,j] (the leading entries in [0, T); the
 * first -1 or out-of-range index ends the row's list), the compressed latent serving
 * as key and value for every head; a row with no entry outputs zeros.
 *  qa  [B, S, HA, D] bf16, 16-byte aligned   kv [B, T, D] bf16, 16-byte aligned
 *  idx [B, S, k] int32 (e.g. si_indexer_topk's out_idx)
 *  out [B, S, HA, D] bf16, 8-byte aligned
 * Arithmetic: logits by bf16 MFMA with fp32 accumulation, times scale * log2(e); exp2;
 * running maximum and sum in fp32; the weights rounded to bf16 for the weight x value
 * MFMA (fp32 accumulation); the output divided by the sum and rounded to bf16.
 * D = 128, 1 <= HA <= 128, k >= 1.  Asynchronous on stream.
 */
si_status si_sparse_attention(const void* qa, const void* kv, const int32_t* idx, int64_t B,
                              int64_t S, int64_t T, int32_t HA, int32_t D, int32_t k, float scale,
                              void* out, void* stream);

/*
 * ---- Two-stage (coarse -> fine) indexer --------------------------------------------
 * The candidate stage of the chengshu blog page "两级稀疏注意力：滑窗、压缩 KV latent 与
 * indexer", section "indexer：在摘要里做'预筛选'": blocks of `block` compressed keys are
 * scored cheaply and the best k_blocks blocks kept (the page: 2048 blocks of 8), then
 * only the kept keys are scored and the top k (512 there) returned.  The page defines
 * no block score; readings used here:
 *   - block key j = bf16(fp32 sum of keys block*j .. block*j + block-1 in key order,
 *     times 1/block), rounded to nearest even (si_block_keys_mean);
 *   - block j is a candidate for query position t once all its keys are visible:
 *     (block*j + block) * m <= t + 1; the coarse stage is the single-stage indexer
 *     over the block keys with mask ratio block * m, k = k_blocks;
 *   - the fine candidates are the keys of the kept blocks plus the visible keys of the
 *     query's trailing incomplete block; the fine score is the single-stage score,
 *     computed by the same MFMA sequence and head order, so equal bit for bit.
 * When a query sees at most k_blocks complete blocks every visible key is a fine
 * candidate and the row equals si_indexer_topk's.
 */
typedef struct si_two_stage_plan {
    int32_t query_chunk;      /* query rows per driver step                         */
    int32_t n_chunks;         /* driver steps per batch entry                       */
    int32_t cand_stride;      /* candidate slots per query row in the workspace     */
    int32_t reserved;
    int64_t workspace_bytes;  /* bytes si_indexer_topk_two_stage needs              */
} si_two_stage_plan;

/*
 * si_block_keys_mean -- block keys kb [B, T / block, D] bf16 from bf16 keys kc [B, T, D]
 * (the reading above; keys past the last complete block have no block key).  block a
 * power of two in 2 .. 64, D = 128, 16-byte aligned pointers.  Asynchronous on stream.
 */
si_status si_block_keys_mean(const void* kc, si_dtype kc_dtype, int64_t B, int64_t T, int32_t D,
                             int32_t block, void* kb, void* stream);

/*
 * si_indexer_two_stage_plan -- validate a two-stage problem and return its plan (host
 * only).  cfg: query_chunk = query rows per driver step (0 = auto, 4096); key_tile and
 * key_partition are passed to the coarse stage.  H <= 64, block a power of two in
 * 2 .. 64, 1 <= k, k_blocks <= 2048.
 */
si_status si_indexer_two_stage_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                    int32_t m, int32_t k, int32_t k_blocks, int32_t block,
                                    int64_t q_pos0, const si_config* cfg,
                                    si_two_stage_plan* out);

/*
 * si_indexer_topk_two_stage -- two-stage top-k.  q [B, S, H, D] bf16, kc [B, T, D] bf16,
 * kb [B, T / block, D] bf16 block keys of kc (si_block_keys_mean), w [B, S, H] fp32.
 * out_idx / out_score [B, S, k]: the same contract as si_indexer_topk (sorted by score
 * desc, index asc; -1 / -inf padding).  workspace: at least plan.workspace_bytes,
 * 256-byte aligned (coarse workspace and kept block lists of one coarse chunk, fine
 * candidate keys and their score ranges of one query chunk).  The coarse indexer runs once per coarse chunk of
 * the largest multiple of query_chunk up to 32768 rows (at least query_chunk), so its
 * query tiles fill the GPU without key partitions; then, per query chunk of it, fine
 * scoring and fine selection.
 */
si_status si_indexer_topk_two_stage(const void* q, si_dtype q_dtype, const void* kc,
                                    si_dtype kc_dtype, const void* kb, const float* w, int64_t B,
                                    int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                                    int32_t k, int32_t k_blocks, int32_t block, int64_t q_pos0,
                                    const si_config* cfg, int32_t* out_idx, float* out_score,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * si_materialize_scores -- reference path, score write-out.  Writes the head-summed
 * scores of query rows [row0, row0 + rows) for every batch entry into
 * scores [B, rows, T] fp32, -inf where the key is masked.  Same arithmetic, bit for
 * bit, as the streaming path.  (This is one [rows, T] slice of the head-summed score
 * tensor that public CSA implementations build in full before their top-k: StreamIndex
 * abstract.)  0 <= row0, row0 + rows <= S.
 */
si_status si_materialize_scores(const void* q, si_dtype q_dtype,
                                const void* kc, si_dtype kc_dtype, const void* kc_scale,
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
                              const void* kc, si_dtype kc_dtype, const void* kc_scale,
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
