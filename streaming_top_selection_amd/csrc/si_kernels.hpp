// Launch-side declarations of the gfx950 kernels (shared by the kernel sources and
// the C-ABI driver).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "si_score.hpp"

namespace si {

// Score bin of the select stage's per-query histogram: 256 bins linear in the score,
// bin = fmaf(score, inv, off) clamped to [0, 255] (inv = 0: every key in bin 0).  The
// select and merge kernels both call this, so they bin every key identically.
__device__ __forceinline__ uint32_t hist_bin(float score, float inv, float off) {
    return (uint32_t)__builtin_fminf(__builtin_fmaxf(__builtin_fmaf(score, inv, off), 0.0f), 255.0f);
}

// Keep rule of one list the select stage left for the merge to cut, read off the
// query's histogram: the list's keys with hist_bin above d number `above` (< k), and
// its top k are those plus the k - above largest keys of bin d.  d = -1: no rule.
struct KeepRule {
    int32_t d;
    uint32_t above;
    float inv, off;
};

// Select stage of one query chunk (fused score + running local top-k).
struct SelectArgs {
    Problem P;
    int32_t k;
    int64_t chunk_row0, chunk_row1;   // q rows [row0, row1) of this chunk
    int32_t n_tiles;                  // ceil((row1 - row0) / 32)
    int32_t P_chunk;                  // partitions launched for this chunk
    int32_t P_ws;                     // partition stride of the workspace
    int32_t QC;                       // row stride of the workspace (query_chunk)
    int64_t KP;                       // keys per partition
    uint64_t* cand;                   // [B][QC][P_ws][CG + kCandPad] selection keys
    int32_t* cnt;                     // [B][QC][P_ws] list lengths when done
    int32_t defer_final;              // 1: lists end holding their top k among <= CG
                                      // keys (the merge selects); 0: exactly their top k
    KeepRule* rule;                   // [B][QC][P_ws] keep rules (written when deferred)
};

// Merge stage of one query chunk.
struct MergeArgs {
    int64_t B, S, T;
    int32_t m, k;
    int64_t q_pos0;
    int64_t chunk_row0, chunk_row1;
    int32_t P_chunk, P_ws, QC, CG;   // CG: list stride (capacity + kCandPad)
    int64_t KP;
    const uint64_t* cand;
    const int32_t* cnt;
    int32_t* out_idx;
    float* out_score;
    int32_t lds_entries;              // dynamic LDS key slots of one merge group
    int32_t list_max;                 // most keys a list holds: k, or the capacity when
                                      // the select stage left the final selection here
    const KeepRule* rule;             // [B][QC][P_ws] keep rules of such lists
};

// Materialise path: score write-out of rows [row0, row0 + rows).
struct MatScoreArgs {
    Problem P;
    int64_t row0, rows;
    int64_t tile_row0;                // row0 rounded down to a multiple of 32
    int32_t n_row_tiles, n_key_tiles;
    float* scores;                    // [B, rows, T]
};

// Materialise path: exact per-row selection from written scores.
struct MatSelectArgs {
    int64_t B, S, T;
    int32_t m, k;
    int64_t q_pos0;
    int64_t row0, rows;
    const float* scores;              // [B, rows, T]
    int32_t* out_idx;
    float* out_score;
};

// E4M3 quantisation of q vectors (rows x heads vectors of kD bf16).
struct QuantArgs {
    const uint16_t* q;     // [nvec, kD] bf16 bits
    const float* w;        // [nvec] head weights
    uint8_t* q8;           // [nvec, kD] E4M3 bytes
    float* w_eff;          // [nvec] w * scale
    float* q_scale;        // [nvec] scale, or null
    int64_t nvec;
};

hipError_t launch_quantize_q(const QuantArgs& a, hipStream_t stream);

// Two-stage indexer: block keys (mean of blk consecutive bf16 keys).
struct BlockKeyArgs {
    const uint16_t* kc;    // [B, T, kD] bf16
    uint16_t* kb;          // [B, T / blk, kD] bf16
    int64_t B, T;
    int32_t blk;
};

// Two-stage indexer: fine scoring and selection of one query chunk of one batch entry.
struct FineArgs {
    const uint16_t* q;     // [rows, H, kD] bf16: the chunk's query rows
    const float* w;        // [rows, H]
    const uint16_t* kc;    // [T, kD] bf16 keys of the batch entry
    const int32_t* cidx;   // [rows, k_blocks] kept block indices (coarse top-k)
    uint64_t* cand;        // [rows, cand_stride] candidate selection keys
    uint32_t* range;       // [rows, 8, 2] min and max score image (ord) of each (row, key shard)'s candidates
    int32_t* out_idx;      // [rows, k] output rows
    float* out_score;      // [rows, k]
    int64_t T, rows;
    int64_t q_pos0;        // absolute position of the chunk's first row
    int64_t cand_stride;
    int32_t H, m, blk, k_blocks, k;
};

// Sparse attention over the selected compressed entries.
struct AttnArgs {
    const uint16_t* qa;    // [B, S, HA, kD] bf16 attention queries
    const uint16_t* kv;    // [B, T, kD] bf16 compressed latents (key = value)
    const int32_t* idx;    // [B, S, k] selected entries, -1 padded at the end
    uint16_t* out;         // [B, S, HA, kD] bf16
    int64_t B, S, T;
    int32_t HA, k;
    float scale_log2;      // softmax scale * log2(e)
};

hipError_t launch_sparse_attention(const AttnArgs& a, hipStream_t stream);
hipError_t launch_block_keys(const BlockKeyArgs& a, hipStream_t stream);
hipError_t launch_fine_score(const FineArgs& a, hipStream_t stream);
hipError_t launch_fine_select(const FineArgs& a, hipStream_t stream);

// op: operand mode (kOpBf16 .. kOpF8K4, si_score.hpp)
hipError_t launch_select(const SelectArgs& a, int nwave, int kb, int nsub, int cg, int op,
                         hipStream_t stream);
// one register-tile shape (NWAVE waves x KB blocks x NSUB register tiles per key tile)
template <int NWAVE, int KB, int NSUB, int OP>
hipError_t launch_select_shape(const SelectArgs& a, int cg, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_mat_score(const MatScoreArgs& a, int op, hipStream_t stream);
hipError_t launch_mat_select(const MatSelectArgs& a, hipStream_t stream);

}  // namespace si
