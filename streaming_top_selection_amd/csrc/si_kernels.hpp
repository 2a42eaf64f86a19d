// Launch-side declarations of the gfx950 kernels (shared by the kernel sources and
// the C-ABI driver).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "si_score.hpp"

namespace si {

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
    int32_t* cnt;                     // [B][QC][P_ws] list lengths (<= k when done)
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

hipError_t launch_select(const SelectArgs& a, int nwave, int kb, int nsub, int cg, bool fp8,
                         hipStream_t stream);
// one register-tile shape (NWAVE waves x KB blocks x NSUB register tiles per key tile)
template <int NWAVE, int KB, int NSUB, bool FP8>
hipError_t launch_select_shape(const SelectArgs& a, int cg, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_mat_score(const MatScoreArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_mat_select(const MatSelectArgs& a, hipStream_t stream);

}  // namespace si
