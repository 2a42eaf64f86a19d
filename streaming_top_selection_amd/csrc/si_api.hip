// C ABI of the indexer library: validation, planning and the chunk driver.
// All device work is enqueued on the caller's stream; nothing here allocates.
#include <string>

#include "../../include/si_indexer.h"
#include "si_kernels.hpp"
#include "si_plan.hpp"

static_assert(si::kCandPad == si::kPlanCandPad, "candidate list padding");

namespace {

thread_local std::string g_last_error;

si_status fail(si_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

si_status hip_fail(hipError_t e, const char* where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return SI_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

si::Problem make_problem(const void* q, const void* kc, const float* kc_scale, const float* w,
                         int64_t B, int64_t S, int64_t T, int32_t H, int32_t m, int64_t q_pos0) {
    si::Problem P;
    P.q = static_cast<const uint16_t*>(q);
    P.kc = kc;
    P.kc_scale = kc_scale;
    P.w = w;
    P.B = B;
    P.S = S;
    P.T = T;
    P.H = H;
    P.m = m;
    P.q_pos0 = q_pos0;
    return P;
}

// Pointer and dtype checks for the inputs of every scoring entry point.  A tensor
// with no elements may have a NULL pointer.
si_status check_inputs(const void* q, si_dtype q_dtype, const void* kc, si_dtype kc_dtype,
                       const float* kc_scale, const float* w, int64_t B, int64_t S,
                       int64_t T) {
    const bool rows = B > 0 && S > 0, keys = B > 0 && T > 0;
    if (q_dtype != SI_BF16) return fail(SI_ERR_UNSUPPORTED, "q must be SI_BF16");
    if ((rows && (!q || !w)) || (keys && !kc))
        return fail(SI_ERR_INVALID_ARG, "q, kc and w must not be NULL");
    if (kc_dtype == SI_FP8_E4M3FN && keys && !kc_scale)
        return fail(SI_ERR_INVALID_ARG, "E4M3 keys need kc_scale");
    if (kc_dtype == SI_BF16 && kc_scale)
        return fail(SI_ERR_INVALID_ARG, "kc_scale must be NULL for bf16 keys");
    if ((rows && (!aligned(q, 16) || !aligned(w, 4))) || (keys && !aligned(kc, 16)) ||
        (kc_scale && !aligned(kc_scale, 4)))
        return fail(SI_ERR_INVALID_ARG, "q and kc must be 16-byte aligned, w and kc_scale 4-byte");
    return SI_OK;
}

si_status plan_or_fail(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                       int32_t k, int64_t q_pos0, si_dtype kc_dtype, const si_config* cfg,
                       si::PlanInternal& pl) {
    std::string msg;
    const si_status st = si::make_plan(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl, msg);
    if (st != SI_OK) return fail(st, msg);
    return SI_OK;
}

si_status check_workspace(const si::PlanInternal& pl, const void* ws, size_t ws_bytes) {
    if ((int64_t)ws_bytes < pl.pub.workspace_bytes)
        return fail(SI_ERR_WORKSPACE, "workspace smaller than si_plan.workspace_bytes");
    if (pl.pub.workspace_bytes > 0 && (!ws || !aligned(ws, 256)))
        return fail(SI_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    return SI_OK;
}

si_status run_select(const si::PlanInternal& pl, const si::Problem& P, int32_t k,
                     int32_t chunk, void* ws, bool fp8, hipStream_t stream) {
    const int64_t qc = pl.pub.query_chunk;
    si::SelectArgs a;
    a.P = P;
    a.k = k;
    a.chunk_row0 = (int64_t)chunk * qc;
    a.chunk_row1 = std::min<int64_t>(P.S, a.chunk_row0 + qc);
    a.n_tiles = (int32_t)si::ceil_div(a.chunk_row1 - a.chunk_row0, si::kPlanTQ);
    a.P_chunk = si::chunk_partitions(pl, P.S, P.T, P.m, P.q_pos0, chunk);
    a.P_ws = pl.pub.n_partitions;
    a.QC = pl.pub.query_chunk;
    a.KP = pl.pub.key_partition;
    a.cand = static_cast<uint64_t*>(ws);
    a.cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.cand_bytes);
    const hipError_t e = si::launch_select(a, pl.nwave, pl.kb, pl.nsub, pl.pub.cand_capacity,
                                           fp8, stream);
    if (e != hipSuccess) return hip_fail(e, "select kernel launch");
    return SI_OK;
}

si_status run_merge(const si::PlanInternal& pl, int64_t B, int64_t S, int64_t T, int32_t m,
                    int32_t k, int64_t q_pos0, int32_t chunk, int32_t* out_idx,
                    float* out_score, const void* ws, hipStream_t stream) {
    const int64_t qc = pl.pub.query_chunk;
    si::MergeArgs a;
    a.B = B;
    a.S = S;
    a.T = T;
    a.m = m;
    a.k = k;
    a.q_pos0 = q_pos0;
    a.chunk_row0 = (int64_t)chunk * qc;
    a.chunk_row1 = std::min<int64_t>(S, a.chunk_row0 + qc);
    a.P_chunk = si::chunk_partitions(pl, S, T, m, q_pos0, chunk);
    a.P_ws = pl.pub.n_partitions;
    a.QC = pl.pub.query_chunk;
    a.CG = pl.pub.cand_capacity + si::kPlanCandPad;   // list stride
    a.KP = pl.pub.key_partition;
    a.cand = static_cast<const uint64_t*>(ws);
    a.cnt = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + pl.cand_bytes);
    a.out_idx = out_idx;
    a.out_score = out_score;
    int32_t n2 = 1;
    while (n2 < k) n2 <<= 1;
    a.lds_entries = std::max<int32_t>(n2, a.P_chunk * k);
    const hipError_t e = si::launch_merge(a, stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return SI_OK;
}

}  // namespace

extern "C" {

int32_t si_abi_version(void) { return SI_ABI_VERSION; }

const char* si_status_str(si_status status) {
    switch (status) {
        case SI_OK: return "SI_OK";
        case SI_ERR_INVALID_ARG: return "SI_ERR_INVALID_ARG: invalid argument";
        case SI_ERR_UNSUPPORTED: return "SI_ERR_UNSUPPORTED: shape, dtype or knob not built";
        case SI_ERR_WORKSPACE: return "SI_ERR_WORKSPACE: workspace missing or too small";
        case SI_ERR_HIP: return "SI_ERR_HIP: HIP runtime error";
    }
    return "unknown si_status";
}

const char* si_last_error(void) { return g_last_error.c_str(); }

si_status si_indexer_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                          int32_t k, int64_t q_pos0, si_dtype kc_dtype, const si_config* cfg,
                          si_plan* out) {
    g_last_error.clear();
    if (!out) return fail(SI_ERR_INVALID_ARG, "out must not be NULL");
    si::PlanInternal pl;
    const si_status st = plan_or_fail(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl);
    if (st != SI_OK) return st;
    *out = pl.pub;
    return SI_OK;
}

si_status si_indexer_select_chunk(const void* q, si_dtype q_dtype, const void* kc,
                                  si_dtype kc_dtype, const float* kc_scale, const float* w,
                                  int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                  int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                                  int32_t chunk, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    g_last_error.clear();
    si::PlanInternal pl;
    si_status st = plan_or_fail(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl);
    if (st != SI_OK) return st;
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T)) != SI_OK) return st;
    if ((st = check_workspace(pl, workspace, workspace_bytes)) != SI_OK) return st;
    if (chunk < 0 || chunk >= pl.pub.n_chunks) {
        if (S == 0 || B == 0) return SI_OK;
        return fail(SI_ERR_INVALID_ARG, "chunk out of range");
    }
    const si::Problem P = make_problem(q, kc, kc_scale, w, B, S, T, H, m, q_pos0);
    return run_select(pl, P, k, chunk, workspace, kc_dtype == SI_FP8_E4M3FN,
                      static_cast<hipStream_t>(stream));
}

si_status si_indexer_merge_chunk(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                 int32_t m, int32_t k, int64_t q_pos0, si_dtype kc_dtype,
                                 const si_config* cfg, int32_t chunk, int32_t* out_idx,
                                 float* out_score, const void* workspace,
                                 size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    si::PlanInternal pl;
    si_status st = plan_or_fail(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl);
    if (st != SI_OK) return st;
    if (B > 0 && S > 0 && (!out_idx || !out_score))
        return fail(SI_ERR_INVALID_ARG, "outputs must not be NULL");
    if ((st = check_workspace(pl, workspace, workspace_bytes)) != SI_OK) return st;
    if (chunk < 0 || chunk >= pl.pub.n_chunks) {
        if (S == 0 || B == 0) return SI_OK;
        return fail(SI_ERR_INVALID_ARG, "chunk out of range");
    }
    return run_merge(pl, B, S, T, m, k, q_pos0, chunk, out_idx, out_score, workspace,
                     static_cast<hipStream_t>(stream));
}

si_status si_indexer_topk(const void* q, si_dtype q_dtype, const void* kc, si_dtype kc_dtype,
                          const float* kc_scale, const float* w, int64_t B, int64_t S,
                          int64_t T, int32_t H, int32_t D, int32_t m, int32_t k,
                          int64_t q_pos0, const si_config* cfg, int32_t* out_idx,
                          float* out_score, void* workspace, size_t workspace_bytes,
                          void* stream) {
    g_last_error.clear();
    si::PlanInternal pl;
    si_status st = plan_or_fail(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl);
    if (st != SI_OK) return st;
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T)) != SI_OK) return st;
    if (B > 0 && S > 0 && (!out_idx || !out_score))
        return fail(SI_ERR_INVALID_ARG, "outputs must not be NULL");
    if ((st = check_workspace(pl, workspace, workspace_bytes)) != SI_OK) return st;
    const si::Problem P = make_problem(q, kc, kc_scale, w, B, S, T, H, m, q_pos0);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t c = 0; c < pl.pub.n_chunks; ++c) {
        if ((st = run_select(pl, P, k, c, workspace, kc_dtype == SI_FP8_E4M3FN, s)) != SI_OK)
            return st;
        if ((st = run_merge(pl, B, S, T, m, k, q_pos0, c, out_idx, out_score, workspace, s)) !=
            SI_OK)
            return st;
    }
    return SI_OK;
}

si_status si_materialize_scores(const void* q, si_dtype q_dtype, const void* kc,
                                si_dtype kc_dtype, const float* kc_scale, const float* w,
                                int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                int32_t m, int64_t q_pos0, int64_t row0, int64_t rows,
                                float* scores, void* stream) {
    g_last_error.clear();
    std::string msg;
    si_status st = si::check_shape(B, S, T, H, D, m, q_pos0, kc_dtype, msg);
    if (st != SI_OK) return fail(st, msg);
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T)) != SI_OK) return st;
    if (row0 < 0 || rows < 0 || row0 + rows > S)
        return fail(SI_ERR_INVALID_ARG, "rows [row0, row0 + rows) must lie in [0, S)");
    if (rows == 0 || B == 0 || T == 0) return SI_OK;
    if (!scores) return fail(SI_ERR_INVALID_ARG, "scores must not be NULL");
    si::MatScoreArgs a;
    a.P = make_problem(q, kc, kc_scale, w, B, S, T, H, m, q_pos0);
    a.row0 = row0;
    a.rows = rows;
    a.tile_row0 = (row0 / si::kPlanTQ) * si::kPlanTQ;
    a.n_row_tiles = (int32_t)si::ceil_div(row0 + rows - a.tile_row0, si::kPlanTQ);
    a.n_key_tiles = (int32_t)si::ceil_div(T, 512);
    a.scores = scores;
    const hipError_t e = si::launch_mat_score(a, kc_dtype == SI_FP8_E4M3FN,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "materialise score kernel launch");
    return SI_OK;
}

si_status si_materialize_topk(const void* q, si_dtype q_dtype, const void* kc, si_dtype kc_dtype,
                              const float* kc_scale, const float* w, int64_t B, int64_t S,
                              int64_t T, int32_t H, int32_t D, int32_t m, int32_t k,
                              int64_t q_pos0, int32_t* out_idx, float* out_score,
                              float* scores_ws, size_t scores_ws_bytes, int64_t row_block,
                              void* stream) {
    g_last_error.clear();
    std::string msg;
    si_status st = si::check_shape(B, S, T, H, D, m, q_pos0, kc_dtype, msg);
    if (st != SI_OK) return fail(st, msg);
    if (k < 1) return fail(SI_ERR_INVALID_ARG, "k must be >= 1");
    if (k > si::kPlanMaxK) return fail(SI_ERR_UNSUPPORTED, "k must be <= 2048");
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T)) != SI_OK) return st;
    if (B > 0 && S > 0 && (!out_idx || !out_score))
        return fail(SI_ERR_INVALID_ARG, "outputs must not be NULL");
    if (row_block < 1) return fail(SI_ERR_INVALID_ARG, "row_block must be >= 1");
    if (S == 0 || B == 0) return SI_OK;
    const int64_t need = B * std::min(row_block, S) * T * 4;
    if (T > 0 && (!scores_ws || (int64_t)scores_ws_bytes < need))
        return fail(SI_ERR_WORKSPACE, "scores_ws smaller than B * row_block * T * 4 bytes");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t r0 = 0; r0 < S; r0 += row_block) {
        const int64_t rows = std::min(row_block, S - r0);
        if (T > 0) {
            st = si_materialize_scores(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T, H, D, m,
                                       q_pos0, r0, rows, scores_ws, stream);
            if (st != SI_OK) return st;
        }
        si::MatSelectArgs a;
        a.B = B;
        a.S = S;
        a.T = T;
        a.m = m;
        a.k = k;
        a.q_pos0 = q_pos0;
        a.row0 = r0;
        a.rows = rows;
        a.scores = scores_ws;
        a.out_idx = out_idx;
        a.out_score = out_score;
        const hipError_t e = si::launch_mat_select(a, s);
        if (e != hipSuccess) return hip_fail(e, "materialise select kernel launch");
    }
    return SI_OK;
}

}  // extern "C"
