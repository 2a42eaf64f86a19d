// C ABI of the indexer library: validation, planning and the chunk driver.
// All device work is enqueued on the caller's stream; nothing here allocates.
#include <mutex>
#include <string>

#include "../../include/si_indexer.h"
#include "si_kernels.hpp"
#include "si_plan.hpp"

static_assert(si::kCandPad == si::kPlanCandPad, "candidate list padding");

// Scratch of si_indexer_topk_noalloc (for callers that cannot allocate): one copy per
// device, held for the life of the process.  Host code never uses the array's name as
// an address (on the host it names a stand-in, not device memory): the device address
// comes from hipGetSymbolAddress, once per device (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[SI_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

si_status fail(si_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

si_status hip_fail(hipError_t e, const char* where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return SI_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

si::Problem make_problem(const void* q, const void* kc, const void* kc_scale, const float* w,
                         int64_t B, int64_t S, int64_t T, int32_t H, int32_t m, int64_t q_pos0) {
    si::Problem P;
    P.q = q;
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

// The score tile's operand mode for a (q, keys) dtype pair, or -1 if not built.
int operand_mode(si_dtype q_dtype, si_dtype kc_dtype) {
    if (q_dtype == SI_BF16 && kc_dtype == SI_BF16) return si::kOpBf16;
    if (q_dtype == SI_BF16 && kc_dtype == SI_FP8_E4M3FN) return si::kOpBf16K8;
    if (q_dtype == SI_FP8_E4M3FN && kc_dtype == SI_FP8_E4M3FN) return si::kOpF8;
    if (q_dtype == SI_FP8_E4M3FN && kc_dtype == SI_MXFP4_E2M1) return si::kOpF8K4;
    return -1;
}

// Pointer and dtype checks for the inputs of every scoring entry point.  A tensor
// with no elements may have a NULL pointer.
si_status check_inputs(const void* q, si_dtype q_dtype, const void* kc, si_dtype kc_dtype,
                       const void* kc_scale, const float* w, int64_t B, int64_t S,
                       int64_t T) {
    const bool rows = B > 0 && S > 0, keys = B > 0 && T > 0;
    if (q_dtype != SI_BF16 && q_dtype != SI_FP8_E4M3FN)
        return fail(SI_ERR_UNSUPPORTED, "q must be SI_BF16 or SI_FP8_E4M3FN");
    if (operand_mode(q_dtype, kc_dtype) < 0)
        return fail(SI_ERR_UNSUPPORTED,
                    q_dtype == SI_BF16 ? "bf16 q takes bf16 or E4M3 keys (MXFP4 keys need E4M3 q)"
                                       : "E4M3 q takes E4M3 or MXFP4 keys");
    if ((rows && (!q || !w)) || (keys && !kc))
        return fail(SI_ERR_INVALID_ARG, "q, kc and w must not be NULL");
    if (kc_dtype == SI_FP8_E4M3FN && keys && !kc_scale)
        return fail(SI_ERR_INVALID_ARG, "E4M3 keys need kc_scale");
    if (kc_dtype == SI_MXFP4_E2M1 && keys && !kc_scale)
        return fail(SI_ERR_INVALID_ARG, "MXFP4 keys need their E8M0 block scales in kc_scale");
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
                     int32_t chunk, void* ws, int op, hipStream_t stream) {
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
    a.defer_final = pl.defer_final ? 1 : 0;
    a.rule = reinterpret_cast<si::KeepRule*>(static_cast<char*>(ws) + pl.rule_offset);
    const hipError_t e = si::launch_select(a, pl.nwave, pl.kb, pl.nsub, pl.pub.cand_capacity,
                                           op, stream);
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
    a.list_max = pl.defer_final ? pl.pub.cand_capacity : k;
    a.rule = reinterpret_cast<const si::KeepRule*>(static_cast<const char*>(ws) + pl.rule_offset);
    const hipError_t e = si::launch_merge(a, stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return SI_OK;
}

// Every query chunk of a planned problem: select then merge, on one stream.
si_status run_indexer(const si::PlanInternal& pl, const si::Problem& P, int32_t k, int op,
                      int32_t* out_idx, float* out_score, void* ws, hipStream_t s) {
    si_status st;
    for (int32_t c = 0; c < pl.pub.n_chunks; ++c) {
        if ((st = run_select(pl, P, k, c, ws, op, s)) != SI_OK) return st;
        if ((st = run_merge(pl, P.B, P.S, P.T, P.m, k, P.q_pos0, c, out_idx, out_score, ws, s)) !=
            SI_OK)
            return st;
    }
    return SI_OK;
}

// ---- two-stage plan ---------------------------------------------------------------
struct TwoStagePlan {
    int64_t qc, n_chunks, cand_stride;
    int64_t cqc;                 // coarse chunk: query rows of one coarse indexer call
    int64_t coarse_ws, cidx_off, cscore_off, cand_off, range_off, total;
};

constexpr int64_t kTwoStageAutoChunk = 4096;
// The coarse stage runs over several fine chunks at once (about this many rows), so
// that its query tiles fill the chip without key partitions and its merge stays a
// register sort.
constexpr int64_t kTwoStageCoarseRows = 32768;

si_config coarse_config(const si_config* cfg) {
    si_config c = cfg ? *cfg : si_config{0, 0, 0, 0};
    c.query_chunk = 0;          // the coarse problem of one two-stage chunk is one chunk
    return c;
}

si_status make_two_stage_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                              int32_t k, int32_t k_blocks, int32_t blk, int64_t q_pos0,
                              const si_config* cfg, TwoStagePlan& tp) {
    std::string msg;
    si_status st = si::check_shape(B, S, T, H, D, m, q_pos0, SI_BF16, msg);
    if (st != SI_OK) return fail(st, msg);
    if (k < 1 || k_blocks < 1) return fail(SI_ERR_INVALID_ARG, "k and k_blocks must be >= 1");
    if (k > si::kPlanMaxK || k_blocks > si::kPlanMaxK)
        return fail(SI_ERR_UNSUPPORTED, "k and k_blocks must be <= 2048");
    if (H > 64) return fail(SI_ERR_UNSUPPORTED, "the two-stage indexer is built for H <= 64");
    if (blk < 2 || blk > 64 || (blk & (blk - 1)) != 0)
        return fail(SI_ERR_UNSUPPORTED, "block must be a power of two in 2 .. 64");
    if (cfg && (cfg->reserved != 0 || cfg->query_chunk < 0))
        return fail(SI_ERR_INVALID_ARG, "invalid si_config");
    const int64_t qc = (cfg && cfg->query_chunk) ? cfg->query_chunk
                                                 : std::min<int64_t>(std::max<int64_t>(S, 1),
                                                                     kTwoStageAutoChunk);
    tp.qc = qc;
    tp.n_chunks = (S == 0 || B == 0) ? 0 : si::ceil_div(S, qc);
    tp.cand_stride = si::round_up((int64_t)blk * k_blocks + blk, 64);
    tp.cqc = std::min<int64_t>(std::max<int64_t>(S, 1),
                               qc * std::max<int64_t>(1, kTwoStageCoarseRows / qc));
    // the coarse workspace of the widest coarse-chunk plan
    const si_config cc = coarse_config(cfg);
    tp.coarse_ws = 0;
    const int64_t n_coarse = (S == 0 || B == 0) ? 0 : si::ceil_div(S, tp.cqc);
    for (int64_t c = 0; c < n_coarse; ++c) {
        const int64_t r0 = c * tp.cqc, rows = std::min(tp.cqc, S - r0);
        si::PlanInternal pl;
        st = si::make_plan(1, rows, T / blk, H, D, blk * m, k_blocks, q_pos0 + r0, SI_BF16, &cc,
                           pl, msg);
        if (st != SI_OK) return fail(st, "coarse stage: " + msg);
        tp.coarse_ws = std::max<int64_t>(tp.coarse_ws, pl.pub.workspace_bytes);
    }
    tp.cidx_off = si::round_up(tp.coarse_ws, 256);
    tp.cscore_off = tp.cidx_off + si::round_up(tp.cqc * k_blocks * 4, 256);
    tp.cand_off = tp.cscore_off + si::round_up(tp.cqc * k_blocks * 4, 256);
    tp.range_off = tp.cand_off + si::round_up(qc * tp.cand_stride * 8, 256);
    tp.total = tp.n_chunks == 0 ? 0 : tp.range_off + qc * 64;   // 8 shards x (min, max)
    return SI_OK;
}

// The device address of `scratch` on the current device, looked up on the first call
// on each device and kept.
si_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SI_ERR_UNSUPPORTED, "device index >= 64");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SI_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
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

size_t si_indexer_topk_workspace_bytes(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                       int32_t m, int32_t k, const si_config* cfg) {
    g_last_error.clear();
    si::PlanInternal pl;
    // the key dtype does not change the plan; bf16 passes the dtype check
    if (plan_or_fail(B, S, T, H, D, m, k, 0, SI_BF16, cfg, pl) != SI_OK) return SIZE_MAX;
    return (size_t)pl.pub.workspace_bytes;
}

si_status si_indexer_select_chunk(const void* q, si_dtype q_dtype, const void* kc,
                                  si_dtype kc_dtype, const void* kc_scale, const float* w,
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
    return run_select(pl, P, k, chunk, workspace, operand_mode(q_dtype, kc_dtype),
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
                          const void* kc_scale, const float* w, int64_t B, int64_t S,
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
        if ((st = run_select(pl, P, k, c, workspace, operand_mode(q_dtype, kc_dtype), s)) !=
            SI_OK)
            return st;
        if ((st = run_merge(pl, B, S, T, m, k, q_pos0, c, out_idx, out_score, workspace, s)) !=
            SI_OK)
            return st;
    }
    return SI_OK;
}

si_status si_indexer_topk_noalloc(const void* q, si_dtype q_dtype, const void* kc,
                                  si_dtype kc_dtype, const void* kc_scale, const float* w,
                                  int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                  int32_t m, int32_t k, int64_t q_pos0, const si_config* cfg,
                                  int32_t* out_idx, float* out_score, void* stream) {
    g_last_error.clear();
    si::PlanInternal pl;
    std::string msg;
    // the automatic query chunk is the largest whose workspace fits the scratch
    si_status st = si::make_plan(B, S, T, H, D, m, k, q_pos0, kc_dtype, cfg, pl, msg,
                                 (int64_t)SI_NOALLOC_SCRATCH_BYTES);
    if (st != SI_OK) return fail(st, msg);
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, kc_scale, w, B, S, T)) != SI_OK) return st;
    if (B > 0 && S > 0 && (!out_idx || !out_score))
        return fail(SI_ERR_INVALID_ARG, "outputs must not be NULL");
    if (pl.pub.workspace_bytes > (int64_t)SI_NOALLOC_SCRATCH_BYTES)
        return fail(SI_ERR_WORKSPACE,
                    "the problem needs " + std::to_string(pl.pub.workspace_bytes) +
                        " bytes of workspace per query chunk, more than the " +
                        std::to_string((int64_t)SI_NOALLOC_SCRATCH_BYTES) +
                        "-byte static scratch: use a smaller query_chunk, or si_indexer_topk "
                        "with a caller workspace");
    if (pl.pub.n_chunks == 0) return SI_OK;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != SI_OK) return st;
    // every count the merge reads is written by the select launch before it, so the
    // scratch needs no clearing
    const si::Problem P = make_problem(q, kc, kc_scale, w, B, S, T, H, m, q_pos0);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t c = 0; c < pl.pub.n_chunks; ++c) {
        if ((st = run_select(pl, P, k, c, ws, operand_mode(q_dtype, kc_dtype), s)) != SI_OK)
            return st;
        if ((st = run_merge(pl, B, S, T, m, k, q_pos0, c, out_idx, out_score, ws, s)) != SI_OK)
            return st;
    }
    return SI_OK;
}

si_status si_quantize_q_e4m3(const void* q, const float* w, int64_t rows, int32_t H, int32_t D,
                             void* q8, float* w_eff, float* q_scale, void* stream) {
    g_last_error.clear();
    if (rows < 0) return fail(SI_ERR_INVALID_ARG, "rows must be >= 0");
    if (H < 1 || D < 1) return fail(SI_ERR_INVALID_ARG, "H and D must be >= 1");
    if (D != si::kPlanD) return fail(SI_ERR_UNSUPPORTED, "only D = 128 is built");
    if (H > si::kPlanMaxH) return fail(SI_ERR_UNSUPPORTED, "H must be <= 128");
    if (rows == 0) return SI_OK;
    if (!q || !w || !q8 || !w_eff) return fail(SI_ERR_INVALID_ARG, "q, w, q8 and w_eff must not be NULL");
    if (!aligned(q, 16) || !aligned(q8, 8) || !aligned(w, 4) || !aligned(w_eff, 4) ||
        (q_scale && !aligned(q_scale, 4)))
        return fail(SI_ERR_INVALID_ARG,
                    "q must be 16-byte aligned, q8 8-byte, w, w_eff and q_scale 4-byte");
    si::QuantArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.w = w;
    a.q8 = static_cast<uint8_t*>(q8);
    a.w_eff = w_eff;
    a.q_scale = q_scale;
    a.nvec = rows * H;
    const hipError_t e = si::launch_quantize_q(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "quantize kernel launch");
    return SI_OK;
}

si_status si_sparse_attention(const void* qa, const void* kv, const int32_t* idx, int64_t B,
                              int64_t S, int64_t T, int32_t HA, int32_t D, int32_t k, float scale,
                              void* out, void* stream) {
    g_last_error.clear();
    if (B < 0 || S < 0 || T < 0) return fail(SI_ERR_INVALID_ARG, "B, S and T must be >= 0");
    if (HA < 1 || k < 1 || D < 1) return fail(SI_ERR_INVALID_ARG, "HA, k and D must be >= 1");
    if (D != si::kPlanD) return fail(SI_ERR_UNSUPPORTED, "only D = 128 is built");
    if (HA > 128) return fail(SI_ERR_UNSUPPORTED, "HA must be <= 128");
    if (T >= int64_t(0x7FFFFFFF)) return fail(SI_ERR_UNSUPPORTED, "T must be < 2^31 - 1");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SI_ERR_INVALID_ARG, "scale must be finite");
    if (B == 0 || S == 0) return SI_OK;
    if (!qa || !idx || !out || (T > 0 && !kv))
        return fail(SI_ERR_INVALID_ARG, "qa, kv, idx and out must not be NULL");
    if (!aligned(qa, 16) || (kv && !aligned(kv, 16)) || !aligned(idx, 4) || !aligned(out, 8))
        return fail(SI_ERR_INVALID_ARG, "qa and kv must be 16-byte aligned, idx 4-byte, out 8-byte");
    si::AttnArgs a;
    a.qa = static_cast<const uint16_t*>(qa);
    a.kv = static_cast<const uint16_t*>(kv);
    a.idx = idx;
    a.out = static_cast<uint16_t*>(out);
    a.B = B;
    a.S = S;
    a.T = T;
    a.HA = HA;
    a.k = k;
    a.scale_log2 = scale * 1.4426950408889634f;
    const hipError_t e = si::launch_sparse_attention(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sparse attention kernel launch");
    return SI_OK;
}

si_status si_block_keys_mean(const void* kc, si_dtype kc_dtype, int64_t B, int64_t T, int32_t D,
                             int32_t block, void* kb, void* stream) {
    g_last_error.clear();
    if (B < 0 || T < 0) return fail(SI_ERR_INVALID_ARG, "B and T must be >= 0");
    if (kc_dtype != SI_BF16) return fail(SI_ERR_UNSUPPORTED, "block keys are built from bf16 keys");
    if (D != si::kPlanD) return fail(SI_ERR_UNSUPPORTED, "only D = 128 is built");
    if (block < 2 || block > 64 || (block & (block - 1)) != 0)
        return fail(SI_ERR_UNSUPPORTED, "block must be a power of two in 2 .. 64");
    if (B == 0 || T / block == 0) return SI_OK;
    if (!kc || !kb) return fail(SI_ERR_INVALID_ARG, "kc and kb must not be NULL");
    if (!aligned(kc, 16) || !aligned(kb, 16))
        return fail(SI_ERR_INVALID_ARG, "kc and kb must be 16-byte aligned");
    si::BlockKeyArgs a;
    a.kc = static_cast<const uint16_t*>(kc);
    a.kb = static_cast<uint16_t*>(kb);
    a.B = B;
    a.T = T;
    a.blk = block;
    const hipError_t e = si::launch_block_keys(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block key kernel launch");
    return SI_OK;
}

si_status si_indexer_two_stage_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                                    int32_t m, int32_t k, int32_t k_blocks, int32_t block,
                                    int64_t q_pos0, const si_config* cfg,
                                    si_two_stage_plan* out) {
    g_last_error.clear();
    if (!out) return fail(SI_ERR_INVALID_ARG, "out must not be NULL");
    TwoStagePlan tp;
    const si_status st = make_two_stage_plan(B, S, T, H, D, m, k, k_blocks, block, q_pos0, cfg, tp);
    if (st != SI_OK) return st;
    out->query_chunk = (int32_t)tp.qc;
    out->n_chunks = (int32_t)tp.n_chunks;
    out->cand_stride = (int32_t)tp.cand_stride;
    out->reserved = 0;
    out->workspace_bytes = tp.total;
    return SI_OK;
}

si_status si_indexer_topk_two_stage(const void* q, si_dtype q_dtype, const void* kc,
                                    si_dtype kc_dtype, const void* kb, const float* w, int64_t B,
                                    int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                                    int32_t k, int32_t k_blocks, int32_t block, int64_t q_pos0,
                                    const si_config* cfg, int32_t* out_idx, float* out_score,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (q_dtype != SI_BF16 || kc_dtype != SI_BF16)
        return fail(SI_ERR_UNSUPPORTED, "the two-stage indexer takes bf16 q and bf16 keys");
    TwoStagePlan tp;
    si_status st = make_two_stage_plan(B, S, T, H, D, m, k, k_blocks, block, q_pos0, cfg, tp);
    if (st != SI_OK) return st;
    if ((st = check_inputs(q, q_dtype, kc, kc_dtype, nullptr, w, B, S, T)) != SI_OK) return st;
    if (B > 0 && T / block > 0 && (!kb || !aligned(kb, 16)))
        return fail(SI_ERR_INVALID_ARG, "kb must be non-NULL and 16-byte aligned");
    if (B > 0 && S > 0 && (!out_idx || !out_score))
        return fail(SI_ERR_INVALID_ARG, "outputs must not be NULL");
    if ((int64_t)workspace_bytes < tp.total)
        return fail(SI_ERR_WORKSPACE, "workspace smaller than si_two_stage_plan.workspace_bytes");
    if (tp.total > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(SI_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* cidx = reinterpret_cast<int32_t*>(ws + tp.cidx_off);
    float* cscore = reinterpret_cast<float*>(ws + tp.cscore_off);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws + tp.cand_off);
    uint32_t* range = reinterpret_cast<uint32_t*>(ws + tp.range_off);
    const int64_t nb = T / block;
    const si_config cc = coarse_config(cfg);
    std::string msg;
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t* qb = static_cast<const uint16_t*>(q) + b * S * H * (int64_t)D;
        const float* wb = w + b * S * H;
        const uint16_t* kcb = static_cast<const uint16_t*>(kc) + b * T * (int64_t)D;
        const uint16_t* kbb = static_cast<const uint16_t*>(kb) + b * nb * (int64_t)D;
        for (int64_t c = 0; c < tp.n_chunks; ++c) {
            const int64_t r0 = c * tp.qc, rows = std::min(tp.qc, S - r0);
            // coarse (once per coarse chunk, for all its fine chunks): the single-stage
            // indexer over the block keys, mask ratio block * m
            const int64_t c0 = (r0 / tp.cqc) * tp.cqc;
            if (r0 == c0) {
                const int64_t crows = std::min(tp.cqc, S - c0);
                si::PlanInternal pl;
                st = si::make_plan(1, crows, nb, H, D, block * m, k_blocks, q_pos0 + c0, SI_BF16,
                                   &cc, pl, msg);
                if (st != SI_OK) return fail(st, "coarse stage: " + msg);
                const si::Problem P = make_problem(qb + c0 * H * (int64_t)D, kbb, nullptr,
                                                   wb + c0 * H, 1, crows, nb, H, block * m,
                                                   q_pos0 + c0);
                if ((st = run_indexer(pl, P, k_blocks, si::kOpBf16, cidx, cscore, ws, s)) != SI_OK)
                    return st;
            }
            // fine: score the candidates, select the top-k into the output rows
            si::FineArgs a;
            a.q = qb + r0 * H * (int64_t)D;
            a.w = wb + r0 * H;
            a.kc = kcb;
            a.cidx = cidx + (r0 - c0) * (int64_t)k_blocks;
            a.cand = cand;
            a.range = range;
            a.out_idx = out_idx + (b * S + r0) * (int64_t)k;
            a.out_score = out_score + (b * S + r0) * (int64_t)k;
            a.T = T;
            a.rows = rows;
            a.q_pos0 = q_pos0 + r0;
            a.cand_stride = tp.cand_stride;
            a.H = H;
            a.m = m;
            a.blk = block;
            a.k_blocks = k_blocks;
            a.k = k;
            hipError_t e = si::launch_fine_score(a, s);
            if (e != hipSuccess) return hip_fail(e, "fine score kernel launch");
            e = si::launch_fine_select(a, s);
            if (e != hipSuccess) return hip_fail(e, "fine select kernel launch");
        }
    }
    return SI_OK;
}

si_status si_materialize_scores(const void* q, si_dtype q_dtype, const void* kc,
                                si_dtype kc_dtype, const void* kc_scale, const float* w,
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
    const hipError_t e = si::launch_mat_score(a, operand_mode(q_dtype, kc_dtype),
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "materialise score kernel launch");
    return SI_OK;
}

si_status si_materialize_topk(const void* q, si_dtype q_dtype, const void* kc, si_dtype kc_dtype,
                              const void* kc_scale, const float* w, int64_t B, int64_t S,
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
