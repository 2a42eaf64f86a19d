// Host-only validation and planning for the indexer entry points (no HIP calls).
#pragma once

#include <stdint.h>

#include <algorithm>
#include <string>

#include "../../include/si_indexer.h"

namespace si {

constexpr int32_t kPlanTQ = 32;              // query rows per workgroup tile
constexpr int32_t kPlanMaxH = 128;
constexpr int32_t kPlanMaxK = 2048;
constexpr int32_t kPlanD = 128;
constexpr int32_t kMaxPartitions = 64;       // lists one merge wave gathers
constexpr int64_t kMergeMaxEntries = 8192;   // 64 KiB of LDS keys in the merge
constexpr int64_t kAutoWorkspaceCap = int64_t(3) << 30;   // 3 GiB: auto query_chunk bound
constexpr int32_t kTargetGroups = 1024;      // workgroups one select launch aims for
constexpr int32_t kPlanCandPad = 64;         // unread slots after each candidate list

struct PlanInternal {
    si_plan pub;
    int32_t nwave, kb, nsub;  // register tile = nwave * kb * 32 keys; key_tile = * nsub
    int64_t t_eff;            // keys visible to the last query row
    int64_t cand_bytes;       // offset of the count array in the workspace
    int64_t rule_offset;      // offset of the keep-rule array (16 B per list)
    bool defer_final;         // one partition, k <= 512: the merge selects the top k
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline int64_t visible_count_host(int64_t t_abs, int32_t m, int64_t T) {
    return std::min<int64_t>(T, (t_abs + 1) / m);
}

// Shape checks shared by every entry point.  Returns SI_OK or an error with `msg`.
inline si_status check_shape(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D,
                             int32_t m, int64_t q_pos0, si_dtype kc_dtype,
                             std::string& msg) {
    if (B < 0 || S < 0 || T < 0) { msg = "B, S and T must be >= 0"; return SI_ERR_INVALID_ARG; }
    if (m < 1) { msg = "m must be >= 1"; return SI_ERR_INVALID_ARG; }
    if (q_pos0 < 0) { msg = "q_pos0 must be >= 0"; return SI_ERR_INVALID_ARG; }
    if (H < 1) { msg = "H must be >= 1"; return SI_ERR_INVALID_ARG; }
    if (D < 1) { msg = "D must be >= 1"; return SI_ERR_INVALID_ARG; }
    if (D != kPlanD) { msg = "only D = 128 is built"; return SI_ERR_UNSUPPORTED; }
    if (H > kPlanMaxH) { msg = "H must be <= 128"; return SI_ERR_UNSUPPORTED; }
    if (T >= int64_t(0x7FFFFFFF)) { msg = "T must be < 2^31 - 1"; return SI_ERR_UNSUPPORTED; }
    if (kc_dtype != SI_BF16 && kc_dtype != SI_FP8_E4M3FN && kc_dtype != SI_MXFP4_E2M1) {
        msg = "key dtype must be SI_BF16, SI_FP8_E4M3FN or SI_MXFP4_E2M1"; return SI_ERR_UNSUPPORTED;
    }
    if (S > (int64_t(1) << 40) || B > (int64_t(1) << 20)) {
        msg = "B or S too large"; return SI_ERR_UNSUPPORTED;
    }
    return SI_OK;
}

// auto_cap: the workspace bound the automatic query chunk is chosen for
inline si_status make_plan(int64_t B, int64_t S, int64_t T, int32_t H, int32_t D, int32_t m,
                           int32_t k, int64_t q_pos0, si_dtype kc_dtype, const si_config* cfg,
                           PlanInternal& pl, std::string& msg,
                           int64_t auto_cap = kAutoWorkspaceCap) {
    si_status st = check_shape(B, S, T, H, D, m, q_pos0, kc_dtype, msg);
    if (st != SI_OK) return st;
    if (k < 1) { msg = "k must be >= 1"; return SI_ERR_INVALID_ARG; }
    if (k > kPlanMaxK) { msg = "k must be <= 2048"; return SI_ERR_UNSUPPORTED; }
    si_config c = cfg ? *cfg : si_config{0, 0, 0, 0};
    if (c.reserved != 0) { msg = "si_config.reserved must be 0"; return SI_ERR_INVALID_ARG; }
    if (c.key_tile < 0 || c.query_chunk < 0 || c.key_partition < 0) {
        msg = "tuning knobs must be >= 0"; return SI_ERR_INVALID_ARG;
    }

    // key tile -> register tile shape
    const int32_t kt = c.key_tile ? c.key_tile : 512;
    switch (kt) {
        case 64:   pl.nwave = 2; pl.kb = 1; pl.nsub = 1; break;
        case 128:  pl.nwave = 4; pl.kb = 1; pl.nsub = 1; break;
        case 256:  pl.nwave = 4; pl.kb = 2; pl.nsub = 1; break;
        case 512:  pl.nwave = 4; pl.kb = 4; pl.nsub = 1; break;
        case 768:  pl.nwave = 4; pl.kb = 2; pl.nsub = 3; break;
        case 1024: pl.nwave = 4; pl.kb = 4; pl.nsub = 2; break;
        default:
            msg = "key_tile must be 64, 128, 256, 512, 768 or 1024"; return SI_ERR_UNSUPPORTED;
    }
    const int64_t t_eff = (S == 0) ? 0 : visible_count_host(q_pos0 + S - 1, m, T);
    const int64_t q_tiles = B * ceil_div(S, kPlanTQ);

    // key partitions
    int64_t kp;
    if (c.key_partition) {
        if (c.key_partition % kt != 0) {
            msg = "key_partition must be a multiple of key_tile"; return SI_ERR_UNSUPPORTED;
        }
        kp = c.key_partition;
    } else {
        // split keys only when the query tiles alone cannot fill the chip, and never
        // into partitions so short that their local top-k keeps most of them
        int64_t want = q_tiles >= kTargetGroups ? 1 : ceil_div(kTargetGroups, std::max<int64_t>(q_tiles, 1));
        want = std::min<int64_t>(want, kMaxPartitions);
        want = std::min<int64_t>(want, std::max<int64_t>(1, kMergeMaxEntries / k));
        const int64_t keys = std::max<int64_t>(t_eff, 1);
        const int64_t min_kp = std::max<int64_t>({4 * (int64_t)kt, 2048, 4 * (int64_t)k});
        kp = round_up(ceil_div(keys, want), kt);
        kp = std::max<int64_t>(kp, std::min<int64_t>(round_up(keys, kt), round_up(min_kp, kt)));
    }
    const int64_t nparts = std::max<int64_t>(1, ceil_div(t_eff, kp));
    if (nparts > kMaxPartitions || nparts * k > kMergeMaxEntries) {
        msg = "too many key partitions for the merge (need partitions <= 64 and "
              "partitions * k <= 8192): raise key_partition";
        return SI_ERR_UNSUPPORTED;
    }
    // One partition and k <= 512: the select stage leaves each list holding its top k
    // among at most 4096 keys, and the merge (many waves per SIMD) selects the k,
    // instead of a final compaction in the MFMA kernel (one wave per SIMD).
    pl.defer_final = nparts == 1 && k <= 512;
    // candidate slots per (query, partition): room for k kept keys plus a key tile of
    // arrivals with slack, and at least 2k so a compaction frees half the buffer; a
    // deferred list gets 4096, so that with the histogram threshold most lists never
    // compact before the partition's end
    const int32_t cg =
        (!pl.defer_final && 2 * k <= 2048 && k + kt + 256 <= 2048) ? 2048 : 4096;

    // query chunk
    const int64_t per_row = B * nparts * (int64_t(cg + kPlanCandPad) * 8 + 4 + 16);
    int64_t qc;
    if (c.query_chunk) {
        qc = round_up(c.query_chunk, kPlanTQ);
    } else {
        qc = std::max<int64_t>(kPlanTQ, (auto_cap / std::max<int64_t>(per_row, 1)) /
                                            kPlanTQ * kPlanTQ);
        qc = std::min<int64_t>(qc, std::max<int64_t>(round_up(S, kPlanTQ), kPlanTQ));
    }
    if (qc > (int64_t(1) << 30)) { msg = "query_chunk too large"; return SI_ERR_UNSUPPORTED; }
    const int64_t nchunks = S == 0 ? 0 : ceil_div(S, qc);

    const int64_t cand_bytes = round_up(B * qc * nparts * int64_t(cg + kPlanCandPad) * 8, 256);
    const int64_t cnt_bytes = round_up(B * qc * nparts * 4, 256);
    const int64_t rule_bytes = round_up(B * qc * nparts * 16, 256);

    pl.pub.key_tile = kt;
    pl.pub.query_chunk = (int32_t)qc;
    pl.pub.key_partition = (int32_t)std::min<int64_t>(kp, 0x7FFFFFFF);
    pl.pub.n_partitions = (int32_t)nparts;
    pl.pub.n_chunks = (int32_t)nchunks;
    pl.pub.cand_capacity = cg;
    pl.pub.workspace_bytes = (S == 0 || B == 0) ? 0 : cand_bytes + cnt_bytes + rule_bytes;
    pl.t_eff = t_eff;
    pl.cand_bytes = cand_bytes;
    pl.rule_offset = cand_bytes + cnt_bytes;
    return SI_OK;
}

// Partitions one chunk's select launch covers (those the chunk's last row reaches).
inline int32_t chunk_partitions(const PlanInternal& pl, int64_t S, int64_t T, int32_t m,
                                int64_t q_pos0, int32_t chunk) {
    const int64_t qc = pl.pub.query_chunk;
    const int64_t r1 = std::min<int64_t>(S, (int64_t)(chunk + 1) * qc);
    const int64_t n_last = visible_count_host(q_pos0 + r1 - 1, m, T);
    const int64_t p = ceil_div(n_last, pl.pub.key_partition);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(p, pl.pub.n_partitions));
}

}  // namespace si
