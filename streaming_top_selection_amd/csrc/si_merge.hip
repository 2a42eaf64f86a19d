// Merge stage: per query row, merge the local top-k lists of its key partitions into
// the final top-k, sorted by (score desc, index asc), padded with -1 / -inf.  This is
// the partition merge of the pages' method: local top-k lists of all blocks merged
// into the final top-k with no global sort of the scores (geoz.com.cn page, FAQ;
// jeff.news page, sequence diagram: merge-topk keeps the final top-k).
//
// General case, one 64-lane workgroup per query row: the lists (at most partitions *
// k keys, bounded by the planner to 8192) are gathered into LDS; if they hold more than k
// keys an exact radix select finds the k-th key and an in-place compaction keeps the
// top k; a bitonic sort orders them.  HBM traffic: read the lists, write the row.
#include "si_compact.hpp"
#include "si_kernels.hpp"
#include "si_sort.hpp"

namespace si {

__global__ void __launch_bounds__(64) merge_kernel(MergeArgs A) {
    extern __shared__ uint64_t sbuf[];
    __shared__ uint32_t hist[256];

    const int lane = lane_id();
    const int64_t nrows = A.chunk_row1 - A.chunk_row0;
    const int64_t b = (int64_t)blockIdx.x / nrows;
    const int64_t r = (int64_t)blockIdx.x - b * nrows;
    const int64_t row = A.chunk_row0 + r;
    const int64_t n_t = visible_keys(A.q_pos0 + row, A.m, A.T);
    const int Pt = n_t > 0 ? (int)min((int64_t)A.P_chunk, (n_t + A.KP - 1) / A.KP) : 0;
    const int64_t slot0 = (b * A.QC + r) * A.P_ws;

    // gather the partition lists
    // each list holds at most k keys; the clamp keeps a corrupted count from driving
    // the loops below past the LDS buffer
    const int c = lane < Pt ? min(max(A.cnt[slot0 + lane], 0), A.k) : 0;
    const int off = wave_excl_scan(c);
    const int total = wave_sum(c);
    for (int p = 0; p < Pt; ++p) {
        const int cp = __shfl(c, p);
        const int op = __shfl(off, p);
        const uint64_t* src = A.cand + (slot0 + p) * (int64_t)A.CG;
        for (int i = lane; i < cp; i += 64) sbuf[op + i] = src[i];
    }
    wave_sync();

    int n = total;
    if (total > A.k) {
        const uint64_t kth = wave_select_kth(LdsKeys{sbuf, total}, A.k, hist);
        int wpos = 0;
        for (int base = 0; base < total; base += 64) {
            const int i = base + lane;
            const uint64_t v = i < total ? sbuf[i] : 0ull;
            const bool keep = i < total && v >= kth;
            wave_sync();
            const uint64_t bal = __ballot(keep);
            if (keep) sbuf[wpos + __popcll(bal & lanemask_lt())] = v;
            wpos += __popcll(bal);
            wave_sync();
        }
        n = A.k;
    }

    // bitonic sort of sbuf[0, n2) into descending order
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = n + lane; i < n2; i += 64) sbuf[i] = 0ull;
    wave_sync();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int pi = lane; pi < (n2 >> 1); pi += 64) {
                const int a = 2 * stride * (pi / stride) + (pi % stride);
                const int bb = a + stride;
                const bool desc = (a & size) == 0;
                const uint64_t x = sbuf[a], y = sbuf[bb];
                if (desc ? (x < y) : (x > y)) {
                    sbuf[a] = y;
                    sbuf[bb] = x;
                }
            }
            wave_sync();
        }
    }

    int32_t* oi = A.out_idx + (b * A.S + row) * (int64_t)A.k;
    float* os = A.out_score + (b * A.S + row) * (int64_t)A.k;
    for (int j = lane; j < A.k; j += 64) {
        if (j < n) {
            const uint64_t key = sbuf[j];
            oi[j] = key_index(key);
            os[j] = key_score(key);
        } else {
            oi[j] = -1;
            os[j] = -__builtin_inff();
        }
    }
}

// ---- one partition per row and k <= 512: a register sort -----------------------
// The row's single list already holds its top-k (the select stage compacted it to at
// most k keys), so the merge is a sort.  One wave per row; lane l holds elements
// EPL*l .. EPL*l + EPL-1 of a 64*EPL-key bitonic network (EPL = 8, 16 or 32 keys per
// lane for k up to 512, 1024, 2048; padding keys are 0, below every real key), so
// strides below EPL compare within a lane and strides EPL .. 32*EPL against lane
// l ^ (stride / EPL).  Loads and stores are contiguous runs per lane.
constexpr int kSortWaves = 4;

template <int LE>
__global__ void __launch_bounds__(kSortWaves * 64) merge_sort_kernel(MergeArgs A) {
    constexpr int EPL = 1 << LE;
    const int lane = lane_id();
    const int64_t nrows = A.chunk_row1 - A.chunk_row0;
    const int64_t id = (int64_t)blockIdx.x * kSortWaves + wave_id();
    if (id >= A.B * nrows) return;
    const int64_t b = id / nrows;
    const int64_t r = id - b * nrows;
    const int64_t row = A.chunk_row0 + r;
    const int64_t slot0 = (b * A.QC + r) * A.P_ws;
    const int64_t n_t = visible_keys(A.q_pos0 + row, A.m, A.T);
    // the clamp keeps a corrupted count inside the list
    const int n = n_t > 0 ? min(max(A.cnt[slot0], 0), A.k) : 0;

    // slots EPL*lane .. EPL*lane + EPL-1 of the list (all inside it: the launcher
    // checks that its stride holds 64*EPL slots)
    const uint64_t* src = A.cand + slot0 * (int64_t)A.CG + EPL * lane;
    uint64_t x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + e);
        x[e] = ((uint64_t)v.y << 32) | v.x;
        x[e + 1] = ((uint64_t)v.w << 32) | v.z;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = EPL * lane + e < n ? x[e] : 0ull;
    sort_desc<LE>(x);

    write_sorted_keys<LE>(A.out_idx + (b * A.S + row) * (int64_t)A.k,
                          A.out_score + (b * A.S + row) * (int64_t)A.k, A.k, x, n, lane);
}

// ---- one partition per row, the final selection left to the merge --------------
// The row's list holds its top k among up to list_max keys (the select stage's
// threshold keeps it short, but it did not cut it to k).  One wave per row streams the
// list once, 128 keys a round: the select stage's histogram gives the keep rule
// (KeepRule), so a key above bin d goes straight to the kept set in LDS and a key of
// bin d to a 64-slot stage, where the k - above largest are found by counting larger
// keys.  A list the rule does not fit (a query whose histogram was off, or more than
// 64 keys in bin d) has its k-th largest key found by radix passes over the list in
// memory and is streamed again.  The k kept keys are read back from LDS in the sort
// layout, sorted in registers (64*EPL >= k) and written.  A list of at most k keys is
// sorted directly.  Few registers per wave, so many waves per SIMD hide the loads.
constexpr int kMergeRounds = 4;   // list rounds of 128 slots loaded ahead of use

template <int LE>
__global__ void __launch_bounds__(kSortWaves * 64) merge_select_sort_kernel(MergeArgs A) {
    constexpr int EPL = 1 << LE;
    __shared__ uint32_t hist[kSortWaves][256];
    __shared__ __attribute__((aligned(16))) uint64_t stage[kSortWaves][64];
    __shared__ __attribute__((aligned(16))) uint64_t kept[kSortWaves][64 * EPL];
    const int lane = lane_id();
    const int wave = wave_id();
    const int64_t nrows = A.chunk_row1 - A.chunk_row0;
    const int64_t id = (int64_t)blockIdx.x * kSortWaves + wave;
    if (id >= A.B * nrows) return;
    const int64_t b = id / nrows;
    const int64_t r = id - b * nrows;
    const int64_t row = A.chunk_row0 + r;
    const int64_t slot0 = (b * A.QC + r) * A.P_ws;
    const int64_t n_t = visible_keys(A.q_pos0 + row, A.m, A.T);
    // the clamp keeps a corrupted count inside the list (the launcher checks that the
    // list stride holds list_max slots and that k <= 64*EPL)
    const int n = __builtin_amdgcn_readfirstlane(n_t > 0 ? min(max(A.cnt[slot0], 0), A.list_max) : 0);
    const uint64_t* src = A.cand + slot0 * (int64_t)A.CG;

    uint64_t x[EPL];
    int nk;
    if (n <= A.k) {
        // slots EPL*lane .. EPL*lane + EPL-1, as in merge_sort_kernel
#pragma unroll
        for (int e = 0; e < EPL; e += 2) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + EPL * lane + e);
            x[e] = ((uint64_t)v.y << 32) | v.x;
            x[e + 1] = ((uint64_t)v.w << 32) | v.z;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = EPL * lane + e < n ? x[e] : 0ull;
        nk = n;
    } else {
        uint64_t* const kw = kept[wave];
        uint64_t* const sw = stage[wave];
        // appends the keys of `keep` (one per lane) at base, in lane order
        auto append = [&](bool keep, uint64_t v, uint64_t* dst, int cap, int& base) {
            const uint64_t m = __ballot(keep);
            const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (keep && at < cap) dst[at] = v;
            base += __popcll(m);
        };
        const KeepRule rl = A.rule[slot0];
        bool fast = rl.d >= 0;
        int base = 0;
        // two keys per lane and load (slots i + 2 lane, i + 2 lane + 1): the launcher
        // checks that the list stride holds list_max rounded up to 128 slots
        // (a slot past the list's last 128-slot round reads that round's last pair
        // instead, so loads need no branch; its keys are dropped as past n)
        const int lim = (n + 127) / 128 * 128 - 2;
        auto load2 = [&](int slot, uint64_t& v0, uint64_t& v1) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + min(slot, lim));
            v0 = slot < n ? (((uint64_t)w.y << 32) | w.x) : 0ull;
            v1 = slot + 1 < n ? (((uint64_t)w.w << 32) | w.z) : 0ull;
        };
        if (fast) {
            sw[lane] = 0ull;
            int nd = 0;
            const uint32_t d = (uint32_t)rl.d;
            // rounds of 128 slots, four loaded before any is used (one load and wait at
            // a time left the stream latency-bound)
            for (int i = 0; i < n; i += kMergeRounds * 128) {
                uint64_t v[kMergeRounds][2];
#pragma unroll
                for (int u = 0; u < kMergeRounds; ++u) load2(i + 128 * u + 2 * lane, v[u][0], v[u][1]);
#pragma unroll
                for (int u = 0; u < kMergeRounds; ++u) {
                    const int slot = i + 128 * u + 2 * lane;
                    const uint32_t b0 = hist_bin(key_score(v[u][0]), rl.inv, rl.off);
                    const uint32_t b1 = hist_bin(key_score(v[u][1]), rl.inv, rl.off);
                    append(slot < n && b0 > d, v[u][0], kw, 64 * EPL, base);
                    append(slot + 1 < n && b1 > d, v[u][1], kw, 64 * EPL, base);
                    append(slot < n && b0 == d, v[u][0], sw, 64, nd);
                    append(slot + 1 < n && b1 == d, v[u][1], sw, 64, nd);
                }
            }
            const int need = A.k - base;
            // the rule holds for this list (it always does; a list it does not fit goes
            // the general way)
            fast = base == (int)rl.above && need >= 1 && need <= nd && nd <= 64;
            if (fast) {
                wave_sync();
                const uint64_t th = stage_kth(sw, nd, need);
                const uint64_t v = sw[lane];
                append(lane < nd && v >= th, v, kw, 64 * EPL, base);
            }
        }
        if (!fast) {
            // the exact k-th largest key by radix passes over the list in memory, then
            // the keys at or above it (exactly k: keys are unique)
            const uint64_t th = wave_select_kth(LdsKeys{src, n}, A.k, hist[wave]);
            base = 0;
            for (int i = 0; i < n; i += kMergeRounds * 128) {
                uint64_t v[kMergeRounds][2];
#pragma unroll
                for (int u = 0; u < kMergeRounds; ++u) load2(i + 128 * u + 2 * lane, v[u][0], v[u][1]);
#pragma unroll
                for (int u = 0; u < kMergeRounds; ++u) {
                    const int slot = i + 128 * u + 2 * lane;
                    append(slot < n && v[u][0] >= th, v[u][0], kw, 64 * EPL, base);
                    append(slot + 1 < n && v[u][1] >= th, v[u][1], kw, 64 * EPL, base);
                }
            }
        }
        wave_sync();
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = EPL * lane + e < A.k ? kw[EPL * lane + e] : 0ull;
        nk = A.k;
    }
    sort_desc<LE>(x);
    write_sorted_keys<LE>(A.out_idx + (b * A.S + row) * (int64_t)A.k,
                          A.out_score + (b * A.S + row) * (int64_t)A.k, A.k, x, nk, lane);
}

// Several partitions whose lists hold at most 64*EPL keys together: gathered into LDS
// (one 64-lane group per row, as in merge_kernel), then sorted in registers; the
// first min(k, total) keys are the row's top-k.
template <int LE>
__global__ void __launch_bounds__(64) merge_gather_sort_kernel(MergeArgs A) {
    constexpr int EPL = 1 << LE;
    __shared__ uint64_t sbuf[64 * EPL];
    const int lane = lane_id();
    const int64_t nrows = A.chunk_row1 - A.chunk_row0;
    const int64_t b = (int64_t)blockIdx.x / nrows;
    const int64_t r = (int64_t)blockIdx.x - b * nrows;
    const int64_t row = A.chunk_row0 + r;
    const int64_t n_t = visible_keys(A.q_pos0 + row, A.m, A.T);
    const int Pt = n_t > 0 ? (int)min((int64_t)A.P_chunk, (n_t + A.KP - 1) / A.KP) : 0;
    const int64_t slot0 = (b * A.QC + r) * A.P_ws;
    // the clamps keep a corrupted count inside the lists and the buffer (the launcher
    // checks partitions * k <= 64*EPL)
    const int c = lane < Pt ? min(max(A.cnt[slot0 + lane], 0), A.k) : 0;
    const int off = wave_excl_scan(c);
    const int total = min(wave_sum(c), 64 * EPL);
    for (int p = 0; p < Pt; ++p) {
        const int cp = __shfl(c, p);
        const int op = __shfl(off, p);
        const uint64_t* src = A.cand + (slot0 + p) * (int64_t)A.CG;
        for (int i = lane; i < cp && op + i < 64 * EPL; i += 64) sbuf[op + i] = src[i];
    }
    wave_sync();
    uint64_t x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = EPL * lane + e < total ? sbuf[EPL * lane + e] : 0ull;
    sort_desc<LE>(x);
    write_sorted_keys<LE>(A.out_idx + (b * A.S + row) * (int64_t)A.k,
                          A.out_score + (b * A.S + row) * (int64_t)A.k, A.k, x, min(total, A.k),
                          lane);
}

template <int LE>
static hipError_t launch_merge_gather_sort(const MergeArgs& a, int64_t rows, hipStream_t stream) {
    hipLaunchKernelGGL(merge_gather_sort_kernel<LE>, dim3((unsigned)rows), dim3(64), 0, stream, a);
    return hipGetLastError();
}

template <int LE>
static hipError_t launch_merge_sort(const MergeArgs& a, int64_t rows, hipStream_t stream) {
    const int64_t grid = (rows + kSortWaves - 1) / kSortWaves;
    hipLaunchKernelGGL(merge_sort_kernel<LE>, dim3((unsigned)grid), dim3(kSortWaves * 64), 0,
                       stream, a);
    return hipGetLastError();
}

template <int LE>
static hipError_t launch_merge_select_sort(const MergeArgs& a, int64_t rows, hipStream_t stream) {
    const int64_t grid = (rows + kSortWaves - 1) / kSortWaves;
    hipLaunchKernelGGL((merge_select_sort_kernel<LE>), dim3((unsigned)grid),
                       dim3(kSortWaves * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    const int64_t rows = a.B * (a.chunk_row1 - a.chunk_row0);
    if (rows <= 0) return hipSuccess;
    // one partition whose list may hold more than k keys: select, then sort
    if (a.list_max > a.k) {
        if (a.P_chunk != 1 || a.k > 512 || a.CG < (a.list_max + 127) / 128 * 128 || a.CG < 512)
            return hipErrorInvalidValue;
        return launch_merge_select_sort<3>(a, rows, stream);
    }
    // one partition: sort the single list in registers (the list stride must hold the
    // network's 64*EPL slots, which every planned capacity does)
    if (a.P_chunk == 1) {
        if (a.k <= 512 && a.CG >= 512) return launch_merge_sort<3>(a, rows, stream);
        if (a.k <= 1024 && a.CG >= 1024) return launch_merge_sort<4>(a, rows, stream);
        if (a.k <= 2048 && a.CG >= 2048) return launch_merge_sort<5>(a, rows, stream);
    }
    // several partitions holding at most 2048 keys together: gather, register sort
    const int64_t entries = (int64_t)a.P_chunk * a.k;
    if (entries <= 512) return launch_merge_gather_sort<3>(a, rows, stream);
    if (entries <= 1024) return launch_merge_gather_sort<4>(a, rows, stream);
    if (entries <= 2048) return launch_merge_gather_sort<5>(a, rows, stream);
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows), dim3(64),
                       (size_t)a.lds_entries * sizeof(uint64_t), stream, a);
    return hipGetLastError();
}

}  // namespace si
