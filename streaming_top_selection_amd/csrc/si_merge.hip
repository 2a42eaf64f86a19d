// Merge stage: per query row, merge the local top-k lists of its key partitions into
// the final top-k, sorted by (score desc, index asc), padded with -1 / -inf.  This is
// the partition merge of the pages' method: local top-k lists of all blocks merged
// into the final top-k with no global sort of the scores (geoz.com.cn page, FAQ;
// jeff.news page, sequence diagram: merge-topk keeps the final top-k).
//
// One 64-lane workgroup per query row.  The lists (at most partitions * k keys,
// bounded by the planner to 8192) are gathered into LDS; if they hold more than k
// keys an exact radix select finds the k-th key and an in-place compaction keeps the
// top k; a bitonic sort orders them.  HBM traffic: read the lists, write the row.
#include "si_kernels.hpp"

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

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    const int64_t grid = a.B * (a.chunk_row1 - a.chunk_row0);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)grid), dim3(64),
                       (size_t)a.lds_entries * sizeof(uint64_t), stream, a);
    return hipGetLastError();
}

}  // namespace si
