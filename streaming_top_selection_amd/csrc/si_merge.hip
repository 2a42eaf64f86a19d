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

// ---- one partition per row and k <= 512: a register sort -----------------------
// The row's single list already holds its top-k (the select stage compacted it to at
// most k keys), so the merge is a sort.  One wave per row; lane l holds elements
// EPL*l .. EPL*l + EPL-1 of a 64*EPL-key bitonic network (EPL = 8, 16 or 32 keys per
// lane for k up to 512, 1024, 2048; padding keys are 0, below every real key), so
// strides below EPL compare within a lane and strides EPL .. 32*EPL against lane
// l ^ (stride / EPL).  Loads and stores are contiguous runs per lane.
constexpr int kSortWaves = 4;

// 64-bit lane exchange: partner lane ^ m (DPP within a quad for m = 1, 2)
template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
    if constexpr (M == 1 || M == 2) {
        constexpr int C = M == 1 ? kDppQuadSwap1 : kDppQuadSwap2;
        const uint32_t lo = dpp<C>(0u, (uint32_t)v), hi = dpp<C>(0u, (uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | lo;
    } else {
        return __shfl_xor(v, M);
    }
}

// One bitonic stage: blocks of 2^S elements, compare distance 2^T, LE = log2(EPL).
// A block sorts descending when bit S of its element index is 0 (the whole network's
// block always); bit S >= LE of the index EPL*lane + e is lane bit S - LE.
template <int LE, int S, int T>
__device__ __forceinline__ void bitonic_stage(uint64_t (&x)[1 << LE], int lane) {
    constexpr int EPL = 1 << LE, LN = LE + 6;   // log2 of the network size
    const bool desc_lane = S == LN || ((lane >> (S >= LE ? S - LE : 0)) & 1) == 0;
    if constexpr (T >= LE) {
        constexpr int M = 1 << (T - LE);
        // the lane with the lower index keeps the larger key in a descending block
        const bool keep_max = ((lane & M) == 0) == desc_lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint64_t p = xor_lane64<M>(x[e]);
            x[e] = (x[e] > p) == keep_max ? x[e] : p;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (e & (1 << T)) continue;
            const int e2 = e | (1 << T);
            const bool desc = S >= LE ? desc_lane : ((e >> S) & 1) == 0;
            const bool swap = (x[e] > x[e2]) != desc;
            const uint64_t a = x[e], b = x[e2];
            x[e] = swap ? b : a;
            x[e2] = swap ? a : b;
        }
    }
}

template <int LE, int S, int T>
__device__ __forceinline__ void bitonic_merge_steps(uint64_t (&x)[1 << LE], int lane) {
    bitonic_stage<LE, S, T>(x, lane);
    if constexpr (T > 0) bitonic_merge_steps<LE, S, T - 1>(x, lane);
}

template <int LE, int S>
__device__ __forceinline__ void bitonic_blocks(uint64_t (&x)[1 << LE], int lane) {
    bitonic_merge_steps<LE, S, S - 1>(x, lane);
    if constexpr (S < LE + 6) bitonic_blocks<LE, S + 1>(x, lane);
}

// Sorts the 64*EPL keys x (element EPL*lane + e in x[e]) into descending order.
template <int LE>
__device__ __forceinline__ void sort_desc(uint64_t (&x)[1 << LE]) {
    bitonic_blocks<LE, 1>(x, lane_id());
}

// Writes row `row` of batch entry b: the first n (<= k) of the sorted keys x (element
// EPL*lane + e in x[e]) as (index, score), then -1 / -inf up to k.
template <int LE>
__device__ __forceinline__ void write_sorted_row(const MergeArgs& A, int64_t b, int64_t row,
                                                 const uint64_t (&x)[1 << LE], int n, int lane) {
    constexpr int EPL = 1 << LE;
    int32_t* oi = A.out_idx + (b * A.S + row) * (int64_t)A.k + EPL * lane;
    float* os = A.out_score + (b * A.S + row) * (int64_t)A.k + EPL * lane;
    if (EPL * lane + EPL <= A.k && (A.k & 3) == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            int32_t vi[4];
            float vs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool real = EPL * lane + e + j < n;
                vi[j] = real ? key_index(x[e + j]) : -1;
                vs[j] = real ? key_score(x[e + j]) : -__builtin_inff();
            }
            *reinterpret_cast<u32x4*>(oi + e) =
                u32x4{(uint32_t)vi[0], (uint32_t)vi[1], (uint32_t)vi[2], (uint32_t)vi[3]};
            *reinterpret_cast<u32x4*>(os + e) =
                u32x4{__float_as_uint(vs[0]), __float_as_uint(vs[1]), __float_as_uint(vs[2]),
                      __float_as_uint(vs[3])};
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (EPL * lane + e < A.k) {
                const bool real = EPL * lane + e < n;
                oi[e] = real ? key_index(x[e]) : -1;
                os[e] = real ? key_score(x[e]) : -__builtin_inff();
            }
        }
    }
}

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

    write_sorted_row<LE>(A, b, row, x, n, lane);
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
    write_sorted_row<LE>(A, b, row, x, min(total, A.k), lane);
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

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    const int64_t rows = a.B * (a.chunk_row1 - a.chunk_row0);
    if (rows <= 0) return hipSuccess;
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
