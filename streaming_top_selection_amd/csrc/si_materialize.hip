// Materialise-then-select reference path (the public CSA approach the StreamIndex
// abstract contrasts with: write the scores, then reduce to top-k), kept for small S
// and for row blocks of large S.  Its score kernel shares score_regs with the
// streaming path; its selection is an independent algorithm: a 32-bit radix select
// on the score values, an index-order pass that takes the lowest indices among
// scores equal to the k-th, and a rank sort.
#include "si_kernels.hpp"
#include "si_score_q8.hpp"

namespace si {

// ---- score write-out: one workgroup = 32 rows x 512 keys --------------------------
template <int OP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mat_score_kernel(MatScoreArgs A) {
    constexpr int NWAVE = 4, KB = 4, RT = NWAVE * KB * kMB;
    __shared__ ScoreLds L;
    SI_DECLARE_QBUFS(Q, OP);
    const Problem& P = A.P;
    const int lane = threadIdx.x & 63, wave = wave_id();

    int64_t id = blockIdx.x;
    const int64_t b = id % P.B;
    id /= P.B;
    const int kt = (int)(id % A.n_key_tiles);
    const int rt = (int)(id / A.n_key_tiles);
    const int64_t trow0 = A.tile_row0 + (int64_t)rt * kTQ;
    const int rows_valid = (int)min((int64_t)kTQ, P.S - trow0);
    const int64_t key0 = (int64_t)kt * RT;
    const int64_t n_last = visible_keys(P.q_pos0 + trow0 + rows_valid - 1, P.m, P.T);

    f32x16 acc[KB];
    const bool live = key0 < n_last;
    if (live) {
        load_w_tile<NWAVE * 64>(P, b, trow0, rows_valid, L);
        __syncthreads();
        score_tile<NWAVE, KB, OP>(P, b, trow0, rows_valid, key0, P.T, L, Q, acc);
    }
    // register r holds row trow0 + mfma_row(r, lane); lanes run along the keys, so
    // each store writes 32 consecutive scores of two rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = trow0 + mfma_row(r, lane);
        if (row >= trow0 + rows_valid || row < A.row0 || row >= A.row0 + A.rows) continue;
        const int64_t nvis = visible_keys(P.q_pos0 + row, P.m, P.T);
        float* out = A.scores + (b * A.rows + (row - A.row0)) * P.T;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t s = key0 + (int64_t)(wave * KB + kb) * kMB + (lane & 31);
            if (s < P.T) out[s] = (live && s < nvis) ? acc[kb][r] : -__builtin_inff();
        }
    }
}

// ---- exact selection from one written score row: one 64-lane group per row -------
__global__ void __launch_bounds__(64) mat_select_kernel(MatSelectArgs A) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t pick[2];
    __shared__ uint64_t sel[kMaxK];
    const int lane = lane_id();
    const int64_t b = (int64_t)blockIdx.x / A.rows;
    const int64_t rr = (int64_t)blockIdx.x - b * A.rows;
    const int64_t row = A.row0 + rr;
    const float* sc = A.scores + (b * A.rows + rr) * A.T;
    const int64_t n = visible_keys(A.q_pos0 + row, A.m, A.T);
    const int need = (int)min((int64_t)A.k, n);

    // value v* of the k-th largest score and how many scores equal to it to take
    uint32_t vstar = 0;
    int eq_take = 0;
    const bool partial = n > A.k;
    if (partial) {
        uint32_t prefix = 0, pmask = 0;
        int rank = A.k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = lane; i < 256; i += 64) hist[i] = 0u;
            __syncthreads();
            for (int64_t i = lane; i < n; i += 64) {
                const uint32_t u = ord_f32(sc[i]);
                if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (lane == 0) {
                uint32_t cum = 0;
                int d = 255;
                for (; d > 0; --d) {
                    if (cum + hist[d] >= (uint32_t)rank) break;
                    cum += hist[d];
                }
                pick[0] = (uint32_t)d;
                pick[1] = cum;
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            pmask |= 0xFFu << shift;
            rank -= (int)pick[1];
            __syncthreads();
        }
        vstar = prefix;
        eq_take = rank;
    }

    // collect in index order: every score above v*, then the lowest-index eq_take
    // scores equal to v* (all visible scores when n <= k)
    int cnt = 0, eq_seen = 0;
    for (int64_t base = 0; base < n; base += 64) {
        const int64_t i = base + lane;
        const bool valid = i < n;
        const uint32_t u = valid ? ord_f32(sc[i]) : 0u;
        const bool gt = valid && (!partial || u > vstar);
        const bool eq = valid && partial && u == vstar;
        const uint64_t eqb = __ballot(eq);
        const int eq_rank = eq_seen + __popcll(eqb & lanemask_lt());
        eq_seen += __popcll(eqb);
        const bool take = gt || (eq && eq_rank < eq_take);
        const uint64_t tb = __ballot(take);
        if (take) sel[cnt + __popcll(tb & lanemask_lt())] = make_key(sc[i], (uint32_t)i);
        cnt += __popcll(tb);
    }
    __syncthreads();

    // rank sort: position = number of selected keys larger than this one
    int32_t* oi = A.out_idx + (b * A.S + row) * (int64_t)A.k;
    float* os = A.out_score + (b * A.S + row) * (int64_t)A.k;
    for (int e = lane; e < need; e += 64) {
        const uint64_t key = sel[e];
        int pos = 0;
        for (int f = 0; f < need; ++f) pos += sel[f] > key ? 1 : 0;
        oi[pos] = key_index(key);
        os[pos] = key_score(key);
    }
    for (int j = need + lane; j < A.k; j += 64) {
        oi[j] = -1;
        os[j] = -__builtin_inff();
    }
}

hipError_t launch_mat_score(const MatScoreArgs& a, int op, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_row_tiles * a.n_key_tiles * a.P.B;
    if (grid <= 0) return hipSuccess;
    switch (op) {
        case kOpBf16:
            hipLaunchKernelGGL(mat_score_kernel<kOpBf16>, dim3((unsigned)grid), dim3(256), 0, stream, a);
            break;
        case kOpBf16K8:
            hipLaunchKernelGGL(mat_score_kernel<kOpBf16K8>, dim3((unsigned)grid), dim3(256), 0, stream, a);
            break;
        case kOpF8:
            hipLaunchKernelGGL(mat_score_kernel<kOpF8>, dim3((unsigned)grid), dim3(256), 0, stream, a);
            break;
        case kOpF8K4:
            hipLaunchKernelGGL(mat_score_kernel<kOpF8K4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mat_select(const MatSelectArgs& a, hipStream_t stream) {
    const int64_t grid = a.B * a.rows;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(mat_select_kernel, dim3((unsigned)grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace si
