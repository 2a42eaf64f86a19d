// Select stage: fused indexer scoring + exact running local top-k per (query, key
// partition).  This is the chunked score-and-reduce step of the pages' method (the
// running top-k kept without the full intermediate: skillsdirectory.com "Streamindex
// Csa Topk", Core Technique 1; per-chunk candidates handed to a merge: jeff.news page,
// sequence diagram), laid out for gfx950.
//
// One workgroup = one tile of 32 query rows x one key partition [p*KP, (p+1)*KP).
// It walks the partition in register tiles of NWAVE*KB*32 keys (score_regs), and
// after each tile:
//   filter   every lane compares its 16*KB scores (one query each) against that
//            query's running threshold theta (an exact selection key, initially 0)
//            and appends the survivors to the query's candidate buffer in the
//            workspace (CG slots, LDS atomic counter);
// and after every key_tile keys (NSUB register tiles):
//   compact  a query whose buffer could overflow in the next key tile is reduced, by
//            one wave, to its exact top-k (wave radix select over the 64-bit keys held
//            in registers), and theta becomes the k-th key.
// At the end of the partition each buffer is compacted to at most k entries; the
// merge stage sorts and merges the partition lists.
//
// Correctness of the threshold: after a compaction the buffer holds the k best keys
// seen so far and theta is the k-th of them; a later key below theta has k better keys
// already and can never enter the top-k.  Keys are unique (score bits, ~index), so
// every comparison is strict and the result is the unique top-k.
#include "si_kernels.hpp"

namespace si {

// Reduces one query's candidate buffer buf[0, cnt) (cnt > k, unique keys) to its exact
// top k, in place, and returns the k-th key.  Called by a whole wave; kept out of
// line so its E keys per lane do not add to the scoring loop's register budget.
template <int E>
__device__ __noinline__ uint64_t compact_to_topk(uint64_t* buf, int cnt, int k,
                                                 uint32_t* hist) {
    const int lane = lane_id();
    RegKeys<E> R;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * 64 + lane;
        R.v[e] = i < cnt ? buf[i] : 0ull;
    }
    const uint64_t kth = wave_select_kth(R, k, hist);
    int mine = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) mine += (R.v[e] >= kth) ? 1 : 0;
    uint64_t* dst = buf + wave_excl_scan(mine);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (R.v[e] >= kth) *dst++ = R.v[e];
    return kth;
}

template <int NWAVE, int KB, int NSUB, int CG, bool FP8>
__global__ void __launch_bounds__(NWAVE * 64)
select_kernel(SelectArgs A) {
    constexpr int NT = NWAVE * 64;
    constexpr int RT = NWAVE * KB * kMB;   // keys per register tile
    constexpr int KT = RT * NSUB;          // keys per key tile
    constexpr int E = CG / 64;             // candidate keys per lane when compacting
    static_assert(CG % 64 == 0, "capacity must be a multiple of the wave size");

    __shared__ ScoreLds L;
    SI_DECLARE_QBUFS(Q);
    __shared__ uint64_t sTheta[kTQ];
    __shared__ int32_t sCnt[kTQ];
    __shared__ int32_t sN[kTQ];
    __shared__ uint32_t sHist[NWAVE][256];

    const Problem& P = A.P;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // heavy tiles (late rows, many visible keys) first
    int64_t id = blockIdx.x;
    const int64_t b = id % P.B;
    id /= P.B;
    const int p = (int)(id % A.P_chunk);
    id /= A.P_chunk;
    const int tile = A.n_tiles - 1 - (int)id;

    const int64_t row0 = A.chunk_row0 + (int64_t)tile * kTQ;
    const int rows_valid = (int)min((int64_t)kTQ, A.chunk_row1 - row0);
    const int64_t t0 = P.q_pos0 + row0;
    const int64_t n_last = visible_keys(t0 + rows_valid - 1, P.m, P.T);
    const int64_t key_lo = (int64_t)p * A.KP;
    const int64_t key_hi = min(key_lo + A.KP, n_last);
    const int64_t slot0 = (b * A.QC + (row0 - A.chunk_row0)) * A.P_ws + p;

    if (key_lo >= key_hi) {
        if (tid < rows_valid) A.cnt[slot0 + (int64_t)tid * A.P_ws] = 0;
        return;
    }

    load_w_tile<NT>(P, b, row0, rows_valid, L);
    if (tid < kTQ) {
        sTheta[tid] = 0ull;
        sCnt[tid] = 0;
        sN[tid] = tid < rows_valid ? (int)min(visible_keys(t0 + tid, P.m, P.T), key_hi) : 0;
    }
    __syncthreads();

    const int qj = lane & 31;                      // this lane's query in the tile
    uint64_t* const my_cand = A.cand + (slot0 + (int64_t)qj * A.P_ws) * CG;

    int sub = 0;
    for (int64_t key0 = key_lo; key0 < key_hi; key0 += RT) {
        f32x16 acc[KB];
        score_regs<NWAVE, KB, FP8>(P, b, row0, rows_valid, key0, L, Q, acc);

        // ---- filter against the running threshold, append survivors ----------
        // A key beats theta iff its score is larger than theta's score, or equal with
        // a lower index; the float compare decides almost every case in one op.  The
        // causal mask only needs checking when the tile crosses this query's end.
        const int nj = sN[qj];
        const uint64_t th = sTheta[qj];
        const float thf = th == 0ull ? -__builtin_inff() : key_score(th);
        const uint32_t th_lo = (uint32_t)th;
        const int64_t kbase = key0 + (int64_t)wave * KB * kMB;
        const bool full = kbase + KB * kMB <= nj;
        uint32_t pass_bits[KB];                        // bit r of block kb: key passes
        int npass = 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint32_t bits = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float v = acc[kb][r];
                const int64_t s = kbase + kb * kMB + mfma_row(r, lane);
                bool pass = v > thf || (v == thf && th != 0ull && ~(uint32_t)s > th_lo);
                if (!full) pass = pass && s < nj;
                bits |= (pass ? 1u : 0u) << r;
            }
            pass_bits[kb] = bits;
            npass += __popc(bits);
        }
        if (npass) {
            const int base = atomicAdd(&sCnt[qj], npass);
            // the compaction policy keeps base + npass <= CG; the bound below only
            // keeps a broken invariant from writing outside this query's buffer
            int pos = base;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (pass_bits[kb] & (1u << r)) {
                        const int64_t s = kbase + kb * kMB + mfma_row(r, lane);
                        if (pos < CG) my_cand[pos] = make_key(acc[kb][r], (uint32_t)s);
                        ++pos;
                    }
                }
        }

        // ---- compaction: keep room for one more key tile; exact top-k at the end ----
        ++sub;
        const bool last = key0 + RT >= key_hi;
        if (sub == NSUB || last) {
            sub = 0;
            __syncthreads();
            const int limit = last ? A.k : CG - KT;
            for (int jj = wave; jj < rows_valid; jj += NWAVE) {
                const int cj = min(sCnt[jj], CG);
                if (cj > limit) {
                    uint64_t* buf = A.cand + (slot0 + (int64_t)jj * A.P_ws) * CG;
                    const uint64_t kth = compact_to_topk<E>(buf, cj, A.k, sHist[wave]);
                    if (lane == 0) {
                        sCnt[jj] = A.k;
                        sTheta[jj] = kth;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (tid < rows_valid) A.cnt[slot0 + (int64_t)tid * A.P_ws] = min(sCnt[tid], A.k);
}

template <int NWAVE, int KB, int NSUB, int CG, bool FP8>
static hipError_t launch_one(const SelectArgs& a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_tiles * a.P_chunk * a.P.B;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((select_kernel<NWAVE, KB, NSUB, CG, FP8>), dim3((unsigned)grid),
                       dim3(NWAVE * 64), 0, stream, a);
    return hipGetLastError();
}

template <bool FP8, int CG>
static hipError_t launch_tile(const SelectArgs& a, int nwave, int kb, int nsub,
                              hipStream_t stream) {
    if (nwave == 2 && kb == 1 && nsub == 1) return launch_one<2, 1, 1, CG, FP8>(a, stream);
    if (nwave == 4 && kb == 1 && nsub == 1) return launch_one<4, 1, 1, CG, FP8>(a, stream);
    if (nwave == 8 && kb == 1 && nsub == 1) return launch_one<8, 1, 1, CG, FP8>(a, stream);
    if (nwave == 8 && kb == 2 && nsub == 1) return launch_one<8, 2, 1, CG, FP8>(a, stream);
    if (nwave == 8 && kb == 2 && nsub == 2) return launch_one<8, 2, 2, CG, FP8>(a, stream);
    if (nwave == 4 && kb == 6 && nsub == 1) return launch_one<4, 6, 1, CG, FP8>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs& a, int nwave, int kb, int nsub, int cg, bool fp8,
                         hipStream_t stream) {
    if (fp8) {
        if (cg == 2048) return launch_tile<true, 2048>(a, nwave, kb, nsub, stream);
        if (cg == 4096) return launch_tile<true, 4096>(a, nwave, kb, nsub, stream);
    } else {
        if (cg == 2048) return launch_tile<false, 2048>(a, nwave, kb, nsub, stream);
        if (cg == 4096) return launch_tile<false, 4096>(a, nwave, kb, nsub, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace si
