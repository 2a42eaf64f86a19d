// Select stage: fused indexer scoring + exact running local top-k per (query, key
// partition).  This is the chunked score-and-reduce step of the pages' method (the
// running top-k kept without the full intermediate: skillsdirectory.com "Streamindex
// Csa Topk", Core Technique 1; per-chunk candidates handed to a merge: jeff.news page,
// sequence diagram), laid out for gfx950.
//
// One workgroup = one tile of 32 query rows x one key partition [p*KP, (p+1)*KP).
// It walks the partition in register tiles of NWAVE*KB*32 keys (score_regs), and
// after each tile:
//   filter   every score is compared with its query's running threshold score and
//            the survivors are appended to the query's candidate buffer in the
//            workspace (CG slots): one LDS atomic per query and wave reserves a
//            range, and each register writes its survivors as contiguous runs;
// and after every key_tile keys (NSUB register tiles):
//   compact  a query whose buffer could overflow in the next key tile is reduced, by
//            one wave with the keys in registers, to its best keys: between k and a
//            little more than k mid-partition (whole score bins, see si_compact.hpp),
//            exactly k at the partition's end; the smallest kept key's score becomes
//            the threshold.
// The merge stage then sorts (one partition) or merges the partition lists.
//
// Correctness of the threshold: after a compaction the buffer holds the best keys
// seen so far, at least k of them, and the threshold key theta is the smallest kept
// one; a later key below theta has k better keys already and can never enter the
// top-k.  Keys are unique (score bits, ~index).  Every key compared with theta comes
// from a later register tile, so its index is larger than theta's and a score equal
// to theta's loses the tie: the exact test "key > theta" is the float compare
// "score > score(theta)".
#pragma once

#include "si_compact.hpp"
#include "si_kernels.hpp"

namespace si {

// Compacts the candidate buffers of the rows in `todo` (a bit per row of the tile),
// each to between k and keep_max keys, and updates their counts and thresholds.  With
// E <= 32 the next row's keys are loaded while the current row is selected.
template <int E, int CG>
__device__ __forceinline__ void compact_rows(uint64_t todo, uint64_t* cand_tile,
                                             int64_t row_stride, int k, int keep_max,
                                             int32_t* sCnt, float* sThf, uint32_t* hist,
                                             uint64_t* stage) {
    const int lane = lane_id();
    auto pop = [&]() {
        if (todo == 0ull) return -1;
        const int j = __ffsll((long long)todo) - 1;
        todo &= todo - 1;
        return j;
    };
    auto count = [&](int j) { return min(__builtin_amdgcn_readfirstlane(sCnt[j]), CG); };
    auto finish = [&](int j, uint64_t (&v)[E]) {
        uint32_t tho;
        const int kept = compact_regs<E>(cand_tile + (int64_t)j * row_stride, v, count(j), k,
                                         keep_max, hist, stage, &tho);
        if (lane == 0) {
            sCnt[j] = kept;
            sThf[j] = unord_f32(tho);
        }
    };
    if constexpr (E <= 32) {
        // the next row's keys load while this row is selected (a row with no successor
        // re-loads itself, so that every iteration issues the same loads)
        uint64_t va[E], vb[E];
        int ja = pop();
        if (ja < 0) return;
        load_keys<E>(cand_tile + (int64_t)ja * row_stride, va);
        for (;;) {
            const int jb = pop();
            load_keys<E>(cand_tile + (int64_t)(jb >= 0 ? jb : ja) * row_stride, vb);
            finish(ja, va);
            if (jb < 0) break;
            ja = pop();
            load_keys<E>(cand_tile + (int64_t)(ja >= 0 ? ja : jb) * row_stride, va);
            finish(jb, vb);
            if (ja < 0) break;
        }
    } else {
        uint64_t v[E];
        for (int j = pop(); j >= 0; j = pop()) {
            load_keys<E>(cand_tile + (int64_t)j * row_stride, v);
            finish(j, v);
        }
    }
}

// Filter and append of one register tile (see the file comment).  Register r of block
// kb holds the score of query q = mfma_row(r, lane) and key kbase + 32*kb + (lane & 31);
// query q sits in register r_q = 4*(q/8) + q%4 of half (q/4)%2 of every block.
// MASKED: the keys cross the end of some query's visible range (or of the partition).
template <int KB, int CG, bool MASKED>
__device__ __forceinline__ void filter_append(const f32x16 (&acc)[KB], int64_t kbase,
                                              const float* sThf, const int32_t* sN,
                                              int32_t* sCnt, uint64_t* cand_tile,
                                              int64_t row_stride) {
    const int lane = lane_id();
    const int il = lane & 31;
    const bool upper = lane >= 32;
    float thf[16];
    int nj[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        thf[r] = sThf[mfma_row(r, lane)];
        if constexpr (MASKED) nj[r] = sN[mfma_row(r, lane)];
    }
    auto passes = [&](int r, int kb) {
        bool p = acc[kb][r] > thf[r];
        if constexpr (MASKED) p = p && kbase + kb * kMB + il < nj[r];
        return p;
    };
    // pass 1: survivors per query (wave-uniform counts), one atomic per query
    int my_count = 0;                       // lane q < 32: survivors of query q
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        uint32_t c_lo = 0, c_hi = 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint64_t m = __ballot(passes(r, kb));
            c_lo += __popc((uint32_t)m);
            c_hi += __popc((uint32_t)(m >> 32));
        }
        if (lane == mfma_row(r, 0)) my_count = (int)c_lo;
        if (lane == mfma_row(r, 32)) my_count = (int)c_hi;
    }
    int my_base = 0;
    if (lane < kTQ && my_count > 0) my_base = atomicAdd(&sCnt[lane], my_count);
    // pass 2: write each (register, block) as one run per half; every lane stores
    // (lanes with no survivor into the list's pad slots), so no store needs a branch,
    // and a group with no survivor at all is not skipped either: with no branch the
    // 16 x KB groups form one block the compiler can overlap (the pass is latency-bound
    // at one wave per SIMD).
    // A lane keeps its row's next free position in a register: its rank among its
    // half's survivors is its rank in the whole wave, less (upper half) the lower
    // half's survivors.  Per-half choices are bit selects on `half` (all ones in the
    // upper half), and the compares are redone on an opaque copy of the thresholds,
    // so no per-(register, block) mask has to survive from pass 1 in scalar registers.
    uint32_t half = upper ? ~0u : 0u;
    asm volatile("" : "+v"(half));
    auto sel = [&](uint32_t hi, uint32_t lo) { return (half & hi) | (~half & lo); };
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(thf[r]));
    uint32_t low[KB];                       // key low bits: ~index
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) low[kb] = ~(uint32_t)(kbase + kb * kMB + il);
    const uint32_t pad = (uint32_t)CG | (uint32_t)il;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int q_lo = mfma_row(r, 0), q_hi = mfma_row(r, 32);
        uint32_t next = sel((uint32_t)__builtin_amdgcn_readlane(my_base, q_hi),
                            (uint32_t)__builtin_amdgcn_readlane(my_base, q_lo));
        uint64_t* const row = cand_tile + (int64_t)(upper ? q_hi : q_lo) * row_stride;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bool pass = passes(r, kb);
            const uint64_t m = __ballot(pass);
            const uint32_t m_lo = (uint32_t)m, m_hi = (uint32_t)(m >> 32);
            const uint32_t n_lo = (uint32_t)__popc(m_lo), n_hi = (uint32_t)__popc(m_hi);
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi(m_hi, __builtin_amdgcn_mbcnt_lo(m_lo, 0u)) -
                                  (half & n_lo);
            // the compaction policy keeps every position below CG; the clamp only
            // keeps a broken invariant inside this query's pad slots
            const uint32_t dst = min(pass ? next + rank : ~0u, pad);
            row[dst] = ((uint64_t)ord_f32(acc[kb][r]) << 32) | low[kb];
            next += sel(n_hi, n_lo);
        }
    }
}

// One wave per SIMD (512 registers each): see score_regs.
template <int NWAVE, int KB, int NSUB, int CG, bool FP8>
__global__ void __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
select_kernel(SelectArgs A) {
    constexpr int NT = NWAVE * 64;
    constexpr int RT = NWAVE * KB * kMB;   // keys per register tile
    constexpr int KT = RT * NSUB;          // keys per key tile
    constexpr int E = CG / 64;             // candidate keys per lane when compacting
    static_assert(CG % 64 == 0, "capacity must be a multiple of the wave size");

    __shared__ ScoreLds L;
    SI_DECLARE_QBUFS(Q);
    __shared__ float sThf[kTQ];            // threshold score (-inf: none; +inf: no row)
    __shared__ int32_t sCnt[kTQ];          // candidates in the query's buffer
    __shared__ int32_t sN[kTQ];            // end of the query's visible keys here
    __shared__ uint32_t sHist[NWAVE][256];
    __shared__ __attribute__((aligned(16))) uint64_t sStage[NWAVE][64];

    const Problem& P = A.P;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();

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
    constexpr int CGS = CG + kCandPad;     // list stride

    if (key_lo >= key_hi) {
        if (tid < rows_valid) A.cnt[slot0 + (int64_t)tid * A.P_ws] = 0;
        return;
    }

    load_w_tile<NT>(P, b, row0, rows_valid, L);
    if (tid < kTQ) {
        sThf[tid] = tid < rows_valid ? -__builtin_inff() : __builtin_inff();
        sCnt[tid] = 0;
        sN[tid] = tid < rows_valid ? (int)min(visible_keys(t0 + tid, P.m, P.T), key_hi) : 0;
    }
    __syncthreads();
    // keys below this bound are visible to every row of the tile and inside the partition
    const int64_t all_visible = min(visible_keys(t0, P.m, P.T), key_hi);
    const int64_t row_stride = (int64_t)A.P_ws * CGS;
    // keys a mid-partition compaction may keep: k plus a quarter of the free room
    const int keep_mid = A.k + (CG - KT - A.k) / 4;

    int sub = 0;
    for (int64_t key0 = key_lo; key0 < key_hi; key0 += RT) {
        f32x16 acc[KB];
        score_regs<NWAVE, KB, FP8>(P, b, row0, rows_valid, key0, key_hi, L, Q, acc);

        const int64_t kbase = key0 + (int64_t)wave * KB * kMB;
        uint64_t* const cand_tile = A.cand + slot0 * CGS;
        if (kbase + KB * kMB <= all_visible)
            filter_append<KB, CG, false>(acc, kbase, sThf, sN, sCnt, cand_tile, row_stride);
        else
            filter_append<KB, CG, true>(acc, kbase, sThf, sN, sCnt, cand_tile, row_stride);

        // ---- compaction: keep room for one more key tile; exact top-k at the end ----
        ++sub;
        const bool last = key0 + RT >= key_hi;
        if (sub == NSUB || last) {
            sub = 0;
            // every wave's reservations have landed once its LDS operations have: the
            // counts are final, and every wave takes the same decision from them (no
            // count changes before the barrier inside the branch)
            lds_barrier();
            // mid-partition: make room for the next key tile, keeping at most keep_mid
            // keys (a few over k saves radix passes); at the end: exactly the top k
            const int limit = last ? A.k : CG - KT;
            const int keep_max = last ? A.k : keep_mid;
            const int c = lane < kTQ ? min(sCnt[lane], CG) : 0;
            if (__ballot(c > limit) != 0ull) {
                // the appended keys of every wave are visible once its stores have landed
                __syncthreads();
                // rows wave, wave + NWAVE, ... of the tile are this wave's
                const uint64_t todo = __ballot(c > limit && lane % NWAVE == wave);
                compact_rows<E, CG>(todo, A.cand + slot0 * CGS, row_stride, A.k, keep_max, sCnt,
                                    sThf, sHist[wave], sStage[wave]);
                __syncthreads();
            }
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

// Launches the select kernel of one register-tile shape for either candidate capacity.
// Each shape is instantiated in a source file of its own (si_select_kt*.hip), so the
// kernels compile in parallel.
template <int NWAVE, int KB, int NSUB, bool FP8>
hipError_t launch_select_shape(const SelectArgs& a, int cg, hipStream_t stream) {
    if (cg == 2048) return launch_one<NWAVE, KB, NSUB, 2048, FP8>(a, stream);
    if (cg == 4096) return launch_one<NWAVE, KB, NSUB, 4096, FP8>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace si
