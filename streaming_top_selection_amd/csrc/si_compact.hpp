// Candidate-buffer compaction of the select stage: one wave reduces one query's buffer
// (keys held in registers, E per lane) to its best keys, in place.
//
// Selection of the threshold: pass 1 builds a 256-bin histogram of the keys' score
// images (the upper 32 bits of a key, monotonic in the score), linear between the
// smallest and the largest; the bin holding the rank-th key is found with a wave scan.
// If keeping that whole bin stays within keep_max the bins decide the kept set.
// Otherwise, a bin of at most 64 keys is ranked directly (one key per lane), and a
// larger one (only with heavy score ties) by radix passes over the full 64-bit keys.
// The bins are monotonic and equal scores share a bin, so keys in lower bins are
// below every kept key.
#pragma once

#include <type_traits>

#include "si_common.hpp"

namespace si {

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp<kDppQuadSwap1>(0u, v));
    v = min(v, dpp<kDppQuadSwap2>(0u, v));
    v = min(v, dpp<kDppRowHalfMirror>(0u, v));
    v = min(v, dpp<kDppRowMirror>(0u, v));
    return min(min(readlane(v, 0), readlane(v, 16)), min(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp<kDppQuadSwap1>(0u, v));
    v = max(v, dpp<kDppQuadSwap2>(0u, v));
    v = max(v, dpp<kDppRowHalfMirror>(0u, v));
    v = max(v, dpp<kDppRowMirror>(0u, v));
    return max(max(readlane(v, 0), readlane(v, 16)), max(readlane(v, 32), readlane(v, 48)));
}

// After a 256-bin histogram (filled, and synced with wave_sync): the bin holding the
// rank-th largest entry; *above = entries in higher bins, *cnt = entries in that bin.
// With fewer than rank entries: -1, *above = all entries, *cnt = 0.
__device__ __forceinline__ int hist_find(const uint32_t* hist, int rank, uint32_t* above,
                                         uint32_t* cnt) {
    const int lane = lane_id();
    const u32x4 h = *reinterpret_cast<const u32x4*>(&hist[4 * lane]);
    const uint32_t local = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_incl_scan(local);
    uint32_t cum = readlane(incl, 63) - incl;       // entries in the lanes above
    int found = -1;
    uint32_t a = 0, c = 0;
    const uint32_t hb[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (found < 0 && cum < (uint32_t)rank && cum + hb[b] >= (uint32_t)rank) {
            found = 4 * lane + b;
            a = cum;
            c = hb[b];
        }
        cum += hb[b];
    }
    const uint64_t bal = __ballot(found >= 0);
    if (bal == 0ull) {                              // fewer than rank entries
        *above = readlane(incl, 63);
        *cnt = 0u;
        return -1;
    }
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)bal) - 1);
    *above = readlane(a, src);
    *cnt = readlane(c, src);
    return (int)readlane((uint32_t)found, src);
}

// Score bin of a key: floor(256 * (o - omin) / (span + 1)) for its score image o,
// computed as a multiply-high by mul = floor(2^40 / (span + 1)) (mul = 0: one bin).
// Monotonic in the key; recomputed where needed rather than held in registers.
__device__ __forceinline__ uint32_t score_bin(uint64_t key, uint32_t omin, uint32_t mul) {
    const uint32_t b = __umulhi((uint32_t)(key >> 32) - omin, mul);
    return b < 255u ? b : 255u;
}

// The rank-th largest (1-based, rank <= n) of the n distinct keys in stage[0, n)
// (64 u64 of LDS owned by the wave, 16-byte aligned, zeros past n), ranked by counting
// the larger ones: 32 broadcast 16-byte reads and no wait per key.
__device__ __forceinline__ uint64_t stage_kth(const uint64_t* stage, int n, int rank) {
    const int lane = lane_id();
    const uint64_t mine = stage[lane];
    int greater = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 2) {
        const u64x2 p = *reinterpret_cast<const u64x2*>(&stage[j]);
        greater += (p.x > mine ? 1 : 0) + (p.y > mine ? 1 : 0);
    }
    const uint64_t hit = __ballot(lane < n && greater == rank - 1);
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
    wave_sync();
    return readlane64(mine, src);
}

// The rank_in_bin-th largest (1-based) of the valid keys in score bin d1, when that
// bin holds at most 64 keys: gathered one per lane through `stage` (64 u64 of LDS
// owned by the wave, 16-byte aligned) and ranked by counting the larger ones.  The
// slots past the bin's keys hold 0, below every key, so every lane compares against
// all 64 slots with no bound: 32 broadcast 16-byte reads and no wait per key.
template <int E>
__device__ __forceinline__ uint64_t select_small_bin(const uint64_t (&v)[E], int cnt,
                                                     uint32_t omin, uint32_t mul, int d1,
                                                     int rank_in_bin, uint64_t* stage) {
    const int lane = lane_id();
    stage[lane] = 0ull;   // LDS operations of one wave complete in order
    int n = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool in = e * 64 + lane < cnt && score_bin(v[e], omin, mul) == (uint32_t)d1;
        const uint64_t m = __ballot(in);
        if (in)
            stage[n + (int)__builtin_amdgcn_mbcnt_hi(
                          (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = v[e];
        n += __popcll(m);
    }
    wave_sync();
    return stage_kth(stage, n, rank_in_bin);
}

// Exact threshold by radix passes over the full keys of the alive set (the valid keys,
// restricted to score bin d1 when use_bins): the smallest key th such that the valid
// keys >= th number between rank and keep_max.  Windows of up to 8 bits start just
// below the highest bit where the alive keys differ.
template <int E>
__device__ uint64_t select_refine(const uint64_t (&v)[E], int cnt, int rank, int keep_max,
                                  uint32_t* hist, uint32_t omin, uint32_t mul, bool use_bins,
                                  int d1) {
    typedef typename std::conditional<(E > 32), uint64_t, uint32_t>::type Mask;
    const int lane = lane_id();
    Mask alive = 0;
    int above1 = 0;
    uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool valid = e * 64 + lane < cnt;
        const uint32_t be = score_bin(v[e], omin, mul);
        if (valid && use_bins && be > (uint32_t)d1) above1 += 1;
        if (valid && (!use_bins || be == (uint32_t)d1)) {
            alive |= Mask(1) << e;
            lo = v[e] < lo ? v[e] : lo;
            hi = v[e] > hi ? v[e] : hi;
        }
    }
    const int above_all = wave_sum(above1);
    rank -= above_all;
    keep_max -= above_all;
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    const uint64_t diff = lo ^ hi;
    if (diff == 0ull) return lo;
    const int top = 63 - __clzll((long long)diff);
    int shift = top >= 7 ? top - 7 : 0;
    int width = top - shift + 1;
    for (;;) {
        const uint32_t dmask = (1u << width) - 1u;
        *reinterpret_cast<u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
        wave_sync();
#pragma unroll
        for (int e = 0; e < E; ++e)
            atomicAdd(&hist[(uint32_t)(v[e] >> shift) & dmask], (uint32_t)((alive >> e) & 1));
        wave_sync();
        uint32_t above, cntd;
        const int d = hist_find(hist, rank, &above, &cntd);
        wave_sync();
        rank -= (int)above;
        keep_max -= (int)above;
        // the last window (bit 0) always ends here: a bin is then one key value
        if ((int)cntd <= keep_max || shift == 0) {
            uint64_t m = ~0ull;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (((alive >> e) & 1) && (int)((uint32_t)(v[e] >> shift) & dmask) >= d)
                    m = v[e] < m ? v[e] : m;
            return wave_min_u64(m);
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (((alive >> e) & 1) && (int)((uint32_t)(v[e] >> shift) & dmask) != d)
                alive &= ~(Mask(1) << e);
        width = shift >= 8 ? 8 : shift;
        shift -= width;
    }
}

// Loads a buffer's E*64 slots into registers (slot e*64 + lane).  Every slot is read,
// with no branch, so that the loads of one buffer can be in flight, with a known
// count, while another buffer's keys are selected; slots past cnt are masked by the
// caller.
template <int E>
__device__ __forceinline__ void load_keys(const uint64_t* buf, uint64_t (&v)[E]) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = buf[e * 64 + lane];
}

// The rule that keeps between k and keep_max of the largest of the cnt keys v (slots
// past cnt hold 0; 1 <= k < cnt): on return *by_bin says whether the kept keys are
// those with score_bin(key, *omin, *mul) >= *d, and otherwise they are those >= the
// returned key.
template <int E>
__device__ __forceinline__ uint64_t find_keep_rule(const uint64_t (&v)[E], int cnt, int k,
                                                   int keep_max, uint32_t* hist,
                                                   uint64_t* stage, uint32_t* omin_out,
                                                   uint32_t* mul_out, int* d_out,
                                                   bool* by_bin_out) {
    const int lane = lane_id();
    uint32_t omin = ~0u, omax = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e * 64 + lane < cnt) {
            const uint32_t o = (uint32_t)(v[e] >> 32);
            omin = o < omin ? o : omin;
            omax = o > omax ? o : omax;
        }
    }
    omin = wave_min_u32(omin);
    omax = wave_max_u32(omax);
    int d = 0;
    bool by_bin = false, exact = false;
    uint64_t th64 = 0;
    uint32_t mul = 0u;
    if (omax > omin) {
        // pass 1: the histogram of the score bins
        mul = (uint32_t)((uint64_t(256) << 32) / (uint64_t(omax - omin) + 1));
        *reinterpret_cast<u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
        wave_sync();
#pragma unroll
        for (int e = 0; e < E; ++e)   // every lane adds (0 past cnt): no branch, no wait
            atomicAdd(&hist[score_bin(v[e], omin, mul)], e * 64 + lane < cnt ? 1u : 0u);
        wave_sync();
        uint32_t above, cntd;
        d = hist_find(hist, k, &above, &cntd);
        wave_sync();
        if ((int)(above + cntd) <= keep_max) {
            by_bin = true;
        } else if (cntd <= 64u) {
            th64 = select_small_bin<E>(v, cnt, omin, mul, d, k - (int)above, stage);
            exact = true;
        }
    }
    if (!by_bin && !exact)
        th64 = select_refine<E>(v, cnt, k, keep_max, hist, omin, mul, omax > omin, d);
    *omin_out = omin;
    *mul_out = mul;
    *d_out = d;
    *by_bin_out = by_bin;
    return th64;
}

// Keeps between k and keep_max of the largest of the cnt keys v (exactly k when
// keep_max == k; 1 <= k < cnt), written back to buf[0, kept) as contiguous runs; the
// dropped keys go to the kCandPad slots after the list (buf[E*64, E*64 + 64)), so every
// store is issued with no branch.  Slots of v past cnt are ignored.  Returns the kept count; *th_ord
// receives the smallest kept key's score image.
template <int E>
__device__ __forceinline__ int compact_regs(uint64_t* buf, uint64_t (&v)[E], int cnt,
                                            int k, int keep_max, uint32_t* hist,
                                            uint64_t* stage, uint32_t* th_ord) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = e * 64 + lane < cnt ? v[e] : 0ull;
    uint32_t omin, mul;
    int d;
    bool by_bin;
    const uint64_t th64 =
        find_keep_rule<E>(v, cnt, k, keep_max, hist, stage, &omin, &mul, &d, &by_bin);
    int base = 0;
    uint32_t tmin = ~0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool keep = e * 64 + lane < cnt &&
                          (by_bin ? score_bin(v[e], omin, mul) >= (uint32_t)d : v[e] >= th64);
        const uint64_t m = __ballot(keep);
        const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                  (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        buf[keep ? at : E * 64 + lane] = v[e];
        const uint32_t o = (uint32_t)(v[e] >> 32);
        tmin = keep && o < tmin ? o : tmin;
        base += __popcll(m);
    }
    *th_ord = wave_min_u32(tmin);
    return base;
}

}  // namespace si
