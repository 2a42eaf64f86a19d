// Device helpers shared by the gfx950 kernels of the indexer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace si {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;          // head dim (the only one built)
constexpr int kTQ = 32;          // query rows per workgroup tile = MFMA N
constexpr int kMB = 32;          // keys per MFMA block = MFMA M
constexpr int kMaxH = 128;       // most indexer heads supported
constexpr int kMaxK = 2048;      // largest top-k supported
constexpr int kWave = 64;
// Slots after each candidate list that absorb the stores of lanes with nothing to
// write, so that appends and compactions store with no branch (never read).
constexpr int kCandPad = 64;

// ---------------------------------------------------------------------------
// MFMA: D[32x32] = A[32x16] * B[16x32] + C, bf16 inputs, fp32 accumulation.
// Lane l supplies row (l & 31) of A and column (l & 31) of B, both at the
// same eight k positions; it receives column (l & 31) of D at the rows
// mfma_row(r, l) for r = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int mfma_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// ---------------------------------------------------------------------------
// Order-preserving 32-bit image of an fp32 value (a > b  <=>  ord(a) > ord(b)
// for non-NaN values, with -0 and +0 mapped apart, so callers canonicalise -0).
// A selection key packs (ord(score), ~index): larger key = better entry, and
// among equal scores the lower index has the larger key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_f32(float x) {
    // negative: all bits flipped; otherwise the sign bit set
    const uint32_t u = __float_as_uint(x);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float score, uint32_t idx) {
    return ((uint64_t)ord_f32(score) << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ int32_t key_index(uint64_t key) {
    return (int32_t)(~(uint32_t)key);
}

__device__ __forceinline__ float key_score(uint64_t key) {
    return unord_f32((uint32_t)(key >> 32));
}

// -0 -> +0, everything else unchanged (IEEE: -0 + +0 = +0, x + 0 = x for x != 0).
__device__ __forceinline__ float canon_zero(float x) { return x + 0.0f; }

// ---------------------------------------------------------------------------
// OCP FP8 E4M3 -> bf16.  Exact: every finite E4M3 value (3 mantissa bits, exponents
// 2^-9 .. 2^8) is representable in bf16.  gfx950 converts two bytes per instruction
// (v_cvt_scalef32_pk_bf16_fp8, scale 1.0); an exhaustive check of all 256 codes in
// each byte position against a field-by-field decode (sign, exponent rebias 7 -> 127,
// subnormals normalised) matched for every finite code.  NaN codes are outside the
// ABI contract.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// four E4M3 bytes (little-endian in a u32) -> four bf16 in two u32 (byte 0 in the low
// half of .x)
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    return r;
}

// ---------------------------------------------------------------------------
// Wavefront primitives (64 lanes).  Reductions and scans move data between lanes
// with DPP (a VALU operand modifier, no LDS round trip): butterflies within each
// row of 16 lanes, then the four row results are combined with readlane or, for
// scans, with the gfx9 row broadcasts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// the workgroup's wave index as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Orders this wave's LDS accesses before/after the call (LDS operations of one
// wave are performed in issue order; this stops the compiler moving them).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that waits for this wave's LDS operations only (global stores
// may still be in flight): for publishing LDS counters between waves.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt unchanged
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// DPP controls (gfx9 encoding)
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowShr = 0x110;        // + n: row_shr:n
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// v from another lane by DPP; lanes the control does not write (row mask, or a
// source outside the row) receive `old`
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    return ((uint64_t)readlane((uint32_t)(v >> 32), l) << 32) | readlane((uint32_t)v, l);
}

// butterfly step within rows of 16 lanes for a 64-bit value
template <int CTRL, class Op>
__device__ __forceinline__ uint64_t dpp_step64(uint64_t v, Op op) {
    const uint32_t lo = dpp<CTRL>(0u, (uint32_t)v), hi = dpp<CTRL>(0u, (uint32_t)(v >> 32));
    return op(v, ((uint64_t)hi << 32) | lo);
}

template <class Op>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v, Op op) {
    v = dpp_step64<kDppQuadSwap1>(v, op);
    v = dpp_step64<kDppQuadSwap2>(v, op);
    v = dpp_step64<kDppRowHalfMirror>(v, op);
    v = dpp_step64<kDppRowMirror>(v, op);      // every lane holds its row's result
    const uint64_t r0 = readlane64(v, 0), r1 = readlane64(v, 16);
    const uint64_t r2 = readlane64(v, 32), r3 = readlane64(v, 48);
    return op(op(r0, r1), op(r2, r3));
}

// wave-uniform max / min of a 64-bit value over the 64 lanes
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
    return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
}

// inclusive prefix sum over lanes 0..lane
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    uint32_t x = v;
    x += dpp<kDppRowShr + 1>(0u, x);
    x += dpp<kDppRowShr + 2>(0u, x);
    x += dpp<kDppRowShr + 4>(0u, x);
    x += dpp<kDppRowShr + 8>(0u, x);           // scans within rows of 16
    x += dpp<kDppRowBcast15, 0xA>(0u, x);      // rows 1, 3 add the row before
    x += dpp<kDppRowBcast31, 0xC>(0u, x);      // rows 2, 3 add rows 0..1
    return x;
}

// exclusive prefix sum over lanes
__device__ __forceinline__ int wave_excl_scan(int v) {
    return (int)wave_incl_scan((uint32_t)v) - v;
}

// wave-uniform sum over the 64 lanes
__device__ __forceinline__ int wave_sum(int v) {
    return (int)readlane(wave_incl_scan((uint32_t)v), 63);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Causal visibility: number of compressed keys visible to absolute position t.
__device__ __forceinline__ int64_t visible_keys(int64_t t_abs, int32_t m, int64_t T) {
    int64_t n = (t_abs + 1) / m;
    return n < T ? n : T;
}

// ---------------------------------------------------------------------------
// Value sources for the wave radix select: each visits the keys one lane holds.
// ---------------------------------------------------------------------------
template <int E>
struct RegKeys {                      // E keys per lane in registers (0 = empty)
    uint64_t v[E];
    template <class F>
    __device__ __forceinline__ void for_each(F f) const {
#pragma unroll
        for (int e = 0; e < E; ++e) f(v[e]);
    }
};

struct LdsKeys {                      // keys buf[0..n) in LDS, strided over lanes
    const uint64_t* buf;
    int n;
    template <class F>
    __device__ __forceinline__ void for_each(F f) const {
        for (int i = lane_id(); i < n; i += 64) f(buf[i]);
    }
};

// ---------------------------------------------------------------------------
// Radix threshold select over the non-zero 64-bit keys held by a wave (unique keys).
// Returns a wave-uniform threshold th > 0 with
//     rank <= #{keys >= th} <= keep_max        (1 <= rank <= keep_max, rank <= #keys)
// keep_max == rank asks for exactly `rank` keys at or above th.  Digits are windows of
// up to 8 bits, the first one just below the highest bit where the keys differ (the
// bits above it are common to all keys and carry no information); each pass narrows
// the window to the bin holding the rank-th key and stops as soon as keeping that
// whole bin stays within keep_max.  `hist` is 256 u32 of LDS owned by this wave.
// ---------------------------------------------------------------------------
template <class Src>
__device__ uint64_t wave_select_threshold(const Src& src, int rank, int keep_max,
                                          uint32_t* hist) {
    const int lane = lane_id();
    uint64_t lo = ~0ull, hi = 0ull;
    src.for_each([&](uint64_t v) {
        if (v != 0ull) {
            lo = v < lo ? v : lo;
            hi = v > hi ? v : hi;
        }
    });
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    const uint64_t diff = lo ^ hi;
    if (diff == 0ull) return lo;                      // a single key
    const int top = 63 - __clzll((long long)diff);    // highest differing bit
    int shift = top >= 7 ? top - 7 : 0;               // window [shift, top]
    int width = top - shift + 1;
    uint64_t pmask = top == 63 ? 0ull : (~0ull << (top + 1));
    uint64_t prefix = lo & pmask;
    for (;;) {
        *reinterpret_cast<u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
        wave_sync();
        const uint32_t dmask = (1u << width) - 1u;
        src.for_each([&](uint64_t v) {
            if (v != 0ull && (v & pmask) == prefix)
                atomicAdd(&hist[(uint32_t)(v >> shift) & dmask], 1u);
        });
        wave_sync();
        // lane l holds bins 4l..4l+3; keys in bins above lane l's: total - inclusive
        const u32x4 h = *reinterpret_cast<const u32x4*>(&hist[4 * lane]);
        const uint32_t local = h.x + h.y + h.z + h.w;
        const uint32_t incl = wave_incl_scan(local);
        uint32_t cum = readlane(incl, 63) - incl;
        int found = -1;
        uint32_t above_d = 0, cnt_d = 0;
        const uint32_t hb[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int b = 3; b >= 0; --b) {
            if (found < 0 && cum < (uint32_t)rank && cum + hb[b] >= (uint32_t)rank) {
                found = 4 * lane + b;
                above_d = cum;
                cnt_d = hb[b];
            }
            cum += hb[b];
        }
        const uint64_t bal = __ballot(found >= 0);
        const int srcl = __builtin_amdgcn_readfirstlane(__ffsll((long long)bal) - 1);
        const int d = (int)readlane((uint32_t)found, srcl);
        above_d = readlane(above_d, srcl);
        cnt_d = readlane(cnt_d, srcl);
        wave_sync();
        rank -= (int)above_d;
        keep_max -= (int)above_d;
        prefix |= (uint64_t)d << shift;
        pmask |= (uint64_t)dmask << shift;
        // keeping the whole bin stays within keep_max: done.  This always happens by
        // the last window (bit 0), where a bin is a single key value: rank <= cnt_d
        // <= 1 <= keep_max.
        if ((int)cnt_d <= keep_max || shift == 0) return prefix;
        width = shift >= 8 ? 8 : shift;
        shift -= width;
    }
}

// The rank-th largest key's threshold: exactly `rank` keys are >= the result.
template <class Src>
__device__ __forceinline__ uint64_t wave_select_kth(const Src& src, int rank, uint32_t* hist) {
    return wave_select_threshold(src, rank, rank, hist);
}

}  // namespace si
