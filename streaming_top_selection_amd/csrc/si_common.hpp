// Device helpers shared by the gfx950 kernels of the indexer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace si {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;          // head dim (the only one built)
constexpr int kTQ = 32;          // query rows per workgroup tile = MFMA N
constexpr int kMB = 32;          // keys per MFMA block = MFMA M
constexpr int kMaxH = 128;       // most indexer heads supported
constexpr int kMaxK = 2048;      // largest top-k supported
constexpr int kWave = 64;

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
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

// -0 -> +0, everything else unchanged.
__device__ __forceinline__ float canon_zero(float x) {
    return (__float_as_uint(x) == 0x80000000u) ? 0.0f : x;
}

// ---------------------------------------------------------------------------
// OCP FP8 E4M3 byte -> bf16 bits.  Exact: every finite E4M3 value (3 mantissa
// bits, exponents 2^-9 .. 2^8) is representable in bf16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t x) {
    const uint32_t sign = (x & 0x80u) << 8;
    const uint32_t e = (x >> 3) & 0xFu;
    const uint32_t m = x & 0x7u;
    uint32_t mag;
    if (e != 0u) {
        mag = ((e + 120u) << 7) | (m << 4);          // bias 7 -> bias 127
    } else if (m == 0u) {
        mag = 0u;
    } else {                                          // subnormal m * 2^-9
        const uint32_t p = 31u - __builtin_clz(m);    // 0..2
        mag = ((p + 118u) << 7) | ((m << (7u - p)) & 0x7Fu);
    }
    return sign | mag;
}

// four E4M3 bytes (little-endian in a u32) -> four bf16 in two u32
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    u32x2 r;
    r.x = e4m3_to_bf16_bits(w & 0xFFu) | (e4m3_to_bf16_bits((w >> 8) & 0xFFu) << 16);
    r.y = e4m3_to_bf16_bits((w >> 16) & 0xFFu) | (e4m3_to_bf16_bits(w >> 24) << 16);
    return r;
}

// ---------------------------------------------------------------------------
// Wavefront primitives (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Orders this wave's LDS accesses before/after the call (LDS operations of one
// wave are performed in issue order; this stops the compiler moving them).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    uint32_t lo = __shfl((unsigned)(v & 0xFFFFFFFFu), src);
    uint32_t hi = __shfl((unsigned)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFu), off);
        uint32_t hi = __shfl_xor((unsigned)(v >> 32), off);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// exclusive prefix sum over lanes
__device__ __forceinline__ int wave_excl_scan(int v) {
    const int lane = lane_id();
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x - v;
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
// Radix select of the rank-th largest (1-based) non-zero 64-bit key held by a
// wave, MSB first over 8-bit digits.  `hist` is 256 u32 of LDS owned by this
// wave.  Keys are unique, so the result is the exact rank-th key.  The result
// is wave-uniform.  Requires 1 <= rank <= number of non-zero keys.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFu), off);
        uint32_t hi = __shfl_xor((unsigned)(v >> 32), off);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

template <class Src>
__device__ uint64_t wave_select_kth(const Src& src, int rank, uint32_t* hist) {
    const int lane = lane_id();
    // Leading bytes shared by every key (those where the smallest and the largest key
    // agree) hold no information: start below them.  Candidates above a threshold
    // usually share their top score bytes, which would otherwise send every key to one
    // histogram bin.
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
    if (diff == 0ull) return lo;              // a single distinct key
    const int top = 63 - __clzll((long long)diff);   // highest differing bit
    int shift = (top / 8) * 8;
    uint64_t pmask = shift == 56 ? 0ull : (~0ull << (shift + 8));
    uint64_t prefix = lo & pmask;
    for (; shift >= 0; shift -= 8) {
        for (int i = lane; i < 256; i += 64) hist[i] = 0u;
        wave_sync();
        src.for_each([&](uint64_t v) {
            if (v != 0ull && (v & pmask) == prefix)
                atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
        });
        wave_sync();
        const u32x4 h = *reinterpret_cast<const u32x4*>(&hist[4 * lane]);
        const uint32_t local = h.x + h.y + h.z + h.w;
        uint32_t suf = local;
        for (int off = 1; off < 64; off <<= 1) {
            uint32_t t = __shfl_down(suf, off);
            if (lane + off < 64) suf += t;
        }
        uint32_t cum = suf - local;       // keys in higher bins (lanes above)
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
        const int srcl = __ffsll((long long)bal) - 1;
        const int d = __shfl(found, srcl);
        above_d = __shfl(above_d, srcl);
        cnt_d = __shfl(cnt_d, srcl);
        rank -= (int)above_d;
        prefix |= (uint64_t)d << shift;
        pmask |= 0xFFull << shift;
        wave_sync();
        if (cnt_d == 1u) {                // the rank-th key is the only one left
            uint64_t best = 0;
            src.for_each([&](uint64_t v) {
                if (v != 0ull && (v & pmask) == prefix) best = v;
            });
            return wave_max_u64(best);
        }
    }
    return prefix;
}

}  // namespace si
