// The score tile: one workgroup scores kTQ = 32 query rows against NWAVE * KB * 32
// compressed keys, all heads, on bf16 MFMA.  Both the streaming kernel and the
// materialise reference kernel call this routine, so their scores agree bit for bit.
//
// Arithmetic per (query t, key s), fixed for every caller and tuning knob:
//   z_h   = MFMA-32x32x16 chain over d (steps 0..7, see below), fp32 accumulate
//   acc   = fmaf(w[t,h], max(z_h, 0), acc)        for h = 0 .. H-1, acc0 = +0
//   score = acc (bf16 keys) or acc * kc_scale[s] (E4M3 keys); -0 -> +0
// (indexer score: per-head dot, ReLU, head-weighted sum; the pages give no formula.)
//
// Data flow (MI355X layout, not the pages' Triton design):
//  * K-stationary: each wave loads its keys once into MFMA A-operand registers and
//    keeps them for all heads (a key tile is the same for every head).
//  * q is streamed head by head through a double-buffered LDS tile of 32 rows x 128
//    bf16 (8 KiB/head) that all waves of the workgroup share as the B operand.
//  * Output layout: lane l owns query column (l & 31) and key rows mfma_row(r, l),
//    so the head weight w[t,h] is one LDS read per lane per head.
#pragma once

#include "si_common.hpp"

namespace si {

struct Problem {
    const uint16_t* q;        // [B, S, H, D] bf16 bits
    const void* kc;           // [B, T, D] bf16 bits or E4M3 bytes
    const float* kc_scale;    // [B, T] (E4M3 keys) or nullptr
    const float* w;           // [B, S, H]
    int64_t B, S, T;
    int32_t H, m;
    int64_t q_pos0;
};

constexpr int kQRow = kD + 8;     // staged q row in bf16 (272 bytes: bank-skewed rows)
constexpr int kWStride = kMaxH + 1;  // w row stride in floats (odd: conflict-free column reads)

struct ScoreLds {
    uint16_t q[2][kTQ * kQRow];   // double-buffered q tile of one head
    float w[kTQ * kWStride];      // head weights of the 32 query rows
};

// Fills L.w for query rows [row0, row0 + rows_valid) of batch entry b (0 past the end).
template <int NT>
__device__ __forceinline__ void load_w_tile(const Problem& P, int64_t b, int64_t row0,
                                            int rows_valid, ScoreLds& L) {
    const int H = P.H;
    for (int f = threadIdx.x; f < kTQ * H; f += NT) {
        const int j = f / H, h = f - j * H;
        L.w[j * kWStride + h] =
            j < rows_valid ? P.w[((b * P.S + row0 + j) * H) + h] : 0.0f;
    }
}

// Scores rows [row0, row0 + rows_valid) against keys key0 + [0, NWAVE*KB*32).
// Requires: L.w filled and a __syncthreads() since; key0 % 32 == 0; every thread of
// the workgroup calls it.  acc[kb][r] receives the score of query (lane & 31) and key
// key0 + (wave*KB + kb)*32 + mfma_row(r, lane).  Keys >= T score as if zero.
template <int NWAVE, int KB, bool FP8>
__device__ __forceinline__ void score_regs(const Problem& P, int64_t b, int64_t row0,
                                           int rows_valid, int64_t key0, ScoreLds& L,
                                           f32x16 (&acc)[KB]) {
    constexpr int NT = NWAVE * kWave;
    constexpr int QCHUNKS = kTQ * (kD * 2 / 16);   // 16-byte pieces of one head tile
    constexpr int QPER = QCHUNKS / NT;
    static_assert(QCHUNKS % NT == 0, "q tile must split evenly over the workgroup");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hh = lane >> 5;       // which 64-wide half of d this lane feeds
    const int il = lane & 31;       // A row (key) and B column (query) of this lane
    const int H = P.H;

    // ---- K fragments: keys stay in registers for the whole head loop ----------
    // step s covers d = 64*hh + 8*s + [0, 8) for lane l (same d for A and B).
    bf16x8 kf[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + il;
        if (key < P.T) {
            if constexpr (!FP8) {
                const u32x4* src = reinterpret_cast<const u32x4*>(
                    static_cast<const uint16_t*>(P.kc) + ((b * P.T + key) * kD + 64 * hh));
#pragma unroll
                for (int s = 0; s < 8; ++s) kf[kb][s] = __builtin_bit_cast(bf16x8, src[s]);
            } else {
                const u32x4* src = reinterpret_cast<const u32x4*>(
                    static_cast<const uint8_t*>(P.kc) + ((b * P.T + key) * kD + 64 * hh));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 x = src[c];
                    const u32x2 a0 = e4m3x4_to_bf16x4(x.x), a1 = e4m3x4_to_bf16x4(x.y);
                    const u32x2 a2 = e4m3x4_to_bf16x4(x.z), a3 = e4m3x4_to_bf16x4(x.w);
                    const u32x4 lo = {a0.x, a0.y, a1.x, a1.y};
                    const u32x4 hi = {a2.x, a2.y, a3.x, a3.y};
                    kf[kb][2 * c] = __builtin_bit_cast(bf16x8, lo);
                    kf[kb][2 * c + 1] = __builtin_bit_cast(bf16x8, hi);
                }
            }
        } else {
            const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int s = 0; s < 8; ++s) kf[kb][s] = __builtin_bit_cast(bf16x8, zero);
        }
    }

    // ---- q staging: 16-byte pieces, row j = f / 16, piece c = f % 16 -----------
    u32x4 qreg[QPER];
    auto qload = [&](int h) {
#pragma unroll
        for (int n = 0; n < QPER; ++n) {
            const int f = tid + n * NT;
            const int j = f >> 4, c = f & 15;
            if (j < rows_valid) {
                qreg[n] = *reinterpret_cast<const u32x4*>(
                    P.q + (((b * P.S + row0 + j) * H + h) * kD + c * 8));
            } else {
                qreg[n] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto qstore = [&](int buf) {
#pragma unroll
        for (int n = 0; n < QPER; ++n) {
            const int f = tid + n * NT;
            const int j = f >> 4, c = f & 15;
            *reinterpret_cast<u32x4*>(&L.q[buf][j * kQRow + c * 8]) = qreg[n];
        }
    };

#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][r] = 0.0f;

    qload(0);
    qstore(0);
    __syncthreads();

    for (int h = 0; h < H; ++h) {
        const int buf = h & 1;
        if (h + 1 < H) qload(h + 1);

        bf16x8 bq[8];
        const uint16_t* qrow = &L.q[buf][il * kQRow + 64 * hh];
#pragma unroll
        for (int s = 0; s < 8; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(qrow + 8 * s);

        f32x16 z[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) z[kb][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < 8; ++s) z[kb] = mfma32x32x16(kf[kb][s], bq[s], z[kb]);
        }

        const float wh = L.w[il * kWStride + h];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[kb][r] = __builtin_fmaf(wh, __builtin_fmaxf(z[kb][r], 0.0f), acc[kb][r]);

        if (h + 1 < H) qstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = acc[kb][r];
            if constexpr (FP8) {
                const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + mfma_row(r, lane);
                v = v * (key < P.T ? P.kc_scale[b * P.T + key] : 1.0f);
            }
            acc[kb][r] = canon_zero(v);
        }
    }
}

}  // namespace si
