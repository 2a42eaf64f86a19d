// The score tile with E4M3 q on the gfx950 f8f6f4 MFMA.  Same contract, output layout
// and epilogue as score_regs_bf16 (si_score.hpp); only the operands and the MFMA differ.
//
// q arrives quantised per (query row, head) to E4M3 with the scale folded into the
// head weight (w_eff = w * q_scale, a positive factor that commutes with the ReLU), so
// the tile needs only the bytes.  Lower indexer precision is the lever the pages name
// besides memory layout (jeff.news "딥시크 V4 인덱서…", 기술 맥락); the MXFP4 key
// format is the indexer key cache dtype of the deployment on the chengshu page
// ("两级稀疏注意力…", 部署视角).
//
// Arithmetic per (query t, key s), fixed for every caller and tuning knob:
//   z_h   = two MFMA-32x32x64 steps over d (d 0..63, then 64..127), fp32 accumulate;
//           the products of E4M3 x E4M3 (and E4M3 x E2M1 x 2^e) values are exact
//   acc   = fmaf(w_eff[t,h], max(z_h, 0), acc)    for h = 0 .. H-1, acc0 = +0
//   score = acc * kc_scale[s] (E4M3 keys) or acc (MXFP4 keys, whose E8M0 block
//           scales enter the MFMA as its B scale); -0 -> +0
//
// Layout:
//  * Keys (B operand) stay in registers for the whole head loop: 32 bytes per lane and
//    step for E4M3 keys, 16 bytes (32 nibbles) for MXFP4 keys plus one E8M0 byte per
//    step (block 2*step + half).
//  * q tiles are 32 rows x 128 bytes (4 KiB per head), staged by buffer->LDS loads
//    six heads ahead exactly as in the bf16 tile.  Piece c (bytes 16c .. 16c+15) of row
//    r sits at piece 8r + (c ^ (r & 7) ^ ((r >> 3) & 1)) of the tile, so the 16-byte
//    A-operand reads of 8 (or 16) consecutive rows fall in distinct bank groups.
//  * Each step covers d = 64 s + [0, 64).  The E4M3 operands of both sides take the
//    same d positions in the same lane bytes (d = 64 s + 32 hh + j in byte j of half
//    hh), so the MFMA's sum is the dot product whatever its K order; with MXFP4 keys
//    the q bytes follow the E4M3/E2M1 pairing of the scaled MFMA (see roff below).
#pragma once

#include "si_score.hpp"

namespace si {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kQ8Chunks = kTQ * 8;    // 16-byte pieces per staged E4M3 q tile

__device__ __forceinline__ int q8_piece(int r, int c) {
    return 8 * r + (c ^ (r & 7) ^ ((r >> 3) & 1));
}

// D[32x32] += A[32x64] * B[64x32], E4M3 x E4M3 (no scales: the plain instruction)
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D[32x32] += A[32x64] * (B[64x32] * 2^(e_B - 127)), A E4M3 with scale 2^0 (E8M0 127),
// B E2M1 (format 4, the low four dwords) with the E8M0 byte OPSEL of sb as the lane's
// block scale
template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_f8f4(i32x8 a, i32x8 b, f32x16 c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, 127, OPSEL, sb);
}

template <int NWAVE, int KB, bool K4>
__device__ __forceinline__ void score_regs_q8(const Problem& P, int64_t b, int64_t row0,
                                              int rows_valid, int64_t key0, int64_t key_end,
                                              ScoreLds& L, const QBufs& Q, f32x16 (&acc)[KB]) {
    constexpr int NT = NWAVE * kWave;
    // per-lane offsets recomputed at each call (see score_regs_bf16)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = wave_id();
    const int hh = lane >> 5;
    const int il = lane & 31;
    const int H = P.H;

    // ---- K fragments (B operand), register-resident for the whole head loop ----
    i32x8 kf[KB][2];
    int ksc[KB];                       // MXFP4: byte 0 = block hh (step 0), byte 2 = block 2 + hh
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + il;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        if (key < key_end) {
            if constexpr (!K4) {
                const u32x4* src = reinterpret_cast<const u32x4*>(
                    static_cast<const uint8_t*>(P.kc) + (b * P.T + key) * kD + 32 * hh);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u32x4 lo = src[4 * s], hi = src[4 * s + 1];
                    kf[kb][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
                ksc[kb] = 0;
            } else {
                const u32x4* src = reinterpret_cast<const u32x4*>(
                    static_cast<const uint8_t*>(P.kc) + (b * P.T + key) * (kD / 2) + 16 * hh);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u32x4 x = src[2 * s];
                    kf[kb][s] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
                }
                const uint32_t sc = *reinterpret_cast<const uint32_t*>(
                    static_cast<const uint8_t*>(P.kc_scale) + (b * P.T + key) * (kD / 32));
                ksc[kb] = (int)(sc >> (8 * hh));
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                kf[kb][s] = i32x8{(int)zero.x, 0, 0, 0, 0, 0, 0, 0};
            ksc[kb] = 0x7F7F7F7F;      // 2^0: the masked keys' zeros stay zeros
        }
    }

    // ---- q staging: buffer -> LDS loads, kQBuf - 2 heads ahead (as in the bf16 tile) ----
    constexpr int QN = kQ8Chunks / NT;
    static_assert(kQ8Chunks % NT == 0, "every wave issues the same number of q loads");
    constexpr int AHEAD = kQBuf - 2;
    const uint64_t qbase = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(P.q) +
                                                      (b * P.S + row0) * H * (int64_t)kD);
    const uint32_t qbytes = (uint32_t)(rows_valid * H * kD);
    int voff[QN];
#pragma unroll
    for (int n = 0; n < QN; ++n) {
        const int piece = n * NT + tid;          // position in the LDS tile
        const int r = piece >> 3;
        const int c = (piece & 7) ^ (r & 7) ^ ((r >> 3) & 1);   // source piece of row r
        voff[n] = min(r, rows_valid - 1) * H * kD + c * 16;
    }
    auto qload = [&](uint16_t* buf, int h) {
        const uint32_t hc = (uint32_t)(h < H ? h : H - 1);
        const i32x4 rsrc = make_rsrc(qbase + hc * kD, qbytes - hc * kD);
#pragma unroll
        for (int n = 0; n < QN; ++n)
            si_raw_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(buf + (n * NT + wave * 64) * 8),
                16, voff[n], 0, 0, 0);
    };
    // A operand of one head, row il, step s.  E4M3 x E4M3: bytes 64 s + 32 hh + [0, 32),
    // i.e. pieces 4 s + 2 hh and 4 s + 2 hh + 1, the same d positions as the key bytes.
    // E4M3 x E2M1: the MFMA pairs byte j of an E4M3 lane half hh with K index
    // 32 (j / 16) + 16 hh + (j % 16), and nibble j of an E2M1 lane half with K index
    // 32 half + j (each E2M1 half holds one 32-element scale block); the key nibbles
    // hold d = 64 s + 32 half + j, so q's bytes 0..15 are d = 64 s + 16 hh + [0, 16)
    // (piece 4 s + hh) and bytes 16..31 are d = 64 s + 32 + 16 hh + [0, 16) (piece
    // 4 s + 2 + hh).  (Pairing measured on gfx950 with one-hot operands.)
    int roff[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            roff[s][j] = 16 * q8_piece(il, K4 ? 4 * s + 2 * j + hh : 4 * s + 2 * hh + j);
    auto qread = [&](const uint16_t* buf, i32x8 (&bq)[2], int s) {
        const char* base = reinterpret_cast<const char*>(buf);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + roff[s][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + roff[s][1]);
        bq[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto wread = [&](int h, f32x4 (&wv)[4]) {
        const f32x4* row = reinterpret_cast<const f32x4*>(L.w + h * kTQ + 4 * hh);
#pragma unroll
        for (int g = 0; g < 4; ++g) wv[g] = row[2 * g];
    };
    auto mfma_block = [&](int kb, const i32x8 (&bq)[2], f32x16& z) {
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
        if constexpr (!K4) {
            z = mfma_f8(bq[0], kf[kb][0], z);
            z = mfma_f8(bq[1], kf[kb][1], z);
        } else {
            z = mfma_f8f4<0>(bq[0], kf[kb][0], z, ksc[kb]);
            z = mfma_f8f4<2>(bq[1], kf[kb][1], z, ksc[kb]);
        }
    };
    auto epilogue_block = [&](int kb, const f32x16& z, const f32x4 (&wv)[4]) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[kb][r] = __builtin_fmaf(wv[r >> 2][r & 3], __builtin_fmaxf(z[r], 0.0f),
                                        acc[kb][r]);
    };
    auto pin = [&](f32x16& v) { asm volatile("" : "+v"(v)); };
    // one MFMA block (2 MFMAs) interleaved with one epilogue block (32 VALU), with a
    // share of the step's 8 LDS reads and, in block KLOAD, its q loads
    constexpr int KLOAD = KB > 1 ? 1 : 0;
    auto interleave = [&](int kb, int nread) {
        const int first = (nread + 1) / 2;       // reads placed after the first MFMA
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // sixteen VALU
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < (i == 0 ? first : nread - first))
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (kb == KLOAD && i < QN) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][r] = 0.0f;

    // the skewed pipeline of score_regs_bf16: the MFMAs of block X + LA run beside the
    // epilogue of block X; head h+1's operands are read in step h; one barrier per two
    // heads publishes the next two staged tiles.  A block's chain here is two MFMAs
    // (against eight bf16 ones), short enough that with one block of lookahead the
    // epilogue would read results still in flight and stall on the MFMA result hazard;
    // two blocks of lookahead (three of four accumulator slots live) hide it.  With
    // fewer than four blocks a head's operands, read one block ahead, would not be in
    // registers in time for a chain two blocks ahead, so those shapes keep one.
    constexpr int LA = (KB >= 4) ? 2 : 1;
    constexpr int ZR = (LA == 2) ? 4 : ((KB % 3 == 0) ? 3 : 2);
    static_assert((kQBuf * KB) % ZR == 0, "slots must repeat every group of 8 heads");
    static_assert(LA <= KB, "lookahead stays within the next head");
    f32x16 z[ZR];
    i32x8 bq[2][2];
    f32x4 wv[2][4];
    auto step = [&](auto rstep, int h) {
        constexpr int R = decltype(rstep)::value;
        constexpr int RB = (R + 1) % kQBuf, LB = (R + kQBuf - 1) % kQBuf;
        constexpr int C = R % 2, N = 1 - C;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int x = R * KB + kb;
            const int ykb = (kb + LA) % KB;
            const bool next_head = kb + LA >= KB;
            int nread = 0;
            if (KB >= 3) {
                if (kb == 0) qread(Q.p[RB], bq[N], 0), nread = 2;
                if (kb == 1) qread(Q.p[RB], bq[N], 1), nread = 2;
                if (kb == 2) wread(h + 1, wv[N]), nread = 4;
            } else if (KB == 2) {
                if (kb == 0) qread(Q.p[RB], bq[N], 0), qread(Q.p[RB], bq[N], 1), nread = 4;
                if (kb == 1) wread(h + 1, wv[N]), nread = 4;
            } else {
                qread(Q.p[RB], bq[N], 0);
                qread(Q.p[RB], bq[N], 1);
                wread(h + 1, wv[N]);
                nread = 8;
            }
            if (kb == KLOAD) qload(Q.p[LB], h + AHEAD + 1);
            mfma_block(ykb, next_head ? bq[N] : bq[C], z[(x + LA) % ZR]);
            epilogue_block(kb, z[x % ZR], wv[C]);
            interleave(kb, nread);
            pin(acc[kb]);
        }
        if constexpr (R % 2 == 1) {
            SI_WAIT_VMCNT((AHEAD - 2) * QN);
            loop_barrier();
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    using I6 = std::integral_constant<int, 6>;
    using I7 = std::integral_constant<int, 7>;
    static_assert(kQBuf == 8 && AHEAD == 6, "the unrolled loop below assumes 8 buffers");

    qload(Q.p[0], 0);
    qload(Q.p[1], 1);
    qload(Q.p[2], 2);
    qload(Q.p[3], 3);
    qload(Q.p[4], 4);
    qload(Q.p[5], 5);
    qload(Q.p[6], 6);
    SI_WAIT_VMCNT((AHEAD - 2) * QN);
    loop_barrier();
    qread(Q.p[0], bq[0], 0);
    qread(Q.p[0], bq[0], 1);
    wread(0, wv[0]);
#pragma unroll
    for (int x = 0; x < LA; ++x) mfma_block(x, bq[0], z[x]);

    for (int h = 0; h < H; h += kQBuf) {
        step(I0{}, h + 0);
        step(I1{}, h + 1);
        step(I2{}, h + 2);
        step(I3{}, h + 3);
        step(I4{}, h + 4);
        step(I5{}, h + 5);
        step(I6{}, h + 6);
        step(I7{}, h + 7);
    }
    SI_WAIT_VMCNT(0);

    float kscale[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        kscale[kb] = 1.0f;
        if constexpr (!K4) {
            const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + il;
            if (key < P.T) kscale[kb] = static_cast<const float*>(P.kc_scale)[b * P.T + key];
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = acc[kb][r];
            if constexpr (!K4) v = v * kscale[kb];
            acc[kb][r] = canon_zero(v);
        }
    }
}

// The score tile of operand mode OP (see the enum in si_score.hpp).
template <int NWAVE, int KB, int OP>
__device__ __forceinline__ void score_tile(const Problem& P, int64_t b, int64_t row0,
                                           int rows_valid, int64_t key0, int64_t key_end,
                                           ScoreLds& L, const QBufs& Q, f32x16 (&acc)[KB]) {
    if constexpr (op_q8(OP))
        score_regs_q8<NWAVE, KB, OP == kOpF8K4>(P, b, row0, rows_valid, key0, key_end, L, Q, acc);
    else
        score_regs_bf16<NWAVE, KB, OP == kOpBf16K8>(P, b, row0, rows_valid, key0, key_end, L, Q,
                                                    acc);
}

}  // namespace si
