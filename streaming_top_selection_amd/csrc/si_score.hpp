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
//  * K-stationary: each wave loads its keys once into MFMA B-operand registers and
//    keeps them for all heads (a key tile is the same for every head).  With one
//    wave per SIMD a wave has 512 registers, so KB = 4 blocks of 32 keys fit beside
//    double-buffered q operands without spilling.
//  * q is streamed head by head into LDS tiles of 32 rows x 128 bf16 (8 KiB/head) by
//    buffer->LDS loads issued several heads ahead (no register staging, two loads
//    per wave and head, no branches); all waves of the workgroup share each tile as
//    the MFMA A operand.
//  * Software pipeline: the MFMAs of the next block are issued interleaved with the
//    VALU epilogue (ReLU, weighted sum) of the current one, so both pipes stay busy
//    in each wave; the LDS reads of head h+1 and the loads of head h+7 are issued in
//    the shadow of step h's MFMAs, so at most a barrier (one per two heads) sits
//    between the last MFMA of a step and the first of the next.
//  * Output layout: queries are MFMA rows and keys columns, so lane l owns key
//    (l & 31) of each block and query rows mfma_row(r, l).  A query's scores for
//    32 consecutive keys sit in one register across 32 lanes, which lets the
//    selection append survivors as contiguous runs.
#pragma once

#include <type_traits>

#include "si_common.hpp"

namespace si {

struct Problem {
    const void* q;            // [B, S, H, D] bf16 bits or E4M3 bytes
    const void* kc;           // [B, T, D] bf16 bits or E4M3 bytes, [B, T, D/2] MXFP4 nibbles
    const void* kc_scale;     // [B, T] fp32 (E4M3 keys), [B, T, D/32] E8M0 (MXFP4), or null
    const float* w;           // [B, S, H] head weights (E4M3 q: the effective w * q_scale)
    int64_t B, S, T;
    int32_t H, m;
    int64_t q_pos0;
};

// Operand modes of the score tile (q format x key format) and the MFMA they run on.
enum : int {
    kOpBf16 = 0,     // bf16 q x bf16 keys: v_mfma_f32_32x32x16_bf16
    kOpBf16K8 = 1,   // bf16 q x E4M3 keys widened exactly to bf16: the same bf16 MFMA
    kOpF8 = 2,       // E4M3 q x E4M3 keys: v_mfma_f32_32x32x64_f8f6f4
    kOpF8K4 = 3      // E4M3 q x MXFP4 keys: v_mfma_scale_f32_32x32x64_f8f6f4, E8M0 scales
};
constexpr bool op_q8(int op) { return op >= kOpF8; }
constexpr bool op_row_scale(int op) { return op == kOpBf16K8 || op == kOpF8; }
// bytes of one staged q tile (32 rows x D elements of one head)
constexpr int op_q_tile_bytes(int op) { return op_q8(op) ? kTQ * kD : kTQ * kD * 2; }

constexpr int kQBuf = 8;             // q tiles in flight: head h+7 loads while h+1 is read
constexpr int kWHeads = kMaxH + kQBuf;       // weight rows: H heads, then zeros
constexpr int kQChunks = kTQ * 16;   // 16-byte chunks per staged q tile (32 rows x 256 B)
constexpr int kQTile = kQChunks * 8;         // bf16 per staged q tile (8 KiB)

struct ScoreLds {
    float w[kWHeads * kTQ];       // [head][query row] weights (0 past H or the tile's rows)
};

// The staged q tiles: kQBuf separate LDS arrays (each its own object, so the
// compiler can tell the direct-to-LDS loads into one from reads of another).  Chunk c
// (d = 8c .. 8c+7) of row r sits at chunk 16*r + (c ^ (r & 15)) of the tile, so an
// A-operand read (16 consecutive rows at a time, the same chunk of each) hits 16
// different 16-byte bank groups.
struct QBufs {
    uint16_t* p[kQBuf];
};

#define SI_DECLARE_QBUFS(name, OP)                                                    \
    constexpr int name##_n = si::op_q_tile_bytes(OP) / 2;                             \
    __shared__ __attribute__((aligned(16))) uint16_t name##0[name##_n],              \
        name##1[name##_n], name##2[name##_n], name##3[name##_n], name##4[name##_n],  \
        name##5[name##_n], name##6[name##_n], name##7[name##_n];                     \
    const si::QBufs name = {{name##0, name##1, name##2, name##3, name##4, name##5,   \
                             name##6, name##7}}

// Workgroup barrier for the head loop.  LDS visibility is managed explicitly: the
// direct-to-LDS loads are awaited with vmcnt before it and every LDS read feeding an
// MFMA is awaited before its use, so only the compiler must not move memory accesses
// across it (a release fence here would wait for every load in flight).
__device__ __forceinline__ void loop_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding).
#define SI_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | 0x70 | 0xF00)

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds: lane L's 16 bytes at rsrc.base + voffset go to LDS at
// lds + 16*L (the LDS address is taken from M0, so it is wave-uniform).
extern "C" __device__ void si_raw_buffer_load_lds(
    i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer resource (gfx9): 48-bit base, stride 0, num_records bytes; reads past
// num_records return zeros.
__device__ __forceinline__ i32x4 make_rsrc(uint64_t base, uint32_t num_records) {
    i32x4 r;
    r.x = (int32_t)(uint32_t)base;
    r.y = (int32_t)((uint32_t)(base >> 32) & 0xFFFFu);
    r.z = (int32_t)num_records;
    r.w = 0x00020000;
    return r;
}

// Fills L.w for query rows [row0, row0 + rows_valid) of batch entry b (0 past the end):
// read along rows of w (coalesced), stored transposed, one head per LDS row.
template <int NT>
__device__ __forceinline__ void load_w_tile(const Problem& P, int64_t b, int64_t row0,
                                            int rows_valid, ScoreLds& L) {
    const int H = P.H;
    for (int f = threadIdx.x; f < kTQ * kWHeads; f += NT) {
        const int j = f / kWHeads, h = f - j * kWHeads;
        L.w[h * kTQ + j] = (j < rows_valid && h < H) ? P.w[((b * P.S + row0 + j) * H) + h] : 0.0f;
    }
}

// Scores rows [row0, row0 + rows_valid) against keys key0 + [0, NWAVE*KB*32).
// Requires: L.w filled and a __syncthreads() since; key0 % 32 == 0; key_end <= T;
// every thread of the workgroup calls it.  acc[kb][r] receives the score of query row
// row0 + mfma_row(r, lane) and key key0 + (wave*KB + kb)*32 + (lane & 31).  Keys >=
// key_end score as if zero: a caller that masks them anyway passes the end of what any
// of its rows sees, and zero operands there cost the MFMAs less power.
template <int NWAVE, int KB, bool FP8>
__device__ __forceinline__ void score_regs_bf16(const Problem& P, int64_t b, int64_t row0,
                                           int rows_valid, int64_t key0, int64_t key_end,
                                           ScoreLds& L, const QBufs& Q, f32x16 (&acc)[KB]) {
    constexpr int NT = NWAVE * kWave;
    static_assert(kQBuf >= 4, "the pipeline reads head h+1 while loading h+kQBuf-1");

    // The empty asm makes every per-lane value below (load and read offsets) a fresh
    // computation at each call: hoisted out of the caller's key loop they would stay
    // live through its selection code and crowd the head loop's registers.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = wave_id();
    const int hh = lane >> 5;       // which 64-wide half of d this lane feeds
    const int il = lane & 31;       // A row (query) and B column (key) of this lane
    const int H = P.H;

    // ---- K fragments (B operand): keys stay in registers for the whole head loop ----
    // step s covers d = 64*hh + 8*s + [0, 8) for lane l (same d for A and B).
    bf16x8 kf[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + il;
        if (key < key_end) {
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

    // ---- q staging: buffer -> LDS loads, kQBuf - 2 heads ahead -----------------
    // In each of QN rounds a wave loads 64 consecutive chunks of the tile: chunk P =
    // n*NT + tid holds row r = P / 16, piece c = (P % 16) ^ (r & 15).  Rows past the
    // tile's end re-load its last row (weight 0, never selected); heads past H-1
    // re-load head H-1, so every step issues the same loads.  The resource covers this
    // tile's rows; its base moves by one head per load.
    constexpr int QN = kQChunks / NT;
    static_assert(kQChunks % NT == 0, "every wave issues the same number of q loads");
    constexpr int AHEAD = kQBuf - 2;
    const uint64_t qbase = reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(P.q) +
                                                      (b * P.S + row0) * H * (int64_t)kD);
    const uint32_t qbytes = (uint32_t)(rows_valid * H * kD * 2);
    int voff[QN];
#pragma unroll
    for (int n = 0; n < QN; ++n) {
        const int chunk = n * NT + tid;
        const int r = chunk >> 4;
        const int c = (chunk & 15) ^ (r & 15);
        voff[n] = (min(r, rows_valid - 1) * H * kD + c * 8) * 2;
    }
    auto qload = [&](uint16_t* buf, int h) {
        const uint32_t hc = (uint32_t)(h < H ? h : H - 1);
        const i32x4 rsrc = make_rsrc(qbase + hc * (kD * 2), qbytes - hc * (kD * 2));
#pragma unroll
        for (int n = 0; n < QN; ++n)
            si_raw_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(buf + (n * NT + wave * 64) * 8),
                16, voff[n], 0, 0, 0);
    };
    // A operand of one head: query row il, d = 64*hh + 8*s + [0, 8), i.e. piece 8*hh + s
    int roff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) roff[s] = il * 256 + 16 * ((8 * hh + s) ^ (il & 15));
    auto qread = [&](const uint16_t* buf, bf16x8 (&bq)[8], int s0, int s1) {
        const char* base = reinterpret_cast<const char*>(buf);
#pragma unroll
        for (int s = s0; s < s1; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(base + roff[s]);
    };
    // head weights of this lane's 16 query rows: rows 8*g + 4*hh + [0, 4), g = 0..3
    // (one 16-byte LDS read per g; the 32 lanes of a half read the same address)
    auto wread = [&](int h, f32x4 (&wv)[4]) {
        const f32x4* row = reinterpret_cast<const f32x4*>(L.w + h * kTQ + 4 * hh);
#pragma unroll
        for (int g = 0; g < 4; ++g) wv[g] = row[2 * g];
    };
    // MFMA chain of key block kb for one head: z = Q_h * K(kb)^T over d, from zero
    auto mfma_block = [&](int kb, const bf16x8 (&bq)[8], f32x16& z) {
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) z = mfma32x32x16(bq[s], kf[kb][s], z);
    };
    auto epilogue_block = [&](int kb, const f32x16& z, const f32x4 (&wv)[4]) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[kb][r] = __builtin_fmaf(wv[r >> 2][r & 3], __builtin_fmaxf(z[r], 0.0f),
                                        acc[kb][r]);
    };
    // Keeps an accumulator block's epilogue inside the step that issues it (without
    // this the compiler sinks every epilogue of the unrolled loop to its end and keeps
    // all their MFMA outputs alive at once).
    auto pin = [&](f32x16& v) { asm volatile("" : "+v"(v)); };
    // one MFMA block (8 MFMAs) interleaved with one epilogue block (32 VALU), with
    // a share of the step's 12 LDS reads (RD[kb] of them, one per MFMA) and, in block
    // KLOAD, its q loads
    constexpr int KLOAD = KB > 1 ? 1 : 0;
    auto interleave = [&](int kb, int nread) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
            if (i < nread) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (kb == KLOAD && i < QN) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][r] = 0.0f;

    // Skewed software pipeline over blocks (head, key block), in the order
    // (0,0), (0,1), ..., (0,KB-1), (1,0), ...: the MFMA chain of block X + ZR - 1 is
    // issued interleaved with the epilogue (ReLU, weighted sum) of block X, so an
    // epilogue never waits on a chain that was just issued, and block X lives in
    // accumulator slot X mod ZR.  The A operand and the weights of head h+1
    // (bq[(h+1) % 2], wv[(h+1) % 2]) are read at the top of step h, ahead of their
    // first use, and a scheduling barrier keeps those reads there.
    //
    // Step h (buffers known at compile time): read head h+1 from buffer (h+1) % 8;
    // for kb = 0..KB-1 run the MFMAs of block (h, kb) + ZR - 1 beside the epilogue of
    // (h, kb); load head h+7 into buffer (h+7) % 8 (last read in step h-2, before the
    // previous barrier).  Barriers come after odd steps only: the one after step h
    // publishes heads h+2 and h+3, read in the next two steps.  Heads run in groups of
    // 8; steps past H-1 see zero head weights (their epilogue adds exact zeros) and
    // re-loaded data of head H-1, so the arithmetic of every real head is the same for
    // any H.
    constexpr int ZR = (KB == 1) ? 2 : ((KB % 3 == 0) ? 3 : 2);   // accumulator slots
    constexpr int LA = ZR - 1;                                     // blocks of lookahead
    static_assert((kQBuf * KB) % ZR == 0, "slots must repeat every group of 8 heads");
    static_assert(LA <= KB, "lookahead stays within the next head");
    f32x16 z[ZR];
    bf16x8 bq[2][8];
    f32x4 wv[2][4];
    auto step = [&](auto rstep, int h) {
        constexpr int R = decltype(rstep)::value;            // h mod 8
        constexpr int RB = (R + 1) % kQBuf, LB = (R + kQBuf - 1) % kQBuf;
        constexpr int C = R % 2, N = 1 - C;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int x = R * KB + kb;                        // block index mod 8*KB
            const int ykb = (kb + LA) % KB;                   // block x + LA
            const bool next_head = kb + LA >= KB;
            // reads of head h+1 (first used by the block of head h+1, the last one):
            // spread over the blocks before it, at most one per MFMA
            int nread = 0;
            if (KB >= 3) {
                if (kb == 0) qread(Q.p[RB], bq[N], 0, 4), nread = 4;
                if (kb == 1) qread(Q.p[RB], bq[N], 4, 8), nread = 4;
                if (kb == 2) wread(h + 1, wv[N]), nread = 4;
            } else if (kb == 0) {
                qread(Q.p[RB], bq[N], 0, 8);
                wread(h + 1, wv[N]);
                nread = 8;
            }
            if (kb == KLOAD) qload(Q.p[LB], h + AHEAD + 1);
            mfma_block(ykb, next_head ? bq[N] : bq[C], z[(x + LA) % ZR]);
            epilogue_block(kb, z[x % ZR], wv[C]);
            interleave(kb, nread);
            pin(acc[kb]);
        }
        // after an odd step h, heads h+2 and h+3 (read in steps h+1, h+2) must have
        // landed: every wave issues QN loads per head, so <= (AHEAD-2)*QN younger
        // loads means they have
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

    // prologue: heads 0..6 in flight into buffers 0..6, heads 0, 1 and 2 published
    qload(Q.p[0], 0);
    qload(Q.p[1], 1);
    qload(Q.p[2], 2);
    qload(Q.p[3], 3);
    qload(Q.p[4], 4);
    qload(Q.p[5], 5);
    qload(Q.p[6], 6);
    SI_WAIT_VMCNT((AHEAD - 2) * QN);
    loop_barrier();
    qread(Q.p[0], bq[0], 0, 8);
    wread(0, wv[0]);
#pragma unroll
    for (int x = 0; x < LA; ++x) mfma_block(x, bq[0], z[x]);   // blocks (0, 0..LA-1)

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

    // the last steps' loads (of padding heads) land before anything else uses LDS
    SI_WAIT_VMCNT(0);

    float kscale[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        kscale[kb] = 1.0f;
        if constexpr (FP8) {
            const int64_t key = key0 + (int64_t)(wave * KB + kb) * kMB + il;
            if (key < P.T) kscale[kb] = static_cast<const float*>(P.kc_scale)[b * P.T + key];
        }
    }

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = acc[kb][r];
            if constexpr (FP8) v = v * kscale[kb];
            acc[kb][r] = canon_zero(v);
        }
    }
}

}  // namespace si
