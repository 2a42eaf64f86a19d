// Two-stage (coarse -> fine) indexer kernels: the candidate stage of the chengshu blog
// page "两级稀疏注意力：滑窗、压缩 KV latent 与 indexer" (section "indexer：在摘要里做
// '预筛选'"): blocks of compressed keys are scored cheaply, the best blocks are kept,
// and only their keys are scored finely.  Readings (the page defines no block score):
// a block key is the bf16-rounded mean of the block's keys; a block is a candidate once
// all of its keys are visible; the fine candidates are the kept blocks' keys plus the
// query's trailing incomplete block.
//
// The coarse stage is the single-stage indexer over the block keys (mask ratio
// block * m), run by the driver.  The kernels here build the block keys, score the fine
// candidates and select the final top-k.
//
// Fine scoring keeps the single-stage arithmetic bit for bit: one wave holds one query's
// heads as MFMA rows (A) and 32 gathered keys as columns (B), with the same
// v_mfma_f32_32x32x16_bf16 chain over the same d positions per step as score_regs_bf16,
// then the same head-ordered epilogue acc = fmaf(w_h, max(z_h, 0), acc).
#include "si_compact.hpp"
#include "si_kernels.hpp"
#include "si_sort.hpp"

namespace si {

// ---------------------------------------------------------------------------
// Block keys: kb[b, j, :] = bf16(fp32(k[b, blk j] + ... + k[b, blk j + blk - 1]) / blk),
// the sum taken in key order, 1/blk a power of two (exact), rounded to nearest even.
// One thread per (block, 8 consecutive d): 16-byte loads and stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite x
}

__global__ void __launch_bounds__(256) block_keys_kernel(BlockKeyArgs A) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nb = A.T / A.blk;
    constexpr int kChunks = kD / 8;
    if (id >= A.B * nb * kChunks) return;
    const int dch = (int)(id % kChunks);
    const int64_t bj = id / kChunks;                 // b * nb + j
    const int64_t b = bj / nb, j = bj - b * nb;
    const uint16_t* src = A.kc + ((b * A.T + j * A.blk) * kD + 8 * dch);
    float acc[8];
    {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __uint_as_float(wd[i] << 16);
            acc[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
        }
    }
    for (int i = 1; i < A.blk; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)i * kD);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = acc[2 * e] + __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] = acc[2 * e + 1] + __uint_as_float(wd[e] & 0xFFFF0000u);
        }
    }
    const float inv = 1.0f / (float)A.blk;           // exact: blk is a power of two
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = f32_to_bf16_rne(acc[2 * e] * inv) | (f32_to_bf16_rne(acc[2 * e + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(A.kb + (bj * kD + 8 * dch)) = u32x4{o[0], o[1], o[2], o[3]};
}

hipError_t launch_block_keys(const BlockKeyArgs& a, hipStream_t stream) {
    const int64_t n = a.B * (a.T / a.blk) * (kD / 8);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(block_keys_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fine scoring.  Candidate position p of row r: p < blk*nk -> key blk * cidx[r][p / blk]
// + p % blk (the kept blocks, nk = min(k_blocks, complete visible blocks)); then the
// trailing keys blk*nb .. n-1; past ncand nothing.  Writes the selection key (ord(score),
// ~index) of each candidate to cand[r][p], and the smallest and largest score image of
// the candidates of each (row, shard) to range[r][shard] (min > max: none).
//
// The keys are split into shards of 512-key granules (granule g -> shard g mod 8, a
// block by its first key), and each row is scored by one wave per shard, in workgroups
// of consecutive rows of one shard.  Workgroups are handed to the chip's eight
// accelerator dies (XCDs) in turn, so workgroup i runs on die i mod 8: the shard of
// workgroup i is i mod 8, and each die gathers keys from one eighth of the key array,
// which its own L2 can hold (2 MiB of the 16 MiB at S = 262,144) instead of streaming
// every key from the shared cache.  A wave first lists its shard's kept blocks (and the
// trailing block) in LDS in rank order, then scores them 64 candidates at a time.
// ---------------------------------------------------------------------------
constexpr int kFineWaves = 4;
constexpr int kFineShards = 8;
constexpr int kFineGranule = 512;
constexpr int kFineMaxBlocks = 2048;   // the two-stage plan bounds k_blocks by this

struct FineRow {
    int64_t n, nb, nk, ncand;
};

__device__ __forceinline__ FineRow fine_row(const FineArgs& A, int64_t t) {
    FineRow f;
    f.n = visible_keys(t, A.m, A.T);
    f.nb = visible_keys(t, A.blk * A.m, A.T / A.blk);
    f.nk = min(f.nb, (int64_t)A.k_blocks);
    f.ncand = A.blk * f.nk + (f.n - A.blk * f.nb);
    return f;
}

__device__ __forceinline__ int fine_shard(int64_t first_key) {
    return (int)((first_key / kFineGranule) % kFineShards);
}

__global__ void __launch_bounds__(kFineWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fine_score_kernel(FineArgs A) {
    // this wave's blocks: rank in the row's kept list (nk: the trailing block) and the
    // block index; at most k_blocks + 1 of them
    __shared__ int32_t sRank[kFineWaves][kFineMaxBlocks + 1];
    __shared__ int32_t sBlk[kFineWaves][kFineMaxBlocks + 1];
    const int lane = lane_id();
    const int wave = wave_id();
    const int hh = lane >> 5, il = lane & 31;
    const int shard = (int)(blockIdx.x % kFineShards);
    const int64_t r = (int64_t)(blockIdx.x / kFineShards) * kFineWaves + wave;
    if (r >= A.rows) return;                          // wave-uniform; no barriers below
    const int64_t t = A.q_pos0 + r;                    // absolute position of this row
    const FineRow f = fine_row(A, t);
    const int32_t* cidx = A.cidx + r * A.k_blocks;
    uint64_t* out = A.cand + r * A.cand_stride;
    const int H = A.H;
    const int blk = A.blk;
    int32_t* const rank = sRank[wave];
    int32_t* const blkj = sBlk[wave];

    // this shard's blocks, in rank order
    int nblk = 0;
    for (int64_t base = 0; base < f.nk; base += 64) {
        const int64_t i = base + lane;
        const int32_t j = i < f.nk ? cidx[i] : 0;
        const bool mine = i < f.nk && fine_shard((int64_t)j * blk) == shard;
        const uint64_t bal = __ballot(mine);
        if (mine) {
            const int at = nblk + __popcll(bal & lanemask_lt());
            rank[at] = (int32_t)i;
            blkj[at] = j;
        }
        nblk += __popcll(bal);
    }
    const int64_t ntail = f.n - blk * f.nb;            // keys of the trailing block
    if (ntail > 0 && fine_shard(blk * f.nb) == shard) {
        if (lane == 0) {
            rank[nblk] = (int32_t)f.nk;
            blkj[nblk] = (int32_t)f.nb;
        }
        ++nblk;
    }
    wave_sync();
    // slot q of this wave's list: block q / blk, key offset q % blk; its key and the
    // candidate position it is written to (-1: none)
    auto slot_key = [&](int64_t q, int64_t* pos) {
        const int64_t sb = q / blk, o = q - sb * blk;
        if (sb >= nblk) return (int64_t)-1;
        const int32_t i = rank[sb];
        if (i >= f.nk && o >= ntail) return (int64_t)-1;
        *pos = (int64_t)i * blk + o;
        return (int64_t)blkj[sb] * blk + o;
    };

    // A operand: heads 32 rb + il of this query, d = 64 hh + 8 s + [0, 8) in step s
    bf16x8 qa[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int head = 32 * rb + il;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < H)
                v = *reinterpret_cast<const u32x4*>(A.q + ((r * H + head) * kD + 64 * hh + 8 * s));
            qa[rb][s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    // the row's head weights, read once (0 past H: those heads' scores are exact zeros,
    // their terms add +0 as in the single-stage tile)
    const float* wrow = A.w + r * H;
    float wr[64];
#pragma unroll
    for (int h = 0; h < 64; ++h) {
        const float wv = wrow[min(h, H - 1)];
        wr[h] = h < H ? wv : 0.0f;
    }

    const int64_t nchunks = ((int64_t)nblk * blk + 63) / 64;
    uint32_t omin = ~0u, omax = 0u;
    for (int64_t c = 0; c < nchunks; ++c) {
        // B operand: key block kb holds slots 64 c + 32 kb + [0, 32); lane il of each
        // half supplies its column, d = 64 hh + 8 s + [0, 8)
        bf16x8 kf[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            int64_t pos_unused;
            const int64_t key = slot_key(64 * c + 32 * kb + il, &pos_unused);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (key >= 0)
                    v = *reinterpret_cast<const u32x4*>(A.kc + (key * kD + 64 * hh + 8 * s));
                kf[kb][s] = __builtin_bit_cast(bf16x8, v);
            }
        }
        f32x16 z[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) z[rb][kb][e] = 0.0f;
#pragma unroll
                for (int s = 0; s < 8; ++s) z[rb][kb] = mfma32x32x16(qa[rb][s], kf[kb][s], z[rb][kb]);
            }
        // Lane il of half hh scores slot 64 c + 32 hh + il, i.e. column il of key
        // block hh.  Register e of lane (il, half g) holds head 32 rb + mfma_row(e, 32 g)
        // of that column.  Swapping the upper half of block 0's registers with the lower
        // half of block 1's (v_permlane32_swap) leaves every lane with both head groups
        // of its own block: g0 holds the heads of group 0, g1 those of group 1.
        float g0[2][16], g1[2][16];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(z[rb][0][e]), __float_as_uint(z[rb][1][e]), false, false);
                g0[rb][e] = __uint_as_float(sw[0]);
                g1[rb][e] = __uint_as_float(sw[1]);
            }
        // acc = fmaf(w_h, max(z_h, 0), acc) for h = 0 .. 63 from +0, as in the tile
        float acc = 0.0f;
#pragma unroll
        for (int h = 0; h < 64; ++h) {
            const int rb = h >> 5, hl = h & 31;
            const int e = 4 * (hl >> 3) + (hl & 3);
            const float zz = ((hl >> 2) & 1) ? g1[rb][e] : g0[rb][e];
            acc = __builtin_fmaf(wr[h], __builtin_fmaxf(zz, 0.0f), acc);
        }
        int64_t p = 0;
        const int64_t key = slot_key(64 * c + lane, &p);
        if (key >= 0) {
            const uint64_t sk = make_key(canon_zero(acc), (uint32_t)key);
            out[p] = sk;
            const uint32_t o = (uint32_t)(sk >> 32);
            omin = o < omin ? o : omin;
            omax = o > omax ? o : omax;
        }
    }
    omin = wave_min_u32(omin);
    omax = wave_max_u32(omax);
    if (lane == 0)
        *reinterpret_cast<u32x2*>(A.range + 2 * (r * kFineShards + shard)) = u32x2{omin, omax};
}

hipError_t launch_fine_score(const FineArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.k_blocks > kFineMaxBlocks) return hipErrorInvalidValue;
    const int64_t grid = (a.rows + kFineWaves - 1) / kFineWaves * kFineShards;
    hipLaunchKernelGGL(fine_score_kernel, dim3((unsigned)grid), dim3(kFineWaves * 64), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fine selection: one wave per row, over the row's keys in the workspace.  With the
// score range fine scoring recorded, one pass counts the keys per score bin
// (hist_bin: 256 bins linear in the score between the row's extremes), and the bin d
// holding the k-th largest key follows; a second pass keeps the keys of higher bins
// and stages bin d's, whose k - above largest are found by counting larger keys.  When
// bin d holds more than 64 keys (or the range is empty) the k-th largest key comes from
// exact radix passes instead and the keys at or above it are kept.  The kept keys
// (exactly k: keys are unique and non-zero) are sorted in registers by the bitonic
// network and written as the row.
// ---------------------------------------------------------------------------
template <int LE>
__global__ void __launch_bounds__(64) fine_select_kernel(FineArgs A) {
    constexpr int EPL = 1 << LE;
    __shared__ uint64_t sbuf[64 * EPL];
    __shared__ uint32_t hist[256];
    __shared__ __attribute__((aligned(16))) uint64_t stage[64];
    const int lane = lane_id();
    const int64_t r = blockIdx.x;
    const int64_t t = A.q_pos0 + r;
    const FineRow f = fine_row(A, t);
    const uint64_t* keys = A.cand + r * A.cand_stride;
    const int ncand = (int)f.ncand;
    const int need = min(ncand, A.k);
    // appends the keys of `keep` (one per lane) at pos, in lane order, below cap
    auto append = [&](bool keep, uint64_t v, uint64_t* dst, int cap, int& pos) {
        const uint64_t bal = __ballot(keep);
        const int at = pos + __popcll(bal & lanemask_lt());
        if (keep && at < cap) dst[at] = v;
        pos += __popcll(bal);
    };
    int pos = 0;
    bool done = ncand <= A.k;
    if (done) {
        for (int base = 0; base < ncand; base += 64) {
            const int i = base + lane;
            append(i < ncand, i < ncand ? keys[i] : 0ull, sbuf, 64 * EPL, pos);
        }
    } else {
        // 256 bins linear in the score between the row's extremes (hist_bin)
        // the row's score range: the extremes over the shards' ranges
        u32x2 rg = {~0u, 0u};
#pragma unroll
        for (int x = 0; x < kFineShards; ++x) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(A.range + 2 * (r * kFineShards + x));
            rg.x = min(rg.x, v.x);
            rg.y = max(rg.y, v.y);
        }
        const float lo = unord_f32(rg.x), span = unord_f32(rg.y) - lo;
        if (rg.y > rg.x && span > 0.0f && span < __builtin_inff()) {
            const float inv = 256.0f / span, off = -(lo * inv);
            *reinterpret_cast<u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
            wave_sync();
            // eight keys per lane in flight per round (one load and wait at a time left
            // each pass latency-bound)
            for (int base = 0; base < ncand; base += 8 * 64) {
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = base + 64 * u + lane;
                    v[u] = i < ncand ? keys[i] : 0ull;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = base + 64 * u + lane;
                    atomicAdd(&hist[hist_bin(key_score(v[u]), inv, off)], i < ncand ? 1u : 0u);
                }
            }
            wave_sync();
            uint32_t above, cntd;
            const int d = hist_find(hist, A.k, &above, &cntd);
            wave_sync();
            if (d >= 0 && cntd <= 64u) {
                stage[lane] = 0ull;
                int nd = 0;
                for (int base = 0; base < ncand; base += 8 * 64) {
                    uint64_t v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int i = base + 64 * u + lane;
                        v[u] = i < ncand ? keys[i] : 0ull;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int i = base + 64 * u + lane;
                        const uint32_t bn = hist_bin(key_score(v[u]), inv, off);
                        append(i < ncand && bn > (uint32_t)d, v[u], sbuf, 64 * EPL, pos);
                        append(i < ncand && bn == (uint32_t)d, v[u], stage, 64, nd);
                    }
                }
                wave_sync();
                if (pos == (int)above && nd == (int)cntd) {
                    const uint64_t th = stage_kth(stage, nd, A.k - pos);
                    const uint64_t v = stage[lane];
                    append(lane < nd && v >= th, v, sbuf, 64 * EPL, pos);
                    done = true;
                }
            }
        }
        if (!done) {
            // exactly k keys are >= th
            const uint64_t th = wave_select_kth(LdsKeys{keys, ncand}, A.k, hist);
            pos = 0;
            for (int base = 0; base < ncand; base += 64) {
                const int i = base + lane;
                const uint64_t v = i < ncand ? keys[i] : 0ull;
                append(i < ncand && v >= th, v, sbuf, 64 * EPL, pos);
            }
        }
    }
    wave_sync();
    uint64_t x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = EPL * lane + e < need ? sbuf[EPL * lane + e] : 0ull;
    sort_desc<LE>(x);
    write_sorted_keys<LE>(A.out_idx + r * (int64_t)A.k, A.out_score + r * (int64_t)A.k, A.k, x,
                          need, lane);
}

hipError_t launch_fine_select(const FineArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.rows), block(64);
    if (a.k <= 512) hipLaunchKernelGGL(fine_select_kernel<3>, grid, block, 0, stream, a);
    else if (a.k <= 1024) hipLaunchKernelGGL(fine_select_kernel<4>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fine_select_kernel<5>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace si
