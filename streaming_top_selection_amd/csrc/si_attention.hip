// Sparse attention over the indexer's selection: the consumer the indexer composes
// with (StreamIndex abstract, aisoku.com page: the sparse attention kernel reads only
// the selected keys, composed with a pipelined attention kernel at S = 262,144; jeff.news
// page, sequence diagram: merge-topk -> sparse attention -> result).  The pages give no
// attention formula; reading: per query row t and head h,
//     o[t,h,:] = sum_j softmax_j(scale <qa[t,h,:], kv[s_j,:]>) kv[s_j,:]
// over the row's selected compressed entries s_j (index -1 = none), the latent being
// both key and value and shared by every head; a row with no entry gives zeros.
//
// One workgroup per query row, one wave per 32 heads.  The selected entries are taken
// 32 at a time: their latents are gathered into LDS twice (row-major for the score
// product, transposed for the weight x value product), then per wave
//   S^T[32 keys x 32 heads] = KV[32 x D] * qa^T          (bf16 MFMA, fp32 accumulate)
//   online softmax per head (exp2 of fp32 logits, running maximum and sum)
//   O^T[D x 32 heads]      += KV^T[D x 32] * P^T[32 x 32] (weights rounded to bf16)
// The score layout puts one head per lane column, so a head's maximum and sum need
// one exchange with lane ^ 32 and the rescale of O is a per-lane multiply.  The next
// two blocks' rows are loaded into registers while the current block is computed
// (the kernel is compiled per wave count, so the gather loops unroll and the staged
// rows stay in registers).
#include "si_kernels.hpp"

namespace si {

constexpr int kAttnKeys = 32;                  // selected entries per block
constexpr int kKvtStride = 36;                 // bf16 per transposed row (32 + 4 pad)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    // round to nearest even (finite inputs)
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const uint32_t ra = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
    const uint32_t rb = (ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16;
    return ra | (rb << 16);
}

template <int NW>
__global__ void __launch_bounds__(NW * 64) sparse_attention_kernel(AttnArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t kvs[kAttnKeys * kD];        // 8 KiB
    __shared__ __attribute__((aligned(16))) uint16_t kvt[kD * kKvtStride];       // 9 KiB
    const int lane = lane_id();
    const int wave = wave_id();
    const int hh = lane >> 5, il = lane & 31;
    constexpr int nthreads = NW * 64;
    const int tid = threadIdx.x;
    const int64_t bt = blockIdx.x;                 // b * S + t
    const int64_t b = bt / A.S;
    const int32_t* sel = A.idx + bt * A.k;
    const uint16_t* kvb = A.kv + b * A.T * kD;

    // selected entries: the valid ones come first (the indexer pads at the end); an
    // index outside [0, T) ends the list as well
    // (only the leading run counts, so every entry below n_sel is a valid index)
    int n_sel = 0;
    for (int base = 0; base < A.k; base += 64) {
        const int i = base + lane;
        const int32_t v = i < A.k ? sel[i] : -1;
        const uint64_t ok = __ballot(i < A.k && v >= 0 && v < A.T);
        const int lead = ok == ~0ull ? 64 : (int)__builtin_ctzll(~ok);
        n_sel += lead;
        if (lead < 64) break;
    }
    n_sel = __builtin_amdgcn_readfirstlane(n_sel);

    const int head = 32 * wave + il;
    const bool head_ok = head < A.HA;
    // B operand of the score product: qa[t, head, 64 hh + 8 s + [0, 8)]
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (head_ok)
            v = *reinterpret_cast<const u32x4*>(A.qa + ((bt * A.HA + head) * kD + 64 * hh + 8 * s));
        qf[s] = __builtin_bit_cast(bf16x8, v);
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -__builtin_inff(), l = 0.0f;

    // gather: piece id = it * nthreads + tid covers key r = id / 16, d = 8 (id % 16) + [0, 8)
    constexpr int npieces = kAttnKeys * (kD / 8);
    constexpr int per_thread = (npieces + nthreads - 1) / nthreads;   // 8, 4, 3 or 2
    u32x4 pre[2][8];      // two blocks in flight
    auto load_block = [&](int blk, u32x4 (&pr)[8]) {
#pragma unroll
        for (int it = 0; it < per_thread; ++it) {
            const int id = it * nthreads + tid;
            if (id >= npieces) break;
            const int r = id >> 4, c = id & 15;
            const int j = blk * kAttnKeys + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (j < n_sel) v = *reinterpret_cast<const u32x4*>(kvb + (int64_t)sel[j] * kD + 8 * c);
            pr[it] = v;
        }
    };
    auto store_block = [&](const u32x4 (&pr)[8]) {
#pragma unroll
        for (int it = 0; it < per_thread; ++it) {
            const int id = it * nthreads + tid;
            if (id >= npieces) break;
            const int r = id >> 4, c = id & 15;
            *reinterpret_cast<u32x4*>(&kvs[(16 * r + (c ^ (r & 15))) * 8]) = pr[it];
            const uint32_t wd[4] = {pr[it].x, pr[it].y, pr[it].z, pr[it].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kvt[(8 * c + 2 * e) * kKvtStride + r] = (uint16_t)(wd[e] & 0xFFFFu);
                kvt[(8 * c + 2 * e + 1) * kKvtStride + r] = (uint16_t)(wd[e] >> 16);
            }
        }
    };

    const int nblocks = (n_sel + kAttnKeys - 1) / kAttnKeys;
    if (nblocks > 0) load_block(0, pre[0]);
    if (nblocks > 1) load_block(1, pre[1]);
    for (int blk = 0; blk < nblocks; ++blk) {
        __syncthreads();                              // the previous block's reads are done
        // blocks blk (slot blk % 2) and blk + 1 are in flight; store blk, then refill
        // its slot with blk + 2
        if (blk & 1) store_block(pre[1]); else store_block(pre[0]);
        __syncthreads();                              // this block is in LDS
        if (blk + 2 < nblocks) {
            if (blk & 1) load_block(blk + 2, pre[1]); else load_block(blk + 2, pre[0]);
        }

        // S^T = KV * qa^T: A = key rows (lane il: key il, d = 64 hh + 8 s + [0, 8))
        f32x16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int c = 8 * hh + s;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kvs[(16 * il + (c ^ (il & 15))) * 8]);
            z = mfma32x32x16(a, qf[s], z);
        }
        // register r of this lane: key mfma_row(r, lane) of the block, head = column il
        float sc[16];
        float bm = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool valid = blk * kAttnKeys + mfma_row(r, lane) < n_sel;
            sc[r] = valid ? z[r] * A.scale_log2 : -__builtin_inff();
            bm = fmaxf(bm, sc[r]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 32));           // the head's other 16 keys
        const float m_new = fmaxf(m, bm);             // finite: block 0 has a valid key
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        float p[16], ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(sc[r] - m_new);
            ps += p[r];
        }
        ps += __shfl_xor(ps, 32);
        l = l * alpha + ps;
        m = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        // B operand of the value product, step s2: this lane's weights r = 8 s2 .. 8 s2 + 7,
        // i.e. keys 16 s2 + 4 hh + [0, 4) and 16 s2 + 8 + 4 hh + [0, 4), rounded to bf16
        bf16x8 pb[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4 v = {pack_bf16x2(p[8 * s2], p[8 * s2 + 1]), pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]),
                             pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]), pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7])};
            pb[s2] = __builtin_bit_cast(bf16x8, v);
        }
        // O^T += KV^T * P^T: A = rows d = 32 db + il of the transposed block, the same keys
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const uint16_t* row = &kvt[(32 * db + il) * kKvtStride];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint64_t lo = *reinterpret_cast<const uint64_t*>(row + 16 * s2 + 4 * hh);
                const uint64_t hi = *reinterpret_cast<const uint64_t*>(row + 16 * s2 + 8 + 4 * hh);
                const u32x4 v = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
                o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, v), pb[s2], o[db]);
            }
        }
    }

    // o[db][r]: head = column il, d = 32 db + mfma_row(r, lane); four consecutive d per
    // group of registers, written as 8 bytes of bf16
    if (!head_ok) return;
    const float inv = nblocks > 0 ? 1.0f / l : 0.0f;
    uint16_t* orow = A.out + (bt * A.HA + head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * hh;
            const uint32_t lo = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
            const uint32_t hi = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d) = u32x2{lo, hi};
        }
}

hipError_t launch_sparse_attention(const AttnArgs& a, hipStream_t stream) {
    const int64_t grid = a.B * a.S;
    if (grid <= 0) return hipSuccess;
    const int waves = (a.HA + 31) / 32;
    const dim3 g((unsigned)grid);
    switch (waves) {
        case 1: hipLaunchKernelGGL(sparse_attention_kernel<1>, g, dim3(64), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(sparse_attention_kernel<2>, g, dim3(128), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(sparse_attention_kernel<3>, g, dim3(192), 0, stream, a); break;
        case 4: hipLaunchKernelGGL(sparse_attention_kernel<4>, g, dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace si
