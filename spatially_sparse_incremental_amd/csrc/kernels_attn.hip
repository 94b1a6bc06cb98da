// kernels_attn.hip -- query-pruned self-attention on gfx950.
//
// nubint.ai review, "Proposed method": attention layers are handled by
// pruning the queries of unedited tokens, so the attention work scales with
// the edited area.  Queries: the tokens of the listed blocks (block x block
// tokens of the h x w grid); keys and values: every token of the same image.
//
// Split over keys (as in flash decoding): a work item is (64-query tile of one
// image, head, key split).  Its 4 waves own 16 queries each and run an online
// softmax over the split's keys, 64 at a time, with both products on the
// matrix cores (v_mfma_f32_16x16x32_{f16,bf16}):
//   S^T  = K Q^T      A = key rows from LDS, B = this wave's Q^T fragments (registers)
//   O^T += V^T P^T    A = rows of a transposed V tile in LDS, B = P^T taken from S^T
// In S^T's accumulator layout a lane holds one query and 4 keys of each
// 16-key subtile.  Two subtiles packed give a B fragment of the second product
// (the order of k inside one MFMA is free, as long as A uses the same order),
// and every softmax statistic of a query lives in the lanes l, l^16, l^32,
// l^48.  O^T's accumulators hold the same query per lane, so the rescale by
// exp(m_old - m_new) needs no lane exchange.  Each item leaves (max, sum,
// unnormalised O) in the caller's workspace; a second kernel combines the
// splits, writes the queries' outputs and copies the cache elsewhere.
//
// Query tiles never straddle two images: each image's listed blocks are
// padded to whole 64-row tiles (per-image block counts come from one pass
// over the list in every workgroup).
#include "device_common.h"

namespace sige {

constexpr int kAttnD = 64;          // head dim
constexpr int kAttnKT = 64;         // keys per LDS tile
constexpr int kAttnQT = 64;         // queries per work item (4 waves x 16)
constexpr int kAttnThreads = 256;
constexpr int kAttnMaxImages = 8;
constexpr int kAttnWsRow = kAttnD + 4;  // floats per query in the workspace: O^T column, max, sum, pad
constexpr int kAttnKPitch = kAttnD + 8;   // halves per key row of the K tile in LDS
constexpr int kAttnVPitch = kAttnKT + 8;  // halves per d row of the transposed V tile

struct AttnArgs {
    const uint8_t *q, *k, *v;
    const int32_t *idx, *count;
    float *ws;
    const uint8_t *cache;
    uint8_t *out;
    Geo g;               // the token grid as a k = 1 geometry: h, w, b, cap; cin = cout = heads * D
    CopyCfg cc;          // copy of the cache (nvec 0: none)
    int heads;
    float scale_log2;    // softmax scale * log2(e)
    int grid1;           // grid of the partial kernel (fixes the key split)
};

template <int DT>
struct AttnMfma {  // one 16x16x32 MFMA
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        if constexpr (DT == 1)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                          0, 0, 0);
    }
};

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    uint16_t a, b;
    if constexpr (DT == 1) {
        a = __builtin_bit_cast(uint16_t, (__bf16)lo);
        b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    } else {
        a = __builtin_bit_cast(uint16_t, (_Float16)lo);
        b = __builtin_bit_cast(uint16_t, (_Float16)hi);
    }
    return (uint32_t)a | ((uint32_t)b << 16);
}

// Per-image bookkeeping of the listed blocks, in LDS: first slot and first
// padded tile of every image, and the total number of tiles.
struct AttnTiles {
    int first_slot[kAttnMaxImages + 1];
    int first_tile[kAttnMaxImages + 1];
};

__device__ void attn_tiles(const Geo &g, const int32_t *__restrict__ idx, int cnt, AttnTiles *t, int *cnt_img) {
    const int per = g.nby * g.nbx, b2 = g.b * g.b;
    if (threadIdx.x < kAttnMaxImages) cnt_img[threadIdx.x] = 0;
    __syncthreads();
    constexpr int U = 4;
    for (int e0 = threadIdx.x; e0 < cnt; e0 += U * kAttnThreads) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = (e0 + u * kAttnThreads < cnt) ? idx[e0 + u * kAttnThreads] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v[u] >= 0 && v[u] < g.cap) atomicAdd(&cnt_img[v[u] / per], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0, tl = 0;
        for (int i = 0; i < g.n; ++i) {
            t->first_slot[i] = s;
            t->first_tile[i] = tl;
            s += cnt_img[i];
            tl += (cnt_img[i] * b2 + kAttnQT - 1) / kAttnQT;
        }
        t->first_slot[g.n] = s;
        t->first_tile[g.n] = tl;
    }
    __syncthreads();
}

// Keys per split: the split count gives the grid about two items per workgroup.
__device__ __forceinline__ void attn_split(int items, int nkt, int grid, int &S, int &ktp) {
    S = items > 0 ? (2 * grid) / items : 1;
    S = max(1, min(S, min(16, nkt)));
    ktp = (nkt + S - 1) / S;
}

// The token of query row `row` of a tile of image n (or -1 past the image's rows
// or outside the grid).
__device__ __forceinline__ int attn_token(const Geo &g, const int32_t *__restrict__ idx, const AttnTiles &t, int n,
                                          int row) {
    const int b2 = g.b * g.b;
    const int nrows = (t.first_slot[n + 1] - t.first_slot[n]) * b2;
    if (row >= nrows) return -1;
    const int slot = t.first_slot[n] + row / b2, pix = row - (row / b2) * b2;
    int nn, by, bx;
    if (!decode_block(g, idx[slot], nn, by, bx) || nn != n) return -1;
    const int y = by * g.b + pix / g.b, x = bx * g.b + pix % g.b;
    if (y >= g.h || x >= g.w) return -1;
    return y * g.w + x;
}

template <int DT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(AttnArgs a) {
    constexpr int D = kAttnD, KT = kAttnKT;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * kAttnKPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * kAttnVPitch];
    __shared__ AttnTiles tiles;
    __shared__ int cnt_img[kAttnMaxImages];
    const Geo &g = a.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = g.h * g.w, C = a.heads * D;
    const int nkt = (L + KT - 1) / KT;
    const int cnt = clamp_count(a.count, g.cap);
    attn_tiles(g, a.idx, cnt, &tiles, cnt_img);
    const int ntiles = tiles.first_tile[g.n];
    const int items = ntiles * a.heads;
    int S, ktp;
    attn_split(items, nkt, gridDim.x, S, ktp);
    const int ql = lane & 15, kg = lane >> 4;  // this lane's query (B/C column) and k group
    for (int p = blockIdx.x; p < items * S; p += gridDim.x) {
        const int split = p % S, item = p / S;
        const int head = item % a.heads, tile = item / a.heads;
        int n = 0;
        while (n + 1 < g.n && tiles.first_tile[n + 1] <= tile) ++n;
        const int row = (tile - tiles.first_tile[n]) * kAttnQT + wave * 16 + ql;
        const int tok = attn_token(g, a.idx, tiles, n, row);
        // this wave's Q^T fragments: query ql, d = 32 * ks + 8 * kg + (0..7)
        u32x4 qf[2];
        const size_t img = (size_t)n * L;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            qf[ks] = ld16(a.q + ((img + (tok < 0 ? 0 : tok)) * C + head * D + ks * 32 + kg * 8) * 2);
        f32x4 oT[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) oT[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;
        const int kt0 = split * ktp, kt1 = min(nkt, kt0 + ktp);
        for (int kt = kt0; kt < kt1; ++kt) {
            const int j0 = kt * KT;
            __syncthreads();  // every wave is done with the previous tile
            // K tile: key rows of 8 16-byte slots and a pad slot, straight into LDS
            for (int qg = wave; qg < (KT * 9 + 63) / 64; qg += 4) {
                const int slot = qg * 64 + lane, key = slot / 9, c = slot - key * 9;
                if (key < KT && c < 8) {
                    const int j = min(j0 + key, L - 1);
                    __builtin_amdgcn_global_load_lds(
                        (const void *)(a.k + ((img + j) * C + head * D + c * 8) * 2),
                        (__attribute__((address_space(3))) void *)((uint8_t *)Ks + qg * 1024), 16, 0, 0);
                }
            }
            // V tile, transposed: 16 bytes of one key row per thread and step
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = tid + i * kAttnThreads, key = c >> 3, dc = c & 7;
                const int j = min(j0 + key, L - 1);
                const u32x4 vv = ld16(a.v + ((img + j) * C + head * D + dc * 8) * 2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Vt[(dc * 8 + 2 * e) * kAttnVPitch + key] = (uint16_t)(vv[e] & 0xFFFFu);
                    Vt[(dc * 8 + 2 * e + 1) * kAttnVPitch + key] = (uint16_t)(vv[e] >> 16);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // S^T = K Q^T for the 4 subtiles of 16 keys
            f32x4 sT[4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {
                sT[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4 kf = *(const u32x4 *)(Ks + (sub * 16 + ql) * kAttnKPitch + ks * 32 + kg * 8);
                    sT[sub] = AttnMfma<DT>::run(kf, qf[ks], sT[sub]);
                }
            }
            // online softmax for query ql: keys 16 * sub + 4 * kg + i of this tile
            float mt = -INFINITY;
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = j0 + sub * 16 + kg * 4 + i < L;
                    const float x = valid ? sT[sub][i] * a.scale_log2 : -INFINITY;
                    sT[sub][i] = x;
                    mt = fmaxf(mt, x);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = exp2f(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = exp2f(sT[sub][i] - m_new);
                    sT[sub][i] = e;
                    ps += e;
                }
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int m = 0; m < 4; ++m) oT[m] *= alpha;
            // O^T += V^T P^T, 32 keys per MFMA: keys 32*pr + 4*kg + (0..3) and 32*pr + 16 + 4*kg + (0..3)
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const u32x4 pb = u32x4{pack2<DT>(sT[2 * pr][0], sT[2 * pr][1]), pack2<DT>(sT[2 * pr][2], sT[2 * pr][3]),
                                       pack2<DT>(sT[2 * pr + 1][0], sT[2 * pr + 1][1]),
                                       pack2<DT>(sT[2 * pr + 1][2], sT[2 * pr + 1][3])};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint16_t *vr = Vt + (m * 16 + ql) * kAttnVPitch + pr * 32 + kg * 4;
                    const uint2 lo = *(const uint2 *)vr, hi = *(const uint2 *)(vr + 16);
                    oT[m] = AttnMfma<DT>::run(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, oT[m]);
                }
            }
        }
        // this item's partial: unnormalised O^T column of query ql, then max and sum
        float *wp = a.ws + ((size_t)p * kAttnQT + wave * 16 + ql) * kAttnWsRow;
#pragma unroll
        for (int m = 0; m < 4; ++m) *(f32x4 *)(wp + m * 16 + kg * 4) = oT[m];
        if (kg == 0) {
            wp[D] = m_run;
            wp[D + 1] = l_run;
        }
    }
}

// Combine the key splits of every query and head, write the outputs, then copy
// the cache elsewhere (copy_cached).
template <int DT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_combine(AttnArgs a) {
    constexpr int D = kAttnD;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ AttnTiles tiles;
    __shared__ int cnt_img[kAttnMaxImages];
    const Geo &g = a.g;
    const int L = g.h * g.w, C = a.heads * D;
    const int nkt = (L + kAttnKT - 1) / kAttnKT;
    const int cnt = clamp_count(a.count, g.cap);
    attn_tiles(g, a.idx, cnt, &tiles, cnt_img);
    const int ntiles = tiles.first_tile[g.n];
    const int items = ntiles * a.heads;
    int S, ktp;
    attn_split(items, nkt, a.grid1, S, ktp);
    // work unit: (item, query, 8-channel chunk)
    const long total = (long)items * kAttnQT * (D / 8);
    for (long u = (long)blockIdx.x * kAttnThreads + threadIdx.x; u < total; u += (long)gridDim.x * kAttnThreads) {
        const int dc = (int)(u % (D / 8));
        const int qi = (int)((u / (D / 8)) % kAttnQT);
        const int item = (int)(u / ((long)(D / 8) * kAttnQT));
        const int head = item % a.heads, tile = item / a.heads;
        int n = 0;
        while (n + 1 < g.n && tiles.first_tile[n + 1] <= tile) ++n;
        const int tok = attn_token(g, a.idx, tiles, n, (tile - tiles.first_tile[n]) * kAttnQT + qi);
        if (tok < 0) continue;
        float mx = -INFINITY;
        for (int s = 0; s < S; ++s)
            mx = fmaxf(mx, a.ws[((size_t)(item * S + s) * kAttnQT + qi) * kAttnWsRow + D]);
        float sum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; ++s) {
            const float *wp = a.ws + ((size_t)(item * S + s) * kAttnQT + qi) * kAttnWsRow;
            const float f = wp[D] == -INFINITY ? 0.f : exp2f(wp[D] - mx);
            sum += f * wp[D + 1];
            const f32x4 x0 = *(const f32x4 *)(wp + dc * 8), x1 = *(const f32x4 *)(wp + dc * 8 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] += f * x0[e];
                o[4 + e] += f * x1[e];
            }
        }
        const float inv = 1.f / sum;
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pack2<DT>(o[2 * e] * inv, o[2 * e + 1] * inv);
        st16(a.out + (((size_t)n * L + tok) * C + head * D + dc * 8) * 2, r);
    }
    if (a.cc.nvec > 0) {
        const long long lo = split_point(a.cc.nvec, blockIdx.x, gridDim.x);
        const long long hi = split_point(a.cc.nvec, blockIdx.x + 1, gridDim.x);
        if (lo < hi) {
            uint32_t *bm = nullptr;
            if (((g.cap + 31) >> 5) * 4 <= 64 * 1024) {
                bm = (uint32_t *)smem;
                build_bitmap<kAttnThreads>(a.idx, cnt, g.cap, bm);
            }
            copy_span<4, kAttnThreads>(g, a.cc, bm, a.idx, cnt, a.cache, a.out, lo, hi);
        }
    }
}

int attn_partial_grid(int cus) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_partial<2>, kAttnThreads, 0) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    return cus * n;
}

hipError_t launch_attention(int dt, const void *q, const void *k, const void *v, const int32_t *idx,
                            const int32_t *count, const Geo &g, int heads, float scale, const void *cached, void *out,
                            const CopyCfg &cc, void *ws, int grid1, int grid2, hipStream_t st) {
    AttnArgs a{(const uint8_t *)q, (const uint8_t *)k, (const uint8_t *)v, idx, count, (float *)ws,
               (const uint8_t *)cached, (uint8_t *)out, g, cc, heads, scale * 1.4426950408889634f, grid1};
    const int bm = cc.nvec > 0 && ((g.cap + 31) / 32) * 4 <= 64 * 1024 ? ((g.cap + 31) / 32) * 4 : 0;
    if (dt == 1) {
        hipLaunchKernelGGL(k_attn_partial<1>, dim3(grid1), dim3(kAttnThreads), 0, st, a);
        hipLaunchKernelGGL(k_attn_combine<1>, dim3(grid2), dim3(kAttnThreads), bm, st, a);
    } else {
        hipLaunchKernelGGL(k_attn_partial<2>, dim3(grid1), dim3(kAttnThreads), 0, st, a);
        hipLaunchKernelGGL(k_attn_combine<2>, dim3(grid2), dim3(kAttnThreads), bm, st, a);
    }
    return hipGetLastError();
}

}  // namespace sige
