// kernels_attn.hip -- query-pruned self-attention on gfx950.
//
// nubint.ai review, "Proposed method": attention layers are handled by
// pruning the queries of unedited tokens, so the attention work scales with
// the edited area.  Queries: the tokens of the listed blocks (block x block
// tokens of the h x w grid); keys and values: every token of the same image.
//
// Split over keys (as in flash decoding): a work item is (128-query tile of one
// image, head, key split).  Its 4 waves own 32 queries each (two groups of 16
// that share every K and V fragment) and run an online softmax over the
// split's keys, 64 at a time, with both products on the matrix cores
// (v_mfma_f32_16x16x32_{f16,bf16}).  The key tiles of a split
// are staged kAttnChunk at a time (K straight into LDS, V through registers
// and written transposed), all loads of a chunk in flight together, so a
// split of up to kAttnChunk tiles costs one memory round trip:
//   S^T  = K Q^T      A = key rows from LDS, B = this wave's Q^T fragments (registers)
//   O^T += V^T P^T    A = rows of a transposed V tile in LDS, B = P^T taken from S^T
// In S^T's accumulator layout a lane holds one query and 4 keys of each
// 16-key subtile.  Two subtiles packed give a B fragment of the second product
// (the order of k inside one MFMA is free, as long as A uses the same order),
// and every softmax statistic of a query lives in the lanes l, l^16, l^32,
// l^48.  O^T's accumulators hold the same query per lane, so the rescale by
// exp(m_old - m_new) needs no lane exchange; the max and sum over the four
// k groups are two lane swaps (v_permlane16_swap, v_permlane32_swap).  Each item leaves (max, sum,
// unnormalised O) in the caller's workspace; a second kernel combines the
// splits, writes the queries' outputs and copies the cache elsewhere.
//
// Query tiles never straddle two images: each image's listed blocks are
// padded to whole 128-row tiles (per-image block counts come from one pass
// over the list in every workgroup).
#include <type_traits>

#include "device_common.h"

namespace sige {

constexpr int kAttnD = 64;          // head dim
constexpr int kAttnKT = 64;         // keys per LDS tile
constexpr int kAttnQW = 32;         // queries per wave (two groups of 16)
constexpr int kAttnQT = 4 * kAttnQW;  // queries per work item
static_assert(kAttnQT == kAttnQueryTile, "query tile");
constexpr int kAttnThreads = 256;
constexpr int kAttnMaxImages = 8;
constexpr int kAttnWsRow = kAttnD + 4;  // floats per query in the workspace: O^T column, max, sum, pad
constexpr int kAttnKPitch = kAttnD + 8;   // halves per key row of the K tile in LDS
constexpr int kAttnVPitch = kAttnKT + 8;  // halves per d row of the transposed V tile
constexpr int kAttnChunk = 4;             // key tiles staged in LDS per round trip
constexpr int kAttnKTile = kAttnKT * kAttnKPitch;
constexpr int kAttnVTile = kAttnD * kAttnVPitch;
constexpr int kAttnPartialLds = kAttnChunk * (kAttnKTile + kAttnVTile) * 2;  // bytes of dynamic LDS

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

// Two floats rounded to nearest even and packed (one v_cvt_pk_{bf16,f16}_f32).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    if constexpr (DT == 1)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}


// Max and sum over the lanes l, l^16, l^32, l^48 (the four k groups that hold
// one query's statistics): each lane swap leaves a lane's own value and its
// partner's in the two outputs, in either order.
__device__ __forceinline__ float qmax(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float qsum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Per-image bookkeeping of the listed blocks, in LDS: first slot and first
// padded tile of every image, and the total number of tiles.
struct AttnTiles {
    int first_slot[kAttnMaxImages + 1];
    int first_tile[kAttnMaxImages + 1];
};

__device__ void attn_tiles(const Geo &g, const int32_t *__restrict__ idx, int cnt, AttnTiles *t, int *cnt_img) {
    const int per = g.nby * g.nbx, b2 = g.b * g.b;
    if (g.n == 1) {  // one image: every slot is its own, no pass over the list
        if (threadIdx.x == 0) {
            t->first_slot[0] = t->first_tile[0] = 0;
            t->first_slot[1] = cnt;
            t->first_tile[1] = (cnt * b2 + kAttnQT - 1) / kAttnQT;
        }
        __syncthreads();
        return;
    }
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

// Keys per split: enough splits for every co-resident workgroup to hold a work
// item, at most 16, and none shorter than one staged chunk of key tiles.
__device__ __forceinline__ void attn_split(int items, int nkt, int grid, int &S, int &ktp) {
    const int one_chunk = (nkt + kAttnChunk - 1) / kAttnChunk;
    S = items > 0 ? grid / items : 1;
    S = max(1, min(S, min(16, one_chunk)));
    ktp = (nkt + S - 1) / S;
}

// The list entry behind query row `row` of a tile of image n is idx[slot]; the
// token it names (or -1: a row past the image's rows, an invalid entry, a
// pixel outside the grid).
__device__ __forceinline__ int attn_slot(const Geo &g, const AttnTiles &t, int n, int row) {
    const int b2 = g.b * g.b;
    const int nrows = (t.first_slot[n + 1] - t.first_slot[n]) * b2;
    const int slot = t.first_slot[n] + min(row, max(nrows - 1, 0)) / b2;
    return min(max(slot, 0), g.cap - 1);
}

__device__ __forceinline__ int attn_token_of(const Geo &g, const AttnTiles &t, int n, int row, int ent) {
    const int b2 = g.b * g.b;
    const int nrows = (t.first_slot[n + 1] - t.first_slot[n]) * b2;
    if (row >= nrows) return -1;
    const int pix = row - (row / b2) * b2;
    int nn, by, bx;
    if (!decode_block(g, ent, nn, by, bx) || nn != n) return -1;
    const int y = by * g.b + pix / g.b, x = bx * g.b + pix % g.b;
    if (y >= g.h || x >= g.w) return -1;
    return y * g.w + x;
}

template <int DT>
__global__ __launch_bounds__(kAttnThreads, 2) void k_attn_partial(AttnArgs a) {
    constexpr int D = kAttnD, KT = kAttnKT;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *const Ks = lds;                            // kAttnChunk K tiles, key rows
    uint16_t *const Vt = lds + kAttnChunk * kAttnKTile;  // kAttnChunk V tiles, transposed
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
    attn_split(items, nkt, a.grid1, S, ktp);
    const int ql = lane & 15, kg = lane >> 4;  // this lane's query (B/C column) and k group
    constexpr int G = kAttnQW / 16;             // 16-query groups per wave
    for (int p = blockIdx.x; p < items * S; p += gridDim.x) {
        const int split = p % S, item = p / S;
        const int head = item % a.heads, tile = item / a.heads;
        int n = 0;
        while (n + 1 < g.n && tiles.first_tile[n + 1] <= tile) ++n;
        const size_t img = (size_t)n * L;
        const int row0 = (tile - tiles.first_tile[n]) * kAttnQT + wave * kAttnQW + ql;  // group q: row0 + 16 q
        const int kt0 = split * ktp, kt1 = min(nkt, kt0 + ktp);
        __syncthreads();  // every wave is done with the staged tiles of the previous item
        // The list entries of this lane's queries first, then the first two key
        // tiles (K and V rows into registers), then the Q fragments; each tile is
        // written to LDS once its registers arrive, and the tile two ahead is
        // requested into them while this one is computed (keys past the end are
        // clamped and their values never used).  Plain loads, not LDS DMA: the
        // compiler's waits for registers are exact, while any LDS access after
        // a DMA load waits for all of them.
        int ent[G];
#pragma unroll
        for (int q = 0; q < G; ++q) ent[q] = a.idx[attn_slot(g, tiles, n, row0 + 16 * q)];
        __builtin_amdgcn_sched_barrier(0);
        u32x4 kv[2][2], vv[2][2];  // the two tiles in flight: 16 bytes of a K and a V row, twice per thread
        auto issue_tile = [&](int c0, int t) __attribute__((always_inline)) {
            // thread cx takes key cx % 64, channels 8 (cx / 64) .. of it, cx = tid, tid + 256
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int cx = tid + i * kAttnThreads, key = cx & 63, dc = cx >> 6;
                const size_t off = ((img + min((c0 + t) * KT + key, L - 1)) * C + head * D + dc * 8) * 2;
                kv[t & 1][i] = ld16(a.k + off);
                vv[t & 1][i] = ld16(a.v + off);
            }
        };
        // tile t's registers into LDS slot t: K rows as they are, V transposed
        // (a wave takes one 8-channel slice of 64 keys: its 16-bit writes go to 64
        // consecutive halves of each row of V^T)
        auto stage_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int cx = tid + i * kAttnThreads, key = cx & 63, dc = cx >> 6;
                *(u32x4 *)(Ks + t * kAttnKTile + key * kAttnKPitch + dc * 8) = kv[t & 1][i];
                uint16_t *vt = Vt + t * kAttnVTile + key;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vt[(dc * 8 + 2 * e) * kAttnVPitch] = (uint16_t)(vv[t & 1][i][e] & 0xFFFFu);
                    vt[(dc * 8 + 2 * e + 1) * kAttnVPitch] = (uint16_t)(vv[t & 1][i][e] >> 16);
                }
            }
        };
        // the first chunk's first two tiles (unconditionally: keys past the end
        // are clamped), then the Q fragments
        issue_tile(kt0, 0);
        issue_tile(kt0, 1);
        __builtin_amdgcn_sched_barrier(0);
        // this wave's Q^T fragments: query ql of group q, d = 32 * ks + 8 * kg + (0..7)
        u32x4 qf[G][2];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int tok = attn_token_of(g, tiles, n, row0 + 16 * q, ent[q]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                qf[q][ks] = ld16(a.q + ((img + (tok < 0 ? 0 : tok)) * C + head * D + ks * 32 + kg * 8) * 2);
        }
        f32x4 oT[G][4];
        float m_run[G], l_run[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int m = 0; m < 4; ++m) oT[q][m] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run[q] = -INFINITY;
            l_run[q] = 0.f;
        }
        // tile t of the chunk at key tile c0, from LDS slot t
        auto compute_tile = [&](int c0, int t) __attribute__((always_inline)) {
            const int j0 = (c0 + t) * KT;
            const uint16_t *kb = Ks + t * kAttnKTile, *vb = Vt + t * kAttnVTile;
            // every fragment of the tile requested at once: K rows for S^T,
            // rows of V^T for O^T (keys 32*pr + 4*kg + (0..3) and 32*pr + 16 + 4*kg + (0..3));
            // both query groups share them
            u32x4 kf[4][2], vf[2][4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    kf[sub][ks] = *(const u32x4 *)(kb + (sub * 16 + ql) * kAttnKPitch + ks * 32 + kg * 8);
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint16_t *vr = vb + (m * 16 + ql) * kAttnVPitch + pr * 32 + kg * 4;
                    const uint2 lo = *(const uint2 *)vr, hi = *(const uint2 *)(vr + 16);
                    vf[pr][m] = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
            // S^T = K Q^T for the 4 subtiles of 16 keys
            f32x4 sT[G][4];
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int sub = 0; sub < 4; ++sub) {
                    sT[q][sub] = AttnMfma<DT>::run(kf[sub][0], qf[q][0], f32x4{0.f, 0.f, 0.f, 0.f});
                    sT[q][sub] = AttnMfma<DT>::run(kf[sub][1], qf[q][1], sT[q][sub]);
                }
            // online softmax for query ql of each group: keys 16 * sub + 4 * kg + i
            // of this tile.  Scores stay unscaled (the scale is positive, so the
            // max commutes with it); only a tile past the last key masks.
            if (j0 + KT > L) {
#pragma unroll
                for (int q = 0; q < G; ++q)
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (j0 + sub * 16 + kg * 4 + i >= L) sT[q][sub][i] = -INFINITY;
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                float mt = -INFINITY;
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sT[q][sub][i]);
                const float m_new = fmaxf(m_run[q], a.scale_log2 * qmax(mt));
                if (__ballot(m_new != m_run[q])) {  // some query's max moved: rescale the wave's sums
                    const float alpha = __builtin_amdgcn_exp2f(m_run[q] - m_new);
                    l_run[q] *= alpha;
#pragma unroll
                    for (int m = 0; m < 4; ++m) oT[q][m] *= alpha;
                    m_run[q] = m_new;
                }
                float ps = 0.f;
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = __builtin_amdgcn_exp2f(fmaf(sT[q][sub][i], a.scale_log2, -m_new));
                        sT[q][sub][i] = e;
                        ps += e;
                    }
                l_run[q] += qsum(ps);
            }
            // O^T += V^T P^T, 32 keys per MFMA; P^T straight from S^T's accumulators
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const u32x4 pb = u32x4{pack2<DT>(sT[q][2 * pr][0], sT[q][2 * pr][1]),
                                           pack2<DT>(sT[q][2 * pr][2], sT[q][2 * pr][3]),
                                           pack2<DT>(sT[q][2 * pr + 1][0], sT[q][2 * pr + 1][1]),
                                           pack2<DT>(sT[q][2 * pr + 1][2], sT[q][2 * pr + 1][3])};
#pragma unroll
                    for (int m = 0; m < 4; ++m) oT[q][m] = AttnMfma<DT>::run(vf[pr][m], pb, oT[q][m]);
                }
        };
        // A chunk of nt key tiles whose first two are requested: each tile is
        // written to LDS, then the tile two ahead is requested into its registers
        // (the next chunk's first two from the third and fourth on) while it is
        // computed.  Full chunks are straight-line code, so the compiler's waits
        // for the registers are exact.
        auto run_chunk = [&](int c0, int nt, auto full_tag) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
            for (int t = 0; t < kAttnChunk; ++t) {
                if (!FULL && t >= nt) continue;
                stage_tile(t);
                __syncthreads();  // tile t is in LDS for every wave
                if (FULL ? t + 2 < kAttnChunk : t + 2 < nt)
                    issue_tile(c0, t + 2);
                else if (c0 + kAttnChunk < kt1 && t + 2 - kAttnChunk >= 0 && (FULL || nt == kAttnChunk))
                    issue_tile(c0 + kAttnChunk, t + 2 - kAttnChunk);
                compute_tile(c0, t);
            }
        };
        for (int c0 = kt0; c0 < kt1; c0 += kAttnChunk) {
            const int nt = min(kAttnChunk, kt1 - c0);
            if (nt == kAttnChunk)
                run_chunk(c0, nt, std::true_type{});
            else
                run_chunk(c0, nt, std::false_type{});
        }
        // this item's partial: unnormalised O^T column of each query, then max and sum
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float *wp = a.ws + ((size_t)p * kAttnQT + wave * kAttnQW + 16 * q + ql) * kAttnWsRow;
#pragma unroll
            for (int m = 0; m < 4; ++m) __builtin_nontemporal_store(oT[q][m], (f32x4 *)(wp + m * 16 + kg * 4));
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            if (kg == 0) __builtin_nontemporal_store(f32x2{m_run[q], l_run[q]}, (f32x2 *)(wp + D));
        }
    }
}

// Combine the key splits of every query and head and write the outputs; the
// workgroups past the ones with combine work copy the cache elsewhere
// (copy_cached).  Four neighbouring lanes share one (query, 8 channels): lane
// r takes the splits r, r + 4, ..., all of its partials requested at once, and
// the four merge by lane exchanges, so the partials' bytes are spread over 4x
// the workgroups of one lane per output.
template <int DT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_combine(AttnArgs a) {
    constexpr int D = kAttnD, SL = 4, SMAX = 16 / SL;  // lanes per output; splits per lane
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
    // work unit: (item, query, 8-channel chunk, split lane); the SL lanes of a
    // unit are consecutive, so every condition below is uniform over them
    const long total = (long)items * kAttnQT * (D / 8) * SL;
    for (long u = (long)blockIdx.x * kAttnThreads + threadIdx.x; u < total; u += (long)gridDim.x * kAttnThreads) {
        const int r = (int)(u % SL);
        const long v = u / SL;
        const int dc = (int)(v % (D / 8));
        const int qi = (int)((v / (D / 8)) % kAttnQT);
        const int item = (int)(v / ((long)(D / 8) * kAttnQT));
        const int head = item % a.heads, tile = item / a.heads;
        int n = 0;
        while (n + 1 < g.n && tiles.first_tile[n + 1] <= tile) ++n;
        const int row = (tile - tiles.first_tile[n]) * kAttnQT + qi;
        const int ent = a.idx[attn_slot(g, tiles, n, row)];
        float2 ml[SMAX];
        f32x4 x0[SMAX], x1[SMAX];
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int s = r + SL * j;
            if (s < S) {
                const float *wp = a.ws + ((size_t)(item * S + s) * kAttnQT + qi) * kAttnWsRow;
                ml[j] = *(const float2 *)(wp + D);
                x0[j] = *(const f32x4 *)(wp + dc * 8);
                x1[j] = *(const f32x4 *)(wp + dc * 8 + 4);
            } else {
                ml[j] = float2{-INFINITY, 0.f};
                x0[j] = x1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        const int tok = attn_token_of(g, tiles, n, row, ent);
        if (tok < 0) continue;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) mx = fmaxf(mx, ml[j].x);
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        float sum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const float f = ml[j].x == -INFINITY ? 0.f : exp2f(ml[j].x - mx);
            sum += f * ml[j].y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] += f * x0[j][e];
                o[4 + e] += f * x1[j][e];
            }
        }
#pragma unroll
        for (int sh = 1; sh < SL; sh *= 2) {
            sum += __shfl_xor(sum, sh);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], sh);
        }
        if (r != 0) continue;
        const float inv = 1.f / sum;
        u32x4 res;
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = pack2<DT>(o[2 * e] * inv, o[2 * e + 1] * inv);
        st16(a.out + (((size_t)n * L + tok) * C + head * D + dc * 8) * 2, res);
    }
    if (a.cc.nvec > 0) {
        const int busy = (int)((total + kAttnThreads - 1) / kAttnThreads);
        const int c0 = busy < (int)gridDim.x / 2 ? busy : 0;  // the copy goes to the idle workgroups
        if ((int)blockIdx.x < c0) return;
        const int i = blockIdx.x - c0, nw = gridDim.x - c0;
        const long long lo = split_point(a.cc.nvec, i, nw), hi = split_point(a.cc.nvec, i + 1, nw);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_partial<2>, kAttnThreads, kAttnPartialLds) !=
            hipSuccess ||
        n < 1) {
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
        hipLaunchKernelGGL(k_attn_partial<1>, dim3(grid1), dim3(kAttnThreads), kAttnPartialLds, st, a);
        hipLaunchKernelGGL(k_attn_combine<1>, dim3(grid2), dim3(kAttnThreads), bm, st, a);
    } else {
        hipLaunchKernelGGL(k_attn_partial<2>, dim3(grid1), dim3(kAttnThreads), kAttnPartialLds, st, a);
        hipLaunchKernelGGL(k_attn_combine<2>, dim3(grid2), dim3(kAttnThreads), bm, st, a);
    }
    return hipGetLastError();
}

}  // namespace sige
