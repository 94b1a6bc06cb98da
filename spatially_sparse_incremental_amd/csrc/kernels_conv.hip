// kernels_conv.hip -- steps 3-5 (gather, block convolution, scatter) and the
// fused layer on gfx950.
//
// SIGE README mirror, "Overview": gather the active blocks (with their halo;
// blocks of a 3x3 stride-1 conv overlap by 2) from the edited activation, stack
// them along the batch dimension, run the convolution on them, and scatter the
// output blocks into the cached output of the original image.  The nubint.ai
// review ("Proposed method") describes the same gather-scatter update.
//
// Layouts: activations NHWC, weights KRSC [c_out][k][k][c_in], block tensors
// [slot][ib][ib][c_in] and [slot][b][b][c_out].  All data moves in 16-byte
// vectors along the channel dimension, which is contiguous in every layout.
// Every memory-bound loop issues a batch of independent 16-byte loads before
// it stores any of them, so a thread waits for memory once per batch rather
// than once per vector.
#include "sige_internal.h"

namespace sige {

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void st16(uint8_t *p, u32x4 v) { *(u32x4 *)p = v; }

// x / d for x * d < 2^31, with m = ceil(2^31 / d) from the host (fast_div_magic)
__device__ __forceinline__ int fdiv(int x, uint32_t m) { return (int)(((uint64_t)(uint32_t)x * m) >> 31); }

__device__ __forceinline__ bool decode_block(const Geo &g, int lin, int &n, int &by, int &bx) {
    if (lin < 0 || lin >= g.cap) return false;
    const int per = g.nby * g.nbx;
    n = lin / per;
    const int r = lin - n * per;
    by = r / g.nbx;
    bx = r - by * g.nbx;
    return true;
}

__device__ __forceinline__ int clamp_count(const int32_t *count, int cap) {
    const int c = *count;
    return c < 0 ? 0 : (c > cap ? cap : c);
}

// Is linear block index `lin` in the ascending list idx[0, cnt)?
__device__ __forceinline__ bool listed(const int32_t *__restrict__ idx, int cnt, int lin) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int v = idx[mid];
        if (v == lin) return true;
        if (v < lin) lo = mid + 1;
        else hi = mid;
    }
    return false;
}

// ---------------------------------------------------------------------------
// Copying the cache outside the listed blocks.  A workgroup first marks every
// listed block in an LDS bitmap (one batched read of idx[0, count)), then copies
// its units.  Unit u = `xw` consecutive pixels of one output row; pixels of
// listed blocks are skipped (the convolution writes them).  CB loads in
// flight per thread.  Without room for the bitmap, a binary search over the ascending
// list decides per block.
// ---------------------------------------------------------------------------

template <int NTHR>
__device__ void build_bitmap(const int32_t *__restrict__ idx, int cnt, int cap, uint32_t *bm) {
    const int words = (cap + 31) >> 5;
    __syncthreads();  // LDS may still be in use by the caller's previous phase
    for (int q = threadIdx.x; q < words; q += NTHR) bm[q] = 0u;
    __syncthreads();
    constexpr int U = 8;
    for (int e0 = threadIdx.x; e0 < cnt; e0 += U * NTHR) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = (e0 + u * NTHR < cnt) ? idx[e0 + u * NTHR] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v[u] >= 0 && v[u] < cap) atomicOr(&bm[v[u] >> 5], 1u << (v[u] & 31));
    }
    __syncthreads();
}

template <int CB, int NTHR>  // CB loads in flight per thread, NTHR threads per workgroup
__device__ void copy_unit(const Geo &g, const int32_t *__restrict__ idx, int cnt, const uint32_t *bm,
                          const uint8_t *__restrict__ cache, uint8_t *__restrict__ out, const CopyCfg &cc, int u,
                          uint8_t *on) {
    const int upr = cc.units_per_row;
    const int row = u / upr;  // n*ho + y
    const int x0 = (u - row * upr) * cc.xw;
    const int x1 = min(g.wo, x0 + cc.xw);
    const int n = row / g.ho, y = row - n * g.ho;
    const int by = y / g.b, j0 = x0 / g.b, j1 = (x1 - 1) / g.b;
    __syncthreads();  // `on` may still be read by the previous unit
    for (int j = threadIdx.x; j <= j1 - j0; j += NTHR) {
        const int lin = (n * g.nby + by) * g.nbx + j0 + j;
        on[j] = bm ? (bm[lin >> 5] >> (lin & 31)) & 1u : (listed(idx, cnt, lin) ? 1 : 0);
    }
    __syncthreads();
    const int row_bytes = cc.row_bytes, vpp = row_bytes >> 4;  // 16-byte vectors per pixel
    const size_t base = ((size_t)row * g.wo + x0) * row_bytes;
    const int nv = (x1 - x0) * vpp;
    for (int v0 = threadIdx.x; v0 < nv; v0 += CB * NTHR) {
        u32x4 r[CB];
        bool go[CB];
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int v = v0 + i * NTHR;
            go[i] = false;
            if (v < nv) {
                const int xl = fdiv(v, cc.m_vpp);
                go[i] = !on[(x0 + xl) / g.b - j0];
                if (go[i]) r[i] = ld16(cache + base + (size_t)v * 16);
            }
        }
#pragma unroll
        for (int i = 0; i < CB; ++i)
            if (go[i]) st16(out + base + (size_t)(v0 + i * NTHR) * 16, r[i]);
    }
}

// ---------------------------------------------------------------------------
// step 3: gather.  One workgroup per listed block (grid-stride over slots).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather(const uint8_t *__restrict__ a, Geo g, int row_bytes, uint32_t m_vpp,
                                                uint32_t m_ib, const int32_t *__restrict__ idx,
                                                const int32_t *__restrict__ count, uint8_t *__restrict__ blocks) {
    constexpr int U = 8;
    const int cnt = clamp_count(count, g.cap);
    const int vpp = row_bytes >> 4;
    const int ib2 = g.ib * g.ib;
    const int nv = ib2 * vpp;
    for (int slot = blockIdx.x; slot < cnt; slot += gridDim.x) {
        int n, by, bx;
        const bool ok = decode_block(g, idx[slot], n, by, bx);
        const int y0 = by * g.b * g.s - g.p, x0 = bx * g.b * g.s - g.p;
        uint8_t *dst = blocks + (size_t)slot * ib2 * row_bytes;
        for (int v0 = threadIdx.x; v0 < nv; v0 += U * 256) {
            u32x4 r[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int v = v0 + i * 256;
                r[i] = u32x4{0u, 0u, 0u, 0u};
                if (v < nv) {
                    const int pix = fdiv(v, m_vpp), cv = v - pix * vpp;
                    const int yy = fdiv(pix, m_ib), xx = pix - yy * g.ib;
                    const int iy = y0 + yy, ix = x0 + xx;
                    if (ok && iy >= 0 && iy < g.h && ix >= 0 && ix < g.w)
                        r[i] = ld16(a + (((size_t)n * g.h + iy) * g.w + ix) * row_bytes + cv * 16);
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (v0 + i * 256 < nv) st16(dst + (size_t)(v0 + i * 256) * 16, r[i]);
        }
    }
}

hipError_t launch_gather(const void *a_edit, int dt, const Geo &g, const int32_t *idx, const int32_t *count,
                         void *blocks, hipStream_t st) {
    const int row_bytes = g.cin * elem_bytes(dt);
    const unsigned grid = (unsigned)(g.cap < 1024 ? g.cap : 1024);
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(256), 0, st, (const uint8_t *)a_edit, g, row_bytes,
                       fast_div_magic(row_bytes >> 4), fast_div_magic(g.ib), idx, count, (uint8_t *)blocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 4 (and the fused layer): implicit GEMM on the matrix cores.
//   M = listed blocks x b*b output pixels (flattened over all blocks, so tiles
//       are not padded per block), N = c_out, K = k*k*c_in.
// A persistent grid of workgroups (8 waves each) walks tiles of 16*MT rows x
// 16*NT output channels.  The 8 waves split each chunk's K steps (tap, one
// 32-channel slice; 16 for fp32) round robin and each accumulates the whole
// tile, so no wave idles on small tiles and every per-wave chain (staging,
// MFMA) is short; the eight partial tiles are summed through LDS at the end.
//   - Weights: a wave's B fragments are used by that wave only, so they go
//     straight from global memory (L2-resident: every tile with the same
//     channel slice reads them) into registers, up to SMAX steps per chunk.
//     They do not depend on the block list: the first chunk's are issued
//     together with the block-index, count and bias reads, so one memory
//     round trip covers all of them.
//   - Input windows: every wave reads every row, so the halo windows of the
//     block slots a tile touches are staged once in LDS, loaded from global
//     memory straight into LDS (global_load_lds_dwordx4: no registers, every
//     load of the stage in flight at once), zero outside the image.
//   - The tile's slots follow from its index alone, so the block indices are
//     read before `count` is known; a tile at or beyond count is dropped.
// MFMA: v_mfma_f32_16x16x32_{bf16,f16} (fp32: four v_mfma_f32_16x16x4_f32).
// Epilogue: partial tiles summed through LDS, bias (prefetched) added, one
// rounding to the storage type, 16-byte row stores into the output image
// (fused) or the block tensor.  With copy_cached, the workgroups that own no
// tile copy the cache outside the listed blocks meanwhile.
// ---------------------------------------------------------------------------
template <int DT>
struct MfmaStep;

template <>
struct MfmaStep<1> {  // bf16: one 16x16x32 MFMA per (16 B of A, 16 B of B)
    static constexpr int KS = 32;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <>
struct MfmaStep<2> {  // fp16
    static constexpr int KS = 32;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};
template <>
struct MfmaStep<0> {  // fp32: four 16x16x4 MFMAs; lane group g holds k = 4g..4g+3
    static constexpr int KS = 16;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
        return c;
    }
};

// Store 8 consecutive channels (fp32: the second 16-byte half only when
// `full`; c_out is a multiple of 4 there, of 8 for 16-bit types).
template <int DT>
__device__ __forceinline__ void store_row8(uint8_t *p, const float *v, bool full) {
    if constexpr (DT == 0) {
        st16(p, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
        if (full)
            st16(p + 16,
                 u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo, hi;
            if constexpr (DT == 1) {
                lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
            } else {
                lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            }
            w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        st16(p, u32x4{w[0], w[1], w[2], w[3]});
    }
}

struct ConvArgs {
    const uint8_t *src;
    const uint8_t *w;
    const float *bias;
    const int32_t *idx;
    const int32_t *count;
    uint8_t *dst;
    const uint8_t *cache;
    Geo g;
    ConvCfg c;
    CopyCfg cc;
};

constexpr int kConvWaves = 8;  // waves per workgroup of the implicit GEMM
constexpr int kConvThreads = 64 * kConvWaves;

// K steps per wave and chunk whose weight fragments a wave holds in registers
template <int NT>
struct Smax {
    static constexpr int v = 10 / NT;
};

template <int DT, int MT, int NT, bool FUSED>
__global__ __launch_bounds__(kConvThreads, 2) void k_conv(ConvArgs a) {
    constexpr int NW = kConvWaves, NTHR = kConvThreads;
    constexpr int ES = elem_bytes(DT);
    constexpr int EPV = 16 / ES;  // elements per 16-byte vector
    constexpr int KS = MfmaStep<DT>::KS;
    constexpr int BM = 16 * MT, BN = 16 * NT;
    constexpr int PSTR = BN + 4;  // padded row of a partial tile (floats)
    constexpr int SMAX = Smax<NT>::v;
    constexpr int VPR = BN / 8;   // 8-channel output vectors per tile row
    constexpr int OPT = (BM * VPR + NTHR - 1) / NTHR;  // output vectors per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // per staged slot: image, input-window origin, output-block origin
    __shared__ int s_n[BM + 1], s_iy[BM + 1], s_ix[BM + 1], s_oy[BM + 1], s_ox[BM + 1];
    __shared__ uint8_t s_on[256];

    const Geo &g = a.g;
    const ConvCfg &c = a.c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib, k2 = g.k * g.k;
    const int mcap = g.cap * b2;            // rows at full capacity (checked on the host)
    const int ntn = (g.cout + BN - 1) / BN;
    const int grid = gridDim.x;
    const int vpc = c.ck / EPV;             // 16-byte vectors per staged pixel
    const int apix = c.a_pix_stride;
    const int kpc = c.ck / KS;              // K steps per tap in a chunk
    const int steps = k2 * kpc;             // K steps per chunk
    const int kl = (lane >> 4) * EPV;       // this lane group's element offset inside a step
    const int cnt_raw = *a.count;           // needed only to drop tiles beyond the list
    int ntiles = -1;
    uint8_t *As = smem;
    float *part = (float *)smem;

    for (int t = blockIdx.x;; t += grid) {
        const int tm = t / ntn, tn = t - tm * ntn;
        const int m0 = tm * BM;
        if (m0 >= mcap) break;
        const int n0 = tn * BN;
        const int s_lo = fdiv(m0, c.m_b2);
        const int s_hi = min(g.cap - 1, fdiv(m0 + BM - 1, c.m_b2));
        const int ns = s_hi - s_lo + 1;
        __syncthreads();  // the previous tile is done with LDS and the slot table
        // Reads that do not depend on the block list go out together: the tile's
        // block indices (before `count` is known), this wave's weight fragments
        // for the first chunk, and the bias.
        int lin = -1;
        if (FUSED && tid < ns) lin = a.idx[s_lo + tid];
        u32x4 bfr[SMAX][NT];
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int stp = wave + NW * j;
            const int tap = stp / kpc, kk = stp - tap * kpc;
            const int cb = kk * KS + kl;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int col = n0 + nt * 16 + (lane & 15);
                bfr[j][nt] = u32x4{0u, 0u, 0u, 0u};
                if (stp < steps && col < g.cout && cb < g.cin)
                    bfr[j][nt] = ld16(a.w + (((size_t)col * k2 + tap) * g.cin + cb) * ES);
            }
        }
        float bias_r[OPT][8];
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int co = n0 + ((tid + o * NTHR) % VPR) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) bias_r[o][j] = (a.bias && co + j < g.cout) ? a.bias[co + j] : 0.f;
        }
        // the list length decides whether this tile exists
        const int cnt = min(max(cnt_raw, 0), g.cap);
        if (ntiles < 0) ntiles = ((cnt * b2 + BM - 1) / BM) * ntn;
        if (t >= ntiles) break;
        const int mrows = cnt * b2;
        if (tid < ns) {
            int n = -1, by = 0, bx = 0;
            if (FUSED) {
                if (!decode_block(g, lin, n, by, bx)) n = -1;
            } else {
                n = 0;  // stacked blocks: positions inside the block tensor only
            }
            s_n[tid] = n;
            s_iy[tid] = by * g.b * g.s - g.p;
            s_ix[tid] = bx * g.b * g.s - g.p;
            s_oy[tid] = by * g.b;
            s_ox[tid] = bx * g.b;
        }
        // LDS byte offset of this lane's row in each M subtile (tap (0,0), channel 0)
        int rb[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int r = m0 + mt * 16 + (lane & 15);
            int off = 0;
            if (r < mrows) {
                const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
                const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
                off = ((slot - s_lo) * ib2 + py * g.s * g.ib + px * g.s) * apix;
            }
            rb[mt] = off;
        }
        f32x4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int nslot = ns * ib2 * (vpc + 1);  // 16-byte LDS slots of the staged windows
        const int nq = (nslot + 63) / 64;        // 64-slot groups, one wave instruction each
        for (int c0 = 0; c0 < g.cin; c0 += c.ck) {
            __syncthreads();  // slot table visible; every wave is done with the previous chunk
            // Input windows straight from global memory into LDS: each wave fills
            // 64 consecutive 16-byte slots per instruction (lane i -> slot base + i;
            // a pixel occupies vpc slots plus one pad slot, left unwritten).
            // Slots outside the image or beyond c_in get zeros from their own lane.
#pragma unroll 2
            for (int q = wave; q < nq; q += NW) {
                const int slot = q * 64 + lane;
                const int P = fdiv(slot, c.m_vpc1), cvv = slot - P * (vpc + 1);
                if (slot < nslot && cvv < vpc) {
                    const int ch = c0 + cvv * EPV;
                    const uint8_t *src = nullptr;
                    if (ch < g.cin) {
                        if (FUSED) {
                            const int ls = fdiv(P, c.m_ib2), pix = P - ls * ib2;
                            const int yy = fdiv(pix, c.m_ib), xx = pix - yy * g.ib;
                            const int n = s_n[ls], iy = s_iy[ls] + yy, ix = s_ix[ls] + xx;
                            if (n >= 0 && iy >= 0 && iy < g.h && ix >= 0 && ix < g.w)
                                src = a.src + ((((size_t)n * g.h + iy) * g.w + ix) * g.cin + ch) * ES;
                        } else {
                            src = a.src + (((size_t)s_lo * ib2 + P) * g.cin + ch) * ES;
                        }
                    }
                    if (src)
                        __builtin_amdgcn_global_load_lds((const void *)src,
                                                         (__attribute__((address_space(3))) void *)(As + q * 1024),
                                                         16, 0, 0);
                    else
                        st16(As + slot * 16, u32x4{0u, 0u, 0u, 0u});
                }
            }
            if (c0 > 0) {  // the next chunk's weight fragments (the first chunk's are in flight)
#pragma unroll
                for (int j = 0; j < SMAX; ++j) {
                    const int stp = wave + NW * j;
                    const int tap = stp / kpc, kk = stp - tap * kpc;
                    const int cb = c0 + kk * KS + kl;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int col = n0 + nt * 16 + (lane & 15);
                        bfr[j][nt] = u32x4{0u, 0u, 0u, 0u};
                        if (stp < steps && col < g.cout && cb < g.cin)
                            bfr[j][nt] = ld16(a.w + (((size_t)col * k2 + tap) * g.cin + cb) * ES);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);  // the LDS loads and the weight fragments have landed
            __syncthreads();
#pragma unroll
            for (int j = 0; j < SMAX; ++j) {
                const int stp = wave + NW * j;
                if (stp < steps) {
                    const int tap = stp / kpc, kk = stp - tap * kpc;
                    const int ky = tap / g.k, kx = tap - ky * g.k;
                    const int aoff = (ky * g.ib + kx) * apix + (kk * KS + kl) * ES;
                    u32x4 av[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) av[mt] = *(const u32x4 *)(As + rb[mt] + aoff);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] = MfmaStep<DT>::run(av[mt], bfr[j][nt], acc[mt][nt]);
                }
            }
        }
        // Sum the 8 waves' partial tiles: waves 4..7 park theirs in LDS, waves 0..3
        // add them in, park the sums, and every thread adds the four.
        // 16x16 accumulator layout: lane l holds rows 4*(l/16)+i, column l%16.
        __syncthreads();  // all waves done reading the staged windows
        const int pw = wave & 3;
        if (wave >= 4) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part[(pw * BM + mt * 16 + (lane >> 4) * 4 + i) * PSTR + nt * 16 + (lane & 15)] =
                            acc[mt][nt][i];
        }
        __syncthreads();
        if (wave < 4) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float *q = &part[(pw * BM + mt * 16 + (lane >> 4) * 4 + i) * PSTR + nt * 16 + (lane & 15)];
                        *q += acc[mt][nt][i];
                    }
        }
        __syncthreads();
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int v = tid + o * NTHR;
            if (v >= BM * VPR) break;
            const int row = v / VPR, col = (v - row * VPR) * 8;
            const int r = m0 + row;
            const int co = n0 + col;
            if (r >= mrows || co >= g.cout) continue;
            const int nval = min(8, g.cout - co);  // 8, or 4 for an fp32 tail
            float sum[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x = bias_r[o][j];
#pragma unroll
                for (int w = 0; w < 4; ++w) x += part[(w * BM + row) * PSTR + col + j];
                sum[j] = x;
            }
            const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
            const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
            if (FUSED) {
                const int ls = slot - s_lo, n = s_n[ls];
                if (n < 0) continue;
                const int y = s_oy[ls] + py, x = s_ox[ls] + px;
                if (y >= g.ho || x >= g.wo) continue;
                store_row8<DT>(a.dst + ((((size_t)n * g.ho + y) * g.wo + x) * g.cout + co) * ES, sum, nval == 8);
            } else {
                store_row8<DT>(a.dst + ((((size_t)slot * g.b + py) * g.b + px) * g.cout + co) * ES, sum, nval == 8);
            }
        }
    }
    if (FUSED && a.cc.units > 0) {
        const int cnt = min(max(cnt_raw, 0), g.cap);
        if (ntiles < 0) ntiles = ((cnt * b2 + BM - 1) / BM) * ntn;
        // Copy units: the workgroups without a tile take up to twice the even
        // share each (they start at once); the rest go round robin to the
        // workgroups with a tile, after it.
        const int units = a.cc.units;
        const int busy = min(ntiles, grid), nfree = grid - busy;
        const int share = (units + grid - 1) / grid;
        const int to_free = nfree > 0 ? min(units, nfree * 2 * share) : 0;
        int first, stride, last;
        if ((int)blockIdx.x >= busy) {
            first = blockIdx.x - busy;
            stride = nfree;
            last = to_free;
        } else {
            first = to_free + blockIdx.x;
            stride = busy;
            last = units;
        }
        if (first < last) {
            uint32_t *bm = nullptr;
            if (((g.cap + 31) >> 5) * 4 <= c.lds_bytes) {  // the GEMM's LDS is free now
                bm = (uint32_t *)smem;
                build_bitmap<NTHR>(a.idx, cnt, g.cap, bm);
            }
            for (int u = first; u < last; u += stride)
                copy_unit<16, NTHR>(g, a.idx, cnt, bm, a.cache, a.dst, a.cc, u, s_on);
        }
    }
}

// Workgroups of `kernel` that fit on one CU with `lds` bytes of dynamic LDS
// (register and LDS limits), from the runtime; cached per kernel and LDS size.
template <typename K>
static int resident_per_cu(K kernel, int lds) {
    struct Entry {
        const void *k;
        int lds, n;
    };
    static thread_local Entry cache[16];
    static thread_local int used = 0;
    for (int i = 0; i < used; ++i)
        if (cache[i].k == (const void *)kernel && cache[i].lds == lds) return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kConvThreads, lds) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    cache[used < 16 ? used++ : 15] = Entry{(const void *)kernel, lds, n};
    return n;
}

// The persistent grid: every resident slot of every CU, and no more (a
// workgroup that cannot start until another ends only delays the kernel).
template <typename K>
static unsigned conv_grid(K kernel, const ConvArgs &args) {
    long grid = (long)args.c.cus * resident_per_cu(kernel, args.c.lds_bytes);
    if (args.c.grid < grid) grid = args.c.grid;  // the host's cap: tiles at full capacity
    if (grid > 8) grid = grid / 8 * 8;           // keep tile t on XCD t % 8 across passes
    return (unsigned)(grid > 0 ? grid : 1);
}

template <int DT, int MT, int NT>
static hipError_t launch_conv_t(int fused, const ConvArgs &args, hipStream_t st) {
    if (fused) {
        auto k = k_conv<DT, MT, NT, true>;
        hipLaunchKernelGGL(k, dim3(conv_grid(k, args)), dim3(kConvThreads), args.c.lds_bytes, st, args);
    } else {
        auto k = k_conv<DT, MT, NT, false>;
        hipLaunchKernelGGL(k, dim3(conv_grid(k, args)), dim3(kConvThreads), args.c.lds_bytes, st, args);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_conv_dt(int fused, const ConvArgs &args, hipStream_t st) {
    const int key = args.c.mt * 10 + args.c.nt;
    switch (key) {
    case 42: return launch_conv_t<DT, 4, 2>(fused, args, st);
    case 41: return launch_conv_t<DT, 4, 1>(fused, args, st);
    case 22: return launch_conv_t<DT, 2, 2>(fused, args, st);
    case 44: return launch_conv_t<DT, 4, 4>(fused, args, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                       const int32_t *count, void *dst, const void *cache, const Geo &g, const ConvCfg &cfg,
                       const CopyCfg &cc, hipStream_t st) {
    ConvArgs args{(const uint8_t *)src, (const uint8_t *)w, bias, idx, count, (uint8_t *)dst,
                  (const uint8_t *)cache, g, cfg, cc};
    switch (dt) {
    case 0: return launch_conv_dt<0>(fused, args, st);
    case 1: return launch_conv_dt<1>(fused, args, st);
    default: return launch_conv_dt<2>(fused, args, st);
    }
}

// ---------------------------------------------------------------------------
// step 5: scatter.  A persistent grid: each workgroup first writes listed
// blocks' valid pixels (slot = workgroup, + grid, ...), then copy units
// (unit u to workgroup (count + u) % grid) when copy_cached.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scatter(const uint8_t *__restrict__ ob, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ count, Geo g, uint32_t m_b,
                                                 const uint8_t *__restrict__ cache, uint8_t *__restrict__ out,
                                                 CopyCfg cc, int bm_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ uint8_t s_on[256];
    constexpr int U = 8;
    const int cnt = clamp_count(count, g.cap);
    const int grid = gridDim.x;
    const int row_bytes = cc.row_bytes, vpp = row_bytes >> 4, b2 = g.b * g.b;
    const int nv = b2 * vpp;
    for (int slot = blockIdx.x; slot < cnt; slot += grid) {
        int n, by, bx;
        if (!decode_block(g, idx[slot], n, by, bx)) continue;
        for (int v0 = threadIdx.x; v0 < nv; v0 += U * 256) {
            u32x4 r[U];
            size_t dst[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int v = v0 + i * 256;
                dst[i] = ~(size_t)0;
                if (v < nv) {
                    const int pix = fdiv(v, cc.m_vpp), cvv = v - pix * vpp;
                    const int py = fdiv(pix, m_b), px = pix - py * g.b;
                    const int y = by * g.b + py, x = bx * g.b + px;
                    if (y < g.ho && x < g.wo) {
                        r[i] = ld16(ob + ((size_t)slot * b2 + pix) * row_bytes + cvv * 16);
                        dst[i] = (((size_t)n * g.ho + y) * g.wo + x) * row_bytes + cvv * 16;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (dst[i] != ~(size_t)0) st16(out + dst[i], r[i]);
        }
    }
    if (cc.units > 0) {
        int u0 = ((int)blockIdx.x - cnt) % grid;
        if (u0 < 0) u0 += grid;
        if (u0 < cc.units) {
            uint32_t *bm = nullptr;
            if (bm_bytes > 0) {
                bm = (uint32_t *)smem;
                build_bitmap<256>(idx, cnt, g.cap, bm);
            }
            for (int u = u0; u < cc.units; u += grid) copy_unit<16, 256>(g, idx, cnt, bm, cache, out, cc, u, s_on);
        }
    }
}

hipError_t launch_scatter(int dt, const void *out_blocks, const int32_t *idx, const int32_t *count, const Geo &g,
                          const void *cached, void *out, int grid, const CopyCfg &cc, hipStream_t st) {
    (void)dt;
    // bitmap of listed blocks for the copy, when it fits in 64 KiB of LDS
    const long bm = cc.units > 0 ? ((long)(g.cap + 31) / 32) * 4 : 0;
    const int bm_bytes = bm <= 64 * 1024 ? (int)bm : 0;
    hipLaunchKernelGGL(k_scatter, dim3(grid), dim3(256), bm_bytes, st, (const uint8_t *)out_blocks, idx, count, g,
                       fast_div_magic(g.b), (const uint8_t *)cached, (uint8_t *)out, cc, bm_bytes);
    return hipGetLastError();
}

}  // namespace sige
