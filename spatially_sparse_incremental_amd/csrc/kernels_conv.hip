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
#include "sige_internal.h"

namespace sige {

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void st16(uint8_t *p, u32x4 v) { *(u32x4 *)p = v; }

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

// Copy unit u: one segment of `xw` pixels of one output row.  Pixels that lie
// in a listed block are skipped (another workgroup writes them).
__device__ void copy_unit(const Geo &g, const int32_t *__restrict__ idx, int cnt, const uint8_t *__restrict__ cache,
                          uint8_t *__restrict__ out, int xw, int u, int row_bytes) {
    __shared__ uint8_t on[256];
    const int upr = (g.wo + xw - 1) / xw;
    const int row = u / upr;  // n*ho + y
    const int x0 = (u - row * upr) * xw;
    const int x1 = min(g.wo, x0 + xw);
    const int n = row / g.ho, y = row - n * g.ho;
    const int by = y / g.b, j0 = x0 / g.b, j1 = (x1 - 1) / g.b;
    for (int j = threadIdx.x; j <= j1 - j0; j += blockDim.x)
        on[j] = listed(idx, cnt, (n * g.nby + by) * g.nbx + j0 + j) ? 1 : 0;
    __syncthreads();
    const int vpp = row_bytes >> 4;  // 16-byte vectors per pixel
    const size_t base = ((size_t)row * g.wo) * row_bytes;
    const int nv = (x1 - x0) * vpp;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        const int x = x0 + v / vpp;
        if (on[x / g.b - j0]) continue;
        const size_t off = base + (size_t)x * row_bytes + (size_t)(v % vpp) * 16;
        st16(out + off, ld16(cache + off));
    }
}

// ---------------------------------------------------------------------------
// step 3: gather.  One workgroup per listed block (grid-stride over slots).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather(const uint8_t *__restrict__ a, Geo g, int row_bytes,
                                                const int32_t *__restrict__ idx, const int32_t *__restrict__ count,
                                                uint8_t *__restrict__ blocks) {
    const int cnt = clamp_count(count, g.cap);
    const int vpp = row_bytes >> 4;
    const int ib2 = g.ib * g.ib;
    for (int slot = blockIdx.x; slot < cnt; slot += gridDim.x) {
        int n, by, bx;
        const bool ok = decode_block(g, idx[slot], n, by, bx);
        const int y0 = by * g.b * g.s - g.p, x0 = bx * g.b * g.s - g.p;
        uint8_t *dst = blocks + (size_t)slot * ib2 * row_bytes;
        for (int v = threadIdx.x; v < ib2 * vpp; v += blockDim.x) {
            const int pix = v / vpp, cv = v - pix * vpp;
            const int yy = pix / g.ib, xx = pix - yy * g.ib;
            const int iy = y0 + yy, ix = x0 + xx;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (ok && iy >= 0 && iy < g.h && ix >= 0 && ix < g.w)
                val = ld16(a + (((size_t)n * g.h + iy) * g.w + ix) * row_bytes + cv * 16);
            st16(dst + (size_t)pix * row_bytes + cv * 16, val);
        }
    }
}

hipError_t launch_gather(const void *a_edit, int dt, const Geo &g, const int32_t *idx, const int32_t *count,
                         void *blocks, hipStream_t st) {
    const int row_bytes = g.cin * elem_bytes(dt);
    const unsigned grid = (unsigned)(g.cap < 1024 ? g.cap : 1024);
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(256), 0, st, (const uint8_t *)a_edit, g, row_bytes, idx, count,
                       (uint8_t *)blocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 4 (and the fused layer): implicit GEMM on the matrix cores.
//   M = listed blocks x b*b output pixels (flattened over all blocks, so tiles
//       are not padded per block), N = c_out, K = k*k*c_in.
// A workgroup (4 waves) owns a tile of 16*MT rows x 16*NT output channels.  Per
// chunk of `ck` input channels it stages into LDS the input windows of the
// block slots its rows touch (16-byte vectors; zero outside the image) and the
// matching k*k*ck slice of the weights of its NT*16 channels.  The 4 waves then
// split the chunk's K steps (tap, 32-channel slice) round robin, each
// accumulating the whole tile with v_mfma_f32_16x16x32_{bf16,f16} (fp32:
// v_mfma_f32_16x16x4_f32, 4 per 16-channel slice), so no wave idles on small
// tiles.  The four partial tiles are summed through LDS, bias added, rounded
// once to the storage type and written as 16-byte row vectors.
// Fused mode stages from A_edited directly and writes into the output image;
// workgroups after the GEMM ones copy the cached output outside listed blocks.
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
};

template <int DT, int MT, int NT, bool FUSED>
__global__ __launch_bounds__(256) void k_conv(ConvArgs a) {
    constexpr int ES = elem_bytes(DT);
    constexpr int EPV = 16 / ES;  // elements per 16-byte vector
    constexpr int KS = MfmaStep<DT>::KS;
    constexpr int BM = 16 * MT, BN = 16 * NT;
    constexpr int PSTR = BN + 4;  // padded row of a partial tile (floats)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int sidx[BM + 1];

    const Geo &g = a.g;
    const int cnt = clamp_count(a.count, g.cap);
    if (FUSED && (int)blockIdx.x >= a.c.compute_grid) {
        copy_unit(g, a.idx, cnt, a.cache, a.dst, a.c.copy_xw, blockIdx.x - a.c.compute_grid, g.cout * ES);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib, k2 = g.k * g.k;
    const long mrows = (long)cnt * b2;
    const int mtiles = (int)((mrows + BM - 1) / BM);
    const int ntn = (g.cout + BN - 1) / BN;
    const int ntiles = mtiles * ntn;
    const int ck = a.c.ck, vpc = ck / EPV;  // 16-byte vectors per staged pixel
    const int apix = a.c.a_pix_stride, brow = a.c.b_row_stride;
    uint8_t *As = smem;
    uint8_t *Bs = smem + a.c.a_bytes;
    float *part = (float *)smem;

    for (int t = blockIdx.x; t < ntiles; t += a.c.compute_grid) {
        // consecutive workgroups take consecutive N tiles of one M tile, so the
        // round-robin placement over the 8 XCDs keeps each XCD on few weight slices
        const int tm = t / ntn, tn = t - tm * ntn;
        const long m0 = (long)tm * BM;
        const int n0 = tn * BN;
        const int s_lo = (int)(m0 / b2);
        const int s_hi = (int)min((long)cnt - 1, (m0 + BM - 1) / b2);
        const int ns = s_hi - s_lo + 1;
        __syncthreads();  // previous tile's partial sums and sidx are consumed
        if (FUSED)
            for (int i = tid; i < ns; i += 256) sidx[i] = a.idx[s_lo + i];

        // LDS byte offset of this lane's row in each M subtile (tap (0,0), channel 0)
        int rb[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const long r = m0 + mt * 16 + (lane & 15);
            int off = 0;
            if (r < mrows) {
                const int slot = (int)(r / b2), pix = (int)(r - (long)slot * b2);
                const int py = pix / g.b, px = pix - py * g.b;
                off = ((slot - s_lo) * ib2 + py * g.s * g.ib + px * g.s) * apix;
            }
            rb[mt] = off;
        }
        f32x4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int c0 = 0; c0 < g.cin; c0 += ck) {
            __syncthreads();  // sidx visible; previous chunk fully read
            // stage the input windows of slots [s_lo, s_hi]
            const int na = ns * ib2 * vpc;
            for (int v = tid; v < na; v += 256) {
                const int ls = v / (ib2 * vpc);
                const int rem = v - ls * ib2 * vpc;
                const int pix = rem / vpc, cv = rem - pix * vpc;
                const int c = c0 + cv * EPV;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (c < g.cin) {
                    const int yy = pix / g.ib, xx = pix - yy * g.ib;
                    if (FUSED) {
                        int n, by, bx;
                        if (decode_block(g, sidx[ls], n, by, bx)) {
                            const int iy = by * g.b * g.s - g.p + yy, ix = bx * g.b * g.s - g.p + xx;
                            if (iy >= 0 && iy < g.h && ix >= 0 && ix < g.w)
                                val = ld16(a.src + ((((size_t)n * g.h + iy) * g.w + ix) * g.cin + c) * ES);
                        }
                    } else {
                        val = ld16(a.src + ((((size_t)(s_lo + ls) * g.ib + yy) * g.ib + xx) * g.cin + c) * ES);
                    }
                }
                st16(As + (ls * ib2 + pix) * apix + cv * 16, val);
            }
            // stage the weight slice [n0, n0+BN) x k*k taps x [c0, c0+ck)
            const int nb = BN * k2 * vpc;
            for (int v = tid; v < nb; v += 256) {
                const int r = v / (k2 * vpc);
                const int rem = v - r * k2 * vpc;
                const int tap = rem / vpc, cv = rem - tap * vpc;
                const int co = n0 + r, c = c0 + cv * EPV;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (co < g.cout && c < g.cin) val = ld16(a.w + (((size_t)co * k2 + tap) * g.cin + c) * ES);
                st16(Bs + r * brow + (tap * ck + cv * EPV) * ES, val);
            }
            __syncthreads();
            const int kpc = ck / KS;  // K steps per tap in this chunk
            const int steps = k2 * kpc;
            const int kl = (lane >> 4) * EPV;  // this lane group's element offset inside a step
            for (int stp = wave; stp < steps; stp += 4) {
                const int tap = stp / kpc, kk = stp - tap * kpc;
                const int ky = tap / g.k, kx = tap - ky * g.k;
                const int aoff = (ky * g.ib + kx) * apix + (kk * KS + kl) * ES;
                const int boff = (tap * ck + kk * KS + kl) * ES;
                u32x4 av[MT], bv[NT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = *(const u32x4 *)(As + rb[mt] + aoff);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bv[nt] = *(const u32x4 *)(Bs + (nt * 16 + (lane & 15)) * brow + boff);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = MfmaStep<DT>::run(av[mt], bv[nt], acc[mt][nt]);
            }
        }
        __syncthreads();  // all waves done reading the staged chunk
        // 16x16 accumulator layout: lane l holds rows 4*(l/16)+i, column l%16
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    part[(wave * BM + mt * 16 + (lane >> 4) * 4 + i) * PSTR + nt * 16 + (lane & 15)] = acc[mt][nt][i];
        __syncthreads();
        constexpr int VPR = BN / 8;  // 8-channel output vectors per tile row
        for (int v = tid; v < BM * VPR; v += 256) {
            const int row = v / VPR, col = (v - row * VPR) * 8;
            const long r = m0 + row;
            const int co = n0 + col;
            if (r >= mrows || co >= g.cout) continue;
            const int nval = min(8, g.cout - co);  // 8, or 4 for an fp32 tail
            float s[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x = (a.bias && j < nval) ? a.bias[co + j] : 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) x += part[(w * BM + row) * PSTR + col + j];
                s[j] = x;
            }
            const int slot = (int)(r / b2), pix = (int)(r - (long)slot * b2);
            const int py = pix / g.b, px = pix - py * g.b;
            if (FUSED) {
                int n, by, bx;
                if (!decode_block(g, sidx[slot - s_lo], n, by, bx)) continue;
                const int y = by * g.b + py, x = bx * g.b + px;
                if (y >= g.ho || x >= g.wo) continue;
                store_row8<DT>(a.dst + ((((size_t)n * g.ho + y) * g.wo + x) * g.cout + co) * ES, s, nval == 8);
            } else {
                store_row8<DT>(a.dst + ((((size_t)slot * g.b + py) * g.b + px) * g.cout + co) * ES, s, nval == 8);
            }
        }
    }
}

template <int DT, int MT, int NT>
static hipError_t launch_conv_t(int fused, const ConvArgs &args, hipStream_t st) {
    const unsigned grid = (unsigned)(args.c.compute_grid + (fused ? args.c.copy_units : 0));
    if (fused)
        hipLaunchKernelGGL((k_conv<DT, MT, NT, true>), dim3(grid), dim3(256), args.c.lds_bytes, st, args);
    else
        hipLaunchKernelGGL((k_conv<DT, MT, NT, false>), dim3(grid), dim3(256), args.c.lds_bytes, st, args);
    return hipGetLastError();
}

hipError_t launch_conv(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                       const int32_t *count, void *dst, const void *cache, const Geo &g, const ConvCfg &cfg,
                       hipStream_t st) {
    ConvArgs args{(const uint8_t *)src, (const uint8_t *)w, bias, idx, count, (uint8_t *)dst,
                  (const uint8_t *)cache, g, cfg};
    if (cfg.mt != 4 || cfg.nt != 2) return hipErrorInvalidValue;
    switch (dt) {
    case 0: return launch_conv_t<0, 4, 2>(fused, args, st);
    case 1: return launch_conv_t<1, 4, 2>(fused, args, st);
    default: return launch_conv_t<2, 4, 2>(fused, args, st);
    }
}

// ---------------------------------------------------------------------------
// step 5: scatter.  Workgroups [0, scatter_grid) write the listed blocks' valid
// pixels; the rest copy the cache outside listed blocks (when copy_cached).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scatter(const uint8_t *__restrict__ ob, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ count, Geo g, int row_bytes,
                                                 const uint8_t *__restrict__ cache, uint8_t *__restrict__ out,
                                                 int scatter_grid, int copy_xw) {
    const int cnt = clamp_count(count, g.cap);
    if ((int)blockIdx.x >= scatter_grid) {
        copy_unit(g, idx, cnt, cache, out, copy_xw, blockIdx.x - scatter_grid, row_bytes);
        return;
    }
    const int vpp = row_bytes >> 4, b2 = g.b * g.b;
    for (int slot = blockIdx.x; slot < cnt; slot += scatter_grid) {
        int n, by, bx;
        if (!decode_block(g, idx[slot], n, by, bx)) continue;
        for (int v = threadIdx.x; v < b2 * vpp; v += blockDim.x) {
            const int pix = v / vpp, cv = v - pix * vpp;
            const int py = pix / g.b, px = pix - py * g.b;
            const int y = by * g.b + py, x = bx * g.b + px;
            if (y >= g.ho || x >= g.wo) continue;
            st16(out + (((size_t)n * g.ho + y) * g.wo + x) * row_bytes + cv * 16,
                 ld16(ob + ((size_t)slot * b2 + pix) * row_bytes + cv * 16));
        }
    }
}

hipError_t launch_scatter(int dt, const void *out_blocks, const int32_t *idx, const int32_t *count, const Geo &g,
                          const void *cached, void *out, int copy_cached, int scatter_grid, int copy_xw,
                          int copy_units, hipStream_t st) {
    const int row_bytes = g.cout * elem_bytes(dt);
    const unsigned grid = (unsigned)(scatter_grid + (copy_cached ? copy_units : 0));
    hipLaunchKernelGGL(k_scatter, dim3(grid), dim3(256), 0, st, (const uint8_t *)out_blocks, idx, count, g,
                       row_bytes, (const uint8_t *)cached, (uint8_t *)out, scatter_grid, copy_xw);
    return hipGetLastError();
}

}  // namespace sige
