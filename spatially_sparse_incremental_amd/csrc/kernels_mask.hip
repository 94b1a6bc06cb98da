// kernels_mask.hip -- step 1 (change mask) and step 2 (active block list) on gfx950.
//
// Step 1 follows the mer.dev notes on "Efficient Spatially Sparse Inference for
// Conditional GANs and Diffusion Models", section 3 (diff the edited image
// against the original to locate the edit) and the SIGE README mirror,
// "Overview" (compute the difference mask).  Step 2 follows the same notes,
// section 3.2 (downsample the mask to several scales, dilate it, use it to pick
// tiles) and the README "Overview" (reduce the mask to active block indices).
#include "sige_internal.h"

namespace sige {

// ---------------------------------------------------------------------------
// step 1: diff.  HBM-bound: two streaming reads of n*h*w*c elements.
// A 64-lane wave handles 16 pixels: four 16-lane groups, each reading one pixel's
// channel row in 16-byte vectors (1 KiB contiguous per wave and load), four
// pixels per group issued before any compare.  The per-pixel OR over the 16
// lanes of a group is one __ballot; the group leader writes 4 mask bytes at once.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ bool vec_differs(u32x4 x, u32x4 y, float tau) {
    bool f = false;
    if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f |= fabsf(__uint_as_float(y[i]) - __uint_as_float(x[i])) > tau;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int hw = 0; hw < 2; ++hw) {
                const uint32_t xo = (x[i] >> (16 * hw)) & 0xFFFFu, ye = (y[i] >> (16 * hw)) & 0xFFFFu;
                float fo, fe;
                if constexpr (DT == 1) {  // bf16 widens exactly by a 16-bit shift
                    fo = __uint_as_float(xo << 16);
                    fe = __uint_as_float(ye << 16);
                } else {  // fp16 -> fp32 is exact
                    fo = (float)__builtin_bit_cast(_Float16, (uint16_t)xo);
                    fe = (float)__builtin_bit_cast(_Float16, (uint16_t)ye);
                }
                f |= fabsf(fe - fo) > tau;
            }
        }
    }
    return f;
}

template <int DT>
__global__ __launch_bounds__(256) void k_diff(const uint8_t *__restrict__ ao, const uint8_t *__restrict__ ae,
                                              long npix, int vpp, float tau, uint8_t *__restrict__ mask) {
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
    const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long p0 = wave * 16 + sub * 4;  // this group's 4 consecutive pixels
    bool flag[4] = {false, false, false, false};
    for (int v0 = 0; v0 < vpp; v0 += 16) {
        const int v = v0 + li;
        u32x4 x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = y[u] = u32x4{0, 0, 0, 0};
            if (p0 + u < npix && v < vpp) {
                const size_t off = ((size_t)(p0 + u) * vpp + v) * 16;
                x[u] = *(const u32x4 *)(ao + off);
                y[u] = *(const u32x4 *)(ae + off);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) flag[u] |= vec_differs<DT>(x[u], y[u], tau);
    }
    uint32_t word = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const unsigned long long bal = __ballot(flag[u]);
        if ((bal >> (sub * 16)) & 0xFFFFull) word |= 1u << (8 * u);
    }
    if (li == 0 && p0 < npix) {
        if (p0 + 3 < npix) {
            *(uint32_t *)(mask + p0) = word;
        } else {
            for (int u = 0; p0 + u < npix; ++u) mask[p0 + u] = (word >> (8 * u)) & 1u;
        }
    }
}

hipError_t launch_diff(int dt, const void *a_orig, const void *a_edit, long npix, int vpp, float tau,
                       uint8_t *mask, hipStream_t st) {
    const long waves = (npix + 15) / 16;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    const uint8_t *ao = (const uint8_t *)a_orig, *ae = (const uint8_t *)a_edit;
    switch (dt) {
    case 0: hipLaunchKernelGGL(k_diff<0>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask); break;
    case 1: hipLaunchKernelGGL(k_diff<1>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask); break;
    default: hipLaunchKernelGGL(k_diff<2>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 2: reduce.  Latency-bound and tiny, so one 1024-thread workgroup does all
// of it in LDS, which also makes the ascending order free:
//   a) OR-pool the mask by (fy, fx) into bit rows (32 pooled pixels per word),
//      reading the mask in 16-byte vectors and merging bits with LDS atomics;
//   b) window test per block: any set bit in its input window (clipped);
//   c) dilation, separable: along x into a second array, then along y;
//   d) compaction 1024 blocks at a time: wave64 __ballot gives each wave's
//      flags, mbcnt the lane's rank inside the wave, a 16-entry LDS table the
//      wave offsets; indices are written in ascending order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_reduce(const uint8_t *__restrict__ mask, int hm, int wm, int fy, int fx,
                                                 Geo g, int dil, int vec16, int32_t *__restrict__ idx,
                                                 int32_t *__restrict__ count) {
    __shared__ uint32_t bits[kReduceBitsWords];
    __shared__ uint8_t act[kReduceMaxBlocks];
    __shared__ uint8_t tmp[kReduceMaxBlocks];
    __shared__ int wcnt[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int H = g.h, W = g.w, WW = (W + 31) >> 5;
    const int nblk = g.nby * g.nbx;
    const int bs = g.b * g.s;
    int running = 0;
    for (int n = 0; n < g.n; ++n) {
        for (int i = tid; i < H * WW; i += 1024) bits[i] = 0u;
        __syncthreads();
        const uint8_t *m = mask + (size_t)n * hm * wm;
        if (vec16) {
            const int vpr = wm >> 4;
            for (int v = tid; v < hm * vpr; v += 1024) {
                const int Y = v / vpr, q = v - Y * vpr;
                const u32x4 d = *(const u32x4 *)(m + (size_t)Y * wm + q * 16);
                if ((d.x | d.y | d.z | d.w) == 0u) continue;
                const int yp = Y / fy;
                const int wlo = ((q * 16) / fx) >> 5;
                uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if ((d[i >> 2] >> ((i & 3) * 8)) & 0xFFu) {
                        const int xp = (q * 16 + i) / fx;
                        const uint32_t bit = 1u << (xp & 31);
                        if ((xp >> 5) == wlo) m0 |= bit;
                        else m1 |= bit;
                    }
                }
                if (m0) atomicOr(&bits[yp * WW + wlo], m0);
                if (m1) atomicOr(&bits[yp * WW + wlo + 1], m1);
            }
        } else {
            for (int v = tid; v < hm * wm; v += 1024) {
                if (!m[v]) continue;
                const int Y = v / wm, X = v - Y * wm;
                const int xp = X / fx, yp = Y / fy;
                atomicOr(&bits[yp * WW + (xp >> 5)], 1u << (xp & 31));
            }
        }
        __syncthreads();
        for (int q = tid; q < nblk; q += 1024) {
            const int i = q / g.nbx, j = q - i * g.nbx;
            const int r0 = max(0, i * bs - g.p), r1 = min(H, i * bs - g.p + g.ib);
            const int c0 = max(0, j * bs - g.p), c1 = min(W, j * bs - g.p + g.ib);
            bool hit = false;
            if (r0 < r1 && c0 < c1) {
                const int w0 = c0 >> 5, w1 = (c1 - 1) >> 5;
                for (int r = r0; r < r1 && !hit; ++r) {
                    for (int wd = w0; wd <= w1; ++wd) {
                        const int lo = (wd == w0) ? (c0 & 31) : 0;
                        const int hi = (wd == w1) ? ((c1 - 1) & 31) : 31;
                        const uint32_t sel = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
                        if (bits[r * WW + wd] & sel) {
                            hit = true;
                            break;
                        }
                    }
                }
            }
            act[q] = hit ? 1 : 0;
        }
        __syncthreads();
        for (int q = tid; q < nblk; q += 1024) {
            const int i = q / g.nbx, j = q - i * g.nbx;
            uint8_t on = 0;
            for (int jj = max(0, j - dil); jj <= min(g.nbx - 1, j + dil); ++jj) on |= act[i * g.nbx + jj];
            tmp[q] = on;
        }
        __syncthreads();
        for (int base = 0; base < nblk; base += 1024) {
            const int q = base + tid;
            bool on = false;
            if (q < nblk) {
                const int i = q / g.nbx, j = q - i * g.nbx;
                for (int ii = max(0, i - dil); ii <= min(g.nby - 1, i + dil); ++ii) on |= tmp[ii * g.nbx + j] != 0;
            }
            const unsigned long long bal = __ballot(on);
            const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
            if (lane == 0) wcnt[wid] = __popcll(bal);
            __syncthreads();
            int off = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w) {
                const int c = wcnt[w];
                off += (w < wid) ? c : 0;
                tot += c;
            }
            if (on) idx[running + off + rank] = n * nblk + q;
            running += tot;
            __syncthreads();
        }
    }
    if (tid == 0) *count = running;
}

hipError_t launch_reduce(const uint8_t *mask, int hm, int wm, const Geo &g, int dilate, int vec16, int32_t *idx,
                         int32_t *count, hipStream_t st) {
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(1024), 0, st, mask, hm, wm, hm / g.h, wm / g.w, g, dilate, vec16,
                       idx, count);
    return hipGetLastError();
}

}  // namespace sige
