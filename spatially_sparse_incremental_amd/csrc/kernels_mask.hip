// kernels_mask.hip -- step 1 (change mask) and step 2 (active block list) on gfx950.
//
// Step 1 follows the mer.dev notes on "Efficient Spatially Sparse Inference for
// Conditional GANs and Diffusion Models", section 3 (diff the edited image
// against the original to locate the edit) and the SIGE README mirror,
// "Overview" (compute the difference mask).  Step 2 follows the same notes,
// section 3.2 (downsample the mask to several scales, dilate it, use it to pick
// tiles) and the README "Overview" (reduce the mask to active block indices).
#include "mask_core.h"

namespace sige {

// ---------------------------------------------------------------------------
// step 1: diff.  HBM-bound: two streaming reads of n*h*w*c elements.
// A 64-lane wave handles 16 pixels: four 16-lane groups, each reading one pixel's
// channel row in 16-byte vectors (1 KiB contiguous per wave and load), four
// pixels per group issued before any compare.  The per-pixel OR over the 16
// lanes of a group is one __ballot; the group leader writes 4 mask bytes at
// once, and lane 0 the wave's 16 bits of the packed mask when one is asked for.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_diff(const uint8_t *__restrict__ ao, const uint8_t *__restrict__ ae,
                                              long npix, int vpp, float tau, uint8_t *__restrict__ mask,
                                              uint16_t *__restrict__ bits) {
    diff16<DT>(ao, ae, npix, vpp, tau, mask, bits, (long)blockIdx.x * 4 + (threadIdx.x >> 6));
}

hipError_t launch_diff(int dt, const void *a_orig, const void *a_edit, long npix, int vpp, float tau,
                       uint8_t *mask, uint32_t *bits, hipStream_t st) {
    const long waves = (npix + 15) / 16;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    const uint8_t *ao = (const uint8_t *)a_orig, *ae = (const uint8_t *)a_edit;
    uint16_t *b16 = (uint16_t *)bits;
    switch (dt) {
    case 0: hipLaunchKernelGGL(k_diff<0>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask, b16); break;
    case 1: hipLaunchKernelGGL(k_diff<1>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask, b16); break;
    default: hipLaunchKernelGGL(k_diff<2>, dim3(grid), dim3(256), 0, st, ao, ae, npix, vpp, tau, mask, b16); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 2 for large inputs, in two launches.
//  k_activity: one workgroup per (image, block row).  It ORs the full-resolution
//    mask rows under the row's input windows into pooled column bits in LDS
//    (16-byte mask loads, 8 in flight, bits merged with LDS atomics), then tests
//    each block's window columns.  The raw activity flags (one byte per block)
//    go into the caller's idx buffer, which is 4x larger than needed for them.
//  k_compact: one 1024-thread workgroup.  It reads every flag into LDS first,
//    then dilates (along x into a second array, then along y) and compacts
//    1024 blocks at a time: wave64 __ballot gives each wave's flags, mbcnt the
//    lane's rank, a 16-entry LDS table the wave offsets.  Indices are written
//    in ascending order over the idx buffer, after all flags were read.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_activity(const uint8_t *__restrict__ mask, int hm, int wm, int fy, int fx,
                                                  Geo g, int vec16, uint8_t *__restrict__ flags, ReduceCopy cp,
                                                  int ncopy) {
    if ((int)blockIdx.x >= g.nby) {  // workgroups past the block rows copy the cache (image row 0 only)
        if (blockIdx.y == 0) {
            const int i = blockIdx.x - g.nby;
            copy_all_span<4, 256>(cp.src, cp.dst, split_point(cp.nvec, i, ncopy), split_point(cp.nvec, i + 1, ncopy));
        }
        return;
    }
    __shared__ uint32_t colbits[kReduceMaxWidth / 32];
    constexpr int U = 8;
    const int tid = threadIdx.x;
    const int i = blockIdx.x, n = blockIdx.y;
    const int H = g.h, W = g.w, WW = (W + 31) >> 5;
    const int bs = g.b * g.s;
    for (int q = tid; q < WW; q += 256) colbits[q] = 0u;
    __syncthreads();
    const int pr0 = max(0, i * bs - g.p), pr1 = min(H, i * bs - g.p + g.ib);
    const size_t pix0 = ((size_t)n * hm + (size_t)pr0 * fy) * wm;  // first pixel of the band
    const uint8_t *m = mask + (vec16 == 2 ? pix0 / 8 : pix0);
    const int rows = (pr1 - pr0) * fy;
    if (vec16 == 2) {  // a bitset (wm a multiple of 32)
        const uint32_t *mb = (const uint32_t *)m;
        const int wpr = wm >> 5, nv = rows * wpr;
        const uint32_t m_fx = fast_div_magic(fx);
        for (int v0 = tid; v0 < nv; v0 += U * 256) {
            uint32_t d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) d[u] = (v0 + u * 256 < nv) ? mb[v0 + u * 256] : 0u;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (d[u]) pool_word(colbits, d[u], ((v0 + u * 256) % wpr) * 32, fx, m_fx);
        }
    } else if (vec16) {
        const int vpr = wm >> 4;
        const int nv = rows * vpr;
        for (int v0 = tid; v0 < nv; v0 += U * 256) {
            u32x4 d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 256;
                d[u] = u32x4{0u, 0u, 0u, 0u};
                if (v < nv) d[u] = *(const u32x4 *)(m + (size_t)(v / vpr) * wm + (v % vpr) * 16);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if ((d[u].x | d[u].y | d[u].z | d[u].w) == 0u) continue;
                const int q = (v0 + u * 256) % vpr;
                const int wlo = ((q * 16) / fx) >> 5;
                uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    if ((d[u][b >> 2] >> ((b & 3) * 8)) & 0xFFu) {
                        const int xp = (q * 16 + b) / fx;
                        const uint32_t bit = 1u << (xp & 31);
                        if ((xp >> 5) == wlo) m0 |= bit;
                        else m1 |= bit;
                    }
                }
                if (m0) atomicOr(&colbits[wlo], m0);
                if (m1) atomicOr(&colbits[wlo + 1], m1);
            }
        }
    } else {
        const int nv = rows * wm;
        for (int v = tid; v < nv; v += 256) {
            if (!m[v]) continue;
            const int xp = (v % wm) / fx;
            atomicOr(&colbits[xp >> 5], 1u << (xp & 31));
        }
    }
    __syncthreads();
    for (int j = tid; j < g.nbx; j += 256) {
        const int c0 = max(0, j * bs - g.p), c1 = min(W, j * bs - g.p + g.ib);
        bool hit = false;
        if (pr0 < pr1 && c0 < c1) {
            const int w0 = c0 >> 5, w1 = (c1 - 1) >> 5;
            for (int wd = w0; wd <= w1 && !hit; ++wd) {
                const int lo = (wd == w0) ? (c0 & 31) : 0;
                const int hi = (wd == w1) ? ((c1 - 1) & 31) : 31;
                const uint32_t sel = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
                hit = (colbits[wd] & sel) != 0u;
            }
        }
        flags[((size_t)n * g.nby + i) * g.nbx + j] = hit ? 1 : 0;
    }
}

__global__ __launch_bounds__(1024) void k_compact(Geo g, int dil, int32_t *__restrict__ idx,
                                                  int32_t *__restrict__ count) {
    __shared__ uint8_t act[kReduceMaxBlocks];
    __shared__ uint8_t tmp[kReduceMaxBlocks];
    __shared__ int wcnt[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int nblk = g.nby * g.nbx, cap = g.cap;
    const uint32_t *fw = (const uint32_t *)idx;  // the flags k_activity left in idx
    for (int q = tid; q < (cap + 3) / 4; q += 1024) {
        const uint32_t v = fw[q];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (4 * q + b < cap) act[4 * q + b] = (v >> (8 * b)) & 0xFFu;
    }
    __syncthreads();
    for (int q = tid; q < cap; q += 1024) {
        const int r = q % nblk, i = r / g.nbx, j = r - i * g.nbx;
        const int rowbase = q - j;
        uint8_t on = 0;
        for (int jj = max(0, j - dil); jj <= min(g.nbx - 1, j + dil); ++jj) on |= act[rowbase + jj];
        tmp[q] = on;
    }
    __syncthreads();
    int running = 0;
    for (int base = 0; base < cap; base += 1024) {
        const int q = base + tid;
        bool on = false;
        if (q < cap) {
            const int r = q % nblk, i = r / g.nbx, j = r - i * g.nbx;
            const int img = q - r;
            for (int ii = max(0, i - dil); ii <= min(g.nby - 1, i + dil); ++ii) on |= tmp[img + ii * g.nbx + j] != 0;
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
        if (on) idx[running + off + rank] = q;
        running += tot;
        __syncthreads();
    }
    if (tid == 0) *count = running;
}

// ---------------------------------------------------------------------------
// step 2 in one launch, for inputs whose pooled mask fits in LDS as bits
// (h * ceil(w/32) <= kReduceBitsWords): one 1024-thread workgroup.
//   a) OR-pool the mask into bit rows (32 pooled pixels per word): every
//      16-byte mask load of a round is in flight before any is used, bits
//      merged with LDS atomics;
//   b) when consecutive input windows touch (k >= stride), the dilated
//      activity of a block is one rectangle test: each block row's rows are
//      ORed into one bit row, and every block tests its column range while
//      being compacted (wave64 __ballot + mbcnt ranks, 16-entry LDS table of
//      wave offsets); otherwise window test, dilation along x, then along y
//      fused with the compaction.
// All divisions by launch constants use host-computed multipliers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_reduce_one(const uint8_t *__restrict__ mask, int hm, int wm, int fy, int fx,
                                                     Geo g, int dil, int vec16, RedCfg rc,
                                                     int32_t *__restrict__ idx, int32_t *__restrict__ count,
                                                     ReduceCopy cp) {
    if (blockIdx.x > 0) {  // the other workgroups copy the cache meanwhile
        const int i = blockIdx.x - 1, nw = gridDim.x - 1;
        copy_all_span<2, 1024, true>(cp.src, cp.dst, split_point(cp.nvec, i, nw), split_point(cp.nvec, i + 1, nw));
        return;
    }
    __shared__ uint32_t bits[kReduceBitsWords];
    // per block row: OR of the bit rows under its (dilated) windows; or, when
    // windows do not touch, the raw and x-dilated block flags
    __shared__ __attribute__((aligned(16))) uint8_t scratch[2 * kReduceMaxBlocks];
    __shared__ int wcnt[16];
    const int running = reduce_list<1024>(mask, hm, wm, fy, fx, g, dil, vec16, rc, bits, scratch, wcnt, idx);
    if (threadIdx.x == 0) *count = running;
}

bool reduce_one_launch_ok(int hm, int wm, const Geo &g, int vec16) {
    const int fy = hm / g.h, fx = wm / g.w;
    const int WW = (g.w + 31) / 32;
    // the one-launch path divides with 31-bit multipliers: every dividend * divisor < 2^31
    const long lim = 1L << 31;
    const int vdiv = vec16 == 2 ? wm / 32 : vec16 ? wm / 16 : 1;  // bitset words or 16-byte vectors per row
    const bool exact = (vec16 ? (long)hm * vdiv * vdiv : (long)hm * wm * wm) < lim && (long)hm * fy < lim &&
                       (long)wm * fx < lim;
    return exact && (long)g.h * WW <= kReduceBitsWords && g.nby * g.nbx <= kReduceMaxBlocks;
}

hipError_t launch_reduce(const uint8_t *mask, int hm, int wm, const Geo &g, int dilate, int vec16, int32_t *idx,
                         int32_t *count, const ReduceCopy &cp, int copy_wgs, hipStream_t st) {
    const int ncopy = cp.nvec > 0 ? copy_wgs : 0;
    const int fy = hm / g.h, fx = wm / g.w;
    const int vdiv = vec16 == 2 ? wm / 32 : vec16 ? wm / 16 : 1;
    if (reduce_one_launch_ok(hm, wm, g, vec16)) {
        RedCfg rc{fast_div_magic(vdiv), fast_div_magic(wm), fast_div_magic(fy), fast_div_magic(fx),
                  fast_div_magic(g.nbx)};
        hipLaunchKernelGGL(k_reduce_one, dim3(1 + ncopy), dim3(1024), 0, st, mask, hm, wm, fy, fx, g, dilate, vec16,
                           rc, idx, count, cp);
        return hipGetLastError();
    }
    const int ncopy4 = ncopy * 4;  // 256-thread workgroups
    hipLaunchKernelGGL(k_activity, dim3(g.nby + ncopy4, g.n), dim3(256), 0, st, mask, hm, wm, fy, fx, g, vec16,
                       (uint8_t *)idx, cp, ncopy4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, g, dilate, idx, count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 2 for the layers of a network at one edit: every layer's list comes
// from the same change mask, pooled to that layer's input (mer.dev notes, 3.2:
// one mask downsampled to several scales), so all of them can be built before
// any layer runs.  Workgroup i < n builds layer i's list as k_reduce_one does
// (packed mask); the other workgroups copy the layers' caches into their
// outputs, the copies taken as one range of 16-byte vectors split evenly.
// ---------------------------------------------------------------------------
struct ReduceLayer {
    Geo g;
    int fy, fx, dil;
    RedCfg rc;
    int32_t *idx, *count;
    const uint8_t *src;
    uint8_t *dst;
    long long nvec;
};
struct ReduceLayers {
    int n;
    long long total_vec;
    ReduceLayer l[kReduceMaxLayers];
};

__global__ __launch_bounds__(1024) void k_reduce_layers(const uint8_t *__restrict__ mask, int hm, int wm,
                                                        ReduceLayers L) {
    if ((int)blockIdx.x >= L.n) {
        const int i = blockIdx.x - L.n, nw = gridDim.x - L.n;
        const long long lo = split_point(L.total_vec, i, nw), hi = split_point(L.total_vec, i + 1, nw);
        long long base = 0;
        for (int l = 0; l < L.n; ++l) {
            const long long nv = L.l[l].nvec;
            const long long a = lo > base ? lo : base, b = hi < base + nv ? hi : base + nv;
            if (a < b) copy_all_span<2, 1024, true>(L.l[l].src, L.l[l].dst, a - base, b - base);
            base += nv;
        }
        return;
    }
    __shared__ uint32_t bits[kReduceBitsWords];
    __shared__ __attribute__((aligned(16))) uint8_t scratch[2 * kReduceMaxBlocks];
    __shared__ int wcnt[16];
    const ReduceLayer &ly = L.l[blockIdx.x];
    const int running =
        reduce_list<1024>(mask, hm, wm, ly.fy, ly.fx, ly.g, ly.dil, 2, ly.rc, bits, scratch, wcnt, ly.idx);
    if (threadIdx.x == 0) *ly.count = running;
}

hipError_t launch_reduce_layers(const uint32_t *bits, int hm, int wm, int n, const ReduceLayerArgs *layers,
                                int copy_wgs, hipStream_t st) {
    if (n < 1 || n > kReduceMaxLayers) return hipErrorInvalidValue;
    ReduceLayers L{};
    L.n = n;
    for (int i = 0; i < n; ++i) {
        const ReduceLayerArgs &a = layers[i];
        if (!reduce_one_launch_ok(hm, wm, a.g, 2)) return hipErrorInvalidValue;  // checked by the caller
        ReduceLayer &d = L.l[i];
        d.g = a.g;
        d.fy = hm / a.g.h;
        d.fx = wm / a.g.w;
        d.dil = a.dilate;
        d.rc = RedCfg{fast_div_magic(wm / 32), fast_div_magic(wm), fast_div_magic(d.fy), fast_div_magic(d.fx),
                      fast_div_magic(a.g.nbx)};
        d.idx = a.idx;
        d.count = a.count;
        d.src = a.src;
        d.dst = a.dst;
        d.nvec = a.src ? a.nvec : 0;
        L.total_vec += d.nvec;
    }
    const int ncopy = L.total_vec > 0 ? copy_wgs : 0;
    hipLaunchKernelGGL(k_reduce_layers, dim3(n + ncopy), dim3(1024), 0, st, (const uint8_t *)bits, hm, wm, L);
    return hipGetLastError();
}

}  // namespace sige
