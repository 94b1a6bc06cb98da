// mask_core.h -- device code of the change mask (step 1) and the active block
// list (step 2): the per-wave diff, the pooling of a mask into bit rows, and
// the bit rows' block list.  The method is described in kernels_mask.hip.
#pragma once
#include "device_common.h"

namespace sige {

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

// One wave's 16 pixels starting at pixel 16 * wave: four 16-lane groups, each
// reading one pixel's channel row in 16-byte vectors (1 KiB contiguous per
// wave and load), four pixels per group issued before any compare.  The
// per-pixel OR over the 16 lanes of a group is one __ballot; the group leader
// writes 4 mask bytes at once (mask not NULL), and lane 0 writes the wave's 16
// pixels as one 16-bit half of a bitset word (bits not NULL; bit p % 32 of word
// p / 32 for pixel p, npix a multiple of 16).  A_o's loads are non-temporal:
// the original activation is read once, and its lines, evicted first, leave
// the caches to A_e (whose active windows the layer reads next), the cached
// output and the weights.  Measured on the 256x256x128 bf16 step: 21.4 ->
// 20.2 us; the diff alone, repeated over the same inputs, gets slower, since
// it then finds less of A_o in the caches.
template <int DT>
__device__ __forceinline__ void diff16(const uint8_t *__restrict__ ao, const uint8_t *__restrict__ ae, long npix,
                                       int vpp, float tau, uint8_t *__restrict__ mask, uint16_t *__restrict__ bits,
                                       long wave) {
    const int lane = threadIdx.x & 63, sub = lane >> 4, li = lane & 15;
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
                x[u] = __builtin_nontemporal_load((const u32x4 *)(ao + off));
                y[u] = *(const u32x4 *)(ae + off);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) flag[u] |= vec_differs<DT>(x[u], y[u], tau);
    }
    uint32_t word = 0, half = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const unsigned long long bal = __ballot(flag[u]);
        if ((bal >> (sub * 16)) & 0xFFFFull) word |= 1u << (8 * u);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
            if ((bal >> (gq * 16)) & 0xFFFFull) half |= 1u << (gq * 4 + u);
    }
    if (bits && lane == 0 && wave * 16 < npix) bits[wave] = (uint16_t)half;
    if (mask && li == 0 && p0 < npix) {
        if (p0 + 3 < npix) {
            *(uint32_t *)(mask + p0) = word;
        } else {
            for (int u = 0; p0 + u < npix; ++u) mask[p0 + u] = (word >> (8 * u)) & 1u;
        }
    }
}

struct RedCfg {
    uint32_t m_vpr;  // fast_div_magic(mask_w / 16)
    uint32_t m_wm;   // fast_div_magic(mask_w)
    uint32_t m_fy, m_fx, m_nbx;
};

__device__ __forceinline__ int fdiv31(int x, uint32_t m) { return (int)(((uint64_t)(uint32_t)x * m) >> 31); }

// Any set bit of bit row `br` in columns [c0, c1)?
__device__ __forceinline__ bool any_bits(const uint32_t *br, int c0, int c1) {
    if (c0 >= c1) return false;
    const int w0 = c0 >> 5, w1 = (c1 - 1) >> 5;
    const uint32_t lo = ~((1u << (c0 & 31)) - 1u);
    const uint32_t hi = ((c1 - 1) & 31) == 31 ? 0xFFFFFFFFu : ((1u << (((c1 - 1) & 31) + 1)) - 1u);
    if (w0 == w1) return (br[w0] & lo & hi) != 0u;
    uint32_t acc = (br[w0] & lo) | (br[w1] & hi);
    for (int wd = w0 + 1; wd < w1; ++wd) acc |= br[wd];
    return acc != 0u;
}

// Compact one round of NW * 64 candidate blocks in ascending order: wave64
// ballot, mbcnt rank, wave offsets through LDS.
template <int NW>
__device__ __forceinline__ int compact_round(bool on, int q_out, int running, int *wcnt, int32_t *out) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const unsigned long long bal = __ballot(on);
    const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
    if (lane == 0) wcnt[wid] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = wcnt[w];
        off += (w < wid) ? c : 0;
        tot += c;
    }
    if (on) out[running + off + rank] = q_out;
    __syncthreads();
    return running + tot;
}

// OR the 32 pixels of one bitset word (columns x0 .. x0 + 31 of a row, x0 a
// multiple of 32) into the bit row `row`, pooled by fx along x (m_fx its
// multiplier).
__device__ __forceinline__ void pool_word(uint32_t *row, uint32_t v, int x0, int fx, uint32_t m_fx) {
    if (fx == 1) {
        atomicOr(&row[x0 >> 5], v);
        return;
    }
    const int wlo = fdiv31(x0, m_fx) >> 5;
    uint32_t m0 = 0u, m1 = 0u;
    while (v) {
        const int i = __builtin_ctz(v);
        v &= v - 1u;
        const int xp = fdiv31(x0 + i, m_fx);
        if ((xp >> 5) == wlo) m0 |= 1u << (xp & 31);
        else m1 |= 1u << (xp & 31);
    }
    if (m0) atomicOr(&row[wlo], m0);
    if (m1) atomicOr(&row[wlo + 1], m1);
}

// One image's mask m [hm, wm], OR-pooled by (fy, fx), as bit rows in LDS:
// bits[y * ceil(w / 32) + x / 32] bit x % 32 for the pooled pixel (y, x).
// Input modes: bytes (vec16 0), bytes read as 16-byte vectors (1), or a bitset
// (2: bit x % 32 of word (y * wm + x) / 32, wm a multiple of 32; rc.m_vpr is
// then the multiplier of wm / 32).
template <int NTHR>
__device__ __forceinline__ void mask_to_bits(const uint8_t *__restrict__ m, int hm, int wm, int fy, int fx,
                                             const Geo &g, int vec16, const RedCfg &rc, uint32_t *bits) {
    constexpr int U = 8;
    const int tid = threadIdx.x;
    const int H = g.h, WW = (g.w + 31) >> 5;
    for (int q = tid; q < H * WW; q += NTHR) bits[q] = 0u;
    __syncthreads();
    if (vec16 == 2) {
        const uint32_t *mb = (const uint32_t *)m;
        const int wpr = wm >> 5, nv = hm * wpr;
        for (int v0 = tid; v0 < nv; v0 += U * NTHR) {
            uint32_t d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) d[u] = (v0 + u * NTHR < nv) ? mb[v0 + u * NTHR] : 0u;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!d[u]) continue;
                const int v = v0 + u * NTHR;
                const int Y = fdiv31(v, rc.m_vpr), q = v - Y * wpr;
                pool_word(bits + fdiv31(Y, rc.m_fy) * WW, d[u], q * 32, fx, rc.m_fx);
            }
        }
    } else if (vec16) {
        const int vpr = wm >> 4, nv = hm * vpr;
        for (int v0 = tid; v0 < nv; v0 += U * NTHR) {
            u32x4 d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * NTHR;
                d[u] = v < nv ? *(const u32x4 *)(m + (size_t)v * 16) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if ((d[u].x | d[u].y | d[u].z | d[u].w) == 0u) continue;
                const int v = v0 + u * NTHR;
                const int Y = fdiv31(v, rc.m_vpr), q = v - Y * vpr;
                const int row = fdiv31(Y, rc.m_fy) * WW;
                const int wlo = fdiv31(q * 16, rc.m_fx) >> 5;
                uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    if ((d[u][b >> 2] >> ((b & 3) * 8)) & 0xFFu) {
                        const int xp = fx == 1 ? q * 16 + b : fdiv31(q * 16 + b, rc.m_fx);
                        const uint32_t bit = 1u << (xp & 31);
                        if ((xp >> 5) == wlo) m0 |= bit;
                        else m1 |= bit;
                    }
                }
                if (m0) atomicOr(&bits[row + wlo], m0);
                if (m1) atomicOr(&bits[row + wlo + 1], m1);
            }
        }
    } else {
        const int nv = hm * wm;
        for (int v0 = tid; v0 < nv; v0 += U * NTHR) {
            uint8_t d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) d[u] = (v0 + u * NTHR < nv) ? m[v0 + u * NTHR] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!d[u]) continue;
                const int v = v0 + u * NTHR;
                const int Y = fdiv31(v, rc.m_wm), X = v - Y * wm;
                const int xp = fdiv31(X, rc.m_fx), yp = fdiv31(Y, rc.m_fy);
                atomicOr(&bits[yp * WW + (xp >> 5)], 1u << (xp & 31));
            }
        }
    }
    __syncthreads();
}

// One image's active blocks from its bit rows: ascending linear indices
// appended to out[running...]; returns the new length in every thread.
template <int NTHR>
__device__ __forceinline__ int bits_to_list(const Geo &g, int dil, const RedCfg &rc, const uint32_t *bits,
                                            uint8_t *scratch, int *wcnt, int32_t *out, int n, int running) {
    const int tid = threadIdx.x;
    const int H = g.h, W = g.w, WW = (W + 31) >> 5;
    const int nblk = g.nby * g.nbx;
    const int bs = g.b * g.s;
    const bool touching = g.ib >= bs;  // consecutive windows overlap or touch
    if (touching) {
        // The dilated activity of block (i, j) is "some set bit in the union of
        // the windows of blocks (i', j'), |i'-i|, |j'-j| <= d", a rectangle when
        // consecutive windows touch: rows [max(0,(i-d)bs-p), min(H,(i+d)bs-p+ib)),
        // columns likewise.  First OR each block row's rows into one bit row.
        uint32_t *rowbits = (uint32_t *)scratch;
        for (int q = tid; q < g.nby * WW; q += NTHR) {
            const int i = q / WW, wd = q - i * WW;
            const int r0 = max(0, max(0, i - dil) * bs - g.p);
            const int r1 = min(H, min(g.nby - 1, i + dil) * bs - g.p + g.ib);
            uint32_t acc = 0u;
            for (int r = r0; r < r1; ++r) acc |= bits[r * WW + wd];
            rowbits[q] = acc;
        }
        __syncthreads();
        for (int base = 0; base < nblk; base += NTHR) {
            const int q = base + tid;
            bool on = false;
            if (q < nblk) {
                const int i = fdiv31(q, rc.m_nbx), j = q - i * g.nbx;
                const int c0 = max(0, max(0, j - dil) * bs - g.p);
                const int c1 = min(W, min(g.nbx - 1, j + dil) * bs - g.p + g.ib);
                on = any_bits(rowbits + i * WW, c0, c1);
            }
            running = compact_round<NTHR / 64>(on, n * nblk + q, running, wcnt, out);
        }
    } else {
        uint8_t *act = scratch, *tmp = scratch + nblk;
        for (int q = tid; q < nblk; q += NTHR) {
            const int i = fdiv31(q, rc.m_nbx), j = q - i * g.nbx;
            const int r0 = max(0, i * bs - g.p), r1 = min(H, i * bs - g.p + g.ib);
            const int c0 = max(0, j * bs - g.p), c1 = min(W, j * bs - g.p + g.ib);
            bool hit = false;
            for (int r = r0; r < r1 && !hit; ++r) hit = any_bits(bits + r * WW, c0, c1);
            act[q] = hit ? 1 : 0;
        }
        __syncthreads();
        for (int q = tid; q < nblk; q += NTHR) {
            const int i = fdiv31(q, rc.m_nbx), j = q - i * g.nbx;
            uint8_t on = 0;
            for (int jj = max(0, j - dil); jj <= min(g.nbx - 1, j + dil); ++jj) on |= act[i * g.nbx + jj];
            tmp[q] = on;
        }
        __syncthreads();
        for (int base = 0; base < nblk; base += NTHR) {
            const int q = base + tid;
            bool on = false;
            if (q < nblk) {
                const int i = fdiv31(q, rc.m_nbx), j = q - i * g.nbx;
                for (int ii = max(0, i - dil); ii <= min(g.nby - 1, i + dil); ++ii)
                    on |= tmp[ii * g.nbx + j] != 0;
            }
            running = compact_round<NTHR / 64>(on, n * nblk + q, running, wcnt, out);
        }
    }
    __syncthreads();  // scratch and bits are reused by the next image
    return running;
}

// The ascending list of active blocks of every image (see the step-2 notes in
// kernels_mask.hip), computed by one workgroup of NTHR threads into `out`;
// returns the count in every thread.  LDS: bits holds h * ceil(w / 32) words;
// scratch max(nby * ceil(w / 32) * 4, 2 * nby * nbx) bytes; wcnt NTHR / 64 ints.
template <int NTHR>
__device__ int reduce_list(const uint8_t *__restrict__ mask, int hm, int wm, int fy, int fx, const Geo &g, int dil,
                           int vec16, const RedCfg &rc, uint32_t *bits, uint8_t *scratch, int *wcnt,
                           int32_t *out) {
    int running = 0;
    const size_t istride = vec16 == 2 ? (size_t)hm * wm / 8 : (size_t)hm * wm;  // bytes per image
    for (int n = 0; n < g.n; ++n) {
        mask_to_bits<NTHR>(mask + (size_t)n * istride, hm, wm, fy, fx, g, vec16, rc, bits);
        running = bits_to_list<NTHR>(g, dil, rc, bits, scratch, wcnt, out, n, running);
    }
    return running;
}

}  // namespace sige
