// device_common.h -- device helpers shared by the kernels of this library:
// 16-byte vector access, exact fast divisions, block-list decoding, and the
// copy of a cache outside the listed blocks.  Each kernel file includes it.
#pragma once
#include "sige_internal.h"

namespace sige {

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4 *)p; }

__device__ __forceinline__ void st16(uint8_t *p, u32x4 v) { *(u32x4 *)p = v; }

// x / d for x * d < 2^31, with m = ceil(2^31 / d) from the host (fast_div_magic)
__device__ __forceinline__ int fdiv(int x, uint32_t m) { return (int)(((uint64_t)(uint32_t)x * m) >> 31); }

// a / b and a % b for 0 <= a < 2^50, 0 < b < 2^31: a quotient from fp64 (off by
// at most one there), then one correction step.  Much cheaper than the
// 64-bit integer division routine.
__device__ __forceinline__ long long div_ll(long long a, long long b, long long &r) {
    long long q = (long long)((double)a / (double)b);
    r = a - q * b;
    if (r < 0) {
        --q;
        r += b;
    } else if (r >= b) {
        ++q;
        r -= b;
    }
    return q;
}

// Split point i of [0, total) into n parts: floor(total * i / n), computed in
// fp64 (exact operands for total * n < 2^53; the rounded quotient is monotone
// in i and exact at i = 0 and i = n, so the parts tile the range).
__device__ __forceinline__ long long split_point(long long total, int i, int n) {
    return (long long)floor((double)total * (double)i / (double)n);
}

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
// listed block in an LDS bitmap (one batched read of idx[0, count)), then
// copies a contiguous span of the output's 16-byte vectors, skipping the
// pixels of listed blocks (the convolution writes them).  Without room for
// the bitmap, a binary search over the ascending list decides per vector.
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

// Vectors [v0, v1) of the output, flattened over (n, y, x, vector).  Thread t
// takes v0 + t, v0 + t + NTHR, ...; its pixel coordinates are divided out once
// and then advanced by addition.
template <int CB, int NTHR>
struct CopyWalk {
    long long v, v1;
    int cv, x, y, n, dp, dcv;

    __device__ void init(const Geo &g, const CopyCfg &cc, long long v0, long long v1_) {
        v = v0 + threadIdx.x;
        v1 = v1_;
        long long r;
        const long long pix = div_ll(v, cc.vpp, r);
        cv = (int)r;
        const long long row = div_ll(pix, g.wo, r);
        x = (int)r;
        n = (int)div_ll(row, g.ho, r);
        y = (int)r;
        dp = NTHR / cc.vpp;  // pixels and vectors per stride
        dcv = NTHR - dp * cc.vpp;
    }
    // block index of the current vector
    __device__ __forceinline__ int lin(const Geo &g, const CopyCfg &cc) const {
        return (n * g.nby + fdiv(y, cc.m_b)) * g.nbx + fdiv(x, cc.m_b);
    }
    // on to this thread's next vector
    __device__ __forceinline__ void step(const Geo &g, const CopyCfg &cc) {
        v += NTHR;
        cv += dcv;
        x += dp;
        if (cv >= cc.vpp) {
            cv -= cc.vpp;
            ++x;
        }
        while (x >= g.wo) {
            x -= g.wo;
            if (++y == g.ho) {
                y = 0;
                ++n;
            }
        }
    }
    // Loads of this thread's next CB vectors and their block indices.  The
    // loads are unconditional (past the span they re-read its last vector,
    // flagged -1), so a later wait can cover just the batch it needs.
    __device__ long long fill(const Geo &g, const CopyCfg &cc, const uint8_t *__restrict__ cache, u32x4 (&r)[CB],
                              int (&lin_)[CB]) {
        const long long vb = v;
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const bool ok = v < v1;
            lin_[i] = ok ? lin(g, cc) : -1;
            r[i] = ld16(cache + (ok ? v : v1 - 1) * 16);
            if (ok) step(g, cc);
        }
        return vb;
    }
};

__device__ __forceinline__ bool block_listed(const uint32_t *bm, const int32_t *__restrict__ idx, int cnt, int lin) {
    return bm ? ((bm[lin >> 5] >> (lin & 31)) & 1u) : listed(idx, cnt, lin);
}

// Stores of one batch, skipping vectors of listed blocks; non-temporal (the
// copy is not read again in its kernel, so it leaves no dirty L2 lines for
// the end of the kernel to write back).
template <int CB, int NTHR>
__device__ __forceinline__ void copy_drain(uint8_t *__restrict__ out, long long vb, const u32x4 (&r)[CB],
                                           const int (&lin)[CB], const uint32_t *bm, const int32_t *__restrict__ idx,
                                           int cnt) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        if (lin[i] >= 0 && !block_listed(bm, idx, cnt, lin[i]))
            __builtin_nontemporal_store(r[i], (u32x4 *)(out + (vb + (long long)i * NTHR) * 16));
    }
}

// The copy of [v0, v1), software pipelined: the next batch's loads are in
// flight while the current batch is stored, so reads and writes overlap.
template <int CB, int NTHR>
__device__ void copy_span(const Geo &g, const CopyCfg &cc, const uint32_t *bm, const int32_t *__restrict__ idx,
                          int cnt, const uint8_t *__restrict__ cache, uint8_t *__restrict__ out, long long v0,
                          long long v1) {
    if (v0 + threadIdx.x >= v1) return;
    CopyWalk<CB, NTHR> w;
    w.init(g, cc, v0, v1);
    u32x4 ra[CB], rb[CB];
    int la[CB], lb[CB];
    long long va = w.fill(g, cc, cache, ra, la);
    for (;;) {
        if (w.v >= v1) {
            copy_drain<CB, NTHR>(out, va, ra, la, bm, idx, cnt);
            return;
        }
        const long long vb = w.fill(g, cc, cache, rb, lb);
        copy_drain<CB, NTHR>(out, va, ra, la, bm, idx, cnt);
        if (w.v >= v1) {
            copy_drain<CB, NTHR>(out, vb, rb, lb, bm, idx, cnt);
            return;
        }
        va = w.fill(g, cc, cache, ra, la);
        copy_drain<CB, NTHR>(out, vb, rb, lb, bm, idx, cnt);
    }
}

// Unconditional copy of the 16-byte vectors [v0, v1) from src to dst: thread t
// takes v0 + t, v0 + t + NTHR, ...; CB loads of the next batch are in flight
// while the current one is stored.  NTS: non-temporal stores (no dirty L2
// lines left for the end of the kernel to write back).
template <int CB, int NTHR, bool NTS = false>
__device__ void copy_all_span(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, long long v0, long long v1) {
    long long v = v0 + threadIdx.x;
    if (v >= v1) return;
    u32x4 ra[CB], rb[CB];
    auto fill = [&](u32x4 (&r)[CB], long long base) {
#pragma unroll
        for (int i = 0; i < CB; ++i) r[i] = ld16(src + min(base + (long long)i * NTHR, v1 - 1) * 16);
    };
    auto drain = [&](const u32x4 (&r)[CB], long long base) {
#pragma unroll
        for (int i = 0; i < CB; ++i)
            if (base + (long long)i * NTHR < v1) {
                if (NTS)
                    __builtin_nontemporal_store(r[i], (u32x4 *)(dst + (base + (long long)i * NTHR) * 16));
                else
                    st16(dst + (base + (long long)i * NTHR) * 16, r[i]);
            }
    };
    constexpr long long step = (long long)CB * NTHR;
    fill(ra, v);
    for (;; v += 2 * step) {
        if (v + step >= v1) {
            drain(ra, v);
            return;
        }
        fill(rb, v + step);
        drain(ra, v);
        if (v + 2 * step >= v1) {
            drain(rb, v + step);
            return;
        }
        fill(ra, v + 2 * step);
        drain(rb, v + step);
    }
}

// ---------------------------------------------------------------------------
// Work split of the copy and of the restore among the workgroups of a launch.
// ---------------------------------------------------------------------------

// The part [lo, hi) of the copy that workgroup `bid` takes.  The workgroups
// without a tile come first (they start at once): up to free_vec vectors each
// per tile of the busiest workgroup.  What remains is split evenly over the
// others, after their tiles.
__device__ __forceinline__ void copy_split(const CopyCfg &cc, int ntiles, int grid, int bid, long long &lo,
                                           long long &hi) {
    const long long nvec = cc.nvec;
    const int busy = min(ntiles, grid), nfree = grid - busy;
    const int rounds = (ntiles + grid - 1) / grid;
    long long to_free = (long long)nfree * cc.free_vec * max(rounds, 1);
    if (busy == 0 || to_free > nvec) to_free = nvec;
    if (bid >= busy) {
        lo = split_point(to_free, bid - busy, nfree);
        hi = split_point(to_free, bid - busy + 1, nfree);
    } else {
        const long long rest = nvec - to_free;
        lo = to_free + split_point(rest, bid, busy);
        hi = to_free + split_point(rest, bid + 1, busy);
    }
}

// ---------------------------------------------------------------------------
// Sequential edits: the previous edit's blocks that the new list does not hold
// get the cache back.  restore_slots takes previous-list slots first, first +
// step, ... below end; a block's valid pixels go as batches of 16-byte vectors.
// ---------------------------------------------------------------------------
template <int NTHR>
__device__ void restore_slots(const Geo &g, const CopyCfg &cc, const int32_t *__restrict__ prev_idx, int first,
                              int step, int end, const uint32_t *bm, const int32_t *__restrict__ idx, int cnt,
                              const uint8_t *__restrict__ cache, uint8_t *__restrict__ out) {
    constexpr int U = 8;
    const int vpp = cc.vpp, row_bytes = vpp * 16, nv = g.b * g.b * vpp;
    for (int slot = first; slot < end; slot += step) {
        const int lin = prev_idx[slot];
        int n, by, bx;
        if (!decode_block(g, lin, n, by, bx)) continue;
        if (idx && block_listed(bm, idx, cnt, lin)) continue;
        for (int v0 = threadIdx.x; v0 < nv; v0 += U * NTHR) {
            u32x4 r[U];
            size_t at[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int v = v0 + i * NTHR;
                at[i] = ~(size_t)0;
                if (v < nv) {
                    const int pix = fdiv(v, cc.m_vpp), cvv = v - pix * vpp;
                    const int py = fdiv(pix, cc.m_b), px = pix - py * g.b;
                    const int y = by * g.b + py, x = bx * g.b + px;
                    if (y < g.ho && x < g.wo) {
                        at[i] = (((size_t)n * g.ho + y) * g.wo + x) * row_bytes + cvv * 16;
                        r[i] = ld16(cache + at[i]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (at[i] != ~(size_t)0) st16(out + at[i], r[i]);
        }
    }
}

// The slots [lo, hi) of the previous list that workgroup `bid` restores: the
// workgroups without a tile share them evenly; without such workgroups, all
// share them after their tiles.
__device__ __forceinline__ void restore_split(int np, int ntiles, int grid, int bid, long long &lo, long long &hi) {
    const int busy = min(ntiles, grid), nfree = grid - busy;
    if (nfree > 0) {
        lo = bid >= busy ? split_point(np, bid - busy, nfree) : 0;
        hi = bid >= busy ? split_point(np, bid - busy + 1, nfree) : 0;
    } else {
        lo = split_point(np, bid, grid);
        hi = split_point(np, bid + 1, grid);
    }
}

}  // namespace sige
