// kernels_layer.hip -- the fused sparse layer (steps 3-5 in one kernel) and
// the block convolution of the three-call path (step 4), as an implicit GEMM
// on the matrix cores of gfx950.
//
// SIGE README mirror, "Overview": the input window of every active block (its
// halo of k-1 pixels included) is gathered from the edited activation, the
// convolution runs on the stacked windows, and each output block is written
// into the cached output of the original image.  Here the three happen in one
// kernel and no block tensor is materialised: windows go from the activation
// into LDS, results from the matrix cores into the output image.
//
// The GEMM: M = listed blocks x b*b output pixels, flattened over the list (so
// 6x6 blocks waste nothing to 16-row MFMA tiles); N = c_out; K = k*k*c_in,
// walked as (tap, slice of KS input channels) steps.  A workgroup of 4 waves
// owns a tile of 16*MT rows x 16*NT output channels; the waves split the K
// steps in contiguous runs and each accumulates the whole tile, so every
// staged window element is read from LDS by one wave only.  16-bit types run
// 32x32x16 MFMAs (a 64 x 32 tile is two 32 x 32 fragments, a 32-channel K
// slice two 16-channel halves): at one or two waves per SIMD they issue about
// 1.3-1.7 times the flops of 16x16x32 ones.  fp32 (and tiles of 16 channels)
// run 16x16 MFMAs.  Two workgroups
// share a CU, so one's memory round trips overlap the other's MFMAs.
//
// The critical path of a tile, at small edits the whole launch:
//   1. the list length and the block index of each of the tile's slots (one
//      vector load per lane, issued first), and this wave's weight fragments
//      (L2 into registers; a wave's fragments are its own);
//   2. each wave decodes the slots' window origins in its own lanes and
//      stages its share of the windows straight into LDS
//      (global_load_lds_dwordx4), lane l taking slot l's origin by
//      ds_bpermute -- no slot table, no barrier before the window loads;
//   3. one barrier, the MFMAs (A from LDS, B from registers);
//   4. the 4 partial tiles parked in LDS in accumulator layout (16-byte
//      writes and reads, no bank conflicts), summed, bias added, rounded
//      once, transposed through LDS and stored as 16-byte rows.
// Tile t runs on XCD t % 8 and the N tiles of one M tile share it, so a
// window is fetched into one XCD's L2.  With TAIL, the workgroups then copy
// the cache outside the listed blocks (copy_cached), or restore the previous
// edit's blocks (sequential edits), as split by copy_split / restore_split.
#include <type_traits>

#include "conv_common.h"

namespace sige {

// Source of the window vectors that are zero (outside the image, past c_in,
// pad slots): every such lane of a staging load reads these 16 bytes.
__device__ __attribute__((aligned(16))) const u32x4 k_zero16 = {0u, 0u, 0u, 0u};

struct LayerArgs {
    const uint8_t *src;   // edited activation (fused) or stacked input blocks
    const uint8_t *w;     // KRSC weights
    const float *bias;    // fp32 [c_out] or NULL
    const int32_t *idx;   // block list (fused)
    const int32_t *count;
    uint8_t *dst;         // output image (fused) or output blocks
    const uint8_t *cache;          // TAIL: the cached output
    const int32_t *prev_idx;       // TAIL restore: the previous edit's list (NULL: copy)
    const int32_t *prev_count;
    Geo g;
    LayerCfg c;
    CopyCfg cc;
    float *ws;                     // wide tiles split over K: the fp32 partial tiles
    const uint8_t *ww;             // wide tiles: the weights in stage-major order (NULL: from w, KRSC)
    const uint8_t *wp;             // k_layer: the weights in fragment order (NULL: from w, KRSC)
};

__device__ __forceinline__ void layer_tile(const LayerCfg &c, int t, int &tm, int &tn) {
    if (c.xcd) {
        const int r8 = t >> 3;
        tn = r8 % c.ntn;
        tm = (r8 / c.ntn) * 8 + (t & 7);
    } else {
        tn = t % c.ntn;
        tm = t / c.ntn;
    }
}

// Tiles (padding included) for a list of cnt blocks.
template <int BM>
__device__ __forceinline__ int layer_tiles(const LayerCfg &c, int cnt, int b2) {
    const int mtn = (cnt * b2 + BM - 1) / BM;
    return (c.xcd ? (mtn + 7) / 8 * 8 : mtn) * c.ntn;
}

// This wave's weight fragments of the K steps st0, st0 + 1, ... of the chunk
// at input channel c0 (16x16: lane l takes column l % 16 of each N subtile
// and the EPV input channels at (l / 16) * EPV of the step's slice; W32:
// column l % 32, fragment h the channels at 16 h + (l / 32) * EPV).  wcol[nt] is the
// lane's column offset into the weights; the step's tap offset is uniform, so
// each load is a scalar base plus a 32-bit lane offset (column, then channel
// within the tap, both non-negative).  Channels past c_in (a partial last
// chunk, whose later K slices may start past c_in) read the last valid vector
// of the tap: their products meet zeros in the staged windows.  `dummy` points
// every lane at the first fragment instead (one cache line), for a workgroup
// that does not know yet whether it has a tile.
// From the fragment-order copy (wp, see k_layer_weights_pack) the same
// fragments are 1 KiB in a row per load: (chunk, N tile, K step, N subtile),
// 64 lanes of 16 bytes.
template <int DT, int NT, int SMAX, bool W32, bool PK>
__device__ __forceinline__ void layer_weights(const uint8_t *w, const uint8_t *wp, const Geo &g, const LayerCfg &c,
                                              u32x4 (&bfr)[SMAX][NT], const int (&wcol)[NT], int c0, int st0,
                                              int kl, bool dummy, int ch, int tn, int lane) {
    constexpr int ES = elem_bytes(DT), EPV = 16 / ES, KS = MfmaStep<DT>::KS;
    const uint32_t keep = dummy ? 0u : ~0u;  // masks instead of selects: no branches between the loads
    if constexpr (PK) {
        const uint8_t *pb = wp + (size_t)(ch * c.ntn + tn) * c.steps * NT * 1024;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int stp = min(st0 + j, c.steps - 1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                bfr[j][nt] = ld16(pb + ((uint32_t)(((stp * NT + nt) * 64 + lane) * 16) & keep));
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int stp = min(st0 + j, c.steps - 1);
        const int tap = stp >> c.lkpc, cb = c0 + (stp & (c.kpc - 1)) * KS;
        const uint8_t *base = w + ((uint32_t)(tap * g.cin * ES) & keep);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int lch = min(cb + kl + (W32 ? nt * 16 : 0), g.cin - EPV) * ES;  // in [0, c_in * ES)
            bfr[j][nt] = ld16(base + ((uint32_t)(wcol[nt] + lch) & keep));
        }
    }
}

template <int DT, int MT, int NT, bool FUSED, bool TAIL, bool PK>
__global__ __launch_bounds__(kLayerThreads, 2) void k_layer(LayerArgs a) {
    constexpr int NW = kLayerWaves, NTHR = kLayerThreads;
    constexpr int ES = elem_bytes(DT), EPV = 16 / ES;
    constexpr int BM = 16 * MT, BN = 16 * NT, NF = MT * NT;
    constexpr int SMAX = kLayerFrags / NT;  // K steps per wave and chunk (weights in registers)
    constexpr int VPR = BN * ES / 16;       // 16-byte output vectors per tile row
    constexpr bool W32 = DT != 0 && NT == 2;  // 32x32x16 MFMAs: one 32-channel N fragment
    constexpr int MF = W32 ? MT / 2 : MT;     // M fragments (32 or 16 rows)
    constexpr int NH = W32 ? 2 : 1;           // A fragments per M fragment and K step
    static_assert(BM <= 64, "a tile touches at most 64 block slots: one per lane");
    static_assert(!W32 || MT % 2 == 0, "32-row M fragments");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const Geo &g = a.g;
    const LayerCfg &c = a.c;
    // Every argument the tile path reads, in SGPRs at once: one batch of scalar
    // loads instead of a round trip at each first use.
    asm volatile("" ::"s"(a.src), "s"(a.w), "s"(a.bias), "s"(a.idx), "s"(a.count), "s"(a.dst), "s"(g.h), "s"(g.w),
                 "s"(g.cin), "s"(g.cout), "s"(g.k), "s"(g.s), "s"(g.p), "s"(g.b), "s"(g.ho), "s"(g.wo));
    asm volatile("" ::"s"(g.nby), "s"(g.nbx), "s"(g.ib), "s"(g.cap), "s"(c.ck), "s"(c.nch), "s"(c.kpc),
                 "s"(c.lkpc), "s"(c.steps), "s"(c.spw), "s"(c.vpc), "s"(c.ps), "s"(c.rs), "s"(c.gps), "s"(c.sb), "s"(c.ntn),
                 "s"(c.xcd));
    asm volatile("" ::"s"(c.tiles_cap), "s"(c.spec), "s"(c.m_ps), "s"(c.m_rs), "s"(c.m_b2),
                 "s"(c.m_b), "s"(c.gate_min));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib, k2 = g.k * g.k;
    const int mcap = g.cap * b2;  // output rows at capacity
    const int grid = gridDim.x;
    const int st0 = wave * c.spw;                                                     // this wave's K steps
    const int nst = __builtin_amdgcn_readfirstlane(max(0, min(c.steps - st0, c.spw)));  // [st0, st0 + nst)
    const int kl = (W32 ? lane >> 5 : lane >> 4) * EPV;  // this lane's channels within a K slice (half)

    // The list length, as a vector load issued before anything else (cap >> 31
    // is 0: the per-lane address keeps the value in a vector register, so the
    // compiler does not move its wait up to the load).
    const int cnt_raw = a.count[lane & (g.cap >> 31)];
    int cnt = -1, ntiles = -1, mrows = 0;
    int tn_w = -1;  // N tile whose (single-chunk) weights are in the registers
    int lin_next = 0;  // the next tile's block indices, loaded during this tile
    u32x4 bfr[SMAX][NT];

    // LDS layout of a staged window, in 16-byte units: pixel (yy, xx) holds its
    // vpc vectors at yy*rs + xx*ps (ps = vpc + 1: one pad unit per pixel; rs
    // = b mod 16: one pad run per window row), so the 16 rows of an MFMA
    // fragment -- consecutive output pixels of a block, row after row -- fall on
    // 16 different 16-byte bank groups at every tap.  Block slot l's window
    // starts at unit l*sb/16 + (l*b*b mod 16), which continues that pattern
    // across the blocks of a tile.  Wave w stages the 64-unit groups w, w + 4,
    // ... of every block slot's window, one global_load_lds_dwordx4 each.
    // this wave's first K step as (tap column kx, unit offset of the tap in the window, slice)
    int kk0, kx0, toff0;
    {
        const int tap = st0 >> c.lkpc;
        kk0 = st0 & (c.kpc - 1);
        const int ky = tap / g.k;
        kx0 = tap - ky * g.k;
        toff0 = ky * c.rs + kx0 * c.ps;
    }

    // One tile.  The first tile of the workgroup is a separate instantiation
    // (FIRST): its loads before the list length is known are unconditional, so
    // the compiler's wait for the block indices does not cover the weights.
    // Returns false when the workgroup has no more tiles.
    auto tile = [&](int t, auto first_tag) __attribute__((always_inline)) -> bool {
        constexpr bool FIRST = decltype(first_tag)::value;
        int tm, tn;
        layer_tile(c, t, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int mc = min(m0, mcap - 1);  // padding tiles past capacity read the last slot
        const int s_lo = fdiv(mc, c.m_b2);
        const int ns = min(g.cap - 1, fdiv(min(m0 + BM - 1, mcap - 1), c.m_b2)) - s_lo + 1;
        // the first round trip: slot s_lo + lane's block index and the bias of
        // this lane's columns; on the first tile also this wave's weight
        // fragments (the first workgroup of a CU fetches them before the list
        // length is known; the others load one line instead, then the weights
        // once the tile is known to exist)
        const int lin = FUSED ? (FIRST ? a.idx[s_lo + min(lane, ns - 1)] : lin_next) : 0;
        float bcol[NT];
        int wcol[NT];
        const float *bsrc = a.bias ? a.bias : (const float *)a.w;  // any readable floats without a bias
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = min(n0 + (W32 ? lane & 31 : nt * 16 + (lane & 15)), g.cout - 1);
            bcol[nt] = bsrc[col];
            wcol[nt] = col * k2 * g.cin * ES;
        }
        const bool early_w = (int)blockIdx.x < c.spec;
        if constexpr (FIRST) {
            layer_weights<DT, NT, SMAX, W32, PK>(a.w, a.wp, g, c, bfr, wcol, 0, st0, kl, !early_w, 0, tn, lane);
            __builtin_amdgcn_sched_barrier(0);
            cnt = min(max(cnt_raw, 0), g.cap);
            // A launch paired with the split over input channels: a list below
            // gate_min blocks is the split's (the whole layer and the copy); one
            // of gate_wide..wide_max blocks is the wide tiles'.
            ntiles = cnt < c.gate_min || (cnt >= c.gate_wide && cnt <= c.wide_max) ? 0 : layer_tiles<BM>(c, cnt, b2);
            mrows = cnt * b2;
            if (t >= ntiles) return false;
        }
        if (FUSED && t + grid < ntiles) {  // this workgroup's next tile: its block indices, one tile early
            int tm2, tn2;
            layer_tile(c, t + grid, tm2, tn2);
            const int s2 = fdiv(min(tm2 * BM, mcap - 1), c.m_b2);
            const int ns2 = min(g.cap - 1, fdiv(min(tm2 * BM + BM - 1, mcap - 1), c.m_b2)) - s2 + 1;
            lin_next = a.idx[s2 + min(lane, ns2 - 1)];
        }
        if (m0 >= mrows) return true;  // a padding tile
        const bool need_w = FIRST ? !early_w : (c.nch > 1 || tn != tn_w);
        tn_w = c.nch > 1 ? -1 : tn;

        // slot l = lane l's image, window origin and output-block origin
        int sn = -1, siy = 0, six = 0, soy = 0, sox = 0;
        if (FUSED) {
            int n, by, bx;
            if (lane < ns && decode_block(g, lin, n, by, bx)) {
                sn = n;
                siy = by * g.b * g.s - g.p;
                six = bx * g.b * g.s - g.p;
                soy = by * g.b;
                sox = bx * g.b;
            }
        }
        // LDS byte offset of this lane's row in each M fragment (tap 0, this lane's channels)
        int rb[MF];
#pragma unroll
        for (int mt = 0; mt < MF; ++mt) {
            const int r = m0 + (W32 ? mt * 32 + (lane & 31) : mt * 16 + (lane & 15));
            int off = 0;
            if (r < mrows) {
                const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
                const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
                const int l = slot - s_lo;
                off = l * c.sb + (((l * b2) & 15) + py * g.s * c.rs + px * g.s * c.ps) * 16;
            }
            rb[mt] = off + kl * ES;
        }
        f32x4 acc[W32 ? 1 : MT][NT];  // 16x16 fragments
        f32x16 acc32[MF];             // 32x32 fragments (W32)
#pragma unroll
        for (int mt = 0; mt < (W32 ? 1 : MT); ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MF; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc32[mt][v] = 0.f;

        for (int ch = 0; ch < c.nch; ++ch) {
            const int c0 = ch * c.ck;
            const bool full = c0 + c.ck <= g.cin;  // every channel of the chunk exists
            if (ch > 0) __syncthreads();  // every wave is done with the previous chunk's windows
            // Stage the windows (the layout above): this wave fills groups wave + 4 jj
            // of every slot's window, lane i writing 16 bytes at the group's base + 16 i.
            for (int l = 0; l < ns; ++l) {
                const int n = FUSED ? __builtin_amdgcn_readlane(sn, l) : 0;
                const int iy0 = FUSED ? __builtin_amdgcn_readlane(siy, l) : 0;
                const int ix0 = FUSED ? __builtin_amdgcn_readlane(six, l) : 0;
                const bool inner = !FUSED || (n >= 0 && iy0 >= 0 && iy0 + g.ib <= g.h && ix0 >= 0 &&
                                              ix0 + g.ib <= g.w);
                const uint8_t *base =
                    FUSED ? a.src + ((((long)n * g.h + iy0) * g.w + ix0) * g.cin + c0) * (long)ES
                          : a.src + (((size_t)(s_lo + l) * ib2) * g.cin + c0) * ES;
                uint8_t *dst0 = smem + l * c.sb + ((l * b2) & 15) * 16;
                // a compact loop: the same few instruction-cache lines for every group
#pragma unroll 1
                for (int gj = wave; gj < c.gps; gj += NW) {
                    const int u = gj * 64 + lane;  // this lane's unit of the window
                    const int yy = fdiv(u, c.m_rs), rem = u - yy * c.rs;
                    const int xx = fdiv(rem, c.m_ps), cv = rem - xx * c.ps;
                    bool ok = yy < g.ib && xx < g.ib && cv < c.vpc;  // else a pad unit
                    if (!(inner && full))
                        ok = ok && n >= 0 && c0 + cv * EPV < g.cin && iy0 + yy >= 0 && iy0 + yy < g.h &&
                             ix0 + xx >= 0 && ix0 + xx < g.w;
                    const uint32_t off = FUSED ? ((yy * g.w + xx) * g.cin + cv * EPV) * ES
                                               : ((yy * g.ib + xx) * g.cin + cv * EPV) * ES;
                    // every lane loads: its vector, or the zero vector
                    const void *src = ok ? (const void *)(base + off) : (const void *)&k_zero16;
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst0 + gj * 1024),
                                                     16, 0, 0);
                }
            }
            // the weights, when the registers do not hold this chunk's yet
            if (ch > 0 || need_w)
                layer_weights<DT, NT, SMAX, W32, PK>(a.w, a.wp, g, c, bfr, wcol, c0, st0, kl, false, ch, tn, lane);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's windows and weights have landed
            __syncthreads();
            // This wave's K steps: A fragments from LDS, B from registers.  Step
            // j + 1's reads are issued (unconditionally, at the last step's
            // address past the wave's run) while step j's MFMAs run, so every
            // LDS wait is exact.
            {
                int kk = kk0, kx = kx0, toff = toff0;
                u32x4 av[2][MF][NH];
                int ua = (toff + kk * 4) * 16;  // a K slice is 4 units (KS * ES = 64 bytes), a half 2
#pragma unroll
                for (int mt = 0; mt < MF; ++mt)
#pragma unroll
                    for (int h = 0; h < NH; ++h) av[0][mt][h] = *(const u32x4 *)(smem + rb[mt] + ua + h * 32);
#pragma unroll
                for (int j = 0; j < SMAX; ++j) {
                    if (j + 1 < SMAX) {
                        if (j + 1 < nst) {
                            if (++kk == c.kpc) {
                                kk = 0;
                                toff += c.ps;
                                if (++kx == g.k) {
                                    kx = 0;
                                    toff += c.rs - g.k * c.ps;
                                }
                            }
                            ua = (toff + kk * 4) * 16;
                        }
#pragma unroll
                        for (int mt = 0; mt < MF; ++mt)
#pragma unroll
                            for (int h = 0; h < NH; ++h)
                                av[(j + 1) & 1][mt][h] = *(const u32x4 *)(smem + rb[mt] + ua + h * 32);
                    }
                    if (j < nst) {
                        if constexpr (W32) {
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int mt = 0; mt < MF; ++mt)
                                    acc32[mt] = Mfma32<DT>::run(av[j & 1][mt][h], bfr[j][h], acc32[mt]);
                        } else {
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt)
                                    acc[mt][nt] = MfmaStep<DT>::run(av[j & 1][mt][0], bfr[j][nt], acc[mt][nt]);
                        }
                    }
                }
            }
        }

        // Epilogue: park the 4 partial tiles in accumulator layout, sum them per
        // (fragment, lane), add the bias, round, transpose through LDS, store rows.
        __syncthreads();  // every wave is done reading the windows (the partials take their LDS)
        if constexpr (W32) {  // fragment (mt, q) = registers 4q..4q+3 of acc32[mt]
#pragma unroll
            for (int mt = 0; mt < MF; ++mt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(f32x4 *)(smem + (((wave * NF + mt * 4 + q) << 6) + lane) * 16) =
                        f32x4{acc32[mt][4 * q], acc32[mt][4 * q + 1], acc32[mt][4 * q + 2], acc32[mt][4 * q + 3]};
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *(f32x4 *)(smem + (((wave * NF + mt * NT + nt) << 6) + lane) * 16) = acc[mt][nt];
        }
        __syncthreads();
        uint8_t *otile = smem + NW * NF * 64 * 16;  // the rounded tile, [BM][BN] in the storage type
#pragma unroll
        for (int e0 = 0; e0 < NF * 64; e0 += NTHR) {
            const int f = (e0 + tid) >> 6;  // fragment f, lane `lane` of it
            f32x4 s = *(const f32x4 *)(smem + ((f << 6) + lane) * 16);
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const f32x4 v = *(const f32x4 *)(smem + (((w * NF + f) << 6) + lane) * 16);
                s += v;
            }
            int row0, col;  // this lane's first row and its column in the tile
            float bv = bcol[0];
            if constexpr (W32) {
                row0 = (f >> 2) * 32 + (f & 3) * 8 + (lane >> 5) * 4;
                col = lane & 31;
            } else {
                const int mt = f / NT, nt = f - mt * NT;
#pragma unroll
                for (int q = 1; q < NT; ++q) bv = nt == q ? bcol[q] : bv;
                row0 = mt * 16 + (lane >> 4) * 4;
                col = nt * 16 + (lane & 15);
            }
            if (!a.bias) bv = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + i;
                const float v = s[i] + bv;
                if constexpr (DT == 0) {
                    *(float *)(otile + (row * BN + col) * 4) = v;
                } else if constexpr (DT == 1) {
                    *(__bf16 *)(otile + (row * BN + col) * 2) = (__bf16)v;
                } else {
                    *(_Float16 *)(otile + (row * BN + col) * 2) = (_Float16)v;
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < BM * VPR; e += NTHR) {
            const int row = e / VPR, v = e - row * VPR;
            const int r = m0 + row, co = n0 + v * EPV;
            const int slot = fdiv(min(r, mcap - 1), c.m_b2), pix = min(r, mcap - 1) - slot * b2;
            const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
            const u32x4 val = *(const u32x4 *)(otile + row * BN * ES + v * 16);
            if (FUSED) {
                const int l = min(max(slot - s_lo, 0), 63);
                const int pn = __builtin_amdgcn_ds_bpermute(l << 2, sn);
                const int y = __builtin_amdgcn_ds_bpermute(l << 2, soy) + py;
                const int x = __builtin_amdgcn_ds_bpermute(l << 2, sox) + px;
                if (r >= mrows || co >= g.cout || pn < 0 || y >= g.ho || x >= g.wo) continue;
                __builtin_nontemporal_store(
                    val, (u32x4 *)(a.dst + ((((size_t)pn * g.ho + y) * g.wo + x) * g.cout + co) * ES));
            } else {
                if (r >= mrows || co >= g.cout) continue;
                __builtin_nontemporal_store(val, (u32x4 *)(a.dst + (((size_t)slot * b2 + pix) * g.cout + co) * ES));
            }
        }
        __syncthreads();  // the next tile's windows reuse this LDS
        return true;
    };

    if ((int)blockIdx.x < c.tiles_cap && tile(blockIdx.x, std::true_type{})) {
        for (int t = blockIdx.x + grid; t < ntiles; t += grid)
            if (!tile(t, std::false_type{})) break;
    }

    if (TAIL) {
        if (cnt < 0) {  // this workgroup had no tile position at all
            cnt = min(max(cnt_raw, 0), g.cap);
            ntiles = layer_tiles<BM>(c, cnt, b2);
        }
        if (cnt < c.gate_min || (cnt >= c.gate_wide && cnt <= c.wide_max))
            return;  // the split or the wide tiles do this list and the copy
        long long lo, hi;
        if (a.prev_idx) {
            const int np = clamp_count(a.prev_count, g.cap);
            restore_split(np, ntiles, grid, blockIdx.x, lo, hi);
        } else {
            copy_split(a.cc, ntiles, grid, blockIdx.x, lo, hi);
        }
        if (lo < hi) {
            uint32_t *bm = nullptr;
            if (((g.cap + 31) >> 5) * 4 <= c.lds_bytes) {  // bitmap of listed blocks in LDS, else binary search
                bm = (uint32_t *)smem;
                build_bitmap<NTHR>(a.idx, cnt, g.cap, bm);
            }
            if (a.prev_idx)
                restore_slots<NTHR>(g, a.cc, a.prev_idx, (int)lo, 1, (int)hi, bm, a.idx, cnt, a.cache, a.dst);
            else
                copy_span<4, NTHR>(g, a.cc, bm, a.idx, cnt, a.cache, a.dst, lo, hi);
        }
    }
}

// ---------------------------------------------------------------------------
// Wide tiles, for long lists (k_layer_wide).  A workgroup owns 256 output
// rows x 128 output channels and walks K in stages of 16 input channels (one
// 32x32x16 MFMA K step per tap), with both operands in LDS: the windows of the
// tile's block slots and the stage's weights for every tap and the 128
// columns, double-buffered (one workgroup per CU holds both buffers).  Of the
// 8 waves, 4 compute and 4 stage: a wave stalls while the CU's memory path
// accepts its loads (about as long as a stage's MFMAs), so the loading waves
// stage s + 1 while the computing ones run stage s.  Computing wave w takes
// rows 64w .. 64w+63 against all 128 columns (2 x 4 fragments of 32 x 32: 128
// accumulator registers), so each staged weight serves the 4 of them and each
// staged window element one.  Against the 64 x 32 tiles, a window is staged once for 128
// output channels instead of once per 32, and the weights once per 256 rows
// instead of once per 64.
// LDS of one stage, in 16-byte units: pixel (yy, xx) of slot l's window holds
// channels 0-7 and 8-15 of the stage at base_l + yy*w_rs + 3*xx (+0, +1), the
// third unit and each row's tail being padding; with w_rs = 3b mod 16 and
// base_l = l*w_sb + (3*l*b*b mod 16), output row r of the tile reads 3r mod
// 16 plus an offset common to all rows at every tap, so the 16 rows that one
// ds_read_b128 serves together fall on 16 different bank groups (stride 1; 8
// at stride 2).  Weight (tap t, column n, half h) sits at unit
// (128t + n)*2 + (h ^ (n/8 mod 2)), likewise conflict-free for 16 columns.
// Tile t runs on XCD t % 8, the N tiles of one M tile on one XCD.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 8, kWideThreads = 64 * kWideWaves;  // 4 computing + 4 staging waves

template <int DT, bool TAIL>
__global__ __launch_bounds__(kWideThreads, 1) void k_layer_wide(LayerArgs a) {
    constexpr int ES = 2, WR = kLayerWideRows, WC = kLayerWideCols, TP = kLayerWidePitch;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const Geo &g = a.g;
    const LayerCfg &c = a.c;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= 4;  // a staging wave (else a computing one)
    const int cw = wave & 3;         // index among the computing or among the staging waves
    const int b2 = g.b * g.b, k2 = g.k * g.k;
    const int cnt = clamp_count(a.count, g.cap);
    if (cnt < c.wide_min || cnt > c.wide_max) return;  // another kernel's list (with the copy)
    const int mrows = cnt * b2;
    const int mtn = (mrows + WR - 1) / WR;
    const int ntiles = (c.w_ntn > 1 ? (mtn + 7) / 8 * 8 : mtn) * c.w_ntn;
    const int nst = (g.cin + 15) / 16;
    // K parts, for lists whose tiles leave CUs idle: work item (tm*np + part)*w_ntn + tn
    // takes stages st0..st1-1 of tile (tm, tn) and writes its fp32 partial tile
    // to workspace slot `item`; k_wide_combine adds the parts up
    const int np = a.ws ? wide_parts(c.cus, c.w_pmax, mtn * c.w_ntn) : 1;
    const int nitems = np > 1 ? mtn * c.w_ntn * np : ntiles;
    const int nld = (g.ib + c.w_rpi - 1) / c.w_rpi;  // staging loads per slot window
    const int buf_bytes = c.w_wofs + k2 * WC * 32;
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        // the lane index made opaque per tile: values derived from it are
        // recomputed here instead of being hoisted out of the loop and kept live
        // beside the accumulators (which made the kernel spill registers)
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int h = lane >> 5;  // K half: channels 8h .. 8h+7 of the stage
        int tm, tn, part = 0;
        if (np > 1) {
            tn = item % c.w_ntn;
            const int q = item / c.w_ntn;
            part = q % np;
            tm = q / np;
        } else if (c.w_ntn > 1) {
            const int r8 = item >> 3;
            tn = r8 % c.w_ntn;
            tm = (r8 / c.w_ntn) * 8 + (item & 7);
        } else {
            tm = item;
            tn = 0;
        }
        if (tm >= mtn) continue;  // padding of the tile order
        const int st0 = part * nst / np, st1 = (part + 1) * nst / np;
        const int m0 = tm * WR, n0 = tn * WC;
        const int s_lo = fdiv(m0, c.m_b2);
        const int ns = fdiv(min(m0 + WR, mrows) - 1, c.m_b2) - s_lo + 1;  // at most 64 (checked on the host)
        const int lin = a.idx[s_lo + min(lane, ns - 1)];
        int sn = -1, siy = 0, six = 0, soy = 0, sox = 0;  // slot `lane`: image, window and block origins
        {
            int n, by, bx;
            if (lane < ns && decode_block(g, lin, n, by, bx)) {
                sn = n;
                siy = by * g.b * g.s - g.p;
                six = bx * g.b * g.s - g.p;
                soy = by * g.b;
                sox = bx * g.b;
            }
        }
        __syncthreads();  // the previous tile's epilogue is done with the LDS
        if (loader) {
            // Stage st + 1 while stage st is computed; one barrier per stage, as in
            // the computing waves.  The sources of this wave's loads are worked out
            // once per tile: a stage adds 16 channels (32 bytes) to each, so issuing
            // a load costs a select and an add.  Window load q of this wave is
            // it = cw + 4q: rows j*rpi .. of slot l's window (it = l*nld + j); lane
            // i takes unit i from the load's first row (the second row's units
            // start at lane w_rs); lanes on padding are masked off.
            const int second = (c.w_rpi == 2 && lane >= c.w_rs) ? 1 : 0;
            const int rem = lane - second * c.w_rs;
            const int xx = (rem * 43) >> 7, hh = rem - 3 * xx;  // rem / 3, rem % 3 (rem < 64)
            const int nqw = (ns * nld - cw + 3) >> 2;            // <= kLayerWideWinLoads (checked on the host)
            const uint8_t *wsrc[kLayerWideWinLoads];
            int wdst[kLayerWideWinLoads];
            uint32_t wact = 0, wok = 0;  // bit q: the lane holds data / its source lies in the image
#pragma unroll
            for (int q = 0; q < kLayerWideWinLoads; ++q) {
                wsrc[q] = a.src;
                wdst[q] = 0;
                if (q < nqw) {
                    const int it = cw + 4 * q, l = it / nld, j = it - l * nld;
                    const int n = __builtin_amdgcn_readlane(sn, l);
                    const int iy0 = __builtin_amdgcn_readlane(siy, l), ix0 = __builtin_amdgcn_readlane(six, l);
                    const int yy = j * c.w_rpi + second;
                    const bool act = hh < 2 && xx < g.ib && yy < g.ib;
                    const int iy = iy0 + yy, ix = ix0 + xx;
                    const bool ok = act && n >= 0 && iy >= 0 && iy < g.h && ix >= 0 && ix < g.w;
                    if (ok) wsrc[q] = a.src + ((((long)n * g.h + iy) * g.w + ix) * g.cin + 8 * hh) * ES;
                    wdst[q] = (l * c.w_sb + ((3 * l * b2) & 15) + j * c.w_rpi * c.w_rs) * 16;
                    wact |= (uint32_t)act << q;
                    wok |= (uint32_t)ok << q;
                }
            }
            // Weight load q is group gi = cw + 4q of 64 units: unit u = gi*64 + lane
            // holds (tap u/256, column (u/2) mod 128, channel half th), th being the
            // same for every group of a lane.  From KRSC weights a load gathers 32
            // bytes of each of 32 columns and a stage adds 32 bytes to its source;
            // from the stage-major copy (ww: the units of one N tile and stage in
            // this LDS order, padding zero) a load reads 1 KiB in a row and a
            // stage adds k*k KiB x 4.
            const int th = (lane & 1) ^ ((lane >> 4) & 1);
            const uint8_t *tsrc[9];
            uint32_t tok = 0;
            const long wstep = a.ww ? (long)k2 * 4096 : 32;  // bytes a stage adds to a weight source
#pragma unroll
            for (int q = 0; q < 9; ++q) {
                tsrc[q] = a.w;
                if (q < k2) {
                    const int u = (cw + 4 * q) * 64 + lane;
                    const int tap = u >> 8, col = n0 + ((u >> 1) & 127);
                    if (a.ww) {
                        tsrc[q] = a.ww + ((long)tn * nst * k2 * 256 + u) * 16;
                        tok |= 1u << q;
                    } else if (col < g.cout) {
                        tsrc[q] = a.w + (((long)col * k2 + tap) * g.cin + 8 * th) * ES;
                        tok |= 1u << q;
                    }
                }
            }
            const uint8_t *const zero = (const uint8_t *)&k_zero16;
            auto stage = [&](int st, int buf) __attribute__((always_inline)) {
                const long dl = (long)st * 32, dw = (long)st * wstep;
                const bool hi_out = st * 16 + 8 >= g.cin;  // channels 8..15 of the stage past c_in
                uint8_t *const wb = smem + buf * buf_bytes;
#pragma unroll
                for (int q = 0; q < kLayerWideWinLoads; ++q) {
                    if (q < nqw && ((wact >> q) & 1)) {
                        const bool ok = ((wok >> q) & 1) && !(hi_out && hh == 1);
                        __builtin_amdgcn_global_load_lds(ok ? wsrc[q] + dl : zero,
                                                         (__attribute__((address_space(3))) void *)(wb + wdst[q]),
                                                         16, 0, 0);
                    }
                }
#pragma unroll
                for (int q = 0; q < 9; ++q) {
                    if (q < k2) {
                        const bool ok = ((tok >> q) & 1) && !(hi_out && th == 1);
                        __builtin_amdgcn_global_load_lds(
                            ok ? tsrc[q] + dw : zero,
                            (__attribute__((address_space(3))) void *)(wb + c.w_wofs + (cw + 4 * q) * 1024), 16, 0,
                            0);
                    }
                }
            };
            stage(st0, 0);
            for (int st = st0; st < st1; ++st) {
                __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage st have landed
                __syncthreads();                // everyone's; and stage st - 1's reads are done
                if (st + 1 < st1) stage(st + 1, (st + 1 - st0) & 1);
            }
            __syncthreads();  // the computing waves are done reading the last stage
        } else {
            int ua[2];  // LDS unit of this lane's row (and K half) in each M fragment, tap 0
#pragma unroll
            for (int mf = 0; mf < 2; ++mf) {
                const int r = m0 + cw * 64 + mf * 32 + (lane & 31);
                ua[mf] = h;
                if (r < mrows) {
                    const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
                    const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
                    const int l = slot - s_lo;
                    ua[mf] = l * c.w_sb + ((3 * l * b2) & 15) + py * g.s * c.w_rs + px * g.s * 3 + h;
                }
            }
            int ub[4];  // LDS unit of this lane's column (and K half) in each N fragment, tap 0
            float bcol[4];
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) {
                const int n = nf * 32 + (lane & 31);
                ub[nf] = n * 2 + (h ^ ((n >> 3) & 1));
                bcol[nf] = a.bias ? a.bias[min(n0 + n, g.cout - 1)] : 0.f;
            }
            f32x16 acc[2][4];
#pragma unroll
            for (int mf = 0; mf < 2; ++mf)
#pragma unroll
                for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mf][nf][v] = 0.f;
            for (int st = st0; st < st1; ++st) {
                __syncthreads();  // stage st is in LDS
                const uint8_t *const wb = smem + ((st - st0) & 1) * buf_bytes;
                const uint8_t *const wl = wb + c.w_wofs;
                // tap by tap (k <= 3): the next tap's fragments are read while this one's MFMAs run
                u32x4 av[2][2], bv[2][4];
                int ky = 0, kx = 0;
#pragma unroll
                for (int mf = 0; mf < 2; ++mf) av[0][mf] = *(const u32x4 *)(wb + ua[mf] * 16);
#pragma unroll
                for (int nf = 0; nf < 4; ++nf) bv[0][nf] = *(const u32x4 *)(wl + ub[nf] * 16);
#pragma unroll
                for (int tp = 0; tp < 9; ++tp) {
                    if (tp >= k2) continue;
                    if (tp + 1 < k2) {
                        if (++kx == g.k) {
                            kx = 0;
                            ++ky;
                        }
                        const int toff = ky * c.w_rs + kx * 3;
#pragma unroll
                        for (int mf = 0; mf < 2; ++mf)
                            av[(tp + 1) & 1][mf] = *(const u32x4 *)(wb + (ua[mf] + toff) * 16);
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf)
                            bv[(tp + 1) & 1][nf] = *(const u32x4 *)(wl + (ub[nf] + (tp + 1) * 256) * 16);
                    }
#pragma unroll
                    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf)
                            acc[mf][nf] = Mfma32<DT>::run(av[tp & 1][mf], bv[tp & 1][nf], acc[mf][nf]);
                }
            }
            // Epilogue: bias, one rounding, the tile transposed through LDS, 16-byte row stores;
            // a K part: its fp32 partial tile, row-major, to the workspace
            __syncthreads();  // every wave is done reading the last stage
            if (np > 1) {
                float *const wp = a.ws + (size_t)item * (WR * WC) + (cw * 64 + h * 4) * WC + (lane & 31);
#pragma unroll
                for (int mf = 0; mf < 2; ++mf)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf)
                            wp[(mf * 32 + (i >> 2) * 8 + (i & 3)) * WC + nf * 32] = acc[mf][nf][i];
            } else {
#pragma unroll
                for (int mf = 0; mf < 2; ++mf)
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int row = cw * 64 + mf * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
                            const int col = nf * 32 + (lane & 31);
                            const float v = acc[mf][nf][i] + bcol[nf];
                            if constexpr (DT == 1)
                                *(__bf16 *)(smem + row * TP + col * 2) = (__bf16)v;
                            else
                                *(_Float16 *)(smem + row * TP + col * 2) = (_Float16)v;
                        }
            }
        }
        __syncthreads();
        if (np > 1) continue;  // k_wide_combine stores the tile
#pragma unroll
        for (int e0 = 0; e0 < WR * (WC / 8); e0 += kWideThreads) {
            const int e = e0 + tid;
            const int row = e >> 4, v = e & 15;
            const int r = m0 + row, co = n0 + v * 8;
            const int slot = fdiv(min(r, mrows - 1), c.m_b2), pix = min(r, mrows - 1) - slot * b2;
            const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
            const int l = min(max(slot - s_lo, 0), 63);
            const int pn = __builtin_amdgcn_ds_bpermute(l << 2, sn);
            const int y = __builtin_amdgcn_ds_bpermute(l << 2, soy) + py;
            const int x = __builtin_amdgcn_ds_bpermute(l << 2, sox) + px;
            const u32x4 val = *(const u32x4 *)(smem + row * TP + v * 16);
            if (r >= mrows || co >= g.cout || pn < 0 || y >= g.ho || x >= g.wo) continue;
            __builtin_nontemporal_store(val,
                                        (u32x4 *)(a.dst + ((((size_t)pn * g.ho + y) * g.wo + x) * g.cout + co) * ES));
        }
    }

    if (TAIL) {  // the cache outside the listed blocks (copy_cached)
        __syncthreads();
        long long lo, hi;
        copy_split(a.cc, nitems, gridDim.x, blockIdx.x, lo, hi);
        if (lo < hi) {
            uint32_t *bm = nullptr;
            if (((g.cap + 31) >> 5) * 4 <= c.w_lds) {
                bm = (uint32_t *)smem;
                build_bitmap<kWideThreads>(a.idx, cnt, g.cap, bm);
            }
            copy_span<4, kWideThreads>(g, a.cc, bm, a.idx, cnt, a.cache, a.dst, lo, hi);
        }
    }
}

// The K parts of the wide tiles added up: per listed output pixel and 8
// channels, the bias plus the parts' fp32 partials in part order, rounded once.
// Exits at once when the list is not the wide tiles' or makes no K parts.
template <int DT>
__global__ __launch_bounds__(256) void k_wide_combine(LayerArgs a) {
    constexpr int WR = kLayerWideRows, WC = kLayerWideCols, VPR = WC / 8;
    const Geo &g = a.g;
    const LayerCfg &c = a.c;
    const int cnt = clamp_count(a.count, g.cap);
    if (cnt < c.wide_min || cnt > c.wide_max) return;
    const int b2 = g.b * g.b, mrows = cnt * b2;
    const int mtn = (mrows + WR - 1) / WR;
    const int np = wide_parts(c.cus, c.w_pmax, mtn * c.w_ntn);
    if (np < 2) return;
    const long total = (long)mrows * c.w_ntn * VPR;  // (row, N tile, 8 channels)
    for (long u = (long)blockIdx.x * 256 + threadIdx.x; u < total; u += (long)gridDim.x * 256) {
        const int v = (int)(u % VPR);
        const long q = u / VPR;
        const int tn = (int)(q % c.w_ntn), r = (int)(q / c.w_ntn);
        const int co = tn * WC + v * 8;
        if (co >= g.cout) continue;
        const int tm = r / WR, row = r - tm * WR;
        const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
        const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
        // the block index and the first parts are requested together (the
        // parts' addresses do not depend on the index), then the sum
        const int lin = a.idx[slot];
        float sum[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] = a.bias ? a.bias[co + j] : 0.f;
        constexpr int PB = 4;  // parts requested at once
        for (int p0 = 0; p0 < np; p0 += PB) {  // the parts' slots (tm*np + p)*w_ntn + tn, in part order
            f32x4 lo[PB], hi[PB];
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const int p = min(p0 + q, np - 1);
                const float *wp = a.ws + ((size_t)((tm * np + p) * c.w_ntn + tn) * WR + row) * WC + v * 8;
                lo[q] = *(const f32x4 *)wp;
                hi[q] = *(const f32x4 *)(wp + 4);
            }
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                if (p0 + q >= np) break;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sum[j] += lo[q][j];
                    sum[4 + j] += hi[q][j];
                }
            }
        }
        int n, by, bx;
        if (!decode_block(g, lin, n, by, bx)) continue;
        const int y = by * g.b + py, x = bx * g.b + px;
        if (y >= g.ho || x >= g.wo) continue;
        store_row8<DT>(a.dst + ((((size_t)n * g.ho + y) * g.wo + x) * g.cout + co) * 2, sum, true);
    }
}

template <int DT, bool TAIL>
static hipError_t launch_wide_k(const LayerArgs &args, hipStream_t st) {
    auto k = k_layer_wide<DT, TAIL>;
    const LayerCfg &c = args.c;
    long grid = c.cus;  // one workgroup per CU (both LDS buffers)
    if (!TAIL && c.w_pmax < 2 && c.w_tiles_cap < grid) grid = c.w_tiles_cap;
    if (grid > 8) grid = grid / 8 * 8;
    hipLaunchKernelGGL(k, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kWideThreads), c.w_lds, st, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !args.ws) return e;
    const long rows = (long)c.w_ws_items * kLayerWideRows * (kLayerWideCols / 8);  // (row, 8 channels) at most
    long cgrid = (rows + 255) / 256;
    if (cgrid > 4L * c.cus) cgrid = 4L * c.cus;
    hipLaunchKernelGGL(k_wide_combine<DT>, dim3((unsigned)(cgrid > 0 ? cgrid : 1)), dim3(256), 0, st, args);
    return hipGetLastError();
}

hipError_t launch_layer_wide(int dt, const void *src, const void *w, const float *bias, const int32_t *idx,
                             const int32_t *count, void *dst, const void *cache, const Geo &g, const LayerCfg &cfg,
                             const CopyCfg &cc, hipStream_t st, float *ws, const void *ww) {
    const LayerArgs a{(const uint8_t *)src, (const uint8_t *)w, bias, idx, count, (uint8_t *)dst,
                      (const uint8_t *)cache, nullptr, nullptr, g, cfg, cc, cfg.w_pmax > 1 ? ws : nullptr,
                      (const uint8_t *)ww};
    const bool tail = cc.nvec > 0;
    if (dt == 1) return tail ? launch_wide_k<1, true>(a, st) : launch_wide_k<1, false>(a, st);
    return tail ? launch_wide_k<2, true>(a, st) : launch_wide_k<2, false>(a, st);
}

// The stage-major copy of KRSC weights that the wide tiles stage from: for N
// tile tn (128 output channels), stage s (16 input channels), tap t, column n
// and channel half h, the 8 channels 16s + 8h .. of output channel 128 tn + n
// at tap t sit at 16-byte unit ((tn * nst + s) * k*k + t) * 256 + 2n +
// (h ^ (n/8 mod 2)) -- the order of the stage's weights in LDS -- and zeros
// stand for output channels past c_out and input channels past c_in.  One
// thread per unit; c_in is a multiple of 8, so a unit is all valid or all zero.
__global__ __launch_bounds__(256) void k_wide_weights_pack(const uint8_t *__restrict__ w, Geo g, uint8_t *ww,
                                                           long units) {
    const int k2 = g.k * g.k, nst = (g.cin + 15) / 16;
    for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < units; v += (long)gridDim.x * 256) {
        const int u = (int)(v % (k2 * 256));
        const long ts = v / (k2 * 256);
        const int s = (int)(ts % nst), tn = (int)(ts / nst);
        const int tap = u >> 8, n = (u >> 1) & 127, h = (u & 1) ^ ((n >> 3) & 1);
        const int col = tn * kLayerWideCols + n, ch = s * 16 + h * 8;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (col < g.cout && ch < g.cin) x = ld16(w + (((size_t)col * k2 + tap) * g.cin + ch) * 2);
        *(u32x4 *)(ww + v * 16) = x;
    }
}

// The fragment-order copy of KRSC weights that k_layer loads from: for chunk
// ch, N tile tn (16*nt output channels), K step s of the chunk, N subtile q
// and lane l, the 16 bytes layer_weights would load from the KRSC weights
// (clamped columns and channels included, so the MFMAs see the same values)
// at unit (((ch * ntn + tn) * steps + s) * nt + q) * 64 + l.  One thread per unit.
__global__ __launch_bounds__(256) void k_layer_weights_pack(const uint8_t *__restrict__ w, Geo g, LayerCfg c, int dt,
                                                            uint8_t *wp, long units) {
    const int es = elem_bytes(dt), epv = 16 / es, ks = dt == 0 ? 16 : 32;
    const bool w32 = dt != 0 && c.nt == 2;
    const int k2 = g.k * g.k;
    for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < units; v += (long)gridDim.x * 256) {
        const int l = (int)(v & 63);
        long q = v >> 6;
        const int nt = (int)(q % c.nt);
        q /= c.nt;
        const int s = (int)(q % c.steps);
        q /= c.steps;
        const int tn = (int)(q % c.ntn), ch = (int)(q / c.ntn);
        const int n0 = tn * 16 * c.nt;
        const int tap = s >> c.lkpc, cb = ch * c.ck + (s & (c.kpc - 1)) * ks;
        const int kl = (w32 ? l >> 5 : l >> 4) * epv;
        const int col = min(n0 + (w32 ? l & 31 : nt * 16 + (l & 15)), g.cout - 1);
        const int lch = min(cb + kl + (w32 ? nt * 16 : 0), g.cin - epv);
        *(u32x4 *)(wp + v * 16) = ld16(w + (((size_t)col * k2 + tap) * g.cin + lch) * es);
    }
}

long layer_weights_units(const Geo &g, const LayerCfg &c) { return (long)c.nch * c.ntn * c.steps * c.nt * 64; }

hipError_t launch_layer_weights_pack(int dt, const void *w, const Geo &g, const LayerCfg &c, void *wp, int cus,
                                     hipStream_t st) {
    const long units = layer_weights_units(g, c);
    long grid = (units + 255) / 256;
    if (grid > 4L * cus) grid = 4L * cus;
    hipLaunchKernelGGL(k_layer_weights_pack, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, st,
                       (const uint8_t *)w, g, c, dt, (uint8_t *)wp, units);
    return hipGetLastError();
}

long wide_weights_units(const Geo &g) {
    return (long)((g.cout + kLayerWideCols - 1) / kLayerWideCols) * ((g.cin + 15) / 16) * g.k * g.k * 256;
}

hipError_t launch_wide_weights_pack(const void *w, const Geo &g, void *ww, int cus, hipStream_t st) {
    const long units = wide_weights_units(g);
    long grid = (units + 255) / 256;
    if (grid > 4L * cus) grid = 4L * cus;
    hipLaunchKernelGGL(k_wide_weights_pack, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, st,
                       (const uint8_t *)w, g, (uint8_t *)ww, units);
    return hipGetLastError();
}

// Workgroups of `kernel` resident on one CU with `lds` bytes of dynamic LDS
// (register and LDS limits), from the runtime; cached per kernel and size.
template <typename K>
static int layer_resident(K kernel, int lds) {
    struct Entry {
        const void *k;
        int lds, n;
    };
    static thread_local Entry cache[32];
    static thread_local int used = 0;
    for (int i = 0; i < used; ++i)
        if (cache[i].k == (const void *)kernel && cache[i].lds == lds) return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kLayerThreads, lds) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    cache[used < 32 ? used++ : 31] = Entry{(const void *)kernel, lds, n};
    return n;
}

template <int DT, int MT, int NT, bool FUSED, bool TAIL, bool PK = false>
static hipError_t launch_layer_k(const LayerArgs &args, hipStream_t st) {
    auto k = k_layer<DT, MT, NT, FUSED, TAIL, PK>;
    const LayerCfg &c = args.c;
    long grid = (long)c.cus * layer_resident(k, c.lds_bytes);
    if (!TAIL && c.tiles_cap < grid) grid = c.tiles_cap;  // nothing past the tiles at capacity
    if (grid > 8) grid = grid / 8 * 8;                     // keep tile t on XCD t % 8 across passes
    LayerArgs a = args;
    // the first workgroup of each CU; none when the launch is gated (most of
    // its lists may be the split's, and the weights would be fetched for nothing)
    a.c.spec = c.gate_min > 0 ? 0 : (int)(grid < c.cus ? grid : c.cus);
    hipLaunchKernelGGL(k, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kLayerThreads), c.lds_bytes, st, a);
    return hipGetLastError();
}

template <int DT, int MT, int NT>
static hipError_t launch_layer_t(int fused, bool tail, const LayerArgs &a, hipStream_t st) {
    if (!fused)
        return a.wp ? launch_layer_k<DT, MT, NT, false, false, true>(a, st) : launch_layer_k<DT, MT, NT, false, false>(a, st);
    if (a.wp)  // the weights from the fragment-order copy
        return tail ? launch_layer_k<DT, MT, NT, true, true, true>(a, st)
                    : launch_layer_k<DT, MT, NT, true, false, true>(a, st);
    return tail ? launch_layer_k<DT, MT, NT, true, true>(a, st) : launch_layer_k<DT, MT, NT, true, false>(a, st);
}

template <int DT>
static hipError_t launch_layer_dt(int fused, bool tail, const LayerArgs &a, hipStream_t st) {
    switch (a.c.mt * 10 + a.c.nt) {
    case 42: return launch_layer_t<DT, 4, 2>(fused, tail, a, st);
    case 41: return launch_layer_t<DT, 4, 1>(fused, tail, a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_layer(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                        const int32_t *count, void *dst, const void *cache, const int32_t *prev_idx,
                        const int32_t *prev_count, const Geo &g, const LayerCfg &cfg, const CopyCfg &cc,
                        hipStream_t st, const void *wp) {
    const LayerArgs a{(const uint8_t *)src, (const uint8_t *)w, bias, idx, count, (uint8_t *)dst,
                      (const uint8_t *)cache, prev_idx, prev_count, g, cfg, cc, nullptr, nullptr,
                      (const uint8_t *)wp};
    const bool tail = fused && (cc.nvec > 0 || prev_idx);
    switch (dt) {
    case 0: return launch_layer_dt<0>(fused, tail, a, st);
    case 1: return launch_layer_dt<1>(fused, tail, a, st);
    default: return launch_layer_dt<2>(fused, tail, a, st);
    }
}

}  // namespace sige
