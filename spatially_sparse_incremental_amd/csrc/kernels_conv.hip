// kernels_conv.hip -- steps 3 and 5 (gather, scatter), the restore of
// sequential edits, and the fused layer split over input channels, on gfx950.
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
#include "conv_common.h"

namespace sige {

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
// The fused layer split over input channels (weight-bound layers), an
// implicit GEMM on the matrix cores like k_layer (kernels_layer.hip, which
// runs the unsplit layer and the block convolution):
//   M = listed blocks x b*b output pixels (flattened over all blocks, so tiles
//       are not padded per block), N = c_out, K = k*k*c_in.
// Workgroups of 8 waves walk tiles of 16*MT rows x 16*NT output channels.  The
// 8 waves split each chunk's K steps (tap, one 32-channel slice; 16 for fp32)
// round robin and each accumulates the whole tile; the eight partial tiles
// are summed through LDS at the end.
//   - Weights: a wave's B fragments are used by that wave only, so they go
//     straight from global memory (L2-resident) into registers, up to SMAX
//     steps per chunk.
//   - Input windows: every wave reads every row, so the halo windows of the
//     block slots a tile touches are staged once in LDS, loaded from global
//     memory straight into LDS (global_load_lds_dwordx4), zero outside the
//     image.
// MFMA: v_mfma_f32_16x16x32_{bf16,f16} (fp32: four v_mfma_f32_16x16x4_f32).
// ---------------------------------------------------------------------------
struct ConvArgs {
    const uint8_t *src;
    const uint8_t *w;
    const float *bias;
    const int32_t *idx;
    const int32_t *count;
    uint8_t *dst;
    const uint8_t *cache;
    const int32_t *prev_idx;    // restore mode: the previous edit's list (NULL: none)
    const int32_t *prev_count;
    float *ws;                  // split mode: fp32 partial tiles (NULL otherwise)
    Geo g;
    ConvCfg c;
    CopyCfg cc;
    const uint8_t *wp;          // split mode: the weights in fragment order (NULL: from w, KRSC)
};

// Split over input channels (the fused layer with a workspace): a work item
// is (group of R consecutive M tiles, range of cpk chunks of input channels,
// N tile).  For each chunk of its range it reads its weight fragments once and
// walks every M tile of the group, so the weights cross the chip once per
// group instead of once per M tile, and the chunks spread one layer's weights
// over many CUs.  Each (M tile, N tile, chunk) leaves an fp32 partial tile;
// the combine adds a tile's chunks in order.  When N tiles x chunks fit in the
// resident slots, a range is one chunk and the groups take the rest of the
// slots (G = slots / (N tiles x chunks), at most one per M tile, evened out);
// otherwise there is one group and as many ranges as the slots allow.  A
// group of one M tile with several chunks per range (acc_range) keeps its
// accumulators over the range and leaves one partial tile per range, at the
// range's first chunk.  Without room for a second LDS buffer of windows
// (dbuf), and when chunk ranges are needed for at most 4 M tiles (streaming
// would reuse each chunk's weights at most 4 times but pay an epilogue per M
// tile and chunk), every group is one M tile.  Both kernels derive the same
// plan from the list length (its arithmetic runs at the start of both
// launches, on the path to the first loads, so it is kept short).  Window group = (group,
// range): the items that stage the same windows.  With at least 8 window
// groups (and no extra round of positions from the padding), position
// p = 8 * (tn + ntn * (wg / 8)) + wg % 8 puts every N tile of window group wg
// on XCD wg % 8, so those windows are fetched into one L2.
struct StreamPlan {
    int mtn, ntn, nch;  // M tiles, N tiles, chunks
    int R, G;           // M tiles per group, groups
    int cpk, S;         // chunks per range, ranges
    int nwg;            // window groups (G * S)
    bool acc_range;     // one partial tile per range (R == 1, cpk > 1)
    bool xcd;
    int positions;      // work positions, padding included
};
// Whether the launch's LDS holds two buffers of windows next to the partial
// tiles of NW waves (see k_conv_stream).
__device__ __forceinline__ bool stream_dbuf(const ConvCfg &c, int bm, int bn, int nw) {
    const int pbytes = nw * bm * (bn + 4) * 4;
    return c.lds_bytes >= (c.a_bytes > pbytes ? c.a_bytes : pbytes) + c.a_bytes;
}

__device__ __forceinline__ StreamPlan stream_plan(int cnt, int b2, int bm, int ntn, int nch, int slots, bool dbuf) {
    StreamPlan p;
    p.mtn = (cnt * b2 + bm - 1) / bm;
    p.ntn = ntn;
    p.nch = nch;
    const int mt = max(p.mtn, 1);
    int G = 1, S = nch;
    if (dbuf && ntn * nch <= slots)
        G = min(slots / max(ntn * nch, 1), mt);
    else if (!dbuf || mt <= 4)
        G = mt;  // one M tile per group, chunk ranges in the accumulators
    if (G * ntn * nch > slots) S = max(1, min(nch, slots / max(G * ntn, 1)));
    p.cpk = (nch + S - 1) / S;
    p.S = (nch + p.cpk - 1) / p.cpk;  // evened: no empty range
    p.R = (mt + G - 1) / G;
    p.G = p.mtn > 0 ? (p.mtn + p.R - 1) / p.R : 0;  // 0 for an empty list
    p.nwg = p.G * p.S;
    p.acc_range = p.R == 1 && p.cpk > 1;
    const int padded = (p.nwg + 7) / 8 * 8 * ntn;
    p.xcd = p.nwg >= 8 && (p.nwg % 8 == 0 || padded <= slots);
    p.positions = p.xcd ? padded : p.nwg * ntn;
    return p;
}

constexpr int kConvWaves = 8;  // waves per workgroup of the implicit GEMM
constexpr int kConvThreads = 64 * kConvWaves;

// This wave's weight fragments for the chunk at input channel c0: K steps
// wave, wave + 8, ... (tap, KS-channel slice), 16 output channels per N
// subtile.  Unconditional loads at clamped addresses (the convolution zeroes
// fragments outside the weight tensor where it uses them).
template <int DT, int NT, int SMAX, bool PK>
__device__ __forceinline__ void load_weights(const ConvArgs &a, u32x4 (&bfr)[SMAX][NT], int c0, int n0, int wave,
                                             int lane, int steps, int kpc) {
    constexpr int ES = elem_bytes(DT), EPV = 16 / ES, KS = MfmaStep<DT>::KS;
    const Geo &g = a.g;
    if constexpr (PK) {  // from the fragment-order copy: (chunk, N tile, K step, N subtile) x 64 lanes
        const int ntn = (g.cout + 16 * NT - 1) / (16 * NT);
        const uint8_t *pb = a.wp + (size_t)((c0 / a.c.ck) * ntn + n0 / (16 * NT)) * steps * NT * 1024;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int stp = min(wave + kConvWaves * j, steps - 1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bfr[j][nt] = ld16(pb + ((stp * NT + nt) * 64 + lane) * 16);
        }
        return;
    }
    const int k2 = g.k * g.k, kl = (lane >> 4) * EPV;
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int stp = min(wave + kConvWaves * j, steps - 1);
        const int tap = stp / kpc, kk = stp - tap * kpc;
        const int cb = min(c0 + kk * KS + kl, g.cin - EPV);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = min(n0 + nt * 16 + (lane & 15), g.cout - 1);
            bfr[j][nt] = ld16(a.w + (((size_t)col * k2 + tap) * g.cin + cb) * ES);
        }
    }
}

// K steps per wave and chunk whose weight fragments a wave holds in registers
template <int NT>
struct Smax {
    static constexpr int v = 10 / NT;
};

// Stage the input windows of one M tile's block slots for the channels
// [c0, c0 + ck) into LDS at As, straight from global memory
// (global_load_lds_dwordx4: no registers, every load in flight at once).  Each
// wave fills 64 consecutive 16-byte slots per instruction (lane i -> slot base
// + i; a pixel occupies vpc slots plus one pad slot, left unwritten).  Slots
// outside the image or beyond c_in get zeros from their own lane.  Batches of
// QB slot groups per wave: decode, then every slot-table read of the batch,
// then every load.  t_n, t_iy, t_ix: image and window origin per block slot
// (fused); the stacked block tensor starts at slot s_lo otherwise.
template <int DT, bool FUSED>
__device__ __forceinline__ void stage_windows(const ConvArgs &a, uint8_t *As, const int *t_n, const int *t_iy,
                                              const int *t_ix, int c0, int nslot, int s_lo, int wave, int lane) {
    constexpr int NW = kConvWaves, ES = elem_bytes(DT), EPV = 16 / ES, QB = 4;
    const Geo &g = a.g;
    const ConvCfg &c = a.c;
    const int vpc = c.ck / EPV, ib2 = g.ib * g.ib;
    const int nq = (nslot + 63) / 64;  // 64-slot groups, one wave instruction each
    for (int qb = wave; qb < nq; qb += NW * QB) {
        int ls[QB], pix[QB], chv[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const int slot = (qb + NW * i) * 64 + lane;
            const int P = fdiv(slot, c.m_vpc1), cvv = slot - P * (vpc + 1);
            const bool act = slot < nslot && cvv < vpc;
            const int l = FUSED ? fdiv(P, c.m_ib2) : 0;
            ls[i] = act ? l : -1;
            pix[i] = FUSED ? P - l * ib2 : P;
            chv[i] = c0 + cvv * EPV;
        }
        int tn_[QB], ty[QB], tx[QB];
        if (FUSED) {
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                const int l = max(ls[i], 0);
                tn_[i] = t_n[l];
                ty[i] = t_iy[l];
                tx[i] = t_ix[l];
            }
        }
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            if (ls[i] < 0) continue;
            const int q = qb + NW * i;
            const uint8_t *src = nullptr;
            if (chv[i] < g.cin) {
                if (FUSED) {
                    const int yy = fdiv(pix[i], c.m_ib), xx = pix[i] - yy * g.ib;
                    const int iy = ty[i] + yy, ix = tx[i] + xx;
                    if (tn_[i] >= 0 && iy >= 0 && iy < g.h && ix >= 0 && ix < g.w)
                        src = a.src + ((((size_t)tn_[i] * g.h + iy) * g.w + ix) * g.cin + chv[i]) * ES;
                } else {
                    src = a.src + (((size_t)s_lo * ib2 + pix[i]) * g.cin + chv[i]) * ES;
                }
            }
            if (src)
                __builtin_amdgcn_global_load_lds((const void *)src,
                                                 (__attribute__((address_space(3))) void *)(As + q * 1024), 16, 0, 0);
            else
                st16(As + (q * 64 + lane) * 16, u32x4{0u, 0u, 0u, 0u});
        }
    }
}

// LDS byte offset of this lane's row in each M subtile of the tile at row m0
// (tap (0,0), channel 0) inside the windows staged from slot s_lo; rows at or
// past mrows read slot 0's first pixel (their results are never stored).
template <int MT>
__device__ __forceinline__ void row_offsets(const Geo &g, const ConvCfg &c, int m0, int mrows, int s_lo, int lane,
                                            int (&rb)[MT]) {
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = m0 + mt * 16 + (lane & 15);
        int off = 0;
        if (r < mrows) {
            const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
            const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
            off = ((slot - s_lo) * ib2 + py * g.s * g.ib + px * g.s) * c.a_pix_stride;
        }
        rb[mt] = off;
    }
}

// This wave's K steps of one chunk (wave, wave + 8, ...) on the staged
// windows: A fragments from LDS (rows at byte offsets rb), B fragments from
// registers (zero outside c_in and c_out).  The A fragments of step j + 1 are
// read from LDS while step j's MFMAs run.
template <int DT, int MT, int NT, int SMAX>
__device__ __forceinline__ void mfma_chunk(const ConvArgs &a, const uint8_t *As, const int (&rb)[MT],
                                           const u32x4 (&bfr)[SMAX][NT], f32x4 (&acc)[MT][NT], int c0, int n0,
                                           int wave, int lane, int steps, int kpc) {
    constexpr int NW = kConvWaves, ES = elem_bytes(DT), EPV = 16 / ES, KS = MfmaStep<DT>::KS;
    const Geo &g = a.g;
    const int apix = a.c.a_pix_stride, kl = (lane >> 4) * EPV;
    u32x4 av[2][MT];
    auto read_a = [&](int j, u32x4 (&dst)[MT]) {
        const int stp = min(wave + NW * j, steps - 1);
        const int tap = stp / kpc, kk = stp - tap * kpc;
        const int ky = tap / g.k, kx = tap - ky * g.k;
        const int aoff = (ky * g.ib + kx) * apix + (kk * KS + kl) * ES;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dst[mt] = *(const u32x4 *)(As + rb[mt] + aoff);
    };
    if (wave < steps) read_a(0, av[0]);
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int stp = wave + NW * j;
        if (stp >= steps) break;
        if (j + 1 < SMAX && stp + NW < steps) read_a(j + 1, av[(j + 1) & 1]);
        const int kk = stp - (stp / kpc) * kpc;
        const bool kin = c0 + kk * KS + kl < g.cin;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = MfmaStep<DT>::run(
                    av[j & 1][mt], (kin && n0 + nt * 16 + (lane & 15) < g.cout) ? bfr[j][nt] : u32x4{0u, 0u, 0u, 0u},
                    acc[mt][nt]);
    }
}

// Every wave parks its partial tile in LDS (16x16 accumulator layout: lane l
// holds rows 4*(l/16)+i, column l%16), rows of PSTR floats, wave-major.
template <int MT, int NT, int PSTR>
__device__ __forceinline__ void park_partials(float *part, const f32x4 (&acc)[MT][NT], int wave, int lane) {
    constexpr int BM = 16 * MT;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[(wave * BM + mt * 16 + (lane >> 4) * 4 + i) * PSTR + nt * 16 + (lane & 15)] = acc[mt][nt][i];
}

// A workgroup barrier for LDS accesses only.  Each wave waits for its own LDS
// accesses (s_waitcnt lgkmcnt(0)); the empty asm statements keep the compiler
// from moving memory accesses across the barrier.  Global loads in flight (the
// next tile's windows, on their way into the other LDS buffer) and global
// stores are not waited for, as the fences of __syncthreads would.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maximum
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The split over input channels (see StreamPlan).  A work item walks its
// group's M tiles with the windows double-buffered in LDS: while tile i's MFMAs
// run, tile i + 1's windows are in flight into the other buffer and tile
// i + 2's block indices into registers.  Per M tile the eight waves' partial
// tiles are summed through LDS and the chunk's fp32 sum goes to the workspace
// (non-temporal stores, issued one tile later so that no wait covers them
// early): partial (M tile tm, N tile tn, chunk ks) at
// ((tm * ntn + tn) * nch + ks) * BM * BN.
// LDS: buffer 0 at 0, buffer 1 at max(W, P), where W is one buffer of windows
// and P the eight partial tiles; the partial tiles of the tile staged in buffer
// b start at b * W, so they overlap only the buffer whose windows are consumed.
// When the launch has no room for buffer 1 (large halos), the plan gives every
// group one M tile, so no tile is staged while another is computed.
// The slot table (image and window origin per block slot) has two copies: one
// for the group's first tile, kept for every chunk of the range, and one for
// the others (written for tile i + 1 after every wave has passed the barriers
// that follow its last read, the staging of tile i).
template <int DT, int MT, int NT, bool PK>
__global__ __launch_bounds__(kConvThreads, 2) void k_conv_stream(ConvArgs a) {
    constexpr int NTHR = kConvThreads;
    constexpr int ES = elem_bytes(DT), EPV = 16 / ES, KS = MfmaStep<DT>::KS;
    constexpr int BM = 16 * MT, BN = 16 * NT;
    constexpr int PSTR = BN + 4;
    constexpr int SMAX = Smax<NT>::v;
    constexpr int VPR = BN / 8;
    static_assert(BM <= 64, "wave 0 fills the slot table: at most 64 slots per tile");
    static_assert(BM * VPR <= NTHR, "one output vector per thread");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_n[2][BM + 1], s_iy[2][BM + 1], s_ix[2][BM + 1];

    const Geo &g = a.g;
    const ConvCfg &c = a.c;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib, k2 = g.k * g.k;
    const int ntn = (g.cout + BN - 1) / BN;
    const int vpc = c.ck / EPV, kpc = c.ck / KS, steps = k2 * kpc;
    const int nch = (g.cin + c.ck - 1) / c.ck;
    const int wbytes = c.a_bytes;                          // one buffer of windows
    const int pbytes = kConvWaves * BM * PSTR * 4;         // the eight partial tiles
    const bool dbuf = stream_dbuf(c, BM, BN, kConvWaves);  // two buffers of windows
    const int buf1 = dbuf ? (wbytes > pbytes ? wbytes : pbytes) : 0;  // byte offset of buffer 1
    const int cnt = clamp_count(a.count, g.cap);
    if (cnt > c.gate_max) return;  // paired with the single-range layer, which takes longer lists
    const int mrows = cnt * b2;
    const StreamPlan pl = stream_plan(cnt, b2, BM, ntn, nch, gridDim.x, dbuf);

    // the block slots of M tile tm: the first, and how many
    auto slots_of = [&](int tm, int &s_lo, int &ns) {
        const int m0 = tm * BM;
        s_lo = fdiv(m0, c.m_b2);
        ns = min(g.cap - 1, fdiv(m0 + BM - 1, c.m_b2)) - s_lo + 1;
    };
    // wave 0: lane l's block index of M tile tm (an unconditional read at a clamped slot)
    auto read_lin = [&](int tm) {
        int s_lo, ns;
        slots_of(tm, s_lo, ns);
        return a.idx[s_lo + min(lane, ns - 1)];
    };
    auto fill_table = [&](int tm, int lin, int tb) {
        int s_lo, ns;
        slots_of(tm, s_lo, ns);
        if (lane < ns) {
            int n, by, bx;
            if (!decode_block(g, lin, n, by, bx)) n = -1;
            s_n[tb][lane] = n;
            s_iy[tb][lane] = by * g.b * g.s - g.p;
            s_ix[tb][lane] = bx * g.b * g.s - g.p;
        }
    };
    auto stage = [&](int tm, int tb, uint8_t *buf, int c0) {
        int s_lo, ns;
        slots_of(tm, s_lo, ns);
        stage_windows<DT, true>(a, buf, s_n[tb], s_iy[tb], s_ix[tb], c0, ns * ib2 * (vpc + 1), s_lo, wave, lane);
    };

    for (int p = blockIdx.x; p < pl.positions; p += gridDim.x) {
        int tn, wg;
        if (pl.xcd) {
            const int r8 = p >> 3;
            tn = r8 % ntn;
            wg = (r8 / ntn) * 8 + (p & 7);
        } else {
            tn = p % ntn;
            wg = p / ntn;
        }
        if (wg >= pl.nwg) continue;  // padding
        const int grp = wg / pl.S, rng = wg - grp * pl.S;
        const int tm0 = grp * pl.R, tm1 = min(pl.mtn, tm0 + pl.R);
        const int n0 = tn * BN;
        __syncthreads();  // the previous item is done with LDS and the slot tables
        if (wave == 0) {  // the first tile's slot table, for every chunk of the range
            const int lin0 = read_lin(tm0);
            fill_table(tm0, lin0, 0);
        }
        const int ks0 = rng * pl.cpk, ks1 = min(nch, ks0 + pl.cpk);
        f32x4 acc[MT][NT];
        for (int ks = ks0; ks < ks1; ++ks) {
            const int c0 = ks * c.ck;
            __syncthreads();  // the first slot table is visible; the previous chunk is done with LDS
            // one round trip: this wave's weight fragments for the chunk (kept for
            // every M tile of the group), the first tile's windows and wave 0's
            // block indices of the second tile
            u32x4 bfr[SMAX][NT];
            load_weights<DT, NT, SMAX, PK>(a, bfr, c0, n0, wave, lane, steps, kpc);
            int lin = 0;
            if (wave == 0 && tm0 + 1 < tm1) lin = read_lin(tm0 + 1);
            stage(tm0, 0, smem, c0);
            // this thread's output vector of the previous tile, stored one tile later
            float *pend = nullptr;
            f32x4 plo{0.f, 0.f, 0.f, 0.f}, phi{0.f, 0.f, 0.f, 0.f};
            const int row = tid / VPR, col = (tid - row * VPR) * 8;
            for (int tm = tm0, i = 0; tm < tm1; ++tm, ++i) {
                const int cur = i & 1;
                uint8_t *As = smem + cur * buf1;
                __builtin_amdgcn_s_waitcnt(0);  // this tile's windows, the weights, the next block indices
                if (pend) {
                    __builtin_nontemporal_store(plo, (f32x4 *)pend);
                    __builtin_nontemporal_store(phi, (f32x4 *)(pend + 4));
                    pend = nullptr;
                }
                if (wave == 0 && tm + 1 < tm1) fill_table(tm + 1, lin, 1);
                lds_barrier();  // windows and the next slot table visible; the other buffer is free
                if (tm + 1 < tm1) stage(tm + 1, 1, smem + (cur ^ 1) * buf1, c0);
                if (wave == 0 && tm + 2 < tm1) lin = read_lin(tm + 2);
                int s_lo, ns;
                slots_of(tm, s_lo, ns);
                int rb[MT];
                row_offsets<MT>(g, c, tm * BM, mrows, s_lo, lane, rb);
                if (!pl.acc_range || ks == ks0) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                mfma_chunk<DT, MT, NT, SMAX>(a, As, rb, bfr, acc, c0, n0, wave, lane, steps, kpc);
                if (pl.acc_range && ks + 1 < ks1) continue;  // the range goes on in the accumulators
                lds_barrier();  // every wave is done reading this tile's windows
                float *part = (float *)(smem + (dbuf ? cur * wbytes : 0));
                park_partials<MT, NT, PSTR>(part, acc, wave, lane);
                lds_barrier();
                if (tid < BM * VPR && tm * BM + row < mrows && n0 + col < g.cout) {
                    float sum[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float x = 0.f;
#pragma unroll
                        for (int w = 0; w < kConvWaves; ++w) x += part[(w * BM + row) * PSTR + col + j];
                        sum[j] = x;
                    }
                    const size_t tile = (size_t)tm * ntn + tn;
                    const int kout = pl.acc_range ? ks0 : ks;
                    pend = a.ws + (((tile * nch + kout) * BM + row) * BN + col);
                    plo = f32x4{sum[0], sum[1], sum[2], sum[3]};
                    phi = f32x4{sum[4], sum[5], sum[6], sum[7]};
                }
            }
            if (pend) {
                __builtin_nontemporal_store(plo, (f32x4 *)pend);
                __builtin_nontemporal_store(phi, (f32x4 *)(pend + 4));
            }
        }
    }
}

// The end of the split: for each listed output row and 8 output channels, the
// partial tiles (per chunk, or per range) added in order, the bias, one
// rounding, a 16-byte store into the output image.  With the copy
// (cc.nvec > 0), the workgroups past the ones with combine work copy the cache
// outside the listed blocks (when the combine work fills at least half of the
// grid, every workgroup takes a share after its rows).  `slots` is the
// convolution's grid, from which it took the plan.
template <int DT, int MT, int NT>
__global__ __launch_bounds__(256) void k_split_combine(ConvArgs a, int slots) {
    constexpr int ES = elem_bytes(DT), BM = 16 * MT, BN = 16 * NT, VPR = BN / 8;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const Geo &g = a.g;
    const ConvCfg &c = a.c;
    const int b2 = g.b * g.b, ntn = (g.cout + BN - 1) / BN;
    const int nch = (g.cin + c.ck - 1) / c.ck;
    const int cnt = clamp_count(a.count, g.cap);
    if (cnt > c.gate_max) return;  // the single-range layer does this list (and the copy)
    const StreamPlan pl = stream_plan(cnt, b2, BM, ntn, nch, slots, stream_dbuf(c, BM, BN, kConvWaves));
    const int mrows = cnt * b2;
    const long total = (long)pl.mtn * ntn * BM * VPR;
    for (long u = (long)blockIdx.x * 256 + threadIdx.x; u < total; u += (long)gridDim.x * 256) {
        const int tile = (int)(u / (BM * VPR)), rem = (int)(u - (long)tile * BM * VPR);
        const int row = rem / VPR, col = (rem - row * VPR) * 8;
        const int tn = tile % ntn, tm = tile / ntn;
        const int r = tm * BM + row, co = tn * BN + col;
        if (r >= mrows || co >= g.cout) continue;
        const int slot = fdiv(r, c.m_b2), pix = r - slot * b2;
        const int py = fdiv(pix, c.m_b), px = pix - py * g.b;
        // the block index and the first partials are requested together (the
        // partials' addresses do not depend on the index), then the sum
        const int lin = a.idx[slot];
        float sum[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] = a.bias ? a.bias[min(co + j, g.cout - 1)] : 0.f;
        const int kstep = pl.acc_range ? pl.cpk : 1;
        constexpr int PB = 4;  // partial tiles requested at once
        for (int ks0 = 0; ks0 < nch; ks0 += PB * kstep) {
            f32x4 lo[PB], hi[PB];
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const int ks = min(ks0 + q * kstep, nch - 1);
                const float *wp = a.ws + (((size_t)tile * nch + ks) * BM + row) * BN + col;
                lo[q] = *(const f32x4 *)wp;
                hi[q] = *(const f32x4 *)(wp + 4);
            }
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                if (ks0 + q * kstep >= nch) break;
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
        store_row8<DT>(a.dst + ((((size_t)n * g.ho + y) * g.wo + x) * g.cout + co) * ES, sum, g.cout - co >= 8);
    }
    if (a.cc.nvec > 0) {
        const int busy = (int)((total + 255) / 256);
        const int c0 = busy < (int)gridDim.x / 2 ? busy : 0;
        if ((int)blockIdx.x < c0) return;
        const int i = blockIdx.x - c0, nw = gridDim.x - c0;
        const long long lo = split_point(a.cc.nvec, i, nw), hi = split_point(a.cc.nvec, i + 1, nw);
        if (lo < hi) {
            uint32_t *bm = nullptr;
            if (((g.cap + 31) >> 5) * 4 <= 64 * 1024) {
                bm = (uint32_t *)smem;
                build_bitmap<256>(a.idx, cnt, g.cap, bm);
            }
            copy_span<4, 256>(g, a.cc, bm, a.idx, cnt, a.cache, a.dst, lo, hi);
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

template <int DT, int MT, int NT>
static hipError_t launch_conv_t(int fused, const ConvArgs &args, hipStream_t st) {
    if (fused && args.ws) {  // the split over input channels, then the combine (and the copy)
        auto k = args.wp ? k_conv_stream<DT, MT, NT, true> : k_conv_stream<DT, MT, NT, false>;
        int slots = args.c.cus * resident_per_cu(k, args.c.lds_bytes);
        if (slots > 8) slots = slots / 8 * 8;  // keep position p on XCD p % 8 across passes
        ConvArgs conv = args;
        conv.cc.nvec = 0;  // the combine copies the cache
        hipLaunchKernelGGL(k, dim3(slots), dim3(kConvThreads), args.c.lds_bytes, st, conv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        constexpr int BM = 16 * MT, BN = 16 * NT;
        const long work = ((long)args.g.cap * args.g.b * args.g.b + BM - 1) / BM *
                          ((args.g.cout + BN - 1) / BN) * BM * (BN / 8);  // rows x vectors at capacity
        long grid = (work + 255) / 256 < 4L * args.c.cus ? (work + 255) / 256 : 4L * args.c.cus;
        if (args.cc.nvec > 0) grid = 4L * args.c.cus;  // room for the copy
        const int bm = args.cc.nvec > 0 && ((args.g.cap + 31) / 32) * 4 <= 64 * 1024 ? ((args.g.cap + 31) / 32) * 4 : 0;
        auto kc = k_split_combine<DT, MT, NT>;
        hipLaunchKernelGGL(kc, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), bm, st, args, slots);
    } else {
        return hipErrorInvalidValue;  // the unsplit layer and the block conv run on k_layer (kernels_layer.hip)
    }
    return hipGetLastError();
}

// Partial tiles the split's workspace must hold: one per (M tile, N tile,
// chunk) at full capacity.
template <int DT, int MT, int NT>
static long split_items_t(const Geo &g, const ConvCfg &c) {
    constexpr int BM = 16 * MT, BN = 16 * NT;
    const long tiles = ((long)g.cap * g.b * g.b + BM - 1) / BM * ((g.cout + BN - 1) / BN);
    return tiles * ((g.cin + c.ck - 1) / c.ck);
}

long split_workspace_bytes(int dt, const Geo &g, const ConvCfg &c) {
    const int key = c.mt * 10 + c.nt;
    long items = 0;
#define SIGE_SPLIT_ITEMS(D)                                         \
    switch (key) {                                                  \
    case 42: items = split_items_t<D, 4, 2>(g, c); break;           \
    case 41: items = split_items_t<D, 4, 1>(g, c); break;           \
    case 22: items = split_items_t<D, 2, 2>(g, c); break;           \
    case 44: items = split_items_t<D, 4, 4>(g, c); break;           \
    default: return -1;                                             \
    }
    switch (dt) {
    case 0: SIGE_SPLIT_ITEMS(0) break;
    case 1: SIGE_SPLIT_ITEMS(1) break;
    default: SIGE_SPLIT_ITEMS(2) break;
    }
#undef SIGE_SPLIT_ITEMS
    return items * (16L * c.mt) * (16L * c.nt) * 4;
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
                       const int32_t *count, void *dst, const void *cache, const int32_t *prev_idx,
                       const int32_t *prev_count, const Geo &g, const ConvCfg &cfg, const CopyCfg &cc,
                       hipStream_t st, float *ws, const void *wp) {
    ConvArgs args{(const uint8_t *)src, (const uint8_t *)w, bias, idx, count, (uint8_t *)dst,
                  (const uint8_t *)cache, prev_idx, prev_count, ws, g, cfg, cc, (const uint8_t *)wp};
    switch (dt) {
    case 0: return launch_conv_dt<0>(fused, args, st);
    case 1: return launch_conv_dt<1>(fused, args, st);
    default: return launch_conv_dt<2>(fused, args, st);
    }
}

// The fragment-order copy of KRSC weights for the split's load_weights: for
// chunk ch (c.ck input channels), N tile tn (16 NT output channels), K step s
// of the chunk, N subtile q and lane l, the 16 bytes that lane loads from the
// KRSC weights (clamped columns and channels included) at unit (((ch * ntn +
// tn) * steps + s) * NT + q) * 64 + l.  One thread per unit.
__global__ __launch_bounds__(256) void k_split_weights_pack(const uint8_t *__restrict__ w, Geo g, ConvCfg c, int dt,
                                                            uint8_t *wp, long units) {
    const int es = elem_bytes(dt), epv = 16 / es, ks = dt == 0 ? 16 : 32;
    const int k2 = g.k * g.k, kpc = c.ck / ks, steps = k2 * kpc;
    const int ntn = (g.cout + 16 * c.nt - 1) / (16 * c.nt);
    for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < units; v += (long)gridDim.x * 256) {
        const int l = (int)(v & 63);
        long q = v >> 6;
        const int nt = (int)(q % c.nt);
        q /= c.nt;
        const int s = (int)(q % steps);
        q /= steps;
        const int tn = (int)(q % ntn), ch = (int)(q / ntn);
        const int tap = s / kpc, kk = s - tap * kpc;
        const int cb = min(ch * c.ck + kk * ks + (l >> 4) * epv, g.cin - epv);
        const int col = min(tn * 16 * c.nt + nt * 16 + (l & 15), g.cout - 1);
        *(u32x4 *)(wp + v * 16) = ld16(w + (((size_t)col * k2 + tap) * g.cin + cb) * es);
    }
}

long split_weights_units(int dt, const Geo &g, const ConvCfg &c) {
    const int ks = dt == 0 ? 16 : 32;
    const long nch = (g.cin + c.ck - 1) / c.ck, ntn = (g.cout + 16 * c.nt - 1) / (16 * c.nt);
    return nch * ntn * (long)g.k * g.k * (c.ck / ks) * c.nt * 64;
}

hipError_t launch_split_weights_pack(int dt, const void *w, const Geo &g, const ConvCfg &c, void *wp, int cus,
                                     hipStream_t st) {
    const long units = split_weights_units(dt, g, c);
    long grid = (units + 255) / 256;
    if (grid > 4L * cus) grid = 4L * cus;
    hipLaunchKernelGGL(k_split_weights_pack, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, st,
                       (const uint8_t *)w, g, c, dt, (uint8_t *)wp, units);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// step 5: scatter.  A persistent grid: each workgroup first writes listed
// blocks' valid pixels (slot = workgroup, + grid, ...), then, when
// copy_cached, an even share of the copy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scatter(const uint8_t *__restrict__ ob, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ count, Geo g, uint32_t m_b,
                                                 const uint8_t *__restrict__ cache, uint8_t *__restrict__ out,
                                                 CopyCfg cc, int bm_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int U = 8;
    const int cnt = clamp_count(count, g.cap);
    const int grid = gridDim.x;
    const int vpp = cc.vpp, row_bytes = vpp * 16, b2 = g.b * g.b;
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
    if (cc.nvec > 0) {
        const long long lo = split_point(cc.nvec, blockIdx.x, grid), hi = split_point(cc.nvec, blockIdx.x + 1, grid);
        if (lo < hi) {
            uint32_t *bm = nullptr;
            if (bm_bytes > 0) {
                bm = (uint32_t *)smem;
                build_bitmap<256>(idx, cnt, g.cap, bm);
            }
            copy_span<4, 256>(g, cc, bm, idx, cnt, cache, out, lo, hi);
        }
    }
}

hipError_t launch_scatter(int dt, const void *out_blocks, const int32_t *idx, const int32_t *count, const Geo &g,
                          const void *cached, void *out, int grid, const CopyCfg &cc, hipStream_t st) {
    (void)dt;
    // bitmap of listed blocks for the copy, when it fits in 64 KiB of LDS
    const long bm = cc.nvec > 0 ? ((long)(g.cap + 31) / 32) * 4 : 0;
    const int bm_bytes = bm <= 64 * 1024 ? (int)bm : 0;
    hipLaunchKernelGGL(k_scatter, dim3(grid), dim3(256), bm_bytes, st, (const uint8_t *)out_blocks, idx, count, g,
                       cc.m_b, (const uint8_t *)cached, (uint8_t *)out, cc, bm_bytes);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The standalone restore: a persistent grid, each workgroup marks the new list
// in an LDS bitmap (when it fits), then takes slots workgroup, + grid, ...
__global__ __launch_bounds__(256) void k_restore(const int32_t *__restrict__ prev_idx,
                                                 const int32_t *__restrict__ prev_count,
                                                 const int32_t *__restrict__ idx, const int32_t *__restrict__ count,
                                                 Geo g, CopyCfg cc, const uint8_t *__restrict__ cache,
                                                 uint8_t *__restrict__ out, int bm_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int np = clamp_count(prev_count, g.cap);
    if ((int)blockIdx.x >= np) return;  // no previous block for this workgroup
    const int nn = idx ? clamp_count(count, g.cap) : 0;
    uint32_t *bm = nullptr;
    if (idx && bm_bytes > 0) {
        bm = (uint32_t *)smem;
        build_bitmap<256>(idx, nn, g.cap, bm);
    }
    restore_slots<256>(g, cc, prev_idx, blockIdx.x, gridDim.x, np, bm, idx, nn, cache, out);
}

hipError_t launch_restore(const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                          const int32_t *count, const Geo &g, const CopyCfg &cc, const void *cached, void *out,
                          int grid, hipStream_t st) {
    // bitmap of the new list, when it fits in 64 KiB of LDS (else a binary search per block)
    const long bm = idx ? ((long)(g.cap + 31) / 32) * 4 : 0;
    const int bm_bytes = bm <= 64 * 1024 ? (int)bm : 0;
    hipLaunchKernelGGL(k_restore, dim3(grid), dim3(256), bm_bytes, st, prev_idx, prev_count, idx, count, g, cc,
                       (const uint8_t *)cached, (uint8_t *)out, bm_bytes);
    return hipGetLastError();
}

}  // namespace sige
