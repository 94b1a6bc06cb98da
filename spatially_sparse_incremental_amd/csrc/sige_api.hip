// sige_api.hip -- the C ABI of libsige.so: argument checks, status codes,
// launch configuration.  Every check runs on the host before anything is
// enqueued; the kernels live in kernels_mask.hip and kernels_conv.hip.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "sige.h"
#include "sige_internal.h"

using sige::ConvCfg;
using sige::Geo;

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dtype_ok(int dt) { return dt == SIGE_F32 || dt == SIGE_BF16 || dt == SIGE_F16; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

// A byte range a launch reads or writes (p NULL: none).
struct Region {
    const void *p;
    size_t n;
};

// Whether any written range overlaps another written range or a read range.
bool regions_overlap(const Region *wr, int nw, const Region *rd, int nr) {
    for (int i = 0; i < nw; ++i) {
        if (!wr[i].p) continue;
        for (int j = i + 1; j < nw; ++j)
            if (wr[j].p && overlap(wr[i].p, wr[i].n, wr[j].p, wr[j].n)) return true;
        for (int j = 0; j < nr; ++j)
            if (rd[j].p && overlap(wr[i].p, wr[i].n, rd[j].p, rd[j].n)) return true;
    }
    return false;
}

int derive(const sige_geom *gp, Geo *g) {
    if (!gp) return fail(SIGE_EINVAL, "geometry pointer is NULL");
    const sige_geom &q = *gp;
    if (q.n < 1 || q.h < 1 || q.w < 1 || q.c_in < 1 || q.c_out < 1)
        return fail(SIGE_EINVAL, "n, h, w, c_in, c_out must be >= 1 (got %d, %d, %d, %d, %d)", q.n, q.h, q.w,
                    q.c_in, q.c_out);
    if (q.k < 1 || q.k > 7) return fail(SIGE_EINVAL, "kernel size k=%d outside [1, 7]", q.k);
    if (q.stride < 1 || q.stride > 4) return fail(SIGE_EINVAL, "stride=%d outside [1, 4]", q.stride);
    if (q.pad < 0 || q.pad >= q.k) return fail(SIGE_EINVAL, "pad=%d outside [0, k-1]", q.pad);
    if (q.block < 1 || q.block > 64) return fail(SIGE_EINVAL, "block=%d outside [1, 64]", q.block);
    if (q.h + 2 * q.pad < q.k || q.w + 2 * q.pad < q.k)
        return fail(SIGE_EINVAL, "padded input %dx%d smaller than the kernel", q.h + 2 * q.pad, q.w + 2 * q.pad);
    Geo r;
    r.n = q.n, r.h = q.h, r.w = q.w, r.cin = q.c_in, r.cout = q.c_out;
    r.k = q.k, r.s = q.stride, r.p = q.pad, r.b = q.block;
    r.ho = (q.h + 2 * q.pad - q.k) / q.stride + 1;
    r.wo = (q.w + 2 * q.pad - q.k) / q.stride + 1;
    r.nby = (r.ho + q.block - 1) / q.block;
    r.nbx = (r.wo + q.block - 1) / q.block;
    r.ib = (q.block - 1) * q.stride + q.k;
    if (r.ib > 64) return fail(SIGE_EINVAL, "input window %d exceeds 64", r.ib);
    const int64_t cap = (int64_t)q.n * r.nby * r.nbx;
    if (cap > 0x7FFFFFFFLL) return fail(SIGE_ERANGE, "block capacity %lld exceeds int32", (long long)cap);
    const int64_t in_elems = (int64_t)q.n * q.h * q.w * q.c_in, out_elems = (int64_t)q.n * r.ho * r.wo * q.c_out;
    if (in_elems > (1LL << 40) || out_elems > (1LL << 40)) return fail(SIGE_ERANGE, "tensor too large");
    if ((int64_t)r.ho * q.block > 0x7FFFFFFFLL || (int64_t)r.wo * q.block > 0x7FFFFFFFLL)
        return fail(SIGE_ERANGE, "output %dx%d too large for block size %d", r.ho, r.wo, q.block);
    r.cap = (int)cap;
    *g = r;
    return SIGE_OK;
}

int channel_rows_ok(int dt, int c, const char *what) {
    const int es = sige::elem_bytes(dt);
    if ((c * es) % 16)
        return fail(SIGE_EALIGN, "%s=%d: a channel row of %d bytes is not a multiple of 16", what, c, c * es);
    if (c * es > sige::kMaxRowBytes)
        return fail(SIGE_ERANGE, "%s=%d: channel rows above %d bytes are not supported", what, c, sige::kMaxRowBytes);
    return SIGE_OK;
}

int device_ready() {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        (void)hipGetLastError();
        return fail(SIGE_ENODEV, "no HIP device available");
    }
    return SIGE_OK;
}

int finish(hipError_t e, const char *what, hipStream_t st) {
    if (e != hipSuccess) return fail(SIGE_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
    static int debug_sync = -1;
    if (debug_sync < 0) {
        const char *v = getenv("SIGE_DEBUG_SYNC");
        debug_sync = (v && v[0] == '1') ? 1 : 0;
    }
    if (debug_sync) {
        e = hipStreamSynchronize(st);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return fail(SIGE_EHIP, "%s failed on the device: %s", what, hipGetErrorString(e));
    }
    g_msg[0] = 0;
    return SIGE_OK;
}

constexpr int kStaticLds = 6144;  // the conv kernel's static LDS (slot table, copy bitmap), rounded up

struct DevInfo {  // defaults: gfx950
    int lds = 160 * 1024;  // LDS per workgroup
    int cus = 256;         // compute units
};

// Per-device limits, queried once per device (160 KiB LDS and 256 CUs on MI355X).
DevInfo dev_info() {
    static DevInfo cache[64];
    static bool have[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return DevInfo{};
    }
    if (!have[dev]) {
        DevInfo d;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            d.lds = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            d.cus = v;
        (void)hipGetLastError();
        cache[dev] = d;
        have[dev] = true;
    }
    return cache[dev];
}

// The copy of the cache outside the listed blocks, in 16-byte vectors.
// free_vec: what a workgroup without a tile copies per tile of a busy one
// (default 8192 vectors = 128 KiB, tuned on MI355X for the 256x256x128 layer;
// SIGE_COPY_FREE_VEC overrides it for tuning).
sige::CopyCfg copy_plan(const Geo &g, int es, bool copy) {
    static int free_vec = -1;
    if (free_vec < 0) {
        const char *v = getenv("SIGE_COPY_FREE_VEC");
        const long x = v ? strtol(v, nullptr, 10) : 0;
        free_vec = (x > 0 && x < (1L << 30)) ? (int)x : 8192;
    }
    sige::CopyCfg c{};
    c.vpp = g.cout * es / 16;
    c.m_vpp = sige::fast_div_magic(c.vpp);
    c.m_b = sige::fast_div_magic(g.b);
    c.nvec = copy ? (long long)g.n * g.ho * g.wo * c.vpp : 0;
    c.free_vec = free_vec;
    return c;
}

// Tile shape override for tuning: SIGE_CONV_TILE="MT,NT" (one of 4,2 4,1 2,2 4,4).
void tile_shape(int *mt, int *nt) {
    *mt = 4;
    *nt = 2;
    const char *v = getenv("SIGE_CONV_TILE");
    int a = 0, b = 0;
    if (v && sscanf(v, "%d,%d", &a, &b) == 2) {
        const int key = a * 10 + b;
        if (key == 42 || key == 41 || key == 22 || key == 44) {
            *mt = a;
            *nt = b;
        }
    }
}

// Tile configuration of the implicit GEMM (see kernels_conv.hip).  Each of the
// 8 waves holds the weight fragments of at most 10/NT K steps of a chunk in
// registers, so a chunk has at most 8*10/NT steps: ck <= floor(80/(NT*k*k)) K
// slices.
// Among those, the fewest chunks whose input windows fit in the device's LDS
// (stream: the split over input channels, which also takes a second buffer of
// windows when it fits, to stage the next M tile during the current one).
// The persistent grid fills every CU with up to two workgroups.
int choose_conv(const Geo &g, int dt, int fused, int copy, ConvCfg *out, int stream = 0) {
    ConvCfg c{};
    tile_shape(&c.mt, &c.nt);
    const int es = sige::elem_bytes(dt);
    const int ks = dt == SIGE_F32 ? 16 : 32;
    const int b2 = g.b * g.b, ib2 = g.ib * g.ib, k2 = g.k * g.k;
    while (c.nt > 1 && (8 * (10 / c.nt)) / k2 < 1) c.nt /= 2;  // large kernels: fewer channels per tile
    const int max_kpc = (8 * (10 / c.nt)) / k2;                 // K slices per tap and chunk
    if (max_kpc < 1) return fail(SIGE_ERANGE, "kernel size %d too large for the register-resident weights", g.k);
    const int BM = 16 * c.mt, BN = 16 * c.nt;
    int ns = (BM - 1) / b2 + 2;
    if (ns > BM) ns = BM;
    if (ns > g.cap) ns = g.cap;
    c.ns_max = ns;
    // output rows r (< cap*b*b + BM) are split with fast divisions by b*b: r * b*b < 2^31
    if (((long)g.cap * b2 + BM) * b2 > 0x7FFFFFFFL) return fail(SIGE_ERANGE, "too many output rows for one launch");
    const DevInfo dv = dev_info();
    const long limit = (long)dv.lds - kStaticLds;
    const long part = 8L * BM * (BN + 4) * 4;  // the 8 waves' partial tiles
    const int kslices = (g.cin + ks - 1) / ks;
    int best = 0;
    long best_lds = 0;
    for (int nch = (kslices + max_kpc - 1) / max_kpc; nch <= kslices && !best; ++nch) {
        const int ck = (kslices + nch - 1) / nch * ks;  // ceil(cin / nch), rounded up to a K slice
        if (ck * es / 16 > 256) continue;               // one 16-byte vector per thread and pixel
        const long apix = ck * es + 16;
        const long lds = (long)ns * ib2 * apix;
        const long need = lds > part ? lds : part;
        if (need <= limit) {
            best = ck;
            best_lds = stream && need + lds <= limit ? need + lds : need;
        }
    }
    if (!best)
        return fail(SIGE_ERANGE, "staged windows (%d slots of %dx%d) do not fit in LDS", ns, g.ib, g.ib);
    c.ck = best;
    c.a_pix_stride = best * es + 16;
    c.a_bytes = ns * ib2 * c.a_pix_stride;
    c.lds_bytes = (int)best_lds;
    c.m_ib2 = sige::fast_div_magic(ib2);
    c.m_ib = sige::fast_div_magic(g.ib);
    c.m_vpc1 = sige::fast_div_magic(best * es / 16 + 1);
    c.m_b2 = sige::fast_div_magic(b2);
    c.m_b = sige::fast_div_magic(g.b);
    c.gate_max = 0x7FFFFFFF;
    long grid = 1L << 30;  // the launch trims this to the CUs' resident capacity
    if (!(fused && copy))  // tiles at capacity, M tiles padded to a multiple of 8 (see the kernel's tile order)
        grid = (((long)g.cap * b2 + BM - 1) / BM + 7) / 8 * 8 * ((g.cout + BN - 1) / BN);
    c.cus = dv.cus;
    c.grid = (int)(grid > 0 ? grid : 1);
    *out = c;
    return SIGE_OK;
}

// Wide tiles (k_layer_wide in kernels_layer.hip): 256 rows x 128 output
// channels, K in stages of 16 input channels, two LDS buffers, for 16-bit
// types and k <= 3.  A slot's staged window (one stage) takes rows of w_rs
// units (w_rs >= 3*ib, w_rs = 3b mod 16: see the kernel's bank layout); a
// staging load covers one or two window rows (64 lanes, those on padding
// masked off), and a slot's LDS holds its window rows plus the bank rotation.
// No wide tiles when both buffers (or the epilogue's tile) exceed the CU's
// LDS, or when a staging wave would have more than kLayerWideWinLoads window
// loads per stage (their sources are kept in registers).  wide_min: the list length from which the wide kernel runs
// (SIGE_WIDE_MIN overrides it for tuning).
void wide_layer(const Geo &g, int dt, const DevInfo &dv, sige::LayerCfg *c) {
    c->wide_min = c->wide_max = c->gate_wide = 0x7FFFFFFF;
    c->w_pmax = 1;
    c->w_ws_items = 0;
    if (dt == SIGE_F32 || g.k > 3 || 3 * g.ib > 64) return;
    const int b2 = g.b * g.b, k2 = g.k * g.k;
    int rs = 3 * g.ib;
    while (rs % 16 != (3 * g.b) % 16) ++rs;
    const int rpi = rs + 3 * g.ib <= 64 ? 2 : 1;
    const int foot = (g.ib - 1) * rs + 3 * g.ib;  // the last window row's last data unit + 1
    const int adj = (3 * b2) % 16 ? 15 : 0;
    const int sb = (foot + adj + 15) / 16 * 16;
    const int WR = sige::kLayerWideRows;
    long nsw = WR % b2 == 0 ? WR / b2 : (WR - 1) / b2 + 2;
    if (nsw > g.cap) nsw = g.cap;
    if (nsw > 64) return;
    const int nld = (g.ib + rpi - 1) / rpi;  // staging loads per slot window
    if ((nsw * nld + 3) / 4 > sige::kLayerWideWinLoads) return;  // sources held in registers
    const long win = nsw * sb * 16, buf = win + (long)k2 * sige::kLayerWideCols * 32;
    const long need_e = (long)WR * sige::kLayerWidePitch;
    const long need = 2 * buf > need_e ? 2 * buf : need_e;
    if (need > (long)dv.lds - 1024) return;
    if (((long)g.cap * b2 + WR) > 0x7FFFFFFFL) return;
    c->w_rs = rs;
    c->w_sb = sb;
    c->w_rpi = rpi;
    c->w_ntn = (g.cout + sige::kLayerWideCols - 1) / sige::kLayerWideCols;
    c->w_wofs = (int)win;
    c->w_lds = (int)need;
    const long mtn = ((long)g.cap * b2 + WR - 1) / WR;
    c->w_tiles_cap = (int)((c->w_ntn > 1 ? (mtn + 7) / 8 * 8 : mtn) * c->w_ntn);
    // K parts for lists too short to give every CU a tile: at least
    // kLayerWideMinStages stages each; the workspace holds the most partial
    // tiles any list length makes
    const int nst = (g.cin + 15) / 16;
    int pmax = nst / sige::kLayerWideMinStages;
    c->w_pmax = pmax < 1 ? 1 : (pmax > 16 ? 16 : pmax);
    c->w_ws_items = 0;
    for (long m = 1; m <= mtn && m * c->w_ntn <= dv.cus / 2; ++m) {
        const int np = sige::wide_parts(dv.cus, c->w_pmax, (int)(m * c->w_ntn));
        const long items = m * c->w_ntn * np;
        if (np > 1 && items > c->w_ws_items) c->w_ws_items = (int)items;
    }
    if (c->w_ws_items == 0) c->w_pmax = 1;
    long wmin = 0x7FFFFFFF;
    const char *e = getenv("SIGE_WIDE_MIN");
    if (e) {
        const long x = strtol(e, nullptr, 10);
        if (x >= 0) wmin = x;
    }
    c->wide_min = (int)(wmin < 0x7FFFFFFF ? wmin : 0x7FFFFFFF);
}

// Launch configuration of k_layer (kernels_layer.hip).  A wave holds the
// weight fragments of at most kLayerFrags/NT K steps of a chunk, so a chunk
// has at most 4*kLayerFrags/NT steps: kpc <= floor(4*kLayerFrags/(NT*k*k))
// K slices per tap, a power of 2.  Among those, the fewest chunks (then the
// fewest K slices in all) whose staged windows fit in half of the CU's LDS
// (two workgroups per CU), else in all of it: a chunk costs a round trip of
// window staging and a barrier, several microseconds, while a K slice of zero
// padding costs a few MFMAs.  A block slot's staged window
// takes gps groups of 64 16-byte units plus 16 units for its bank rotation
// (see kernels_layer.hip); the LDS also holds the
// epilogue's 4 partial tiles and the rounded tile.
int choose_layer(const Geo &g, int dt, sige::LayerCfg *out) {
    sige::LayerCfg c{};
    c.mt = 4;
    c.nt = 2;
    const int es = sige::elem_bytes(dt);
    const int ks = dt == SIGE_F32 ? 16 : 32;
    const int b2 = g.b * g.b, k2 = g.k * g.k;
    const int nw = sige::kLayerWaves;
    if ((nw * (sige::kLayerFrags / c.nt)) / k2 < 1) c.nt = 1;  // large kernels: 16 channels per tile
    const int max_kpc = (nw * (sige::kLayerFrags / c.nt)) / k2;  // K slices per tap and chunk
    if (max_kpc < 1) return fail(SIGE_ERANGE, "kernel size %d too large for the register-resident weights", g.k);
    const int BM = 16 * c.mt, BN = 16 * c.nt;
    int ns = (BM - 1) / b2 + 2;
    if (ns > BM) ns = BM;
    if (ns > g.cap) ns = g.cap;
    if (((long)g.cap * b2 + BM) * b2 > 0x7FFFFFFFL) return fail(SIGE_ERANGE, "too many output rows for one launch");
    // 32-bit offsets of a staged vector from its window origin, and of a weight column
    if (((long)(g.ib - 1) * g.w + g.ib) * (long)g.cin * es > 0x7FFFFFFFL)
        return fail(SIGE_ERANGE, "a %dx%d window of %d-wide rows of %d channels exceeds 32-bit offsets", g.ib, g.ib,
                    g.w, g.cin);
    const DevInfo dv = dev_info();
    const long epi = (long)nw * c.mt * c.nt * 64 * 16 + (long)BM * BN * es;  // partial tiles + rounded tile
    const int kslices = (g.cin + ks - 1) / ks;
    int best_kpc = 0, best_gps = 0;
    long best_lds = 0;
    for (int pass = 0; pass < 2 && !best_kpc; ++pass) {
        const long limit = (pass == 0 ? dv.lds / 2 : (long)dv.lds) - 1024;  // 1 KiB: static LDS, alignment
        long best_cost = 0;
        for (int kpc = 1; kpc <= max_kpc; kpc *= 2) {
            const int nch = (kslices + kpc - 1) / kpc;
            const int ck = kpc * ks;
            if (ck * es / 16 > 255) break;
            const int ps = ck * es / 16 + 1;
            const int rs = g.ib * ps + (((g.b - g.ib * ps) % 16) + 16) % 16;
            const int gps = (g.ib * rs + 63) / 64;
            const long need_w = (long)ns * (64 * gps + 16) * 16;
            const long need = need_w > epi ? need_w : epi;
            if (need > limit) break;
            const long cost = (long)nch * 4096 + nch * kpc;  // chunks, then K slices in all
            if (!best_kpc || cost < best_cost) {
                best_kpc = kpc;
                best_gps = gps;
                best_lds = need;
                best_cost = cost;
            }
        }
    }
    if (!best_kpc) return fail(SIGE_ERANGE, "staged windows (%d slots of %dx%d) do not fit in LDS", ns, g.ib, g.ib);
    c.kpc = best_kpc;
    c.lkpc = 0;
    while ((1 << c.lkpc) < best_kpc) ++c.lkpc;
    c.ck = best_kpc * ks;
    c.nch = (kslices + best_kpc - 1) / best_kpc;
    c.steps = k2 * c.kpc;
    c.spw = (c.steps + nw - 1) / nw;
    c.vpc = c.ck * es / 16;
    c.ps = c.vpc + 1;
    c.rs = g.ib * c.ps + (((g.b - g.ib * c.ps) % 16) + 16) % 16;
    c.gps = best_gps;
    c.sb = (64 * best_gps + 16) * 16;
    c.lds_bytes = (int)best_lds;
    c.ntn = (g.cout + BN - 1) / BN;
    const long mtn = ((long)g.cap * b2 + BM - 1) / BM;
    c.xcd = mtn >= 8;
    const long tiles = (c.xcd ? (mtn + 7) / 8 * 8 : mtn) * c.ntn;
    if (tiles > 0x7FFFFFFFL) return fail(SIGE_ERANGE, "too many tiles for one launch");
    c.tiles_cap = (int)tiles;
    c.cus = dv.cus;
    c.spec = 0;
    c.gate_min = 0;
    c.m_ps = sige::fast_div_magic(c.ps);
    c.m_rs = sige::fast_div_magic(c.rs);
    c.m_b2 = sige::fast_div_magic(b2);
    c.m_b = sige::fast_div_magic(g.b);
    wide_layer(g, dt, dv, &c);
    *out = c;
    return SIGE_OK;
}

// Attention: the token grid as a k = 1 geometry, and the workspace the two kernels need.
int attn_geom(int n, int h, int w, int heads, int head_dim, int block, Geo *g) {
    if (head_dim != sige::kAttnHeadDim) return fail(SIGE_ERANGE, "head_dim %d: only 64 is supported", head_dim);
    if (heads < 1) return fail(SIGE_EINVAL, "heads=%d", heads);
    if (n < 1 || n > sige::kAttnImages) return fail(SIGE_ERANGE, "n=%d: 1 to %d images", n, sige::kAttnImages);
    const sige_geom q{n, h, w, heads * head_dim, heads * head_dim, 1, 1, 0, block};
    return derive(&q, g);
}

int attn_grid1() {
    static int grid[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return sige::attn_partial_grid(dev_info().cus);
    }
    if (!grid[dev]) {  // SIGE_ATTN_GRID overrides the partial kernel's grid (tuning)
        const char *v = getenv("SIGE_ATTN_GRID");
        const long x = v ? strtol(v, nullptr, 10) : 0;
        grid[dev] = (x > 0 && x <= 65536) ? (int)x : sige::attn_partial_grid(dev_info().cus);
    }
    return grid[dev];
}

int64_t attn_ws_bytes(const Geo &g, int heads, int grid1) {
    const long per = (long)g.nby * g.nbx, b2 = (long)g.b * g.b;
    const long max_items = (long)g.n * ((per * b2 + sige::kAttnQueryTile - 1) / sige::kAttnQueryTile) * heads;
    const long items = max_items > 2L * grid1 ? max_items : 2L * grid1;
    return (int64_t)items * sige::kAttnWsBytesPerItem;
}

// bitset: the mask as one bit per pixel (bit p % 32 of word p / 32), mask_w a
// multiple of 32
int reduce_common(const uint8_t *mask, int mask_h, int mask_w, const sige_geom *gp, int dilate_blocks, int32_t *idx,
                  int32_t *count, int dtype, const void *cached, void *out, void *stream, const char *what,
                  int bitset = 0) {
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!mask || !idx || !count) return fail(SIGE_EINVAL, "NULL pointer");
    if (bitset && (mask_w % 32 || !aligned(mask, 4)))
        return fail(mask_w % 32 ? SIGE_EINVAL : SIGE_EALIGN, "bitset mask: width %d must be a multiple of 32 and "
                    "the words 4-byte aligned", mask_w);
    if (mask_h < g.h || mask_w < g.w || mask_h % g.h || mask_w % g.w)
        return fail(SIGE_EINVAL, "mask %dx%d is not an integer multiple of the conv input %dx%d", mask_h, mask_w,
                    g.h, g.w);
    if (dilate_blocks < 0 || dilate_blocks > 16) return fail(SIGE_EINVAL, "dilate_blocks=%d outside [0, 16]", dilate_blocks);
    if (g.w > sige::kReduceMaxWidth)
        return fail(SIGE_ERANGE, "conv input width %d exceeds the reduce limit %d", g.w, sige::kReduceMaxWidth);
    if (g.cap > sige::kReduceMaxBlocks)
        return fail(SIGE_ERANGE, "%d blocks (n*nby*nbx) exceed the reduce limit %d", g.cap, sige::kReduceMaxBlocks);
    if (!aligned(idx, 4) || !aligned(count, 4)) return fail(SIGE_EALIGN, "idx/count must be 4-byte aligned");
    const size_t mbytes = (size_t)g.n * mask_h * mask_w / (bitset ? 8 : 1);
    if (overlap(idx, (size_t)g.cap * 4, mask, mbytes) || overlap(count, 4, mask, mbytes) ||
        overlap(count, 4, idx, (size_t)g.cap * 4))
        return fail(SIGE_EINVAL, "idx, count and mask must not overlap");
    sige::ReduceCopy cp{nullptr, nullptr, 0};
    if (out) {  // the reduce with the cache copy
        if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
        if (!cached) return fail(SIGE_EINVAL, "NULL pointer");
        if ((rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
        if (!aligned(cached, 16) || !aligned(out, 16)) return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
        const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * sige::elem_bytes(dtype);
        if (overlap(out, obytes, cached, obytes) || overlap(out, obytes, mask, mbytes) ||
            overlap(out, obytes, idx, (size_t)g.cap * 4) || overlap(out, obytes, count, 4))
            return fail(SIGE_EINVAL, "out overlaps cached, mask, idx or count");
        cp = sige::ReduceCopy{(const uint8_t *)cached, (uint8_t *)out, (long long)(obytes / 16)};
    }
    if ((rc = device_ready())) return rc;
    const int vec16 = bitset ? 2 : (mask_w % 16 == 0) && aligned(mask, 16);
    static int copy_wgs = -1;  // SIGE_REDUCE_COPY_WGS overrides the copy's workgroups (tuning)
    if (copy_wgs < 0) {
        const char *v = getenv("SIGE_REDUCE_COPY_WGS");
        const long x = v ? strtol(v, nullptr, 10) : 0;
        copy_wgs = (x > 0 && x < 65536) ? (int)x : 0;
    }
    return finish(sige::launch_reduce(mask, mask_h, mask_w, g, dilate_blocks, vec16, idx, count, cp,
                                      copy_wgs ? copy_wgs : dev_info().cus / 2, (hipStream_t)stream),
                  what, (hipStream_t)stream);
}

// The static scratch of sige_sparse_conv_layer_split_noalloc: one array per
// GPU in the library's code object, for callers that cannot allocate (under
// graph capture, in serving loops).  Host code never passes `scratch` itself:
// its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device on the entry point's first call there and kept.
constexpr size_t kScratchBytes = 64u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fail(SIGE_ENODEV, "no current HIP device below 64");
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SIGE_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    return SIGE_OK;
}

int split_common(const void *a_edit, const void *w_krsc, const float *bias, const void *cached, const int32_t *idx,
                 const int32_t *count, int dtype, const sige_geom *gp, void *out, int copy_cached, void *workspace,
                 int64_t workspace_bytes, void *stream, const char *what, bool use_scratch = false) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !w_krsc || !idx || !count || !out || (!workspace && !use_scratch) || (copy_cached && !cached))
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(w_krsc, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
        (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors and workspace must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    const size_t ibytes = (size_t)g.n * g.h * g.w * g.cin * es;
    const Region rd[] = {{a_edit, ibytes}, {copy_cached ? cached : nullptr, obytes},
                         {w_krsc, (size_t)g.cout * g.k * g.k * g.cin * es}, {bias, (size_t)g.cout * 4},
                         {idx, (size_t)g.cap * 4}, {count, 4}};
    {
        const Region wr[] = {{out, obytes}};
        if (regions_overlap(wr, 1, rd, 6))
            return fail(SIGE_EINVAL, "out overlaps a_edit, cached, the weights, bias, idx or count");
    }
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 1, 1, &cfg, 1))) return rc;
    const long need = sige::split_workspace_bytes(dtype, g, cfg);
    if (need < 0) return fail(SIGE_EINVAL, "unknown tile shape");
    if (use_scratch && (size_t)need > kScratchBytes)
        return fail(SIGE_ERANGE, "this layer's split needs %ld bytes of scratch, above the static %zu bytes of "
                    "sige_sparse_conv_layer_split_noalloc (use sige_sparse_conv_layer_split with a workspace)",
                    need, kScratchBytes);
    if ((rc = device_ready())) return rc;
    if (use_scratch) {
        if ((rc = scratch_address(&workspace))) return rc;
        workspace_bytes = (int64_t)kScratchBytes;
    }
    if (workspace_bytes < need)
        return fail(SIGE_ERANGE, "workspace of %lld bytes, %ld needed", (long long)workspace_bytes, need);
    {
        const Region wr[] = {{out, obytes}, {workspace, (size_t)need}};
        if (regions_overlap(wr, 2, rd, 6)) return fail(SIGE_EINVAL, "the workspace overlaps another argument");
    }
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    return finish(sige::launch_conv(dtype, 1, a_edit, w_krsc, bias, idx, count, out, copy_cached ? cached : nullptr,
                                    nullptr, nullptr, g, cfg, cc, (hipStream_t)stream, (float *)workspace),
                  what, (hipStream_t)stream);
}


// ---- The kernel choice of sige_sparse_conv_layer_auto ----
//
// Three kernels compute the fused layer.  k_layer gives each 64 x 32 tile of
// output rows and channels its whole K range, chunk after chunk, and every
// row tile reads its own copy of the weights; the split spreads (row group,
// input-channel chunk, channel tile) work items over all CUs, reads each
// weight once per row group and adds the chunks in a second launch;
// k_layer_wide runs 256 x 128 tiles, one per CU, staging windows and weights
// once per tile.  A long K range over few blocks -- the deep, low-resolution
// layers, where the mer.dev notes (5 "Conclusion & Discussion") find the
// block-sparse method least effective -- favours the split; many blocks favour
// k_layer, and long lists of large edits (nubint.ai review, "ABSTRACT": large
// edits) the wide tiles.  The list length is on the device, so the host
// prices the kernels for every list length with the cost model below and
// derives two thresholds: the split does lists of at most split_max blocks,
// the wide tiles those of at least wide_min, k_layer the ones between.  Every
// kernel whose range can occur is launched and checks *count on the device
// (ConvCfg::gate_max, LayerCfg::gate_min and gate_wide, LayerCfg::wide_min):
// the ones not chosen exit at once.
//
// The model, in microseconds for a list of `cnt` blocks (M tiles of 64 rows
// and N tiles of 32 channels, `tiles` of them):
//   k_layer: s0 + chunks * (s1 + s2 * stage_groups) * max(1, s3 * tiles * steps / slots)
//     (a chunk's round trip grows with the 1 KiB staging loads of its windows,
//      stage_groups per tile; once the tiles' MFMA steps exceed what the
//      resident slots overlap, time grows with the tiles)
//   split:   p0 + p1 * weight MB + p2 * GFLOP + p3 * tiles
//            + p4 * ceil(tiles * split_chunks / split_slots) * split_stage_kb
//     (the weights stream once; the work items' rounds each stage a tile's
//      windows of split_stage_kb KiB)
//   wide:    w0 + ceil(wide tiles * parts / CUs) * (w1 * stages * loads + w2)
//            + w3 * MB of fp32 partial tiles (parts > 1)
//     (a stage of 16 input channels takes as long as the CU's memory path
//      needs to accept its `loads` staging loads; a round of work items adds
//      its set-up, first stage and epilogue; `stages` are those of the longest
//      of a tile's K parts, and the parts' partials are written and read back
//      once)
// Constants fitted (least squares on log time) to the kernels timed on MI355X
// on edits of seeds other than the benchmark's, seven edit areas from 0.5% to
// 80% of the frame, the U-Net, GauGAN and latent-diffusion layers
// (calibrate_layer_choice.py in the package).  The k_layer model is the
// loosest (rms error of log time 0.17, the others 0.07 and 0.06 for the wide
// tiles, fitted on lists that fill a wide tile's block slots), so a list goes from k_layer to the wide tiles only where the model
// puts them ahead by more than that: kWideMargin.
struct ChoiceModel {
    double s[4], p[5], w[4];
};
constexpr ChoiceModel kChoice = {
    {4.395, 1.916, 0.06717, 0.04092}, {10.76, 0.2046, 2.133, 0.003156, 0.0456}, {0.9554, 0.03757, 10.8, 0.4737}};

struct LayerFeat {
    int cap, b2, ntn;
    int chunks, steps, groups, slots;  // k_layer
    int split_chunks, split_slots;     // the split
    double split_kb;                   // KiB of one tile's staged windows in the split
    double wmb, gflop_per_block;       // all
    int wide_stages, wide_loads;       // the wide tiles: K stages, staging loads per stage (0: no wide tiles)
    int wide_ntn, cus;
    int wide_pmax;                     // most K parts of a wide tile (1: no split)
};

LayerFeat layer_features(const Geo &g, int dt, const sige::LayerCfg &lc) {
    LayerFeat f{};
    const int es = sige::elem_bytes(dt);
    const int b2 = g.b * g.b, BM = 16 * lc.mt;
    int ns = (BM - 1) / b2 + 2;
    if (ns > BM) ns = BM;
    if (ns > g.cap) ns = g.cap;
    const DevInfo dv = dev_info();
    f.cap = g.cap;
    f.b2 = b2;
    f.ntn = (g.cout + 31) / 32;
    f.chunks = lc.nch;
    f.steps = lc.steps;
    f.groups = ns * lc.gps;
    f.slots = dv.cus * (lc.lds_bytes <= dv.lds / 2 - 1024 ? 2 : 1);
    f.wmb = (double)g.cout * g.k * g.k * g.cin * es * 1e-6;
    f.gflop_per_block = 2.0 * b2 * g.cout * g.k * g.k * (double)g.cin * 1e-9;
    f.cus = dv.cus;
    if (lc.w_lds > 0) {
        const int WR = sige::kLayerWideRows;
        long nsw = WR % b2 == 0 ? WR / b2 : (WR - 1) / b2 + 2;
        if (nsw > g.cap) nsw = g.cap;
        f.wide_stages = (g.cin + 15) / 16;
        f.wide_loads = (int)(nsw * ((g.ib + lc.w_rpi - 1) / lc.w_rpi) + 4 * g.k * g.k);
        f.wide_ntn = lc.w_ntn;
        f.wide_pmax = lc.w_pmax;
    }
    ConvCfg cc;
    if (choose_conv(g, dt, 1, 1, &cc, 1) == SIGE_OK) {
        f.split_chunks = (g.cin + cc.ck - 1) / cc.ck;
        f.split_slots = dv.cus * (cc.lds_bytes <= dv.lds / 2 ? 2 : 1);
        f.split_kb = cc.a_bytes / 1024.0;
    }
    return f;
}

// Microseconds a launch adds when its kernel exits at once (measured on
// MI355X against the kernel alone): k_layer (a persistent grid, one round
// trip for *count and the indices), the split (two launches), the wide tiles
// (one workgroup per CU) and, when their tiles are split over K, its second
// launch that adds the parts up.
constexpr double kGateOffSingle = 3.0, kGateOffSplit = 3.2, kGateOffWide = 1.4;
constexpr double kGateOffCombine = 1.5;
constexpr double kWideMargin = 1.2;

double cost_single(const LayerFeat &f, int cnt) {
    const double tiles = (double)(((long)cnt * f.b2 + 63) / 64) * f.ntn;
    const double per = kChoice.s[1] + kChoice.s[2] * f.groups;
    const double fill = kChoice.s[3] * tiles * f.steps / f.slots;
    return kChoice.s[0] + f.chunks * per * (fill > 1.0 ? fill : 1.0);
}

double cost_split(const LayerFeat &f, int cnt) {
    const long tiles = (((long)cnt * f.b2 + 63) / 64) * f.ntn;
    const long rounds = (tiles * f.split_chunks + f.split_slots - 1) / f.split_slots;
    return kChoice.p[0] + kChoice.p[1] * f.wmb + kChoice.p[2] * f.gflop_per_block * cnt + kChoice.p[3] * tiles +
           kChoice.p[4] * rounds * f.split_kb;
}

double cost_wide(const LayerFeat &f, int cnt) {
    const long mtn = ((long)cnt * f.b2 + sige::kLayerWideRows - 1) / sige::kLayerWideRows;
    const int np = sige::wide_parts(f.cus, f.wide_pmax, (int)(mtn * f.wide_ntn));
    const long items = np > 1 ? mtn * f.wide_ntn * np : (f.wide_ntn > 1 ? (mtn + 7) / 8 * 8 : mtn) * f.wide_ntn;
    const long rounds = (items + f.cus - 1) / f.cus;
    const int stages = (f.wide_stages + np - 1) / np;  // the longest part
    const double mb = np > 1 ? items * (sige::kLayerWideRows * sige::kLayerWideCols * 4e-6) : 0.0;
    return kChoice.w[0] + (double)rounds * (kChoice.w[1] * stages * f.wide_loads + kChoice.w[2]) +
           kChoice.w[3] * mb + (f.wide_pmax > 1 && np == 1 ? kGateOffCombine : 0.0);
}

// The plan: the split for lists of at most split_max blocks, the wide tiles
// for lists of at least wide_min, k_layer for the ones between (split_max -1:
// no split; wide_min > cap: no wide tiles).  Each nonempty subset of the
// available kernels, in that order by list length, is priced: a list goes to
// the cheapest kernel of the subset (the split for lengths up to the last one
// where it is, the wide tiles from the first one after that where they are,
// ahead of k_layer by kWideMargin),
// plus the empty launches of the subset's other kernels.  The plan is the
// subset whose worst relative loss against the cheapest kernel over list
// lengths 1..cap is smallest (fewer kernels on a tie).
void plan_thresholds(const LayerFeat &f, int *split_max, int *wide_min, int *wide_max) {
    const bool have[3] = {f.split_chunks > 0, true, f.wide_stages > 0};  // split, k_layer, wide
    const double off[3] = {kGateOffSplit, kGateOffSingle, kGateOffWide + (f.wide_pmax > 1 ? kGateOffCombine : 0.0)};
    std::vector<double> c[3];
    for (int k = 0; k < 3; ++k) c[k].assign(f.cap + 1, 1e30);
    std::vector<double> best(f.cap + 1, 1e30);
    for (int cnt = 1; cnt <= f.cap; ++cnt) {
        if (have[0]) c[0][cnt] = cost_split(f, cnt);
        c[1][cnt] = cost_single(f, cnt);
        if (have[2]) c[2][cnt] = cost_wide(f, cnt);
        for (int k = 0; k < 3; ++k) best[cnt] = fmin(best[cnt], c[k][cnt]);
    }
    double best_loss = 1e30;
    int best_n = 4;
    *split_max = -1;
    *wide_min = *wide_max = 0x7FFFFFFF;
    for (int mask = 1; mask < 8; ++mask) {
        bool ok = true;
        int n = 0;
        for (int k = 0; k < 3; ++k)
            if (mask >> k & 1) {
                ok = ok && have[k];
                ++n;
            }
        if (!ok) continue;
        // thresholds within the subset
        const bool S = mask & 1, L = mask & 2, W = mask & 4;
        int t1 = S ? 0 : -1, t2 = f.cap + 1, t3 = f.cap;
        if (S && !L && !W) t1 = f.cap;
        if (S && (L || W))
            for (int cnt = 1; cnt <= f.cap; ++cnt) {
                const double other = fmin(L ? c[1][cnt] : 1e30, W ? c[2][cnt] : 1e30);
                if (c[0][cnt] < other) t1 = cnt;
            }
        if (W && !L && !S) t2 = 1;
        if (W && (L || S)) {
            t2 = f.cap + 1;
            for (int cnt = t1 + 1; cnt <= f.cap; ++cnt)
                if (c[2][cnt] * (L ? kWideMargin : 1.0) < (L ? c[1][cnt] : c[0][cnt])) {
                    if (t2 > f.cap) t2 = cnt;
                    t3 = cnt;  // with k_layer, the last length where the wide tiles lead
                }
            if (!L) t3 = f.cap;
        }
        // kernels that actually get a range of lengths
        const bool runS = S && t1 >= 1, runW = W && t2 <= f.cap, runL = L && (t2 > t1 + 1 || t3 < f.cap);
        if (S && !runS) continue;  // priced as the smaller subset
        if (W && !runW) continue;
        if (L && !runL) continue;
        double loss = 0;
        for (int cnt = 1; cnt <= f.cap; ++cnt) {
            const int k = cnt <= t1 ? 0 : (cnt >= t2 && cnt <= t3 ? 2 : 1);
            double t = c[k][cnt];
            for (int j = 0; j < 3; ++j)
                if (j != k && (mask >> j & 1)) t += off[j];
            loss = fmax(loss, t / best[cnt]);
        }
        if (loss < best_loss - 1e-9 || (loss < best_loss + 1e-9 && n < best_n)) {
            best_loss = loss;
            best_n = n;
            *split_max = runS ? (runL || runW ? t1 : f.cap) : -1;
            *wide_min = runW ? (runL || runS ? t2 : 0) : 0x7FFFFFFF;
            *wide_max = runW ? (t3 < f.cap ? t3 : 0x7FFFFFFF) : 0x7FFFFFFF;
        }
    }
}

struct AutoPlan {
    sige::LayerCfg lc;
    ConvCfg cc;
    LayerFeat f;
    int split_max;  // -1: k_layer only; >= cap: the split only; else both, gated on *count
    int wide_min;   // lists of wide_min..wide_max blocks go to the wide tiles (min > cap: never)
    int wide_max;
    long ws_bytes;  // workspace: the split's partials (lists of at most split_max blocks), the wide tiles' K parts
};

// The plan of a layer, remembered per (geometry, dtype, device): the
// threshold scan prices every list length once.
int plan_auto(const Geo &g, int dt, AutoPlan *out) {
    struct Entry {
        Geo g;
        int dt, dev;
        AutoPlan p;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0, next = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = -1;
    }
    {
        std::lock_guard<std::mutex> lk(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].dt == dt && cache[i].dev == dev && !memcmp(&cache[i].g, &g, sizeof(Geo))) {
                *out = cache[i].p;
                return SIGE_OK;
            }
    }
    AutoPlan p{};
    int rc;
    if ((rc = choose_layer(g, dt, &p.lc))) return rc;
    p.f = layer_features(g, dt, p.lc);
    // the split's limits (LDS, register-resident weights) may exclude it, and
    // the wide tiles' (16-bit types, k <= 3, LDS) them
    plan_thresholds(p.f, &p.split_max, &p.wide_min, &p.wide_max);
    if (p.lc.wide_min < 0x7FFFFFFF && p.f.wide_stages > 0) {  // SIGE_WIDE_MIN (tuning): from there on, wide tiles
        p.wide_min = p.lc.wide_min;
        p.wide_max = 0x7FFFFFFF;
        if (p.split_max >= p.wide_min) p.split_max = p.wide_min - 1;
    }
    p.ws_bytes = 0;
    if (p.split_max >= 0) {
        if (choose_conv(g, dt, 1, 1, &p.cc, 1) != SIGE_OK) {
            p.split_max = -1;
        } else {
            Geo gt = g;
            gt.cap = p.split_max < g.cap ? p.split_max : g.cap;
            p.ws_bytes = sige::split_workspace_bytes(dt, gt, p.cc);
            if (p.ws_bytes < 0) return fail(SIGE_EINVAL, "unknown tile shape");
        }
    }
    if (p.split_max >= g.cap) {
        p.cc.gate_max = 0x7FFFFFFF;
    } else if (p.split_max >= 0) {
        p.cc.gate_max = p.split_max;
        p.lc.gate_min = p.split_max + 1;
    }
    if (p.f.wide_stages == 0) p.wide_min = p.wide_max = 0x7FFFFFFF;
    if (p.wide_min <= g.cap) {
        p.lc.gate_wide = p.wide_min;
        p.lc.wide_min = p.wide_min;
        p.lc.wide_max = p.wide_max;
    }
    // K parts of the wide tiles only when a list of their range makes any (the
    // shortest makes the fewest tiles); their partials share the workspace with
    // the split's, which never runs on the same list
    if (p.wide_min <= g.cap && p.lc.w_pmax > 1) {
        const long WR = sige::kLayerWideRows;
        const long mtn0 = ((long)(p.wide_min > 1 ? p.wide_min : 1) * g.b * g.b + WR - 1) / WR;
        if (sige::wide_parts(p.lc.cus, p.lc.w_pmax, (int)(mtn0 * p.lc.w_ntn)) < 2) {
            p.lc.w_pmax = 1;
        } else {
            const long wb = (long)p.lc.w_ws_items * WR * sige::kLayerWideCols * 4;
            if (wb > p.ws_bytes) p.ws_bytes = wb;
        }
    } else {
        p.lc.w_pmax = 1;
    }
    std::lock_guard<std::mutex> lk(mu);
    Entry &e = cache[used < 64 ? used++ : (next++ & 63)];
    e.g = g;
    e.dt = dt;
    e.dev = dev;
    e.p = p;
    *out = p;
    return SIGE_OK;
}

}  // namespace

extern "C" {

const char *sige_strerror(int code) {
    switch (code) {
    case SIGE_OK: return "SIGE_OK";
    case SIGE_EINVAL: return "SIGE_EINVAL: invalid argument";
    case SIGE_EDTYPE: return "SIGE_EDTYPE: unsupported dtype";
    case SIGE_EALIGN: return "SIGE_EALIGN: misaligned pointer or channel row";
    case SIGE_EHIP: return "SIGE_EHIP: HIP runtime error";
    case SIGE_ENODEV: return "SIGE_ENODEV: no GPU";
    case SIGE_ERANGE: return "SIGE_ERANGE: size beyond a kernel limit";
    default: return "unknown status code";
    }
}

const char *sige_last_error(void) { return g_msg; }

int sige_geom_derive(const sige_geom *g, sige_derived *out) {
    Geo d;
    const int rc = derive(g, &d);
    if (rc) return rc;
    if (!out) return fail(SIGE_EINVAL, "output pointer is NULL");
    out->ho = d.ho;
    out->wo = d.wo;
    out->nby = d.nby;
    out->nbx = d.nbx;
    out->ib = d.ib;
    out->cap = d.cap;
    g_msg[0] = 0;
    return SIGE_OK;
}

int64_t sige_max_blocks(const sige_geom *g) {
    Geo d;
    const int rc = derive(g, &d);
    if (rc) return rc;
    g_msg[0] = 0;
    return (int64_t)d.cap;
}

int sige_diff_mask_bits(const void *a_orig, const void *a_edit, int dtype, int n, int h, int w, int c, float thresh,
                        uint8_t *mask, uint32_t *bits, void *stream) {
    const char *what = bits ? "sige_diff_mask_bits" : "sige_diff_mask";
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    if (n < 0 || h < 0 || w < 0 || c < 1) return fail(SIGE_EINVAL, "bad shape n=%d h=%d w=%d c=%d", n, h, w, c);
    if (!(thresh >= 0.0f) || thresh > 3.0e38f) return fail(SIGE_EINVAL, "threshold must be finite and >= 0");
    if (bits && w % 32) return fail(SIGE_EINVAL, "bitset mask: width %d must be a multiple of 32", w);
    const long npix = (long)n * h * w;
    if (npix == 0) {
        g_msg[0] = 0;
        return SIGE_OK;
    }
    if (!a_orig || !a_edit || (!mask && !bits)) return fail(SIGE_EINVAL, "NULL tensor pointer");
    int rc = channel_rows_ok(dtype, c, "c");
    if (rc) return rc;
    if (!aligned(a_orig, 16) || !aligned(a_edit, 16)) return fail(SIGE_EALIGN, "activations must be 16-byte aligned");
    if (!aligned(mask, 4) || !aligned(bits, 4)) return fail(SIGE_EALIGN, "mask and bits must be 4-byte aligned");
    const size_t bytes = (size_t)npix * c * sige::elem_bytes(dtype);
    if (mask && (overlap(mask, (size_t)npix, a_orig, bytes) || overlap(mask, (size_t)npix, a_edit, bytes)))
        return fail(SIGE_EINVAL, "mask overlaps an input");
    if (bits && (overlap(bits, (size_t)npix / 8, a_orig, bytes) || overlap(bits, (size_t)npix / 8, a_edit, bytes) ||
                 (mask && overlap(bits, (size_t)npix / 8, mask, (size_t)npix))))
        return fail(SIGE_EINVAL, "bits overlap an input or the mask");
    if ((rc = device_ready())) return rc;
    const int vpp = c * sige::elem_bytes(dtype) / 16;
    return finish(sige::launch_diff(dtype, a_orig, a_edit, npix, vpp, thresh, mask, bits, (hipStream_t)stream), what,
                  (hipStream_t)stream);
}

int sige_diff_mask(const void *a_orig, const void *a_edit, int dtype, int n, int h, int w, int c, float thresh,
                   uint8_t *mask, void *stream) {
    return sige_diff_mask_bits(a_orig, a_edit, dtype, n, h, w, c, thresh, mask, nullptr, stream);
}


int sige_reduce_mask(const uint8_t *mask, int mask_h, int mask_w, const sige_geom *gp, int dilate_blocks,
                     int32_t *idx, int32_t *count, void *stream) {
    return reduce_common(mask, mask_h, mask_w, gp, dilate_blocks, idx, count, 0, nullptr, nullptr, stream,
                         "sige_reduce_mask");
}

int sige_reduce_bits(const uint32_t *bits, int mask_h, int mask_w, const sige_geom *gp, int dilate_blocks,
                     int32_t *idx, int32_t *count, void *stream) {
    return reduce_common((const uint8_t *)bits, mask_h, mask_w, gp, dilate_blocks, idx, count, 0, nullptr, nullptr,
                         stream, "sige_reduce_bits", 1);
}

int sige_reduce_bits_copy(const uint32_t *bits, int mask_h, int mask_w, const sige_geom *gp, int dilate_blocks,
                          int32_t *idx, int32_t *count, int dtype, const void *cached, void *out, void *stream) {
    if (!out) return fail(SIGE_EINVAL, "NULL pointer");
    return reduce_common((const uint8_t *)bits, mask_h, mask_w, gp, dilate_blocks, idx, count, dtype, cached, out,
                         stream, "sige_reduce_bits_copy", 1);
}

int sige_reduce_bits_layers(const uint32_t *bits, int mask_h, int mask_w, int nlayers, const sige_geom *geoms,
                            const int *dilate_blocks, int32_t *const *idx, int32_t *const *count, int dtype,
                            const void *const *cached, void *const *out, void *stream) {
    if (nlayers < 1 || nlayers > sige::kReduceMaxLayers)
        return fail(SIGE_EINVAL, "nlayers=%d outside [1, %d]", nlayers, sige::kReduceMaxLayers);
    if (!bits || !geoms || !dilate_blocks || !idx || !count) return fail(SIGE_EINVAL, "NULL pointer");
    if (mask_w % 32 || !aligned(bits, 4))
        return fail(mask_w % 32 ? SIGE_EINVAL : SIGE_EALIGN, "bitset mask: width %d must be a multiple of 32 and "
                    "the words 4-byte aligned", mask_w);
    sige::ReduceLayerArgs L[sige::kReduceMaxLayers];
    Region wr[3 * sige::kReduceMaxLayers], rd[1 + sige::kReduceMaxLayers];
    int nw = 0, nr = 0, rc;
    for (int l = 0; l < nlayers; ++l) {
        Geo g;
        if ((rc = derive(&geoms[l], &g))) return rc;
        if (!idx[l] || !count[l]) return fail(SIGE_EINVAL, "layer %d: NULL idx or count", l);
        if (l == 0) {
            rd[nr++] = Region{bits, (size_t)g.n * mask_h * mask_w / 8};
        } else if (g.n != geoms[0].n) {
            return fail(SIGE_EINVAL, "layer %d: n=%d differs from layer 0 (one mask for every layer)", l, g.n);
        }
        if (mask_h < g.h || mask_w < g.w || mask_h % g.h || mask_w % g.w)
            return fail(SIGE_EINVAL, "layer %d: mask %dx%d is not an integer multiple of the conv input %dx%d", l,
                        mask_h, mask_w, g.h, g.w);
        if (dilate_blocks[l] < 0 || dilate_blocks[l] > 16)
            return fail(SIGE_EINVAL, "layer %d: dilate_blocks=%d outside [0, 16]", l, dilate_blocks[l]);
        if (g.w > sige::kReduceMaxWidth)
            return fail(SIGE_ERANGE, "layer %d: conv input width %d exceeds the reduce limit %d", l, g.w,
                        sige::kReduceMaxWidth);
        if (g.cap > sige::kReduceMaxBlocks)
            return fail(SIGE_ERANGE, "layer %d: %d blocks (n*nby*nbx) exceed the reduce limit %d", l, g.cap,
                        sige::kReduceMaxBlocks);
        if (!sige::reduce_one_launch_ok(mask_h, mask_w, g, 2))
            return fail(SIGE_ERANGE, "layer %d: its pooled mask or block grid exceeds one workgroup "
                        "(build its list with sige_reduce_bits)", l);
        if (!aligned(idx[l], 4) || !aligned(count[l], 4))
            return fail(SIGE_EALIGN, "layer %d: idx/count must be 4-byte aligned", l);
        wr[nw++] = Region{idx[l], (size_t)g.cap * 4};
        wr[nw++] = Region{count[l], 4};
        L[l] = sige::ReduceLayerArgs{g, dilate_blocks[l], idx[l], count[l], nullptr, nullptr, 0};
        const void *c = cached ? cached[l] : nullptr;
        void *o = out ? out[l] : nullptr;
        if (!c != !o) return fail(SIGE_EINVAL, "layer %d: cached and out must both be given or both NULL", l);
        if (o) {
            if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
            if ((rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
            if (!aligned(c, 16) || !aligned(o, 16)) return fail(SIGE_EALIGN, "layer %d: tensors must be 16-byte aligned", l);
            const size_t ob = (size_t)g.n * g.ho * g.wo * g.cout * sige::elem_bytes(dtype);
            wr[nw++] = Region{o, ob};
            rd[nr++] = Region{c, ob};
            L[l].src = (const uint8_t *)c;
            L[l].dst = (uint8_t *)o;
            L[l].nvec = (long long)(ob / 16);
        }
    }
    if (regions_overlap(wr, nw, rd, nr))  // what the launch writes overlaps nothing else it touches
        return fail(SIGE_EINVAL, "an output of the layers overlaps another output, the mask or a cache");
    if ((rc = device_ready())) return rc;
    static int copy_wgs = -1;  // SIGE_REDUCE_COPY_WGS overrides the copy's workgroups (tuning)
    if (copy_wgs < 0) {
        const char *v = getenv("SIGE_REDUCE_COPY_WGS");
        const long x = v ? strtol(v, nullptr, 10) : 0;
        copy_wgs = (x > 0 && x < 65536) ? (int)x : 0;
    }
    return finish(sige::launch_reduce_layers(bits, mask_h, mask_w, nlayers, L, copy_wgs ? copy_wgs : dev_info().cus / 2,
                                             (hipStream_t)stream),
                  "sige_reduce_bits_layers", (hipStream_t)stream);
}

int sige_reduce_mask_copy(const uint8_t *mask, int mask_h, int mask_w, const sige_geom *gp, int dilate_blocks,
                          int32_t *idx, int32_t *count, int dtype, const void *cached, void *out, void *stream) {
    if (!out) return fail(SIGE_EINVAL, "NULL pointer");
    return reduce_common(mask, mask_h, mask_w, gp, dilate_blocks, idx, count, dtype, cached, out, stream,
                         "sige_reduce_mask_copy");
}

int sige_gather(const void *a_edit, int dtype, const sige_geom *gp, const int32_t *idx, const int32_t *count,
                void *blocks, void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !idx || !count || !blocks) return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(blocks, 16)) return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    const int es = sige::elem_bytes(dtype);
    {
        const Region wr[] = {{blocks, (size_t)g.cap * g.ib * g.ib * g.cin * es}};
        const Region rd[] = {{a_edit, (size_t)g.n * g.h * g.w * g.cin * es}, {idx, (size_t)g.cap * 4}, {count, 4}};
        if (regions_overlap(wr, 1, rd, 3)) return fail(SIGE_EINVAL, "blocks overlap the input, idx or count");
    }
    if ((rc = device_ready())) return rc;
    return finish(sige::launch_gather(a_edit, dtype, g, idx, count, blocks, (hipStream_t)stream), "sige_gather",
                  (hipStream_t)stream);
}

// The packed copy of a layer's weights (sige_pack_weights): the single-range
// kernel's fragment-order section, then (16-bit types, where the wide tiles
// can run) the wide tiles' stage-major section at a 256-byte aligned offset.
struct PackedLayout {
    sige::LayerCfg lc;
    ConvCfg cc;  // the split's configuration (split_bytes 0: the split cannot run)
    int64_t layer_bytes, wide_off, wide_bytes, split_off, split_bytes, total;
};

static int packed_layout(const Geo &g, int dtype, PackedLayout *pl) {
    int rc = choose_layer(g, dtype, &pl->lc);
    if (rc) return rc;
    pl->layer_bytes = (int64_t)sige::layer_weights_units(g, pl->lc) * 16;
    pl->wide_off = (pl->layer_bytes + 255) / 256 * 256;
    pl->wide_bytes = dtype != SIGE_F32 && pl->lc.w_lds > 0 ? (int64_t)sige::wide_weights_units(g) * 16 : 0;
    pl->split_off = (pl->wide_off + pl->wide_bytes + 255) / 256 * 256;
    pl->split_bytes = choose_conv(g, dtype, 1, 1, &pl->cc, 1) == SIGE_OK
                          ? (int64_t)sige::split_weights_units(dtype, g, pl->cc) * 16
                          : 0;
    pl->total = pl->split_off + pl->split_bytes;
    return SIGE_OK;
}

// Checks of a caller's packed weights against the layout: non-NULL, aligned,
// large enough, not overlapping the written regions wr[0, nwr).
static int check_packed(const void *w_packed, int64_t w_packed_bytes, const PackedLayout &pl, const Region *wr,
                        int nwr);

static int conv_blocks(const void *blocks, const void *w_krsc, const float *bias, int dtype, const sige_geom *gp,
                       const int32_t *count, void *out_blocks, const void *w_packed, int64_t w_packed_bytes,
                       void *stream, const char *name) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!blocks || !w_krsc || !count || !out_blocks) return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(blocks, 16) || !aligned(w_krsc, 16) || !aligned(out_blocks, 16))
        return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    const int es = sige::elem_bytes(dtype);
    {
        const Region wr[] = {{out_blocks, (size_t)g.cap * g.b * g.b * g.cout * es}};
        const Region rd[] = {{blocks, (size_t)g.cap * g.ib * g.ib * g.cin * es},
                             {w_krsc, (size_t)g.cout * g.k * g.k * g.cin * es}, {bias, (size_t)g.cout * 4}, {count, 4}};
        if (regions_overlap(wr, 1, rd, 4)) return fail(SIGE_EINVAL, "out_blocks overlaps blocks, weights, bias or count");
    }
    sige::LayerCfg cfg;
    if ((rc = choose_layer(g, dtype, &cfg))) return rc;
    if (w_packed) {
        PackedLayout pl;
        if ((rc = packed_layout(g, dtype, &pl))) return rc;
        const Region wr[] = {{out_blocks, (size_t)g.cap * g.b * g.b * g.cout * es}};
        if ((rc = check_packed(w_packed, w_packed_bytes, pl, wr, 1))) return rc;
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, false);
    return finish(sige::launch_layer(dtype, 0, blocks, w_krsc, bias, nullptr, count, out_blocks, nullptr, nullptr,
                                     nullptr, g, cfg, cc, (hipStream_t)stream, w_packed),
                  name, (hipStream_t)stream);
}

int sige_conv_blocks(const void *blocks, const void *w_krsc, const float *bias, int dtype, const sige_geom *gp,
                     const int32_t *count, void *out_blocks, void *stream) {
    return conv_blocks(blocks, w_krsc, bias, dtype, gp, count, out_blocks, nullptr, 0, stream, "sige_conv_blocks");
}

int sige_conv_blocks_packed(const void *blocks, const void *w_krsc, const float *bias, int dtype,
                            const sige_geom *gp, const int32_t *count, void *out_blocks, const void *w_packed,
                            int64_t w_packed_bytes, void *stream) {
    if (!w_packed) return fail(SIGE_EINVAL, "NULL pointer");
    return conv_blocks(blocks, w_krsc, bias, dtype, gp, count, out_blocks, w_packed, w_packed_bytes, stream,
                       "sige_conv_blocks_packed");
}

int sige_scatter(const void *out_blocks, const int32_t *idx, const int32_t *count, const sige_geom *gp, int dtype,
                 const void *cached, void *out, int copy_cached, void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!out_blocks || !idx || !count || !out || (copy_cached && !cached)) return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(out_blocks, 16) || !aligned(out, 16) || (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    {
        const Region wr[] = {{out, obytes}};
        const Region rd[] = {{copy_cached ? cached : nullptr, obytes},
                             {out_blocks, (size_t)g.cap * g.b * g.b * g.cout * es}, {idx, (size_t)g.cap * 4}, {count, 4}};
        if (regions_overlap(wr, 1, rd, 4)) return fail(SIGE_EINVAL, "out overlaps cached, out_blocks, idx or count");
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    const DevInfo dv = dev_info();
    const int grid = dv.cus * 4;
    return finish(sige::launch_scatter(dtype, out_blocks, idx, count, g, copy_cached ? cached : nullptr, out, grid, cc,
                                       (hipStream_t)stream),
                  "sige_scatter", (hipStream_t)stream);
}


static int layer_single(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                        const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                        int copy_cached, const void *w_packed, int64_t w_packed_bytes, void *stream,
                        const char *name) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !w_krsc || !idx || !count || !out || (copy_cached && !cached))
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(w_krsc, 16) || !aligned(out, 16) || (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    {
        const Region wr[] = {{out, obytes}};
        const Region rd[] = {{a_edit, (size_t)g.n * g.h * g.w * g.cin * es}, {copy_cached ? cached : nullptr, obytes},
                             {w_krsc, (size_t)g.cout * g.k * g.k * g.cin * es}, {bias, (size_t)g.cout * 4},
                             {idx, (size_t)g.cap * 4}, {count, 4}};
        if (regions_overlap(wr, 1, rd, 6))
            return fail(SIGE_EINVAL, "out overlaps a_edit, cached, the weights, bias, idx or count");
    }
    sige::LayerCfg cfg;
    if ((rc = choose_layer(g, dtype, &cfg))) return rc;
    if (w_packed) {
        PackedLayout pl;
        if ((rc = packed_layout(g, dtype, &pl))) return rc;
        const Region wr[] = {{out, obytes}};
        if ((rc = check_packed(w_packed, w_packed_bytes, pl, wr, 1))) return rc;
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    return finish(sige::launch_layer(dtype, 1, a_edit, w_krsc, bias, idx, count, out, copy_cached ? cached : nullptr,
                                     nullptr, nullptr, g, cfg, cc, (hipStream_t)stream, w_packed),
                  name, (hipStream_t)stream);
}

int sige_sparse_conv_layer(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                           const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                           int copy_cached, void *stream) {
    return layer_single(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, nullptr, 0, stream,
                        "sige_sparse_conv_layer");
}

int sige_sparse_conv_layer_packed(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                  const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp,
                                  void *out, int copy_cached, const void *w_packed, int64_t w_packed_bytes,
                                  void *stream) {
    if (!w_packed) return fail(SIGE_EINVAL, "NULL pointer");
    return layer_single(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, w_packed,
                        w_packed_bytes, stream, "sige_sparse_conv_layer_packed");
}

int sige_sparse_conv_layer_plan(const sige_geom *gp, int dtype, sige_layer_plan *out) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!out) return fail(SIGE_EINVAL, "output pointer is NULL");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    AutoPlan p;
    if ((rc = plan_auto(g, dtype, &p))) return rc;
    out->split_max = p.split_max;
    out->cap = g.cap;
    out->workspace_bytes = p.ws_bytes;
    out->chunks = p.f.chunks;
    out->steps = p.f.steps;
    out->stage_groups = p.f.groups;
    out->slots = p.f.slots;
    out->n_tiles = p.f.ntn;
    out->weight_mb = p.f.wmb;
    out->gflop_per_block = p.f.gflop_per_block;
    out->split_chunks = p.f.split_chunks;
    out->split_slots = p.f.split_slots;
    out->split_stage_kb = p.f.split_kb;
    out->wide_min = p.wide_min;
    out->wide_max = p.wide_max;
    out->wide_parts_max = p.f.wide_stages > 0 ? p.f.wide_pmax : 0;
    out->wide_stages = p.f.wide_stages;
    out->wide_loads = p.f.wide_loads;
    out->wide_n_tiles = p.f.wide_ntn;
    g_msg[0] = 0;
    return SIGE_OK;
}


static int layer_auto(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                      const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                      int copy_cached, void *workspace, int64_t workspace_bytes, const void *w_packed,
                      int64_t w_packed_bytes, void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !w_krsc || !idx || !count || !out || (copy_cached && !cached))
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(w_krsc, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
        (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors and workspace must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    if (workspace_bytes < 0) return fail(SIGE_EINVAL, "negative workspace size");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    const Region rd[] = {{a_edit, (size_t)g.n * g.h * g.w * g.cin * es}, {copy_cached ? cached : nullptr, obytes},
                         {w_krsc, (size_t)g.cout * g.k * g.k * g.cin * es}, {bias, (size_t)g.cout * 4},
                         {idx, (size_t)g.cap * 4}, {count, 4}};
    {
        const Region wr[] = {{out, obytes}};
        if (regions_overlap(wr, 1, rd, 6))
            return fail(SIGE_EINVAL, "out overlaps a_edit, cached, the weights, bias, idx or count");
    }
    AutoPlan p;
    if ((rc = plan_auto(g, dtype, &p))) return rc;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes)
            return fail(SIGE_ERANGE, "workspace of %lld bytes, %ld needed", (long long)workspace_bytes, p.ws_bytes);
        const Region wr[] = {{out, obytes}, {workspace, (size_t)p.ws_bytes}};
        if (regions_overlap(wr, 2, rd, 6)) return fail(SIGE_EINVAL, "the workspace overlaps another argument");
    }
    const uint8_t *wp = nullptr, *ww = nullptr, *wsp = nullptr;  // the packed sections, when given
    if (w_packed) {
        PackedLayout pl;
        if ((rc = packed_layout(g, dtype, &pl))) return rc;
        const Region wr[] = {{out, obytes}, {workspace, (size_t)(p.ws_bytes > 0 ? p.ws_bytes : 0)}};
        if ((rc = check_packed(w_packed, w_packed_bytes, pl, wr, 2))) return rc;
        wp = (const uint8_t *)w_packed;
        ww = pl.wide_bytes > 0 ? wp + pl.wide_off : nullptr;
        // the split's section follows the split's configuration of the plan
        wsp = pl.split_bytes > 0 && pl.cc.ck == p.cc.ck && pl.cc.nt == p.cc.nt ? wp + pl.split_off : nullptr;
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    const hipStream_t st = (hipStream_t)stream;
    // k_layer: every list when the split never wins, else those above split_max
    // (and below wide_min)
    if (p.split_max < g.cap && (p.wide_min > p.split_max + 1 || p.wide_max < g.cap)) {
        if ((rc = finish(sige::launch_layer(dtype, 1, a_edit, w_krsc, bias, idx, count, out,
                                            copy_cached ? cached : nullptr, nullptr, nullptr, g, p.lc, cc, st, wp),
                         "sige_sparse_conv_layer_auto", st)))
            return rc;
    }
    if (p.wide_min <= g.cap) {  // the wide tiles: lists of at least wide_min blocks
        if ((rc = finish(sige::launch_layer_wide(dtype, a_edit, w_krsc, bias, idx, count, out,
                                                 copy_cached ? cached : nullptr, g, p.lc, cc, st, (float *)workspace,
                                                 ww),
                         "sige_sparse_conv_layer_auto", st)))
            return rc;
    }
    if (p.split_max >= 0)  // the split: lists of at most split_max blocks
        return finish(sige::launch_conv(dtype, 1, a_edit, w_krsc, bias, idx, count, out,
                                        copy_cached ? cached : nullptr, nullptr, nullptr, g, p.cc, cc, st,
                                        (float *)workspace, wsp),
                      "sige_sparse_conv_layer_auto", st);
    return SIGE_OK;
}

int sige_sparse_conv_layer_auto(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                                int copy_cached, void *workspace, int64_t workspace_bytes, void *stream) {
    return layer_auto(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, workspace,
                      workspace_bytes, nullptr, 0, stream);
}

int sige_sparse_conv_layer_auto_packed(const void *a_edit, const void *w_krsc, const float *bias,
                                       const void *cached, const int32_t *idx, const int32_t *count, int dtype,
                                       const sige_geom *gp, void *out, int copy_cached, void *workspace,
                                       int64_t workspace_bytes, const void *w_packed, int64_t w_packed_bytes,
                                       void *stream) {
    if (!w_packed) return fail(SIGE_EINVAL, "NULL pointer");
    return layer_auto(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, workspace,
                      workspace_bytes, w_packed, w_packed_bytes, stream);
}

static int check_packed(const void *w_packed, int64_t w_packed_bytes, const PackedLayout &pl, const Region *wr,
                        int nwr) {
    if (!w_packed) return fail(SIGE_EINVAL, "NULL pointer");
    if (!aligned(w_packed, 256)) return fail(SIGE_EALIGN, "packed weights must be 256-byte aligned");
    if (w_packed_bytes < pl.total)
        return fail(SIGE_ERANGE, "packed weights of %lld bytes, %lld needed", (long long)w_packed_bytes,
                    (long long)pl.total);
    const Region rd[] = {{w_packed, (size_t)pl.total}};
    if (regions_overlap(wr, nwr, rd, 1)) return fail(SIGE_EINVAL, "the packed weights overlap an output");
    return SIGE_OK;
}

int64_t sige_packed_weights_bytes(const sige_geom *gp, int dtype) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    PackedLayout pl;
    if ((rc = packed_layout(g, dtype, &pl))) return rc;
    return pl.total;
}

int sige_pack_weights(const void *w_krsc, int dtype, const sige_geom *gp, void *w_packed, int64_t w_packed_bytes,
                      void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!w_krsc || !w_packed) return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(w_krsc, 16)) return fail(SIGE_EALIGN, "weights must be 16-byte aligned");
    PackedLayout pl;
    if ((rc = packed_layout(g, dtype, &pl))) return rc;
    const Region wr[] = {{w_krsc, (size_t)g.cout * g.k * g.k * g.cin * sige::elem_bytes(dtype)}};
    if ((rc = check_packed(w_packed, w_packed_bytes, pl, wr, 1))) return rc;
    if ((rc = device_ready())) return rc;
    const hipStream_t st = (hipStream_t)stream;
    const int cus = dev_info().cus;
    if ((rc = finish(sige::launch_layer_weights_pack(dtype, w_krsc, g, pl.lc, w_packed, cus, st), "sige_pack_weights",
                     st)))
        return rc;
    if (pl.wide_bytes > 0 &&
        (rc = finish(sige::launch_wide_weights_pack(w_krsc, g, (uint8_t *)w_packed + pl.wide_off, cus, st),
                     "sige_pack_weights", st)))
        return rc;
    if (pl.split_bytes > 0)
        return finish(sige::launch_split_weights_pack(dtype, w_krsc, g, pl.cc, (uint8_t *)w_packed + pl.split_off,
                                                      cus, st),
                      "sige_pack_weights", st);
    return SIGE_OK;
}

int64_t sige_sparse_conv_layer_split_workspace(const sige_geom *gp, int dtype) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 1, 1, &cfg, 1))) return rc;
    const long bytes = sige::split_workspace_bytes(dtype, g, cfg);
    if (bytes < 0) return fail(SIGE_EINVAL, "unknown tile shape");
    g_msg[0] = 0;
    return (int64_t)bytes;
}

int sige_sparse_conv_layer_split(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                 const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                                 int copy_cached, void *workspace, int64_t workspace_bytes, void *stream) {
    return split_common(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, workspace,
                        workspace_bytes, stream, "sige_sparse_conv_layer_split");
}

int64_t sige_noalloc_scratch_bytes(void) { return (int64_t)kScratchBytes; }

int sige_sparse_conv_layer_split_noalloc(const void *a_edit, const void *w_krsc, const float *bias,
                                         const void *cached, const int32_t *idx, const int32_t *count, int dtype,
                                         const sige_geom *gp, void *out, int copy_cached, void *stream) {
    return split_common(a_edit, w_krsc, bias, cached, idx, count, dtype, gp, out, copy_cached, nullptr, 0, stream,
                        "sige_sparse_conv_layer_split_noalloc", true);
}

int sige_sparse_conv_layer_restore(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                   const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                                   const int32_t *count, int dtype, const sige_geom *gp, void *out, void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !w_krsc || !cached || !prev_idx || !prev_count || !idx || !count || !out)
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(w_krsc, 16) || !aligned(out, 16) || !aligned(cached, 16))
        return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    {
        const Region wr[] = {{out, obytes}};
        const Region rd[] = {{a_edit, (size_t)g.n * g.h * g.w * g.cin * es}, {cached, obytes},
                             {w_krsc, (size_t)g.cout * g.k * g.k * g.cin * es}, {bias, (size_t)g.cout * 4},
                             {idx, (size_t)g.cap * 4}, {count, 4}, {prev_idx, (size_t)g.cap * 4}, {prev_count, 4}};
        if (regions_overlap(wr, 1, rd, 8))
            return fail(SIGE_EINVAL, "out overlaps a_edit, cached, the weights, bias or a list");
    }
    sige::LayerCfg cfg;
    if ((rc = choose_layer(g, dtype, &cfg))) return rc;
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, false);
    return finish(sige::launch_layer(dtype, 1, a_edit, w_krsc, bias, idx, count, out, cached, prev_idx, prev_count,
                                     g, cfg, cc, (hipStream_t)stream),
                  "sige_sparse_conv_layer_restore", (hipStream_t)stream);
}

int64_t sige_sparse_attention_workspace(int n, int h, int w, int heads, int head_dim, int block) {
    Geo g;
    const int rc = attn_geom(n, h, w, heads, head_dim, block, &g);
    if (rc) return rc;
    g_msg[0] = 0;
    return attn_ws_bytes(g, heads, attn_grid1());
}

int sige_sparse_attention(const void *q, const void *k, const void *v, const int32_t *idx, const int32_t *count,
                          int dtype, int n, int h, int w, int heads, int head_dim, int block, float scale,
                          const void *cached, void *out, int copy_cached, void *workspace, int64_t workspace_bytes,
                          void *stream) {
    if (dtype != SIGE_BF16 && dtype != SIGE_F16) return fail(SIGE_EDTYPE, "dtype %d: bf16 or fp16 only", dtype);
    Geo g;
    int rc = attn_geom(n, h, w, heads, head_dim, block, &g);
    if (rc) return rc;
    if (!q || !k || !v || !idx || !count || !out || !workspace || (copy_cached && !cached))
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cout, "heads*head_dim"))) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
        (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors and workspace must be 16-byte aligned");
    if (!(scale > 0.f) || scale > 1e6f) return fail(SIGE_EINVAL, "scale must be positive and finite");
    const size_t tbytes = (size_t)n * h * w * g.cout * 2;
    const Region rd[] = {{q, tbytes}, {k, tbytes}, {v, tbytes}, {copy_cached ? cached : nullptr, tbytes},
                         {idx, (size_t)g.cap * 4}, {count, 4}};
    {
        const Region wr[] = {{out, tbytes}};
        if (regions_overlap(wr, 1, rd, 6)) return fail(SIGE_EINVAL, "out overlaps q, k, v, cached, idx or count");
    }
    const int grid1 = attn_grid1();  // from the device's CU count (gfx950's 256 when none is visible)
    const int64_t need = attn_ws_bytes(g, heads, grid1);
    if (workspace_bytes < need)
        return fail(SIGE_ERANGE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
    {
        const Region wr[] = {{out, tbytes}, {workspace, (size_t)need}};
        if (regions_overlap(wr, 2, rd, 6)) return fail(SIGE_EINVAL, "the workspace overlaps another argument");
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, 2, copy_cached != 0);
    return finish(sige::launch_attention(dtype, q, k, v, idx, count, g, heads, scale, copy_cached ? cached : nullptr,
                                         out, cc, workspace, grid1, dev_info().cus * 4, (hipStream_t)stream),
                  "sige_sparse_attention", (hipStream_t)stream);
}

int sige_restore_blocks(const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                        const int32_t *count, const sige_geom *gp, int dtype, const void *cached, void *out,
                        void *stream) {
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!prev_idx || !prev_count || !cached || !out) return fail(SIGE_EINVAL, "NULL pointer");
    if ((idx == nullptr) != (count == nullptr)) return fail(SIGE_EINVAL, "idx and count must both be given or both NULL");
    if ((rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(cached, 16) || !aligned(out, 16)) return fail(SIGE_EALIGN, "tensors must be 16-byte aligned");
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * sige::elem_bytes(dtype);
    {
        const Region wr[] = {{out, obytes}};
        const Region rd[] = {{cached, obytes}, {prev_idx, (size_t)g.cap * 4}, {prev_count, 4},
                             {idx, (size_t)g.cap * 4}, {count, 4}};
        if (regions_overlap(wr, 1, rd, 5)) return fail(SIGE_EINVAL, "out overlaps cached or a list");
    }
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, sige::elem_bytes(dtype), true);
    const DevInfo dv = dev_info();
    const int grid = g.cap < dv.cus ? g.cap : dv.cus;
    return finish(sige::launch_restore(prev_idx, prev_count, idx, count, g, cc, cached, out, grid, (hipStream_t)stream),
                  "sige_restore_blocks", (hipStream_t)stream);
}

}  // extern "C"
