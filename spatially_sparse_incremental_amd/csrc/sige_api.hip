// sige_api.hip -- the C ABI of libsige.so: argument checks, status codes,
// launch configuration.  Every check runs on the host before anything is
// enqueued; the kernels live in kernels_mask.hip and kernels_conv.hip.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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
    long grid = 1L << 30;  // the launch trims this to the CUs' resident capacity
    if (!(fused && copy))  // tiles at capacity, M tiles padded to a multiple of 8 (see the kernel's tile order)
        grid = (((long)g.cap * b2 + BM - 1) / BM + 7) / 8 * 8 * ((g.cout + BN - 1) / BN);
    c.cus = dv.cus;
    c.grid = (int)(grid > 0 ? grid : 1);
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
    struct Region {
        const void *p;
        size_t n;
    } wr[3 * sige::kReduceMaxLayers], rd[1 + sige::kReduceMaxLayers];
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
    for (int i = 0; i < nw; ++i) {  // what the launch writes overlaps nothing else it touches
        for (int j = i + 1; j < nw; ++j)
            if (overlap(wr[i].p, wr[i].n, wr[j].p, wr[j].n)) return fail(SIGE_EINVAL, "outputs of the layers overlap");
        for (int j = 0; j < nr; ++j)
            if (overlap(wr[i].p, wr[i].n, rd[j].p, rd[j].n))
                return fail(SIGE_EINVAL, "an output overlaps the mask or a cache");
    }
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
    if (overlap(blocks, (size_t)g.cap * g.ib * g.ib * g.cin * es, a_edit, (size_t)g.n * g.h * g.w * g.cin * es))
        return fail(SIGE_EINVAL, "blocks overlap the input");
    if ((rc = device_ready())) return rc;
    return finish(sige::launch_gather(a_edit, dtype, g, idx, count, blocks, (hipStream_t)stream), "sige_gather",
                  (hipStream_t)stream);
}

int sige_conv_blocks(const void *blocks, const void *w_krsc, const float *bias, int dtype, const sige_geom *gp,
                     const int32_t *count, void *out_blocks, void *stream) {
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
    if (overlap(out_blocks, (size_t)g.cap * g.b * g.b * g.cout * es, blocks, (size_t)g.cap * g.ib * g.ib * g.cin * es))
        return fail(SIGE_EINVAL, "out_blocks overlaps blocks");
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 0, 0, &cfg))) return rc;
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, false);
    return finish(sige::launch_conv(dtype, 0, blocks, w_krsc, bias, nullptr, count, out_blocks, nullptr, nullptr,
                                    nullptr, g, cfg, cc,
                                    (hipStream_t)stream),
                  "sige_conv_blocks", (hipStream_t)stream);
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
    if (copy_cached && overlap(out, obytes, cached, obytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    if (overlap(out, obytes, out_blocks, (size_t)g.cap * g.b * g.b * g.cout * es))
        return fail(SIGE_EINVAL, "out overlaps out_blocks");
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    const DevInfo dv = dev_info();
    const int grid = dv.cus * 4;
    return finish(sige::launch_scatter(dtype, out_blocks, idx, count, g, copy_cached ? cached : nullptr, out, grid, cc,
                                       (hipStream_t)stream),
                  "sige_scatter", (hipStream_t)stream);
}

int sige_sparse_conv_layer(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                           const int32_t *idx, const int32_t *count, int dtype, const sige_geom *gp, void *out,
                           int copy_cached, void *stream) {
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
    if (overlap(out, obytes, a_edit, (size_t)g.n * g.h * g.w * g.cin * es))
        return fail(SIGE_EINVAL, "out overlaps a_edit");
    if (copy_cached && overlap(out, obytes, cached, obytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 1, copy_cached, &cfg))) return rc;
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    return finish(sige::launch_conv(dtype, 1, a_edit, w_krsc, bias, idx, count, out, copy_cached ? cached : nullptr,
                                    nullptr, nullptr, g, cfg, cc, (hipStream_t)stream),
                  "sige_sparse_conv_layer", (hipStream_t)stream);
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
    if (!dtype_ok(dtype)) return fail(SIGE_EDTYPE, "dtype %d", dtype);
    Geo g;
    int rc = derive(gp, &g);
    if (rc) return rc;
    if (!a_edit || !w_krsc || !idx || !count || !out || !workspace || (copy_cached && !cached))
        return fail(SIGE_EINVAL, "NULL pointer");
    if ((rc = channel_rows_ok(dtype, g.cin, "c_in")) || (rc = channel_rows_ok(dtype, g.cout, "c_out"))) return rc;
    if (!aligned(a_edit, 16) || !aligned(w_krsc, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
        (copy_cached && !aligned(cached, 16)))
        return fail(SIGE_EALIGN, "tensors and workspace must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(SIGE_EALIGN, "bias must be 4-byte aligned");
    const int es = sige::elem_bytes(dtype);
    const size_t obytes = (size_t)g.n * g.ho * g.wo * g.cout * es;
    const size_t ibytes = (size_t)g.n * g.h * g.w * g.cin * es;
    if (overlap(out, obytes, a_edit, ibytes)) return fail(SIGE_EINVAL, "out overlaps a_edit");
    if (copy_cached && overlap(out, obytes, cached, obytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 1, 1, &cfg, 1))) return rc;
    if ((rc = device_ready())) return rc;
    const long need = sige::split_workspace_bytes(dtype, g, cfg);
    if (need < 0) return fail(SIGE_EINVAL, "unknown tile shape");
    if (workspace_bytes < need)
        return fail(SIGE_ERANGE, "workspace of %lld bytes, %ld needed", (long long)workspace_bytes, need);
    if (overlap(workspace, (size_t)need, out, obytes) || overlap(workspace, (size_t)need, a_edit, ibytes) ||
        overlap(workspace, (size_t)need, idx, (size_t)g.cap * 4) || overlap(workspace, (size_t)need, count, 4) ||
        (copy_cached && overlap(workspace, (size_t)need, cached, obytes)))
        return fail(SIGE_EINVAL, "the workspace overlaps another argument");
    const sige::CopyCfg cc = copy_plan(g, es, copy_cached != 0);
    return finish(sige::launch_conv(dtype, 1, a_edit, w_krsc, bias, idx, count, out, copy_cached ? cached : nullptr,
                                    nullptr, nullptr, g, cfg, cc, (hipStream_t)stream, (float *)workspace),
                  "sige_sparse_conv_layer_split", (hipStream_t)stream);
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
    if (overlap(out, obytes, a_edit, (size_t)g.n * g.h * g.w * g.cin * es))
        return fail(SIGE_EINVAL, "out overlaps a_edit");
    if (overlap(out, obytes, cached, obytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    ConvCfg cfg;
    if ((rc = choose_conv(g, dtype, 1, 1, &cfg))) return rc;  // the full persistent grid: free workgroups restore
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, es, false);
    return finish(sige::launch_conv(dtype, 1, a_edit, w_krsc, bias, idx, count, out, cached, prev_idx, prev_count, g,
                                    cfg, cc, (hipStream_t)stream),
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
    if (overlap(out, tbytes, q, tbytes) || overlap(out, tbytes, k, tbytes) || overlap(out, tbytes, v, tbytes))
        return fail(SIGE_EINVAL, "out overlaps q, k or v");
    if (copy_cached && overlap(out, tbytes, cached, tbytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    if ((rc = device_ready())) return rc;
    const int grid1 = attn_grid1();
    const int64_t need = attn_ws_bytes(g, heads, grid1);
    if (workspace_bytes < need)
        return fail(SIGE_ERANGE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
    if (overlap(out, tbytes, workspace, (size_t)need)) return fail(SIGE_EINVAL, "out overlaps the workspace");
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
    if (overlap(out, obytes, cached, obytes)) return fail(SIGE_EINVAL, "out overlaps cached");
    if ((rc = device_ready())) return rc;
    const sige::CopyCfg cc = copy_plan(g, sige::elem_bytes(dtype), true);
    const DevInfo dv = dev_info();
    const int grid = g.cap < dv.cus ? g.cap : dv.cus;
    return finish(sige::launch_restore(prev_idx, prev_count, idx, count, g, cc, cached, out, grid, (hipStream_t)stream),
                  "sige_restore_blocks", (hipStream_t)stream);
}

}  // extern "C"
