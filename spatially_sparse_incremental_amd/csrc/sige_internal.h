// sige_internal.h -- types and launchers shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sige {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// storage types: 0 = fp32, 1 = bf16, 2 = fp16 (same values as SIGE_F32/BF16/F16)
__host__ __device__ constexpr int elem_bytes(int dt) { return dt == 0 ? 4 : 2; }

// Geometry with everything derived, passed to kernels by value.
struct Geo {
    int n, h, w, cin, cout, k, s, p, b;
    int ho, wo, nby, nbx, ib;
    int cap;  // n * nby * nbx
};

// Multiplier for exact division x / d when x * d < 2^31: x / d = (x * m) >> 31.
__host__ __device__ inline uint32_t fast_div_magic(uint32_t d) {
    return (uint32_t)(((1ull << 31) + d - 1) / d);
}

// Launch parameters of the implicit-GEMM convolution.
struct ConvCfg {
    int mt, nt;          // 16x16 tiles per workgroup along M (rows) and N (output channels)
    int ck;              // input channels staged per chunk
    int a_pix_stride;    // LDS bytes per staged input pixel (ck*es + 16)
    int a_bytes;         // LDS bytes of the staged input windows
    int lds_bytes;       // dynamic LDS per workgroup
    int ns_max;          // most block slots one M tile can touch
    int grid;            // most persistent workgroups worth launching (tiles at capacity; copy: no cap)
    int cus;             // compute units of the device
    uint32_t m_ib2, m_ib;  // fast_div_magic(ib*ib), fast_div_magic(ib)
    uint32_t m_vpc1;       // fast_div_magic(ck*es/16 + 1): 16-byte LDS slots per staged pixel
    uint32_t m_b2, m_b;    // fast_div_magic(b*b), fast_div_magic(b): output rows -> block slot, pixel
    int gate_max;          // the split runs only for lists of at most this many blocks (else it exits at once)
};

// Launch configuration of the fused layer / block convolution (kernels_layer.hip).
constexpr int kLayerWaves = 4;                  // waves per workgroup (they split the K steps)
constexpr int kLayerThreads = 64 * kLayerWaves;
constexpr int kLayerFrags = 18;                 // weight fragments per lane and chunk (SMAX * NT)
struct LayerCfg {
    int mt, nt;          // 16x16 subtiles per tile along M (rows) and N (output channels)
    int ck, nch;         // input channels per chunk (kpc K slices), chunks
    int kpc, lkpc;       // K slices per tap and chunk (a power of 2), its log2
    int steps, spw;      // K steps per chunk (k*k*kpc), steps per wave
    int vpc, ps, rs;     // 16-byte vectors of a staged pixel (ck*es/16); LDS units (16 B) per pixel (vpc + 1)
                         // and per window row (ib*ps + pad, = b mod 16)
    int gps, sb;         // 64-unit groups of one block slot's staged window; LDS bytes per slot (64 gps + 16 units)
    int lds_bytes;       // dynamic LDS per workgroup
    int ntn, xcd;        // N tiles; tile order keeping an M tile's N tiles on one XCD
    int tiles_cap;       // tiles (padding included) at full capacity
    int cus;             // compute units of the device
    int spec;            // workgroups below this fetch their first weights before the list length (set at launch)
    int gate_min;        // runs only for lists of at least this many blocks (else every workgroup exits at once)
    uint32_t m_ps, m_rs, m_b2, m_b;  // fast_div_magic of ps, rs, b*b, b
    // Wide tiles (kLayerWideRows x kLayerWideCols, 16-channel stages) for long lists
    int wide_min, wide_max;  // the wide kernel runs for lists of wide_min..wide_max blocks (min 0x7FFFFFFF: never)
    int w_rs, w_sb;      // LDS units (16 B) per staged window row and per block slot
    int w_rpi;           // window rows per staging load (1 or 2)
    int w_ntn;           // N tiles of kLayerWideCols channels
    int w_wofs;          // LDS byte offset of the staged weights within one of the two buffers
    int w_lds;           // dynamic LDS of the wide kernel (two buffers, or the epilogue's tile)
    int w_tiles_cap;     // wide tiles (padding included) at full capacity
    int gate_wide;       // k_layer: lists of gate_wide..wide_max blocks are the wide kernel's (it exits)
    int w_pmax;          // most K parts a wide tile's stages are split into (1: none); parts > 1 leave
                         // fp32 partial tiles in the workspace for k_wide_combine
    int w_ws_items;      // partial tiles (kLayerWideRows x kLayerWideCols fp32) the workspace holds
};
constexpr int kLayerWideRows = 256;  // output rows (block pixels) of a wide tile
constexpr int kLayerWideCols = 128;  // output channels of a wide tile
constexpr int kLayerWidePitch = kLayerWideCols * 2 + 16;  // LDS bytes per row of the rounded wide tile
constexpr int kLayerWideWinLoads = 16;  // window loads per staging wave and stage of a wide tile, at most
constexpr int kLayerWideMinStages = 4;   // 16-channel stages per K part of a wide tile, at least

// K parts of the wide tiles for a list that makes `ntr` of them (padding not
// counted): as many as give every CU a work item, at most pmax.
__host__ __device__ inline int wide_parts(int cus, int pmax, int ntr) {
    const int p = ntr > 0 ? cus / ntr : 1;
    return p < 1 ? 1 : (p > pmax ? pmax : p);
}

// Copy of the cache outside the listed blocks, in 16-byte vectors of the
// output flattened over (n, y, x, vector of the channel row).
struct CopyCfg {
    long long nvec;      // n * ho * wo * vpp (0: no copy)
    int vpp;             // 16-byte vectors per output pixel
    uint32_t m_vpp;      // fast_div_magic(vpp)
    uint32_t m_b;        // fast_div_magic(b)
    int free_vec;        // vectors a workgroup without a tile takes per tile of a busy one
};

hipError_t launch_diff(int dt, const void *a_orig, const void *a_edit, long npix, int vpp, float tau,
                       uint8_t *mask, uint32_t *bits, hipStream_t st);
// An unconditional copy of nvec 16-byte vectors from src to dst, done by extra
// workgroups of the reduce launch (nvec 0: none).
struct ReduceCopy {
    const uint8_t *src;
    uint8_t *dst;
    long long nvec;
};
// vec16: the mask as bytes (0), bytes read in 16-byte vectors (1), or a bitset
// (2: bit p % 32 of 32-bit word p / 32 for pixel p, wm a multiple of 32)
hipError_t launch_reduce(const uint8_t *mask, int hm, int wm, const Geo &g, int dilate, int vec16, int32_t *idx,
                         int32_t *count, const ReduceCopy &cp, int copy_wgs, hipStream_t st);
// Whether one workgroup can build the list of geometry g from an hm x wm mask
// (vec16 as above): the pooled bits fit in LDS and the fast divisions are exact.
bool reduce_one_launch_ok(int hm, int wm, const Geo &g, int vec16);
// Several layers' lists from one packed mask in one launch, with their cache copies.
constexpr int kReduceMaxLayers = 16;
struct ReduceLayerArgs {
    Geo g;
    int dilate;
    int32_t *idx, *count;
    const uint8_t *src;  // cache to copy (NULL: none for this layer)
    uint8_t *dst;
    long long nvec;      // 16-byte vectors of the copy
};
hipError_t launch_reduce_layers(const uint32_t *bits, int hm, int wm, int n, const ReduceLayerArgs *layers,
                                int copy_wgs, hipStream_t st);
hipError_t launch_gather(const void *a_edit, int dt, const Geo &g, const int32_t *idx, const int32_t *count,
                         void *blocks, hipStream_t st);
// fused = 0: src = stacked blocks, dst = output blocks.  fused = 1: src = a_edit, dst = out;
// with prev_idx (fused only), the previous list's blocks not in idx are restored from cache.
// ws (fused only): the fp32 workspace of the split over input channels (NULL: no split).
hipError_t launch_conv(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                       const int32_t *count, void *dst, const void *cache, const int32_t *prev_idx,
                       const int32_t *prev_count, const Geo &g, const ConvCfg &cfg, const CopyCfg &cc,
                       hipStream_t st, float *ws = nullptr, const void *wp = nullptr);
// The split's fragment-order copy of KRSC weights (wp above) for configuration c:
// 16-byte units of it, and the launch that writes it.
long split_weights_units(int dt, const Geo &g, const ConvCfg &c);
hipError_t launch_split_weights_pack(int dt, const void *w, const Geo &g, const ConvCfg &c, void *wp, int cus,
                                     hipStream_t st);
// The fused layer (fused = 1: src = a_edit, dst = out; with cc.nvec > 0 the
// cache is copied outside the listed blocks, with prev_idx the previous
// list's blocks are restored) or the block convolution (fused = 0: src =
// stacked blocks, dst = output blocks), on kernels_layer.hip's k_layer.
// wp: the weights in k_layer's fragment order (launch_layer_weights_pack), or NULL
// to load them from the KRSC weights w.
hipError_t launch_layer(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                        const int32_t *count, void *dst, const void *cache, const int32_t *prev_idx,
                        const int32_t *prev_count, const Geo &g, const LayerCfg &cfg, const CopyCfg &cc,
                        hipStream_t st, const void *wp = nullptr);
// The fragment-order copy of KRSC weights for k_layer with configuration cfg: 16-byte
// units of it, and the launch that writes it.
long layer_weights_units(const Geo &g, const LayerCfg &cfg);
hipError_t launch_layer_weights_pack(int dt, const void *w, const Geo &g, const LayerCfg &cfg, void *wp, int cus,
                                     hipStream_t st);
// The wide tiles of the fused layer (16-bit types), run for lists of
// cfg.wide_min..cfg.wide_max blocks (the launches exit at once for others).
// With cfg.w_pmax > 1 a short list's tiles are split over K into parts whose
// fp32 partials go to ws (cfg.w_ws_items tiles), and a second launch adds
// them up into dst.
// ww: the weights in the wide tiles' stage-major order (launch_wide_weights_pack), or
// NULL to stage them from the KRSC weights w.
hipError_t launch_layer_wide(int dt, const void *src, const void *w, const float *bias, const int32_t *idx,
                             const int32_t *count, void *dst, const void *cache, const Geo &g, const LayerCfg &cfg,
                             const CopyCfg &cc, hipStream_t st, float *ws, const void *ww);
// The stage-major copy of KRSC weights (16-bit types) for the wide tiles: 16-byte units
// of it, and the launch that writes it.
long wide_weights_units(const Geo &g);
hipError_t launch_wide_weights_pack(const void *w, const Geo &g, void *ww, int cus, hipStream_t st);
// Bytes of that workspace for g and the launch configuration c (< 0: unknown tile shape).
long split_workspace_bytes(int dt, const Geo &g, const ConvCfg &c);
hipError_t launch_restore(const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                          const int32_t *count, const Geo &g, const CopyCfg &cc, const void *cached, void *out,
                          int grid, hipStream_t st);
hipError_t launch_scatter(int dt, const void *out_blocks, const int32_t *idx, const int32_t *count, const Geo &g,
                          const void *cached, void *out, int grid, const CopyCfg &cc, hipStream_t st);

// Query-pruned attention (kernels_attn.hip): head dim 64, at most 8 images.
constexpr int kAttnHeadDim = 64;
constexpr int kAttnImages = 8;
constexpr long kAttnQueryTile = 128;  // queries per work item
constexpr long kAttnWsBytesPerItem = kAttnQueryTile * (64 + 4) * 4;  // partial of one (query tile, head, key split)
int attn_partial_grid(int cus);
hipError_t launch_attention(int dt, const void *q, const void *k, const void *v, const int32_t *idx,
                            const int32_t *count, const Geo &g, int heads, float scale, const void *cached, void *out,
                            const CopyCfg &cc, void *ws, int grid1, int grid2, hipStream_t st);

// reduce limits (LDS of its workgroups)
constexpr int kReduceMaxWidth = 8192;    // conv input width (pooled column bits of one block row)
constexpr int kReduceBitsWords = 8192;   // pooled mask as bits, for the one-launch reduce (32 KiB)
constexpr int kReduceMaxBlocks = 16384;  // n * nby * nbx (flags of all blocks in one workgroup)
// channel rows of at most this many bytes (keeps the fast divisions exact)
constexpr int kMaxRowBytes = 8192;

}  // namespace sige
