/*
 * sige.h -- C ABI of the tile-sparse incremental convolution library (libsige.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are cited per call below):
 *   mer.dev notes, "Efficient Spatially Sparse Inference for Conditional GANs
 *   and Diffusion Models", sections 3, 3.1, 3.2; the SIGE project README
 *   (dongaigc.com mirror), section "Overview"; the nubint.ai review of the same
 *   paper, "Proposed method".  The activations of the original image are
 *   computed once and cached.  For an edited image: (1) diff the original and
 *   edited activations into a change mask; (2) reduce the mask, pooled to each
 *   layer's scale and dilated, to a list of active output blocks; (3) gather
 *   the active blocks' input windows (with halo) from the edited activation,
 *   stacked along a block dimension; (4) run the convolution on the stacked
 *   blocks; (5) scatter the output blocks into (a copy of) the cached output of
 *   the original image.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and never synchronises.
 *   - Activations, caches and outputs are NHWC and contiguous.  Weights are
 *     KRSC: [c_out][k][k][c_in], contiguous.  Bias is fp32 [c_out] or NULL.
 *   - `dtype` is one of SIGE_F32, SIGE_BF16, SIGE_F16.  Convolutions multiply
 *     in the storage type on the matrix cores, accumulate in fp32 and round
 *     once (to nearest, ties to even) into the storage type.
 *   - Tensors read or written in 16-byte vectors must be 16-byte aligned and
 *     their channel rows a multiple of 16 bytes (c % 8 == 0 for 16-bit types,
 *     c % 4 == 0 for fp32); otherwise SIGE_EALIGN.  Channel rows are at most
 *     8192 bytes (c <= 4096 for 16-bit types, 2048 for fp32); else SIGE_ERANGE.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it; results are ready when the stream reaches them.
 *   - The number of active blocks stays on the device: `count` points to one
 *     int32 in device memory written by sige_reduce_mask and read by the later
 *     steps, so no step waits for the host.  Lists (idx) and block buffers
 *     hold sige_max_blocks() entries: a kernel may read idx entries past
 *     *count (a tile's block indices are fetched before the count arrives)
 *     and ignores their values; only slots [0, *count) are written or used.
 *   - Every call returns SIGE_OK (0) or a negative code.  Arguments are checked
 *     on the host before anything is enqueued; a rejected call enqueues
 *     nothing.  sige_strerror() names a code; sige_last_error() returns the
 *     calling thread's last message.  Device faults surface at the caller's
 *     next synchronisation (or inside the call when the environment variable
 *     SIGE_DEBUG_SYNC=1 is set, which synchronises after every launch).
 */
#ifndef SIGE_H
#define SIGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SIGE_OK 0
#define SIGE_EINVAL (-1)  /* null pointer, bad shape/geometry, aliasing, unsupported parameter */
#define SIGE_EDTYPE (-2)  /* dtype is not SIGE_F32 / SIGE_BF16 / SIGE_F16 */
#define SIGE_EALIGN (-3)  /* pointer or channel row not 16-byte aligned */
#define SIGE_EHIP (-4)    /* the HIP runtime reported an error (message in sige_last_error) */
#define SIGE_ENODEV (-5)  /* no usable GPU */
#define SIGE_ERANGE (-6)  /* a size exceeds a documented limit of a kernel */

enum { SIGE_F32 = 0, SIGE_BF16 = 1, SIGE_F16 = 2 };

/* Geometry of one convolution and its block grid.
 *   input  [n, h, w, c_in];  k x k kernel, stride, zero padding pad;
 *   output [n, ho, wo, c_out] with ho = (h + 2*pad - k)/stride + 1 (wo alike);
 *   output blocks of block x block pixels: nby = ceil(ho/block), nbx = ceil(wo/block)
 *   (the last row/column of blocks may be partial);
 *   input window of block (by, bx): rows [by*block*stride - pad, ... + ib),
 *   columns alike, ib = (block-1)*stride + k (neighbouring windows of a 3x3
 *   stride-1 conv overlap by 2, SIGE README, "Overview").
 * Supported: n, h, w, c_in, c_out >= 1; 1 <= k <= 7; 1 <= stride <= 4;
 * 0 <= pad < k; 1 <= block <= 64; ib <= 64; h + 2*pad >= k (w alike). */
typedef struct {
    int32_t n, h, w;
    int32_t c_in, c_out;
    int32_t k, stride, pad;
    int32_t block;
} sige_geom;

typedef struct {
    int32_t ho, wo;   /* output size */
    int32_t nby, nbx; /* block grid per image */
    int32_t ib;       /* input window edge */
    int64_t cap;      /* n * nby * nbx: capacity of idx and of block buffers */
} sige_derived;

/* Validate a geometry and fill its derived sizes.  Host only; no GPU needed. */
int sige_geom_derive(const sige_geom *g, sige_derived *out);

/* Capacity n*nby*nbx of a geometry, or a negative code. Host only. */
int64_t sige_max_blocks(const sige_geom *g);

/* Step 1 -- change mask (mer.dev notes, section 3; SIGE README, "Overview").
 *   mask[p] = 1 if some channel of pixel p has |float(a_edit) - float(a_orig)| > thresh,
 *   the difference taken in IEEE fp32; else 0.  p runs over the n*h*w pixels.
 *   a_orig, a_edit: [n, h, w, c] in `dtype`, 16-byte aligned.
 *   mask: uint8 [n, h, w], 4-byte aligned; written completely.
 *   thresh: finite, >= 0.  NaN differences do not flag a pixel. */
int sige_diff_mask(const void *a_orig, const void *a_edit, int dtype, int n, int h, int w, int c, float thresh,
                   uint8_t *mask, void *stream);

/* Step 1 with the mask also (or only) packed one bit per pixel: the same change
 * mask as sige_diff_mask, written to `bits` as bit p % 32 of 32-bit word p / 32
 * for pixel p (p = (n*h + y)*w + x).  The packed form is what
 * sige_reduce_bits reads: one eighth of the mask bytes through the single
 * workgroup that pools it.
 *   w must be a multiple of 32 (whole words per row), else SIGE_EINVAL.
 *   bits: uint32 [n*h*w/32], 4-byte aligned; written completely.
 *   mask: as sige_diff_mask, or NULL to write the bits only (not both NULL).
 *   Other arguments as sige_diff_mask. */
int sige_diff_mask_bits(const void *a_orig, const void *a_edit, int dtype, int n, int h, int w, int c, float thresh,
                        uint8_t *mask, uint32_t *bits, void *stream);

/* Step 2 -- active block list (mer.dev notes, 3.2: downsample the mask to each
 * scale and dilate it; SIGE README, "Overview": reduce it to active block indices).
 *   mask: uint8 [g->n, mask_h, mask_w], nonzero = changed.  mask_h = fy * g->h and
 *     mask_w = fx * g->w for integers fy, fx >= 1; the mask is OR-pooled by (fy, fx).
 *   A block is active when a changed pooled pixel lies in its input window
 *     (clipped to the image); the block grid is then dilated by `dilate_blocks`
 *     (square element, clipped at the grid edge).  0 <= dilate_blocks <= 16.
 *   idx: int32 [cap] -- receives the linear indices (n*nby + by)*nbx + bx of the
 *     active blocks in ascending order; entries at and after *count are not written.
 *   count: one int32 in device memory; receives the number of active blocks.
 *   The idx buffer doubles as scratch: a first launch writes one activity byte per
 *     block into it, a second launch reads them all before writing the list.
 *   Limits (else SIGE_ERANGE): g->w <= 8192, n*nby*nbx <= 16384.
 *   c_in/c_out of g are not used. */
int sige_reduce_mask(const uint8_t *mask, int mask_h, int mask_w, const sige_geom *g, int dilate_blocks,
                     int32_t *idx, int32_t *count, void *stream);

/* Step 2 with the cache copy of step 5 in the same launch: sige_reduce_mask,
 * while the other workgroups copy `cached` into `out` (all of it:
 * out = cached).  sige_sparse_conv_layer(..., copy_cached = 0) or
 * sige_scatter(..., copy_cached = 0) on that `out` then gives the
 * copy_cached = 1 result; the copy runs beside the single-workgroup reduce
 * instead of on the convolution's critical path.
 *   cached, out: [n, ho, wo, c_out] in `dtype` for the conv geometry g; out
 *   must not overlap cached, mask, idx or count.  Other arguments and limits
 *   as sige_reduce_mask. */
int sige_reduce_mask_copy(const uint8_t *mask, int mask_h, int mask_w, const sige_geom *g, int dilate_blocks,
                          int32_t *idx, int32_t *count, int dtype, const void *cached, void *out, void *stream);

/* sige_reduce_mask and sige_reduce_mask_copy with the mask packed one bit per
 * pixel, as sige_diff_mask_bits writes it: bit p % 32 of word p / 32 for pixel
 * p = (n*mask_h + y)*mask_w + x.  Same results (bit for bit) as the byte-mask
 * calls on the unpacked mask.
 *   bits: uint32 [g->n*mask_h*mask_w/32], 4-byte aligned (else SIGE_EALIGN);
 *   mask_w a multiple of 32 (else SIGE_EINVAL).  Other arguments and limits as
 *   the byte-mask calls. */
int sige_reduce_bits(const uint32_t *bits, int mask_h, int mask_w, const sige_geom *g, int dilate_blocks,
                     int32_t *idx, int32_t *count, void *stream);
int sige_reduce_bits_copy(const uint32_t *bits, int mask_h, int mask_w, const sige_geom *g, int dilate_blocks,
                          int32_t *idx, int32_t *count, int dtype, const void *cached, void *out, void *stream);

/* Step 2 for the layers of a network at one edit, in one launch (mer.dev notes,
 * 3.2: the one change mask downsampled to every layer's scale).  Layer l's list
 * is what sige_reduce_bits(bits, mask_h, mask_w, &geoms[l], dilate_blocks[l],
 * idx[l], count[l]) writes (bit for bit); one workgroup builds each list, and
 * the launch's other workgroups meanwhile copy cached[l] into out[l] (all of
 * it) for every layer that has a copy, as sige_reduce_bits_copy does.  All
 * lists depend on the mask only, so they can be built before any layer runs;
 * each layer then calls sige_sparse_conv_layer(..., copy_cached = 0) (or its
 * split) on out[l] with idx[l] and count[l].
 *   geoms, dilate_blocks, idx, count: host arrays of nlayers entries (idx[l],
 *     count[l] device pointers as in sige_reduce_bits); 1 <= nlayers <= 16.
 *     Every layer has the same n.
 *   cached, out: host arrays of nlayers device pointers ([n, ho, wo, c_out] of
 *     layer l in `dtype`), or NULL for no copies; cached[l] and out[l] both
 *     NULL skips layer l's copy.  dtype is checked only when some layer copies.
 *   Nothing a layer writes (idx, count, out) may overlap what any layer writes
 *   or reads (bits, cached).
 *   Limits: every layer's pooled mask and block grid must fit one workgroup
 *   (conv input h * ceil(w/32) <= 8192 words, n*nby*nbx <= 16384), else
 *   SIGE_ERANGE; other checks as sige_reduce_bits_copy. */
int sige_reduce_bits_layers(const uint32_t *bits, int mask_h, int mask_w, int nlayers, const sige_geom *geoms,
                            const int *dilate_blocks, int32_t *const *idx, int32_t *const *count, int dtype,
                            const void *const *cached, void *const *out, void *stream);

/* Step 3 -- gather (SIGE README, "Overview": collect the active blocks from the
 * edited activation and stack them along the batch dimension).
 *   blocks[slot, yy, xx, c] = a_edit[n, by*block*stride - pad + yy, bx*block*stride - pad + xx, c]
 *   (zero outside the image) for slot < *count, where idx[slot] = (n*nby + by)*nbx + bx.
 *   a_edit: [n, h, w, c_in];  blocks: [cap, ib, ib, c_in];  both in `dtype`. */
int sige_gather(const void *a_edit, int dtype, const sige_geom *g, const int32_t *idx, const int32_t *count,
                void *blocks, void *stream);

/* Step 4 -- convolution of the stacked blocks (SIGE README, "Overview": feed
 * the stacked blocks to F_l).  A valid k x k conv with the layer's stride on
 * each block, as an implicit GEMM on the matrix cores:
 *   out_blocks[slot, py, px, co] = bias[co] + sum_{ky,kx,ci} w[co,ky,kx,ci] * blocks[slot, py*stride+ky, px*stride+kx, ci]
 *   for slot < *count.  blocks: [cap, ib, ib, c_in]; w_krsc: [c_out, k, k, c_in];
 *   out_blocks: [cap, block, block, c_out]; bias: fp32 [c_out] or NULL. */
int sige_conv_blocks(const void *blocks, const void *w_krsc, const float *bias, int dtype, const sige_geom *g,
                     const int32_t *count, void *out_blocks, void *stream);

/* Step 5 -- scatter (SIGE README, "Overview": scatter the output blocks back
 * into the cached output of the original image).
 *   copy_cached = 1: out = cached outside the listed blocks (a copy), and the
 *     valid pixels of each listed block come from out_blocks.  `out` must not
 *     overlap `cached`.  idx must be ascending (as sige_reduce_mask writes it).
 *   copy_cached = 0: only the listed blocks' pixels of `out` are written; the
 *     caller keeps `out` equal to the cache elsewhere (a persistent buffer).
 *   Pixels of partial edge blocks beyond (ho, wo) are dropped.
 *   out_blocks: [cap, block, block, c_out]; cached, out: [n, ho, wo, c_out]. */
int sige_scatter(const void *out_blocks, const int32_t *idx, const int32_t *count, const sige_geom *g, int dtype,
                 const void *cached, void *out, int copy_cached, void *stream);

/* Steps 3-5 fused into one kernel: the input windows of the listed blocks are
 * staged from a_edit into LDS, convolved on the matrix cores and written
 * straight into `out`; with copy_cached = 1 the same launch copies `cached`
 * into `out` outside the listed blocks.  Result as sige_gather ->
 * sige_conv_blocks -> sige_scatter, without the intermediate block tensors.
 *   a_edit: [n, h, w, c_in]; w_krsc: [c_out, k, k, c_in]; bias fp32 [c_out] or NULL;
 *   cached, out: [n, ho, wo, c_out]; idx ascending, count in device memory.
 *   `out` must overlap neither `a_edit` nor (when copy_cached = 1) `cached`. */
int sige_sparse_conv_layer(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                           const int32_t *idx, const int32_t *count, int dtype, const sige_geom *g, void *out,
                           int copy_cached, void *stream);

/* The fused layer split over input channels, for weight-bound layers (many
 * input channels: the low-resolution latent-diffusion levels, where the
 * mer.dev notes, 5 "Conclusion & Discussion", find tiles least effective, and
 * the GauGAN-sized convolutions).  Same arguments and result as
 * sige_sparse_conv_layer up to the fp32 summation order, in two launches: a
 * work item (group of output-row tiles, one chunk of input channels, one tile
 * of output channels) reads its weights once and walks its row tiles, leaving
 * one fp32 partial tile per (row tile, channel tile, chunk) in `workspace`;
 * the second kernel adds a tile's chunks in chunk order with the bias, writes
 * the listed blocks and, with copy_cached, copies the cache elsewhere.  The
 * row groups are chosen on the device from *count, as many as fill the GPU's
 * resident slots.
 *   workspace: caller-owned device memory of at least
 *   sige_sparse_conv_layer_split_workspace() bytes (a partial tile per row
 *   tile, channel tile and chunk at full capacity), 16-byte aligned, needing
 *   no initialisation; its contents afterwards are meaningless.  Calls that
 *   share a workspace must not overlap in time. */
int64_t sige_sparse_conv_layer_split_workspace(const sige_geom *g, int dtype);
int sige_sparse_conv_layer_split(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                 const int32_t *idx, const int32_t *count, int dtype, const sige_geom *g, void *out,
                                 int copy_cached, void *workspace, int64_t workspace_bytes, void *stream);

/* The fused layer with the kernel chosen by the library: the single-range
 * kernel of sige_sparse_conv_layer (64 x 32 tiles), the split of
 * sige_sparse_conv_layer_split, or wide tiles of 256 rows x 128 output
 * channels (16-bit types, k <= 3; no entry point of their own), whichever a
 * cost model fixed in the library prices fastest for the list length *count.
 * The mer.dev notes (5 "Conclusion & Discussion") name small blocks at low
 * resolution as the method's weak spot: there the K range is long and the
 * blocks few, and the split is the faster kernel; long lists of large edits
 * (nubint.ai review, "ABSTRACT") go to the wide tiles, which stage each
 * window once for 128 output channels.  The list length is read on the
 * device, so the host derives thresholds per layer: lists of at most
 * sige_layer_plan.split_max blocks go to the split, lists of wide_min ..
 * wide_max blocks to the wide tiles, the rest to the single-range kernel.
 * Every kernel whose range can occur is enqueued and the ones not chosen exit
 * as soon as they have read *count (about three microseconds on MI355X for
 * the single-range kernel and the split, 1.4 for the wide tiles); no host
 * timing, no synchronisation, nothing allocated.  The first call for a
 * geometry, dtype and device prices every list length up to the capacity
 * (host work proportional to sige_max_blocks); later calls reuse the plan
 * (SIGE_WIDE_MIN, read when a plan is made, sends lists of at least that many
 * blocks to the wide tiles where they can run: a tuning knob).
 *   Same arguments, checks and result as sige_sparse_conv_layer (up to the
 *   fp32 summation order of the kernel that runs), plus a workspace for the
 *   split's partial tiles and for the wide tiles' K parts (lists too short
 *   to give every compute unit a wide tile split their 16-channel stages
 *   into up to wide_parts_max parts, whose fp32 partials a second launch
 *   adds up): at least sige_layer_plan.workspace_bytes of caller-owned
 *   device memory (16-byte aligned, no initialisation, contents afterwards
 *   meaningless, not shared by calls that overlap in time); NULL and 0 when
 *   workspace_bytes is 0 (neither is ever chosen).  SIGE_ERANGE when the
 *   workspace is smaller.
 * sige_sparse_conv_layer_plan reports the choice for a geometry: split_max
 * (-1: never the split; >= cap: always), wide_min and wide_max (the wide
 * tiles for lists of that many blocks; 0x7FFFFFFF: never, or no upper bound),
 * the workspace size, and the cost
 * model's inputs (the single-range kernel's K chunks per tile, K steps per
 * chunk, 1 KiB staging groups per tile and chunk, resident workgroup slots,
 * tiles of 32 output channels; the split's chunks, resident workgroup slots
 * and KiB of staged windows per tile (0 when the split cannot run); the
 * layer's weight megabytes and GFLOP per listed block; the wide tiles' K
 * stages of 16 channels, staging loads per stage and tiles of 128 output
 * channels (0 when they cannot run), and the most K parts a wide tile is
 * split into (1: none)). */
typedef struct {
    int32_t split_max;        /* the split takes lists of at most this many blocks (-1: none) */
    int32_t cap;              /* blocks at full capacity (sige_max_blocks) */
    int64_t workspace_bytes;  /* workspace sige_sparse_conv_layer_auto needs (0: none) */
    int32_t chunks, steps, stage_groups, slots, n_tiles;
    int32_t split_chunks, split_slots;
    double split_stage_kb, weight_mb, gflop_per_block;
    int32_t wide_min;         /* the wide tiles take lists of wide_min..wide_max blocks (wide_min > cap: none) */
    int32_t wide_stages, wide_loads, wide_n_tiles;
    int32_t wide_max;
    int32_t wide_parts_max;   /* most K parts of a wide tile (1: never split; 0: no wide tiles) */
} sige_layer_plan;
int sige_sparse_conv_layer_plan(const sige_geom *g, int dtype, sige_layer_plan *out);
int sige_sparse_conv_layer_auto(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                const int32_t *idx, const int32_t *count, int dtype, const sige_geom *g, void *out,
                                int copy_cached, void *workspace, int64_t workspace_bytes, void *stream);

/* A layer's weights packed once in the order the layer kernels load them.
 * From KRSC weights a 1 KiB load of the single-range kernel gathers 32 bytes
 * of each of 32 output channels (two lanes per channel: a K slice's weight
 * fragment of the 32x32 MFMA), and a staging load of the wide tiles
 * (nubint.ai review, "ABSTRACT": large edits) 32 bytes of each of 32 output
 * channels of a 16-channel stage; from the packed copy every such load reads
 * 1 KiB in a row.  Measured on MI355X: the 1.2% single-range layer of the
 * 256x256x128 U-Net conv about 9% faster, the wide tiles 6-10%, the split
 * about 4%.
 * The copy has two sections, both in the library's own load order for the
 * geometry and dtype (they follow the kernel configuration the library picks,
 * so a copy is valid for that geometry, dtype and library build only):
 *   - the single-range kernel's: for chunk ch of the K range, N tile tn of
 *     the layer's output-channel tiles, K step s of the chunk (tap, K slice),
 *     N subtile q and lane l, the 16 bytes that lane loads from w_krsc
 *     (output channels past c_out and input channels past c_in clamped as the
 *     kernel clamps them), at unit (((ch * tiles + tn) * steps + s) *
 *     subtiles + q) * 64 + l;
 *   - from the next 256-byte boundary, for 16-bit types where the wide tiles
 *     can run (k <= 3, the stage buffers within the LDS): for N tile tn of
 *     128 output channels, stage s of 16 input channels, tap t = ky * k + kx,
 *     column n < 128 and half h < 2, the 8 values W[128 tn + n][ky][kx][16 s
 *     + 8 h .. + 7] at unit ((tn * ceil(c_in / 16) + s) * k * k + t) * 256 +
 *     2 n + (h XOR ((n / 8) mod 2)), zeros past c_out and c_in;
 *   - from the next 256-byte boundary, where the split over input channels
 *     can run: its fragments, as the first section's but in the split's own
 *     chunks and N tiles (16 lanes per output channel of a 16x16 MFMA
 *     fragment).
 *   sige_packed_weights_bytes: the size of the copy (a negative status code
 *   for invalid arguments).
 *   sige_pack_weights: writes it from w_krsc (the KRSC weights of
 *   sige_sparse_conv_layer) into w_packed, caller-owned device memory of
 *   w_packed_bytes >= sige_packed_weights_bytes, 256-byte aligned, not
 *   overlapping w_krsc; enqueued on `stream`, nothing synchronised or
 *   allocated.  SIGE_ERANGE when w_packed_bytes is too small, SIGE_EINVAL /
 *   SIGE_EALIGN for NULL, overlapping or misaligned pointers. */
int64_t sige_packed_weights_bytes(const sige_geom *g, int dtype);
int sige_pack_weights(const void *w_krsc, int dtype, const sige_geom *g, void *w_packed, int64_t w_packed_bytes,
                      void *stream);

/* sige_conv_blocks, sige_sparse_conv_layer and sige_sparse_conv_layer_auto
 * with the single-range kernel (the block convolution's too), the wide tiles
 * and (auto) the split loading their weights from w_packed
 * (sige_pack_weights of the same w_krsc) instead of w_krsc.  Same arguments, checks and result as the unpacked calls, bit
 * for bit (the same values reach the same registers and LDS slots in the same
 * order).  w_packed: non-NULL (SIGE_EINVAL), 256-byte aligned (SIGE_EALIGN),
 * w_packed_bytes at least sige_packed_weights_bytes (SIGE_ERANGE), not
 * overlapping out, out_blocks or the workspace (SIGE_EINVAL). */
int sige_conv_blocks_packed(const void *blocks, const void *w_krsc, const float *bias, int dtype, const sige_geom *g,
                            const int32_t *count, void *out_blocks, const void *w_packed, int64_t w_packed_bytes,
                            void *stream);
int sige_sparse_conv_layer_packed(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                  const int32_t *idx, const int32_t *count, int dtype, const sige_geom *g, void *out,
                                  int copy_cached, const void *w_packed, int64_t w_packed_bytes, void *stream);
int sige_sparse_conv_layer_auto_packed(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                       const int32_t *idx, const int32_t *count, int dtype, const sige_geom *g,
                                       void *out, int copy_cached, void *workspace, int64_t workspace_bytes,
                                       const void *w_packed, int64_t w_packed_bytes, void *stream);

/* sige_sparse_conv_layer_split without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The partial tiles go to a static
 * device array of the library, sige_noalloc_scratch_bytes() = 64 MiB per GPU,
 * held until the process ends; the call itself allocates nothing.  Same
 * arguments (minus the workspace), checks and result as
 * sige_sparse_conv_layer_split, whose kernels it runs.
 *   SIGE_ERANGE when the layer's split needs more scratch than that
 *   (sige_sparse_conv_layer_split_workspace(g, dtype) > 64 MiB); nothing is
 *   enqueued then.
 *   Every call on one GPU shares that GPU's array: calls whose executions
 *   overlap on one GPU (two streams, two threads) race on it and give wrong
 *   results; calls ordered on one stream are safe.  Nothing in it needs to
 *   start at zero. */
int64_t sige_noalloc_scratch_bytes(void);
int sige_sparse_conv_layer_split_noalloc(const void *a_edit, const void *w_krsc, const float *bias,
                                         const void *cached, const int32_t *idx, const int32_t *count, int dtype,
                                         const sige_geom *g, void *out, int copy_cached, void *stream);

/* Sequential edits (nubint.ai review, "ABSTRACT": results with sequential
 * edits; "Proposed method": the engine keeps its state between edits).  `out`
 * is a persistent buffer that holds the previous edit's result: `cached`
 * outside the blocks of prev_idx[0, *prev_count) and recomputed values inside
 * them.  Every valid pixel of a block that prev_idx lists and idx[0, *count)
 * does not gets its cached value back (a copy); blocks of both lists are left
 * alone.  Then sige_sparse_conv_layer(..., copy_cached = 0) (or sige_scatter
 * with copy_cached = 0) with idx on the same `out` gives the copy_cached = 1
 * result without copying the whole tensor.  idx and count may both be NULL
 * (restore every previous block).  Both lists ascending, as sige_reduce_mask
 * writes them; entries outside [0, cap) are skipped.
 *   cached, out: [n, ho, wo, c_out] in `dtype`, not overlapping.  c_in, k,
 *   stride and pad of g only fix ho and wo. */
int sige_restore_blocks(const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                        const int32_t *count, const sige_geom *g, int dtype, const void *cached, void *out,
                        void *stream);

/* Sequential edits in one launch: sige_restore_blocks(prev_idx, prev_count,
 * idx, count, ...) followed by sige_sparse_conv_layer(..., copy_cached = 0) on
 * the persistent buffer `out`, with the restore done by the workgroups that
 * have no tile of the convolution.  Same arguments and conventions as those two
 * calls; every pointer except bias is required. */
int sige_sparse_conv_layer_restore(const void *a_edit, const void *w_krsc, const float *bias, const void *cached,
                                   const int32_t *prev_idx, const int32_t *prev_count, const int32_t *idx,
                                   const int32_t *count, int dtype, const sige_geom *g, void *out, void *stream);

/* Query-pruned self-attention (nubint.ai review, "Proposed method": attention
 * layers are handled by pruning the queries of unedited tokens, so that the
 * attention work scales with the edited area).
 *   Tokens are the pixels of an h x w grid in row-major order; q, k, v, cached
 *   and out are [n, h*w, heads*head_dim] in dtype (SIGE_F16 or SIGE_BF16), head
 *   hd owning channels [hd*head_dim, (hd+1)*head_dim).  idx[0, *count) lists
 *   blocks of block x block tokens, ascending (as sige_reduce_mask writes it
 *   for the k = 1, stride 1, pad 0 geometry of the token grid).  For every token
 *   t of a listed block (clipped at the grid edge) and every head:
 *     out[t] = sum_j softmax_j(scale * q[t] . k[j]) v[j], j over the tokens of t's image,
 *   with fp32 products and softmax on the matrix cores, the probabilities
 *   rounded to dtype for the second product.
 *   copy_cached = 1: out = cached for every other token (a copy; out must not
 *   overlap cached); 0: those tokens of out are left alone.
 *   workspace: caller-owned device scratch of at least
 *   sige_sparse_attention_workspace() bytes, 16-byte aligned, needing no
 *   initialisation; its contents afterwards are meaningless.
 *   Limits: head_dim 64, n <= 8 (else SIGE_ERANGE).  Two kernel launches. */
int64_t sige_sparse_attention_workspace(int n, int h, int w, int heads, int head_dim, int block);
int sige_sparse_attention(const void *q, const void *k, const void *v, const int32_t *idx, const int32_t *count,
                          int dtype, int n, int h, int w, int heads, int head_dim, int block, float scale,
                          const void *cached, void *out, int copy_cached, void *workspace, int64_t workspace_bytes,
                          void *stream);

/* Name of a status code (static string). */
const char *sige_strerror(int code);

/* Message of the calling thread's most recent call: "" when it succeeded. */
const char *sige_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SIGE_H */
