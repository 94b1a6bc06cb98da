/*
 * sige_oracle.c -- plain CPU oracle for tile-sparse incremental convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle.so and is
 * loaded by the tests, by the smoke check and by the bench's CPU-baseline leg.
 * Nothing in the GPU library includes, links or calls it, and it uses nothing
 * from there: its geometry, its number formats and its convolution are written
 * out here from the pages alone.
 *
 * Sources (page title, section):
 *  [NOTES]  mer.dev reading notes, "Efficient Spatially Sparse Inference for
 *           Conditional GANs and Diffusion Models": section 3 (Method: cache the
 *           original activations, diff the edited image against the original,
 *           recompute only edited regions), 3.1 (Activation Sparsity: by
 *           linearity the edited output is the original output plus the conv of
 *           the activation difference), 3.2 (Sparse Engine SIGE: tile-based
 *           sparsity; downsample the diff mask to several scales, dilate it, use
 *           it to select tiles).
 *  [README] dongaigc.com mirror of the SIGE project README, section "Overview":
 *           compute the difference mask, reduce it to active block indices,
 *           gather active blocks from the edited activation (blocks of a 3x3
 *           stride-1 conv overlap by width 2), stack them along the batch
 *           dimension, run F_l, scatter the output blocks back into the cached
 *           F_l(A_original).
 *  [REVIEW] nubint.ai review of the same paper, "Proposed method": gather-scatter
 *           sparse update that reuses cached activations.
 *
 * Readings the pages leave open (each one is listed with its reason in the
 * design notes):
 *  - the diff flags a pixel when any channel differs by more than tau; the
 *    difference is taken in IEEE fp32 (the kernel's precision), strictly > tau;
 *  - a mask at a finer resolution is OR-pooled by the integer ratio;
 *  - a block is active when any flagged pixel falls in its input window (the
 *    gathered block, halo included), then the block grid is dilated by
 *    `dilate` blocks with a square element, clipped at the grid edge;
 *  - block list: ascending linear index (n*nby + by)*nbx + bx;
 *  - convolution: fp64 accumulation from the exactly-widened stored values,
 *    bias added, one round-to-nearest-even into the storage format.
 *
 * Everything is a straight loop over output pixels; no blocking, no reordering
 * beyond what the definitions state.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_F64 = 3 };

static int elem_size(int dt) {
    switch (dt) {
    case OR_F32: return 4;
    case OR_BF16: return 2;
    case OR_F16: return 2;
    case OR_F64: return 8;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* number formats (IEEE 754 binary16, bfloat16 = top half of binary32)        */
/* ------------------------------------------------------------------------ */
static double half_bits_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round x to the nearest number with `frac` fraction bits, minimum normal
 * exponent `emin` and maximum exponent `emax`; ties go to the even neighbour;
 * results beyond the largest finite value become infinity. */
static double quantize(double x, int frac, int emin, int emax) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e = ilogb(x);
    if (e < emin) e = emin; /* subnormals share the quantum of the smallest binade */
    double q = ldexp(1.0, e - frac);
    double r = nearbyint(x / q) * q; /* default rounding mode: nearest, ties to even */
    double maxfin = ldexp(2.0 - ldexp(1.0, -frac), emax);
    if (fabs(r) > maxfin) return copysign(INFINITY, x);
    return r;
}

double oracle_round(double x, int dt) {
    switch (dt) {
    case OR_F32: return quantize(x, 23, -126, 127);
    case OR_BF16: return quantize(x, 7, -126, 127);
    case OR_F16: return quantize(x, 10, -14, 15);
    default: return x;
    }
}

static uint16_t double_to_half_bits(double x) {
    if (isnan(x)) return 0x7E00;
    double r = quantize(x, 10, -14, 15);
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < -14) return sign | (uint16_t)(a * ldexp(1.0, 24)); /* subnormal */
    uint16_t m = (uint16_t)(a * ldexp(1.0, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | m;
}

static uint16_t double_to_bf16_bits(double x) {
    if (isnan(x)) return 0x7FC0;
    float f = (float)quantize(x, 7, -126, 127); /* exact: the value fits binary32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double load_elem(const void *base, long i, int dt) {
    switch (dt) {
    case OR_F32: return (double)((const float *)base)[i];
    case OR_BF16: return bf16_bits_to_double(((const uint16_t *)base)[i]);
    case OR_F16: return half_bits_to_double(((const uint16_t *)base)[i]);
    case OR_F64: return ((const double *)base)[i];
    }
    return NAN;
}

static void store_elem(void *base, long i, int dt, double v) {
    switch (dt) {
    case OR_F32: ((float *)base)[i] = (float)quantize(v, 23, -126, 127); break;
    case OR_BF16: ((uint16_t *)base)[i] = double_to_bf16_bits(v); break;
    case OR_F16: ((uint16_t *)base)[i] = double_to_half_bits(v); break;
    case OR_F64: ((double *)base)[i] = v; break;
    }
}

/* Encode doubles into a storage format (used by tests to pin the rounding). */
void oracle_encode(const double *x, long n, int dt, void *out) {
    for (long i = 0; i < n; i++) store_elem(out, i, dt, x[i]);
}

void oracle_decode(const void *x, long n, int dt, double *out) {
    for (long i = 0; i < n; i++) out[i] = load_elem(x, i, dt);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

/* ------------------------------------------------------------------------ */
/* geometry                                                                   */
/* ------------------------------------------------------------------------ */
/* Output size of a k x k conv with stride s and zero padding p; block grid of
 * b x b output blocks (the last row/column of blocks may be partial); input
 * window of one block = ib x ib with ib = (b-1)*s + k, so neighbouring windows
 * of a 3x3 stride-1 conv overlap by k - 1 = 2 ([README] Overview).
 * out[0..4] = ho, wo, nby, nbx, ib. */
int oracle_geometry(int h, int w, int k, int s, int p, int b, int *out) {
    if (h <= 0 || w <= 0 || k <= 0 || s <= 0 || p < 0 || b <= 0) return -1;
    if (h + 2 * p < k || w + 2 * p < k) return -1;
    int ho = (h + 2 * p - k) / s + 1;
    int wo = (w + 2 * p - k) / s + 1;
    out[0] = ho;
    out[1] = wo;
    out[2] = (ho + b - 1) / b;
    out[3] = (wo + b - 1) / b;
    out[4] = (b - 1) * s + k;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* step 1: difference mask ([NOTES] 3; [README] Overview)                     */
/* ------------------------------------------------------------------------ */
/* mask[n,y,x] = 1 iff some channel c has |A_e - A_o| > tau, the difference
 * taken in fp32.  Element (n,c,y,x) of either tensor sits at
 * n*sn + c*sc + y*sh + x*sw (strides in elements), so NCHW and NHWC both work. */
int oracle_diff_mask(const void *a_orig, const void *a_edit, int dt, int n, int h, int w, int c,
                     long sn, long sh, long sw, long sc, float tau, uint8_t *mask) {
    if (dt != OR_F32 && dt != OR_BF16 && dt != OR_F16) return -1;
    long npix = (long)n * h * w;
#pragma omp parallel for schedule(static)
    for (long q = 0; q < npix; q++) {
        long nn = q / ((long)h * w), y = (q / w) % h, x = q % w;
        uint8_t flag = 0;
        for (int ch = 0; ch < c; ch++) {
            long off = nn * sn + ch * sc + y * sh + x * sw;
            float fo = (float)load_elem(a_orig, off, dt); /* exact widening */
            float fe = (float)load_elem(a_edit, off, dt);
            float d = fe - fo; /* IEEE fp32, round to nearest even */
            if (fabsf(d) > tau) flag = 1;
        }
        mask[q] = flag;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* step 2: multi-scale reduce to active blocks ([NOTES] 3.2; [README] Overview) */
/* ------------------------------------------------------------------------ */
/* mask: [n, hm, wm] at a resolution that is an integer multiple (fy, fx) of the
 * conv input (h, w).  Pooled mask m_f[y,x] = OR of the fy x fx cell.
 * a0[n,i,j] = OR of m_f over the block's input window, rows
 * [i*b*s - p, i*b*s - p + ib) and columns likewise, clipped to the image.
 * active = a0 dilated by `dilate` blocks (square element, in-grid neighbours). */
int oracle_block_activity(const uint8_t *mask, int n, int hm, int wm, int h, int w, int k, int s, int p,
                          int b, int dilate, uint8_t *active) {
    int g[5];
    if (oracle_geometry(h, w, k, s, p, b, g)) return -1;
    if (hm % h || wm % w || dilate < 0) return -1;
    int fy = hm / h, fx = wm / w, nby = g[2], nbx = g[3], ib = g[4];
    long nblk = (long)n * nby * nbx;
    uint8_t *a0 = (uint8_t *)calloc(nblk ? nblk : 1, 1);
    if (!a0) return -2;
    for (int nn = 0; nn < n; nn++)
        for (int i = 0; i < nby; i++)
            for (int j = 0; j < nbx; j++) {
                int hit = 0;
                for (int yy = i * b * s - p; yy < i * b * s - p + ib && !hit; yy++) {
                    if (yy < 0 || yy >= h) continue;
                    for (int xx = j * b * s - p; xx < j * b * s - p + ib && !hit; xx++) {
                        if (xx < 0 || xx >= w) continue;
                        for (int dy = 0; dy < fy && !hit; dy++)
                            for (int dx = 0; dx < fx && !hit; dx++)
                                if (mask[((long)nn * hm + (long)yy * fy + dy) * wm + (long)xx * fx + dx]) hit = 1;
                    }
                }
                a0[((long)nn * nby + i) * nbx + j] = (uint8_t)hit;
            }
    for (int nn = 0; nn < n; nn++)
        for (int i = 0; i < nby; i++)
            for (int j = 0; j < nbx; j++) {
                uint8_t on = 0;
                for (int di = -dilate; di <= dilate; di++)
                    for (int dj = -dilate; dj <= dilate; dj++) {
                        int ii = i + di, jj = j + dj;
                        if (ii < 0 || ii >= nby || jj < 0 || jj >= nbx) continue;
                        if (a0[((long)nn * nby + ii) * nbx + jj]) on = 1;
                    }
                active[((long)nn * nby + i) * nbx + j] = on;
            }
    free(a0);
    return 0;
}

/* Ascending linear indices of the active blocks; returns the count. */
long oracle_index_list(const uint8_t *active, long total, int32_t *idx) {
    long cnt = 0;
    for (long q = 0; q < total; q++)
        if (active[q]) idx[cnt++] = (int32_t)q;
    return cnt;
}

/* ------------------------------------------------------------------------ */
/* steps 3-5 as one definition: the edited layer output                        */
/* ------------------------------------------------------------------------ */
/* out[n,co,y,x] = bias[co] + sum_{ci,ky,kx} W[co,ci,ky,kx] * A[n,ci,y*s-p+ky,x*s-p+kx]
 * (zero outside the image), accumulated in fp64, for every output pixel whose
 * block (y/b, x/b) is active; the cached value, copied bit for bit, elsewhere.
 * active == NULL means every block is active (the dense conv); cache may then
 * be NULL.  W is OIHW in the storage dtype; bias is fp32 or NULL.  out_dt is
 * the storage dtype, or OR_F64 to keep the unrounded sums.  Output and cache
 * elements (n,co,y,x) sit at n*osn + co*osc + y*osh + x*osw. */
int oracle_sparse_layer(const void *a, int dt, int n, int h, int w, int cin, long sn, long sh, long sw, long sc,
                        const void *wt, const float *bias, int cout, int k, int s, int p, int b,
                        const uint8_t *active, const void *cache, void *out, int out_dt, long osn, long osh,
                        long osw, long osc) {
    int g[5];
    if (oracle_geometry(h, w, k, s, p, b, g)) return -1;
    if (!elem_size(dt)) return -1; /* f32, bf16, f16 storage; f64 for the pins */
    if (out_dt != dt && out_dt != OR_F64) return -1;
    if (active && !cache) return -1;
    int ho = g[0], wo = g[1], nby = g[2], nbx = g[3];
    long nw = (long)cout * cin * k * k;
    double *wd = (double *)malloc(sizeof(double) * (nw ? nw : 1));
    if (!wd) return -2;
    for (long q = 0; q < nw; q++) wd[q] = load_elem(wt, q, dt);
    int err = 0;
#pragma omp parallel
    {
        double *patch = (double *)malloc(sizeof(double) * (size_t)cin * k * k);
        if (!patch) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int nn = 0; nn < n; nn++)
            for (int y = 0; y < ho; y++) {
                if (!patch) continue;
                for (int x = 0; x < wo; x++) {
                    int on = active ? active[((long)nn * nby + y / b) * nbx + x / b] : 1;
                    if (!on) {
                        for (int co = 0; co < cout; co++) {
                            long o = nn * osn + co * osc + y * osh + x * osw;
                            if (out_dt == dt)
                                memcpy((char *)out + o * elem_size(dt), (const char *)cache + o * elem_size(dt),
                                       elem_size(dt));
                            else
                                ((double *)out)[o] = load_elem(cache, o, dt);
                        }
                        continue;
                    }
                    /* the receptive field of (y, x), in OIHW order, zero outside */
                    for (int ci = 0; ci < cin; ci++)
                        for (int ky = 0; ky < k; ky++)
                            for (int kx = 0; kx < k; kx++) {
                                int iy = y * s - p + ky, ix = x * s - p + kx;
                                double v = 0.0;
                                if (iy >= 0 && iy < h && ix >= 0 && ix < w)
                                    v = load_elem(a, nn * sn + ci * sc + iy * sh + ix * sw, dt);
                                patch[((long)ci * k + ky) * k + kx] = v;
                            }
                    for (int co = 0; co < cout; co++) {
                        double acc = 0.0;
                        const double *wr = wd + (long)co * cin * k * k;
                        for (long q = 0; q < (long)cin * k * k; q++) acc += wr[q] * patch[q];
                        if (bias) acc += (double)bias[co];
                        store_elem(out, nn * osn + co * osc + y * osh + x * osw, out_dt, acc);
                    }
                }
            }
        free(patch);
    }
    free(wd);
    return err;
}

/* ------------------------------------------------------------------------ */
/* the three separate steps, NHWC ([README] Overview)                          */
/* ------------------------------------------------------------------------ */
static void block_coords(int32_t lin, int nby, int nbx, int *nn, int *i, int *j) {
    *nn = lin / (nby * nbx);
    *i = (lin / nbx) % nby;
    *j = lin % nbx;
}

/* Gather: blocks[slot, yy, xx, c] = A[n, i*b*s - p + yy, j*b*s - p + xx, c]
 * (zero outside the image) for slot < count, where idx[slot] names (n, i, j).
 * A is NHWC [n, h, w, cin]; blocks is [count, ib, ib, cin]; both in dt. */
int oracle_gather(const void *a, int dt, int n, int h, int w, int cin, int k, int s, int p, int b,
                  const int32_t *idx, long count, void *blocks) {
    int g[5];
    if (oracle_geometry(h, w, k, s, p, b, g)) return -1;
    int nby = g[2], nbx = g[3], ib = g[4], es = elem_size(dt);
    for (long slot = 0; slot < count; slot++) {
        int nn, i, j;
        block_coords(idx[slot], nby, nbx, &nn, &i, &j);
        if (nn < 0 || nn >= n) return -1;
        for (int yy = 0; yy < ib; yy++)
            for (int xx = 0; xx < ib; xx++) {
                int iy = i * b * s - p + yy, ix = j * b * s - p + xx;
                char *dst = (char *)blocks + (((slot * ib + yy) * (long)ib + xx) * cin) * es;
                if (iy < 0 || iy >= h || ix < 0 || ix >= w)
                    memset(dst, 0, (size_t)cin * es);
                else
                    memcpy(dst, (const char *)a + ((((long)nn * h + iy) * w + ix) * cin) * es, (size_t)cin * es);
            }
    }
    return 0;
}

/* Conv on stacked blocks: a valid k x k conv with stride s on each block.
 * out_blocks[slot, py, px, co] = bias[co] + sum W[co,ci,ky,kx] * blk[slot, py*s+ky, px*s+kx, ci],
 * fp64 accumulation, rounded to out_dt (dt or OR_F64).  W is OIHW. */
int oracle_conv_blocks(const void *blocks, int dt, long count, int ib, int cin, const void *wt, const float *bias,
                       int cout, int k, int s, int b, void *out_blocks, int out_dt) {
    if ((b - 1) * s + k != ib) return -1;
    if (out_dt != dt && out_dt != OR_F64) return -1;
    long total = count * b * b;
#pragma omp parallel for schedule(dynamic, 4)
    for (long q = 0; q < total; q++) {
        long slot = q / (b * b);
        int py = (int)((q / b) % b), px = (int)(q % b);
        for (int co = 0; co < cout; co++) {
            double acc = 0.0;
            for (int ci = 0; ci < cin; ci++)
                for (int ky = 0; ky < k; ky++)
                    for (int kx = 0; kx < k; kx++) {
                        double wv = load_elem(wt, (((long)co * cin + ci) * k + ky) * k + kx, dt);
                        double xv =
                            load_elem(blocks, ((slot * ib + py * s + ky) * (long)ib + px * s + kx) * cin + ci, dt);
                        acc += wv * xv;
                    }
            if (bias) acc += (double)bias[co];
            store_elem(out_blocks, q * cout + co, out_dt, acc);
        }
    }
    return 0;
}

/* Scatter: out = cache (bit copy) when copy_cached, then every valid pixel of
 * every block slot < count is overwritten from out_blocks; pixels of partial
 * edge blocks beyond (ho, wo) are dropped.  NHWC [n, ho, wo, cout]. */
int oracle_scatter(const void *out_blocks, int dt, long count, const int32_t *idx, int n, int ho, int wo, int cout,
                   int b, const void *cache, void *out, int copy_cached) {
    int es = elem_size(dt);
    int nby = (ho + b - 1) / b, nbx = (wo + b - 1) / b;
    if (copy_cached) memcpy(out, cache, (size_t)n * ho * wo * cout * es);
    for (long slot = 0; slot < count; slot++) {
        int nn, i, j;
        block_coords(idx[slot], nby, nbx, &nn, &i, &j);
        if (nn < 0 || nn >= n) return -1;
        for (int py = 0; py < b; py++)
            for (int px = 0; px < b; px++) {
                int y = i * b + py, x = j * b + px;
                if (y >= ho || x >= wo) continue;
                memcpy((char *)out + ((((long)nn * ho + y) * wo + x) * cout) * es,
                       (const char *)out_blocks + (((slot * b + py) * (long)b + px) * cout) * es, (size_t)cout * es);
            }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* sequential edits ([REVIEW] ABSTRACT: results with sequential edits;          */
/* Proposed method: the engine keeps its state between edits)                   */
/* ------------------------------------------------------------------------ */
/* `out` holds the previous edit's result: the cache outside the blocks of
 * prev_idx[0, prev_count) and recomputed values inside them.  Every valid
 * pixel of a block that prev_idx lists and idx[0, count) does not gets its
 * cached value back (bit copy); blocks of both lists are left alone, since the
 * new edit recomputes them.  idx may be NULL with count 0 (restore every
 * previous block).  NHWC [n, ho, wo, cout]. */
int oracle_restore_blocks(const int32_t *prev_idx, long prev_count, const int32_t *idx, long count, int n, int ho,
                          int wo, int cout, int b, int dt, const void *cache, void *out) {
    int es = elem_size(dt);
    int nby = (ho + b - 1) / b, nbx = (wo + b - 1) / b;
    for (long slot = 0; slot < prev_count; slot++) {
        int32_t lin = prev_idx[slot];
        int in_new = 0;
        for (long e = 0; e < count; e++)
            if (idx[e] == lin) in_new = 1;
        if (in_new) continue;
        int nn, i, j;
        block_coords(lin, nby, nbx, &nn, &i, &j);
        if (lin < 0 || nn >= n) return -1;
        for (int py = 0; py < b; py++)
            for (int px = 0; px < b; px++) {
                int y = i * b + py, x = j * b + px;
                if (y >= ho || x >= wo) continue;
                long off = ((((long)nn * ho + y) * wo + x) * cout) * es;
                memcpy((char *)out + off, (const char *)cache + off, (size_t)cout * es);
            }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* query-pruned self-attention ([REVIEW] Proposed method: attention layers are */
/* handled by pruning the queries of unedited tokens, so that the attention    */
/* work scales with the edited area)                                            */
/* ------------------------------------------------------------------------ */
/* Tokens are the pixels of an h x w grid in row-major order; q, k, v, cache
 * and out are [n, h*w, heads*d] (head hd owns channels [hd*d, hd*d + d)).  For
 * every token of an active block (b x b tokens, clipped at the grid edge;
 * active NULL: every token) and every head:
 *   out[t] = sum over the tokens j of the same image of
 *            softmax_j(scale * q[t] . k[j]) * v[j],
 * the scores, the softmax (its maximum subtracted) and the weighted sum in
 * fp64 from the exactly widened stored values, then one rounding to out_dt
 * (the storage dtype, or OR_F64).  Every other token: the cached value. */
int oracle_sparse_attention(const void *q, const void *kt, const void *v, int dt, int n, int h, int w, int heads,
                            int d, double scale, int b, const uint8_t *active, const void *cache, void *out,
                            int out_dt) {
    if (!elem_size(dt) || n < 1 || h < 1 || w < 1 || heads < 1 || d < 1 || b < 1) return -1;
    if (out_dt != dt && out_dt != OR_F64) return -1;
    if (active && !cache) return -1;
    const long L = (long)h * w, C = (long)heads * d;
    const int nby = (h + b - 1) / b, nbx = (w + b - 1) / b;
    int err = 0;
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * L);
        double *acc = (double *)malloc(sizeof(double) * d);
        if (!sc || !acc) {
#pragma omp critical
            err = -2;
        }
#pragma omp for schedule(dynamic, 4) collapse(2)
        for (int nn = 0; nn < n; nn++)
            for (long t = 0; t < L; t++) {
                if (!sc || !acc) continue;
                const int y = (int)(t / w), x = (int)(t % w);
                const long base = ((long)nn * L + t) * C;
                if (active && !active[((long)nn * nby + y / b) * nbx + x / b]) {
                    for (long c = 0; c < C; c++) store_elem(out, base + c, out_dt, load_elem(cache, base + c, dt));
                    continue;
                }
                for (int hd = 0; hd < heads; hd++) {
                    double mx = -INFINITY;
                    for (long j = 0; j < L; j++) {
                        const long kb = ((long)nn * L + j) * C + (long)hd * d;
                        double s = 0.0;
                        for (int c = 0; c < d; c++) s += load_elem(q, base + (long)hd * d + c, dt) * load_elem(kt, kb + c, dt);
                        sc[j] = scale * s;
                        if (sc[j] > mx) mx = sc[j];
                    }
                    double sum = 0.0;
                    for (int c = 0; c < d; c++) acc[c] = 0.0;
                    for (long j = 0; j < L; j++) {
                        const double e = exp(sc[j] - mx);
                        const long vb = ((long)nn * L + j) * C + (long)hd * d;
                        sum += e;
                        for (int c = 0; c < d; c++) acc[c] += e * load_elem(v, vb + c, dt);
                    }
                    for (int c = 0; c < d; c++) store_elem(out, base + (long)hd * d + c, out_dt, acc[c] / sum);
                }
            }
        free(sc);
        free(acc);
    }
    return err;
}
