// sige_internal.h -- types and launchers shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sige {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// Launch parameters of the implicit-GEMM convolution.
struct ConvCfg {
    int mt, nt;          // 16x16 tiles per workgroup along M (rows) and N (output channels)
    int ck;              // input channels staged per chunk
    int a_pix_stride;    // LDS bytes per staged input pixel (ck*es + 16)
    int b_row_stride;    // LDS bytes per staged weight row (k*k*ck*es + 16)
    int a_bytes;         // LDS bytes of the staged input windows
    int lds_bytes;       // dynamic LDS per workgroup
    int ns_max;          // most block slots one M tile can touch
    int compute_grid;    // persistent workgroups doing the GEMM
    int copy_xw;         // output pixels per copy unit (one image row segment)
    int copy_units;      // workgroups copying the cache (0 without copy)
};

hipError_t launch_diff(int dt, const void *a_orig, const void *a_edit, long npix, int vpp, float tau,
                       uint8_t *mask, hipStream_t st);
hipError_t launch_reduce(const uint8_t *mask, int hm, int wm, const Geo &g, int dilate, int vec16, int32_t *idx,
                         int32_t *count, hipStream_t st);
hipError_t launch_gather(const void *a_edit, int dt, const Geo &g, const int32_t *idx, const int32_t *count,
                         void *blocks, hipStream_t st);
// fused = 0: src = stacked blocks, dst = output blocks.  fused = 1: src = a_edit, dst = out.
hipError_t launch_conv(int dt, int fused, const void *src, const void *w, const float *bias, const int32_t *idx,
                       const int32_t *count, void *dst, const void *cache, const Geo &g, const ConvCfg &cfg,
                       hipStream_t st);
hipError_t launch_scatter(int dt, const void *out_blocks, const int32_t *idx, const int32_t *count, const Geo &g,
                          const void *cached, void *out, int copy_cached, int scatter_grid, int copy_xw,
                          int copy_units, hipStream_t st);

// reduce limits (LDS of its single workgroup)
constexpr int kReduceBitsWords = 8192;   // pooled mask rows, 32 pixels per word
constexpr int kReduceMaxBlocks = 12288;  // block grid of one image

}  // namespace sige
