// conv_common.h -- device pieces shared by the implicit-GEMM convolution
// kernels (kernels_conv.hip, kernels_layer.hip): one K step on the matrix
// cores per storage type, and the rounding store of 8 output channels.
#pragma once
#include "device_common.h"

namespace sige {

template <int DT>
struct MfmaStep;

template <>
struct MfmaStep<1> {  // bf16: one 16x16x32 MFMA per (16 B of A, 16 B of B)
    static constexpr int KS = 32;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <>
struct MfmaStep<2> {  // fp16
    static constexpr int KS = 32;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};
template <>
struct MfmaStep<0> {  // fp32: four 16x16x4 MFMAs; lane group g holds k = 4g..4g+3
    static constexpr int KS = 16;
    __device__ static __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
        return c;
    }
};

// One 32x32x16 MFMA (bf16, fp16): lane l holds A row l % 32 and B column
// l % 32, each at k = 8 * (l / 32) .. +7; accumulator register v of lane l
// is D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].
template <int DT>
struct Mfma32;
template <>
struct Mfma32<1> {
    __device__ static __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <>
struct Mfma32<2> {
    __device__ static __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

// Store 8 consecutive channels (fp32: the second 16-byte half only when
// `full`; c_out is a multiple of 4 there, of 8 for 16-bit types).
template <int DT>
__device__ __forceinline__ void store_row8(uint8_t *p, const float *v, bool full) {
    if constexpr (DT == 0) {
        st16(p, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
        if (full)
            st16(p + 16,
                 u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo, hi;
            if constexpr (DT == 1) {
                lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
            } else {
                lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            }
            w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        st16(p, u32x4{w[0], w[1], w[2], w[3]});
    }
}

}  // namespace sige
