// Device helpers shared by the GEMM kernels: vector types, per-dtype MFMA and
// conversions, and the four-output epilogue store.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lt.h"

namespace lt {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

#define LDS_AS __attribute__((address_space(3)))

template <int DT>
struct Tr;

template <>
struct Tr<LT_F16> {
    using V8 = f16x8;
    static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return static_cast<float>(__builtin_bit_cast(_Float16, x));
    }
    static __device__ __forceinline__ uint16_t from_f32(float x) {   // round to nearest even
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
};

template <>
struct Tr<LT_BF16> {
    using V8 = bf16x8;
    static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
    }
    static __device__ __forceinline__ uint16_t from_f32(float x) {   // round to nearest even
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
};

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return static_cast<uint32_t>(Tr<DT>::from_f32(a)) | (static_cast<uint32_t>(Tr<DT>::from_f32(b)) << 16);
}

// Epilogue of four consecutive N outputs of one row: alpha*acc + beta*c,
// rounded to the output format and stored as one 8-byte write.
template <int DT>
__device__ __forceinline__ void store4(uint16_t* D, const uint16_t* C, int64_t dof, int64_t cof, float a0,
                                       float a1, float a2, float a3, float alpha, float beta) {
    float v0 = alpha * a0, v1 = alpha * a1, v2 = alpha * a2, v3 = alpha * a3;
    if (beta != 0.0f) {
        u32x2 c = *reinterpret_cast<const u32x2*>(C + cof);
        v0 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x & 0xffff));
        v1 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x >> 16));
        v2 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y & 0xffff));
        v3 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y >> 16));
    }
    u32x2 o;
    o.x = pack2<DT>(v0, v1);
    o.y = pack2<DT>(v2, v3);
    *reinterpret_cast<u32x2*>(D + dof) = o;
}

// The same for the first cnt (1..3) of four outputs, one 2-byte store each:
// the last, partial group of a row that ends inside a tile.
template <int DT>
__device__ __forceinline__ void store_n(uint16_t* D, const uint16_t* C, int64_t dof, int64_t cof, const float* a,
                                        int cnt, float alpha, float beta) {
    for (int e = 0; e < cnt; ++e) {
        float v = alpha * a[e];
        if (beta != 0.0f) v += beta * Tr<DT>::to_f32(C[cof + e]);
        D[dof + e] = Tr<DT>::from_f32(v);
    }
}

}  // namespace lt
