// Device helpers shared by the GEMM kernels: vector types, per-dtype MFMA and
// conversions, and the four-output epilogue store.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "gemm_kernels.hpp"
#include "lt.h"

namespace lt {

// s_waitcnt with vmcnt = n (0 <= n <= 63, a constant), other counters
// untouched. (A macro: a __device__ helper template around the target builtin
// would not be instantiable in the host compilation pass.)
#define LT_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (0x7 << 4) | (0xf << 8) | (((n) >> 4) << 14))

template <int I>
using ic = std::integral_constant<int, I>;

// Compile-time loop: f(ic<I>) for I in [B, E).
template <int B, int E, class F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

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

// alpha*acc + beta*c of four consecutive N outputs with the four C values
// already loaded (c = 0 when beta == 0), rounded to the output format and
// packed: the one arithmetic of the plain epilogue, whichever way the
// result is then stored.
template <int DT>
__device__ __forceinline__ u32x2 epi4(const float* a, float alpha, float beta, u32x2 c) {
    const float v0 = alpha * a[0] + beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x & 0xffff));
    const float v1 = alpha * a[1] + beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x >> 16));
    const float v2 = alpha * a[2] + beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y & 0xffff));
    const float v3 = alpha * a[3] + beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y >> 16));
    u32x2 o;
    o.x = pack2<DT>(v0, v1);
    o.y = pack2<DT>(v2, v3);
    return o;
}

// epi4 stored as one 8-byte write, so a caller can issue all its C loads
// before the first one is waited on.
template <int DT>
__device__ __forceinline__ void store4_c(uint16_t* D, int64_t dof, const float* a, float alpha, float beta,
                                         u32x2 c) {
    *reinterpret_cast<u32x2*>(D + dof) = epi4<DT>(a, alpha, beta, c);
}

// The activation of the fused epilogue, in fp32.
__device__ __forceinline__ float activate(float v, int act) {
    if (act == LT_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (act == LT_ACT_GELU) return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    return v;
}

// One fused output: alpha*acc + beta*c + bias, then the activation (ReLU:
// x > 0 ? x : 0; GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))), in fp32.
template <int DT>
__device__ __forceinline__ float fused_value(float acc, float alpha, float beta, const uint16_t* C, int64_t cof,
                                             const EpiArgs& e, int m, int n) {
    float v = alpha * acc;
    if (beta != 0.0f) v += beta * Tr<DT>::to_f32(C[cof]);
    if (e.bias) v += Tr<DT>::to_f32(e.bias[(int64_t)(e.bias_on_rows ? m : n) * e.bias_stride]);
    return activate(v, e.act);
}

// Fused epilogue of the first cnt (1..4) of four consecutive N outputs of row
// m (C and D N-major): one 8-byte store when all four are in, else 2-byte
// stores. Updates the lane's running max of |stored value|.
template <int DT>
__device__ __forceinline__ void store4_fused(uint16_t* D, const uint16_t* C, int64_t dof, int64_t cof,
                                             const float* a, int cnt, float alpha, float beta,
                                             const EpiArgs& e, int m, int n, float* amax) {
    uint16_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < cnt) {
            o[i] = Tr<DT>::from_f32(fused_value<DT>(a[i], alpha, beta, C, cof + i, e, m, n + i));
            *amax = fmaxf(*amax, fabsf(Tr<DT>::to_f32(o[i])));
        }
    }
    if (cnt == 4) {
        u32x2 w;
        w.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
        w.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
        *reinterpret_cast<u32x2*>(D + dof) = w;
    } else {
        for (int i = 0; i < cnt; ++i) D[dof + i] = o[i];
    }
}

// Max of the lanes' values over the wave, then one atomic max per wave on the
// float's bits (the values are >= 0, so their bit patterns order as
// unsigned integers).
__device__ __forceinline__ void amax_commit(float* amax_out, float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(v));
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

// Raise a kernel's dynamic LDS limit to `bytes`, once per device (the
// attribute belongs to the device the call is made on); `done` holds one bit
// per device id. Returns 0 or the hipError_t.
inline int set_lds_limit_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return 0;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return static_cast<int>(e);
    done.fetch_or(bit, std::memory_order_release);
    return 0;
}

}  // namespace lt
