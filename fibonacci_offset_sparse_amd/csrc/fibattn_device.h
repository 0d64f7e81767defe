// Device helpers for the gfx950 kernels: storage-type conversion, row loads and stores,
// accurate RoPE angles, and the workgroup mapping. Included by the .hip files only.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "fibattn_internal.h"

namespace fibattn {

using bf16_t = uint16_t;  // bfloat16 storage
using f16_t = _Float16;   // half storage of the staged keys and values
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Four consecutive elements starting at p, as float.
template <typename T> __device__ __forceinline__ float4 load4(const T* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
    uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
}

template <> __device__ __forceinline__ float4 load4<f16_t>(const f16_t* p) {
    uint2 w = *reinterpret_cast<const uint2*>(p);
    const h2_t a = __builtin_bit_cast(h2_t, w.x), b = __builtin_bit_cast(h2_t, w.y);
    return make_float4(static_cast<float>(a.x), static_cast<float>(a.y), static_cast<float>(b.x),
                       static_cast<float>(b.y));
}

template <typename T> __device__ __forceinline__ void store4(T* p, float4 x);
template <> __device__ __forceinline__ void store4<float>(float* p, float4 x) {
    *reinterpret_cast<float4*>(p) = x;
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 x) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
}
template <> __device__ __forceinline__ void store4<f16_t>(f16_t* p, float4 x) {
    const h2_t a = {static_cast<_Float16>(x.x), static_cast<_Float16>(x.y)};
    const h2_t b = {static_cast<_Float16>(x.z), static_cast<_Float16>(x.w)};
    *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Stores with the non-temporal hint (global_store ... nt), for a kernel's final outputs: written
// once, read by no later stage of the call. In a grid whose workgroups all load first and store
// last, plain stores drained far slower than hinted ones (a one-round 32 MiB load-then-store: 21.4
// us plain, 13.4 us hinted, on one MI355X). Intermediates that a later kernel of the same call
// reads (staged rows, weights) keep plain stores: hinting them slowed their reader more.
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void* p, const uint4& v) {
    const u32x4_nt_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, static_cast<u32x4_nt_t*>(p));
}
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

// One element as float, and one float stored in the storage type.
template <typename T> __device__ __forceinline__ float load_elem(const T* p);
template <> __device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
template <typename T> __device__ __forceinline__ void store_elem(T* p, float x);
template <> __device__ __forceinline__ void store_elem<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, float x) {
    *p = static_cast<bf16_t>(f32_to_bf16_bits(x));
}

// A 64-element row into registers.
template <typename T> __device__ __forceinline__ void load_row(const T* p, float (&x)[kD]) {
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        float4 v = load4<T>(p + 4 * c);
        x[4 * c + 0] = v.x;
        x[4 * c + 1] = v.y;
        x[4 * c + 2] = v.z;
        x[4 * c + 3] = v.w;
    }
}

template <typename T> __device__ __forceinline__ void store_row(T* p, const float (&x)[kD]) {
#pragma unroll
    for (int c = 0; c < kD / 4; ++c)
        store4<T>(p + 4 * c, make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]));
}

// cos and sin of pos * omega_j. The angle is reduced in revolutions against omega_j / (2 pi)
// held as hi + lo (double accuracy): n is the nearest whole revolution, fma(pos, hi, -n) takes the
// exact product minus n and rounds once, and pos * lo is added, so the reduced angle is good to
// about 2^-25 revolutions for every position below 2^24. Only explicit fmas appear, so no
// contraction can change what is computed.
__device__ __forceinline__ void rope_cos_sin(int pos, float hi, float lo, float& c, float& s) {
    const float fp = static_cast<float>(pos);
    const float n = rintf(fp * hi);
    const float frac = fmaf(fp, lo, fmaf(fp, hi, -n));
    sincosf(frac * 6.28318530717958647692f, &s, &c);
}

// Rotate (x_j, x_{j+32}) by the angle whose cos/sin are cs[j].
__device__ __forceinline__ void rope_apply(float (&x)[kD], const float2* cs) {
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const float2 r = cs[j];
        const float a = x[j], b = x[j + kPairs];
        x[j] = a * r.x - b * r.y;
        x[j + kPairs] = b * r.x + a * r.y;
    }
}

// Transpose of the rotation (used for gradients).
__device__ __forceinline__ void rope_apply_t(float (&x)[kD], const float2* cs) {
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const float2 r = cs[j];
        const float a = x[j], b = x[j + kPairs];
        x[j] = a * r.x + b * r.y;
        x[j + kPairs] = b * r.x - a * r.y;
    }
}

}  // namespace fibattn
