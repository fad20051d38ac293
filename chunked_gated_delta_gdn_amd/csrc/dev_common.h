// Device helpers shared by the kernels: element types and conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bfloat16 stored as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;

// load_raw / from_raw split a load from its conversion, so that a value
// fetched ahead of its use does not make the loading wave wait for it.
template <> struct Elem<float> {
    typedef float raw_t;
    static __device__ __forceinline__ float load(const void *p, int64_t i) {
        return static_cast<const float *>(p)[i];
    }
    static __device__ __forceinline__ raw_t load_raw(const void *p, int64_t i) {
        return static_cast<const float *>(p)[i];
    }
    static __device__ __forceinline__ float from_raw(raw_t x) { return x; }
    static __device__ __forceinline__ void store(void *p, int64_t i, float x) {
        static_cast<float *>(p)[i] = x;
    }
};

template <> struct Elem<bf16_t> {
    typedef uint16_t raw_t;
    static __device__ __forceinline__ float load(const void *p, int64_t i) {
        return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    static __device__ __forceinline__ raw_t load_raw(const void *p, int64_t i) {
        return static_cast<const uint16_t *>(p)[i];
    }
    static __device__ __forceinline__ float from_raw(raw_t x) { return bf16_to_f32(x); }
    static __device__ __forceinline__ void store(void *p, int64_t i, float x) {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    }
};

// Eight consecutive elements fetched as one (bf16: 16 B) or two (fp32: 2 x 16 B)
// loads and converted where used; `at` takes a constant index after unrolling.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const void *p, int64_t i) {
        v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
    }
    __device__ __forceinline__ float at(int j) const {
        const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
        return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const void *p, int64_t i) {
        a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i + 4);
    }
    __device__ __forceinline__ float at(int j) const {
        const float4 &x = j < 4 ? a : b;
        const int k = j & 3;
        return k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w;
    }
};

}  // namespace gdn
