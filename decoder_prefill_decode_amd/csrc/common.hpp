// Shared device helpers for the gfx950 kernels: bf16 conversion, vector
// types, 64-lane wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vlm {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Round a float to the nearest bf16 value, kept as float.
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// Element loads/stores for the two storage types.
template <class T> struct Elt;
template <> struct Elt<float> {
    __device__ __forceinline__ static float ld(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void st(float* p, size_t i, float v) { p[i] = v; }
    __device__ __forceinline__ static float rnd(float v) { return v; }
};
template <> struct Elt<bf16_t> {
    __device__ __forceinline__ static float ld(const bf16_t* p, size_t i) { return bf2f(p[i]); }
    __device__ __forceinline__ static void st(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }
    __device__ __forceinline__ static float rnd(float v) { return round_bf(v); }
};

// 16-byte vector load of 8 bf16 or 4 floats, unpacked to floats.
__device__ __forceinline__ void ld16(const bf16_t* p, float* out) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        out[2 * i] = __uint_as_float(v[i] << 16);
        out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void ld16(const float* p, float* out) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) out[i] = v[i];
}
template <class T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Block-wide sum for blockDim.x == NT (multiple of 64); `red` holds NT/64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) t += red[i];
    __syncthreads();
    return t;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_tanh_f(float z) {
    const float k0 = 0.7978845608028654f, k1 = 0.044715f;
    return 0.5f * z * (1.0f + tanhf(k0 * (z + k1 * z * z * z)));
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace vlm
