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

// float -> bfloat16, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, one instruction with no branch.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

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

// 16 raw bytes already in registers, widened to float (the type argument picks the layout).
__device__ __forceinline__ void unpack16(const u32x4& v, const bf16_t*, float* o) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o[2 * i] = __uint_as_float(v[i] << 16);
        o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const u32x4& v, const float*, float* o) {
#pragma unroll
    for (int i = 0; i < 4; i++) o[i] = __uint_as_float(v[i]);
}
template <class T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

// Cross-lane steps without the LDS crossbar (gfx950 DPP and permlane swaps).
// A "row" is 16 consecutive lanes. dpp_f<CTRL> reads the lane selected by a
// DPP16 control within the row: 0xB1 = quad_perm[1,0,3,2] (lane ^ 1),
// 0x4E = quad_perm[2,3,0,1] (lane ^ 2), 0x141 = row_half_mirror (7 - i within
// each 8 lanes), 0x140 = row_mirror (15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Pairs lanes l and l ^ 16 (swap16) or l and l ^ 32 (swap32): both lanes of a
// pair get {value of the lower lane, value of the upper lane}, so any
// symmetric combination of the two is bitwise identical in both lanes.
struct LanePair { float lo, hi; };
__device__ __forceinline__ LanePair swap16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // {lower row's, upper row's}
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair swap32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // {lower half's, upper half's}
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Sum / max over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const LanePair a = swap16(v);
    v = a.lo + a.hi;
    const LanePair b = swap32(v);
    return b.lo + b.hi;
}
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    const LanePair a = swap16(v);
    v = fmaxf(a.lo, a.hi);
    const LanePair b = swap32(v);
    return fmaxf(b.lo, b.hi);
}

// LDS destination of global_load_lds (direct global-to-LDS loads).
typedef __attribute__((address_space(3))) void lds_void;

template <int V>
__device__ __forceinline__ void wait_vm() {  // s_waitcnt vmcnt(V), other counters untouched (gfx9 encoding)
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
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
