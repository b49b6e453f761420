// Memory-bound helper kernels: embedding lookup and image-row injection
// (Youtu-VL-4B ncnn port, 实现流程 §5), row norms feeding the GEMMs, QK-Norm +
// rotate-half RoPE + KV-cache write (Youtu-VL-4B ncnn port, 实现难点 §2 and
// 实现流程 §7; Penguin-VL ncnn port §2.3 for the two-segment form), RoPE table
// construction, row gathers and weight packing.
#include "common.hpp"
#include "internal.hpp"

namespace vlm {

// ---------------------------------------------------------------- embedding
template <class T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ table, int V, int H,
                                                    const int32_t* __restrict__ ids, float* __restrict__ x) {
    const int s = blockIdx.x;
    const int id = ids[s];
    float* row = x + (size_t)s * H;
    if (id < 0 || id >= V) {
        for (int j = threadIdx.x; j < H; j += 256) row[j] = __uint_as_float(0x7fc00000u);
        return;
    }
    const T* src = table + (size_t)id * H;
    for (int j = threadIdx.x; j < H; j += 256) row[j] = Elt<T>::ld(src, j);
}

// One row: the embedding of tok[0], or a copy of xin when xin != null.
template <class T>
__global__ __launch_bounds__(256) void embed_row_kernel(const T* __restrict__ table, int V, int H,
                                                        const int32_t* __restrict__ tok, const float* __restrict__ xin,
                                                        float* __restrict__ x, const int32_t* __restrict__ len,
                                                        const float* __restrict__ cosv, const float* __restrict__ sinv,
                                                        int D, float* __restrict__ rope) {
    // the RoPE row of this token's position (slot len), staged once for every layer's attention
    if (rope) {
        const int t = len[0];
        for (int j = threadIdx.x; j < D; j += 256) {
            rope[j] = cosv[(size_t)t * D + j];
            rope[D + j] = sinv[(size_t)t * D + j];
        }
    }
    if (xin) {
        for (int j = threadIdx.x; j < H; j += 256) x[j] = xin[j];
        return;
    }
    const int id = tok[0];
    if (id < 0 || id >= V) {
        for (int j = threadIdx.x; j < H; j += 256) x[j] = __uint_as_float(0x7fc00000u);
        return;
    }
    const T* src = table + (size_t)id * H;
    for (int j = threadIdx.x; j < H; j += 256) x[j] = Elt<T>::ld(src, j);
}

// ---------------------------------------------------------------- injection
// Row s with ids[s] == pid gets image row rank(s) = #{j < s : ids[j] == pid}.
template <class T>
__global__ __launch_bounds__(256) void inject_kernel(float* __restrict__ x, int H, const int32_t* __restrict__ ids,
                                                     int pid, const T* __restrict__ img, int n_img) {
    __shared__ int red[4];
    const int s = blockIdx.x;
    if (ids[s] != pid) return;
    int c = 0;
    for (int j = threadIdx.x; j < s; j += 256) c += (ids[j] == pid);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, kWave);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = c;
    __syncthreads();
    const int rank = red[0] + red[1] + red[2] + red[3];
    if (rank >= n_img) return;
    const T* src = img + (size_t)rank * H;
    float* dst = x + (size_t)s * H;
    for (int j = threadIdx.x; j < H; j += 256) dst[j] = Elt<T>::ld(src, j);
}

__global__ void set_len_kernel(int32_t* len, int v) {
    if (threadIdx.x == 0 && blockIdx.x == 0) len[0] = v;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__global__ void inc_len_kernel(int32_t* len) {
    if (threadIdx.x == 0 && blockIdx.x == 0) len[0] = len[0] + 1;
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ s, float* __restrict__ d, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) d[i] = s[i];
}

// ---------------------------------------------------------------- row norms
// RMSNorm: y = x * rsqrt(mean(x^2) + eps) * g. LayerNorm: y = (x - mu) * rsqrt(var + eps) * g + b.
// Output rounded to the operand type. One block per row.
// Rows of up to NPT * 256 elements: every load of the row and its gain/shift is issued before
// the first arithmetic (indices clamped, lanes past H masked), and the row stays in registers
// between the reduction and the output.
template <class T, bool LAYER, int NPT>
__global__ __launch_bounds__(256) void norm_rows_reg_kernel(const float* __restrict__ x, int H, int ldx,
                                                            const T* __restrict__ g, const T* __restrict__ b,
                                                            float eps, T* __restrict__ out) {
    __shared__ float red[4];
    const float* row = x + (size_t)blockIdx.x * ldx;
    const int tid = threadIdx.x;
    float v[NPT], gv[NPT], bv[NPT];
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const int j = min(tid + 256 * i, H - 1);
        v[i] = row[j];
        gv[i] = Elt<T>::ld(g, j);
        bv[i] = (LAYER && b) ? Elt<T>::ld(b, j) : 0.f;
    }
    float mu = 0.f;
    if (LAYER) {
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < NPT; i++) sm += tid + 256 * i < H ? v[i] : 0.f;
        mu = block_sum<256>(sm, red) / (float)H;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const float c = v[i] - mu;
        ss += tid + 256 * i < H ? c * c : 0.f;
    }
    const float r = rsqrtf(block_sum<256>(ss, red) / (float)H + eps);
    T* o = out + (size_t)blockIdx.x * H;
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const int j = tid + 256 * i;
        if (j < H) Elt<T>::st(o, j, (v[i] - mu) * r * gv[i] + bv[i]);
    }
}

template <class T, bool LAYER>
__global__ __launch_bounds__(256) void norm_rows_kernel(const float* __restrict__ x, int H, int ldx,
                                                        const T* __restrict__ g, const T* __restrict__ b, float eps,
                                                        T* __restrict__ out) {
    __shared__ float red[4];
    const float* row = x + (size_t)blockIdx.x * ldx;
    float mu = 0.f;
    if (LAYER) {
        float s = 0.f;
        for (int j = threadIdx.x; j < H; j += 256) s += row[j];
        mu = block_sum<256>(s, red) / (float)H;
    }
    float ss = 0.f;
    for (int j = threadIdx.x; j < H; j += 256) {
        const float v = row[j] - mu;
        ss += v * v;
    }
    const float r = rsqrtf(block_sum<256>(ss, red) / (float)H + eps);
    T* o = out + (size_t)blockIdx.x * H;
    for (int j = threadIdx.x; j < H; j += 256) {
        float y = (row[j] - mu) * r * Elt<T>::ld(g, j);
        if (LAYER && b) y += Elt<T>::ld(b, j);
        Elt<T>::st(o, j, y);
    }
}

// ---------------------------------------------------------------- QK-Norm + RoPE + cache write
// One block per row s: the row's q, k, v projections (fp32, nh * d) and the
// cos / sin row of its position are read once into LDS with 16-byte loads;
// then wavefront w takes heads w, w + 16, ..., and lane p < d/2 owns rotation
// pair p, i.e. the output elements i0 = g*sd + j and i1 = i0 + sd/2 of
// segment g (sd = d/segments). rotate_half(a, b) = (-b, a): y[i0] = a cos -
// b sin, y[i1] = b cos + a sin, where (a, b) are the inputs at (i0, i1), or at
// (g*sd + 2j, g*sd + 2j + 1) for interleaved RoPE (the adjacent pair,
// de-interleaved into the rotate-half order; V is copied unpermuted). The
// per-head RMSNorm gain is indexed by where the element sits when the norm
// runs: input order before the rotation, output order after it.
constexpr int kRopeThreads = 1024;  // 16 wavefronts: a 48-head row is 3 heads per wavefront
template <class T>
__global__ __launch_bounds__(kRopeThreads) void rope_qkv_kernel(RopeArgs a) {
    constexpr int NT = kRopeThreads, NWV = NT / kWave;
    extern __shared__ __attribute__((aligned(16))) float rs[];  // [nh * d] projections, [d] cos, [d] sin
    const int s = blockIdx.x, tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
    const int nh = a.nq + 2 * a.nkv, d = a.d, half = d / 2, nrow = nh * d;
    const int pos = (a.pos_dev ? a.pos_dev[0] : a.pos0) + s;
    float* cs = rs + nrow;
    float* sn = cs + d;
    {
        const f32x4* src = reinterpret_cast<const f32x4*>(a.qkv + (size_t)s * nrow);
        for (int i = tid; i < nrow / 4; i += NT) reinterpret_cast<f32x4*>(rs)[i] = src[i];
        for (int i = tid; i < d; i += NT) {
            cs[i] = a.cos[(size_t)pos * d + i];
            sn[i] = a.sin[(size_t)pos * d + i];
        }
    }
    __syncthreads();
    const bool on = lane < half;
    const int sd = d / a.segments, sh = sd / 2;
    const int g = on ? lane / sh : 0, j = on ? lane % sh : 0;
    const int i0 = g * sd + j, i1 = i0 + sh;
    const int r0 = a.interleave ? g * sd + 2 * j : i0, r1 = a.interleave ? r0 + 1 : i1;
    const float c0 = cs[i0], c1 = cs[i1], s0 = sn[i0], s1 = sn[i1];
    for (int h = w; h < nh; h += NWV) {  // uniform per wavefront
        const float* x = rs + h * d;
        if (h >= a.nq + a.nkv) {  // V head: plain copy (rounded to the cache type)
            if (on) {
                T* dst = (T*)a.vdst + ((size_t)(h - a.nq - a.nkv) * a.ldkv + pos) * d;
                Elt<T>::st(dst, i0, x[i0]);
                Elt<T>::st(dst, i1, x[i1]);
            }
            continue;
        }
        float u0 = on ? x[r0] : 0.f, u1 = on ? x[r1] : 0.f;
        const bool isq = h < a.nq;
        const T* gn = (const T*)(isq ? a.qn : a.kn);
        if (gn && !a.norm_after) {
            const float r = rsqrtf(wave_sum(u0 * u0 + u1 * u1) / (float)d + a.eps);
            if (on) {
                u0 = u0 * r * Elt<T>::ld(gn, r0);
                u1 = u1 * r * Elt<T>::ld(gn, r1);
            }
        }
        float y0 = on ? u0 * c0 - u1 * s0 : 0.f;
        float y1 = on ? u1 * c1 + u0 * s1 : 0.f;
        if (gn && a.norm_after) {  // the rotation keeps the sum of squares; the norm sees the rotated values
            const float r = rsqrtf(wave_sum(y0 * y0 + y1 * y1) / (float)d + a.eps);
            if (on) {
                y0 = y0 * r * Elt<T>::ld(gn, i0);
                y1 = y1 * r * Elt<T>::ld(gn, i1);
            }
        }
        if (!on) continue;
        T* dst = isq ? (T*)a.q + ((size_t)h * a.ldq + s) * d : (T*)a.kdst + ((size_t)(h - a.nq) * a.ldkv + pos) * d;
        Elt<T>::st(dst, i0, y0);
        Elt<T>::st(dst, i1, y1);
    }
}

// ---------------------------------------------------------------- expanded MLA: assembly + RoPE + cache write
// One wavefront per (row, head). The dn unrotated elements of q and k are
// copied, v is copied, and rotation pair j (j < dr/2) of the rope parts turns
// the inputs at (2j, 2j+1) (interleaved) or (j, j + dr/2) into the outputs at
// dn + j and dn + j + dr/2 with the angle of table column j. The rotated key
// is the shared one of the row, the same for every head.
template <class T>
__global__ __launch_bounds__(256) void mla_rope_kernel(MlaRopeArgs a) {
    const int wave = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (wave >= a.S * a.nq) return;
    const int s = wave / a.nq, h = wave % a.nq;
    const int d = a.d, dr = a.dr, dn = d - dr, dv = a.dv, hr = dr / 2;
    const int pos = (a.pos_dev ? a.pos_dev[0] : a.pos0) + s;
    const float* qi = a.q + (size_t)s * a.nq * d + (size_t)h * d;
    const float* kvi = a.kv + (size_t)s * a.nq * (dn + dv) + (size_t)h * (dn + dv);
    const float* kr = a.ka + (size_t)s * a.lda + a.kcol;
    T* qo = (T*)a.qout + ((size_t)h * a.ldq + s) * d;
    T* ko = (T*)a.kdst + ((size_t)h * a.ldkv + pos) * d;
    T* vo = (T*)a.vdst + ((size_t)h * a.ldkv + pos) * dv;
    for (int e = lane; e < dn; e += kWave) {
        Elt<T>::st(qo, e, qi[e]);
        Elt<T>::st(ko, e, kvi[e]);
    }
    for (int e = lane; e < dv; e += kWave) Elt<T>::st(vo, e, kvi[dn + e]);
    for (int j = lane; j < hr; j += kWave) {
        const int r0 = a.interleave ? 2 * j : j, r1 = a.interleave ? 2 * j + 1 : j + hr;
        const float c = a.cos[(size_t)pos * dr + j], sn = a.sin[(size_t)pos * dr + j];
        const float q0 = qi[dn + r0], q1 = qi[dn + r1], k0 = kr[r0], k1 = kr[r1];
        Elt<T>::st(qo, dn + j, q0 * c - q1 * sn);
        Elt<T>::st(qo, dn + j + hr, q1 * c + q0 * sn);
        Elt<T>::st(ko, dn + j, k0 * c - k1 * sn);
        Elt<T>::st(ko, dn + j + hr, k1 * c + k0 * sn);
    }
}

hipError_t launch_mla_rope(int dtype, const MlaRopeArgs& a, hipStream_t st) {
    const int waves = a.S * a.nq;
    if (waves <= 0) return hipSuccess;
    const int blocks = (waves + 3) / 4;
    if (dtype == 1)
        mla_rope_kernel<bf16_t><<<blocks, 256, 0, st>>>(a);
    else
        mla_rope_kernel<float><<<blocks, 256, 0, st>>>(a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- RoPE tables
struct AxisMap { int32_t ax[64]; };
__global__ __launch_bounds__(64) void rope_table_kernel(const int32_t* __restrict__ pos, int n_rows, AxisMap am,
                                                        int segments, int d, double theta, float* __restrict__ cosv,
                                                        float* __restrict__ sinv) {
    const int row = blockIdx.x;
    const int p = threadIdx.x;
    if (p >= d / 2) return;
    const int sd = d / segments, sh = sd / 2;
    const int g = p / sh, j = p % sh;
    const double inv = pow(theta, -2.0 * (double)j / (double)sd);
    const double ang = (double)pos[(size_t)am.ax[p] * n_rows + row] * inv;
    const float c = (float)cos(ang), s = (float)sin(ang);
    const size_t o = (size_t)row * d + g * sd + j;
    cosv[o] = c;
    cosv[o + sh] = c;
    sinv[o] = s;
    sinv[o + sh] = s;
}

// ---------------------------------------------------------------- gathers / packing
__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ src, int n_src,
                                                          const int32_t* __restrict__ idx, int row_len,
                                                          float* __restrict__ dst) {
    const int r = blockIdx.x;
    const int i = idx[r];
    float* o = dst + (size_t)r * row_len;
    if (i < 0 || i >= n_src) {
        for (int j = threadIdx.x; j < row_len; j += 256) o[j] = __uint_as_float(0x7fc00000u);
        return;
    }
    const float* s = src + (size_t)i * row_len;
    for (int j = threadIdx.x; j < row_len; j += 256) o[j] = s[j];
}

// out row 64g + r (r < 32) = wg row 32g + r; out row 64g + 32 + r = wu row 32g + r.
template <class T>
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const T* __restrict__ wg, const T* __restrict__ wu, int H,
                                                           T* __restrict__ out) {
    const int orow = blockIdx.x;
    const int g = orow / 64, r = orow % 64;
    const T* src = (r < 32 ? wg : wu) + (size_t)(32 * g + (r % 32)) * H;
    T* o = out + (size_t)orow * H;
    for (int j = threadIdx.x; j < H; j += 256) o[j] = src[j];
}

// ---------------------------------------------------------------- launchers
hipError_t launch_embed(int dtype, const void* table, int V, int H, const int32_t* ids, int S, float* x,
                        hipStream_t st) {
    if (S <= 0) return hipSuccess;
    if (dtype == 1)
        embed_kernel<bf16_t><<<S, 256, 0, st>>>((const bf16_t*)table, V, H, ids, x);
    else
        embed_kernel<float><<<S, 256, 0, st>>>((const float*)table, V, H, ids, x);
    return hipGetLastError();
}

hipError_t launch_embed_or_copy(int dtype, const void* table, int V, int H, const int32_t* tok, const float* xin,
                                float* x, const int32_t* len, const float* cosv, const float* sinv, int D, float* rope,
                                hipStream_t st) {
    if (dtype == 1)
        embed_row_kernel<bf16_t><<<1, 256, 0, st>>>((const bf16_t*)table, V, H, tok, xin, x, len, cosv, sinv, D, rope);
    else
        embed_row_kernel<float><<<1, 256, 0, st>>>((const float*)table, V, H, tok, xin, x, len, cosv, sinv, D, rope);
    return hipGetLastError();
}

hipError_t launch_inject(int img_dtype, float* x, int S, int H, const int32_t* ids, int pid, const void* img,
                         int n_img, hipStream_t st) {
    if (S <= 0 || n_img <= 0) return hipSuccess;
    if (img_dtype == 1)
        inject_kernel<bf16_t><<<S, 256, 0, st>>>(x, H, ids, pid, (const bf16_t*)img, n_img);
    else
        inject_kernel<float><<<S, 256, 0, st>>>(x, H, ids, pid, (const float*)img, n_img);
    return hipGetLastError();
}

hipError_t launch_set_len(int32_t* len, int value, hipStream_t st) {
    set_len_kernel<<<1, 64, 0, st>>>(len, value);
    return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st) {
    zero_i32_kernel<<<1, 256, 0, st>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_inc_len(int32_t* len, hipStream_t st) {
    inc_len_kernel<<<1, 64, 0, st>>>(len);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    copy_f32_kernel<<<blocks, 256, 0, st>>>(src, dst, n);
    return hipGetLastError();
}

template <class T, bool LAYER>
static void norm_rows_dispatch(const float* x, int R, int H, int ldx, const void* gain, const void* shift, float eps,
                               void* out, hipStream_t st) {
    const T* g = (const T*)gain;
    const T* b = (const T*)shift;
    const int npt = (H + 255) / 256;
#define VLM_NORM_REG(N) norm_rows_reg_kernel<T, LAYER, N><<<R, 256, 0, st>>>(x, H, ldx, g, b, eps, (T*)out)
    if (npt <= 2) VLM_NORM_REG(2);
    else if (npt <= 4) VLM_NORM_REG(4);
    else if (npt <= 8) VLM_NORM_REG(8);
    else if (npt <= 12) VLM_NORM_REG(12);
    else if (npt <= 16) VLM_NORM_REG(16);
    else norm_rows_kernel<T, LAYER><<<R, 256, 0, st>>>(x, H, ldx, g, b, eps, (T*)out);
#undef VLM_NORM_REG
}

hipError_t launch_norm_rows(int dtype, bool layer, const float* x, int R, int H, const void* gain, const void* shift,
                            float eps, void* out, hipStream_t st, int ldx) {
    if (ldx <= 0) ldx = H;
    if (R <= 0 || H <= 0) return hipSuccess;
    if (dtype == 1) {
        if (layer) norm_rows_dispatch<bf16_t, true>(x, R, H, ldx, gain, shift, eps, out, st);
        else norm_rows_dispatch<bf16_t, false>(x, R, H, ldx, gain, nullptr, eps, out, st);
    } else {
        if (layer) norm_rows_dispatch<float, true>(x, R, H, ldx, gain, shift, eps, out, st);
        else norm_rows_dispatch<float, false>(x, R, H, ldx, gain, nullptr, eps, out, st);
    }
    return hipGetLastError();
}

hipError_t launch_rope_qkv(int dtype, const RopeArgs& a, hipStream_t st) {
    if (a.S <= 0) return hipSuccess;
    const size_t smem = ((size_t)(a.nq + 2 * a.nkv) * a.d + 2 * a.d) * sizeof(float);
    if (a.d % 4 != 0 || a.d > 128 || smem > 64 * 1024) return hipErrorInvalidValue;
    if (dtype == 1)
        rope_qkv_kernel<bf16_t><<<a.S, kRopeThreads, smem, st>>>(a);
    else
        rope_qkv_kernel<float><<<a.S, kRopeThreads, smem, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_rope_table(const int32_t* pos, int n_axes, int n_rows, const int32_t* axis_of_pair, int segments,
                             int d, double theta, float* cos, float* sin, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    AxisMap am;
    for (int i = 0; i < 64; i++) am.ax[i] = i < d / 2 ? axis_of_pair[i] : 0;
    (void)n_axes;
    rope_table_kernel<<<n_rows, 64, 0, st>>>(pos, n_rows, am, segments, d, theta, cos, sin);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const float* src, int n_src, const int32_t* idx, int n_rows, int row_len, float* dst,
                              hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    gather_rows_kernel<<<n_rows, 256, 0, st>>>(src, n_src, idx, row_len, dst);
    return hipGetLastError();
}

hipError_t launch_pack_gate_up(int dtype, const void* wg, const void* wu, int F, int H, void* out, hipStream_t st) {
    if (dtype == 1)
        pack_gate_up_kernel<bf16_t><<<2 * F, 256, 0, st>>>((const bf16_t*)wg, (const bf16_t*)wu, H, (bf16_t*)out);
    else
        pack_gate_up_kernel<float><<<2 * F, 256, 0, st>>>((const float*)wg, (const float*)wu, H, (float*)out);
    return hipGetLastError();
}

}  // namespace vlm
