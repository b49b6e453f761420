// Decode-step projections (one row against a weight matrix) and the fused
// lm_head + greedy argmax.
//
// Decode moves every weight byte once per token and is bandwidth-bound
// (MNN llm_demo Omni article §6.1: more threads slowed decode through
// bandwidth contention); the lm_head is one [V][H] table read as a GEMV with
// only the argmax kept (Youtu-VL-4B ncnn port, 实现流程 §6; HunyuanOCR v1.5
// ncnn port §3.4).
//
// Layout on gfx950: the input row is normalised once per block into LDS
// (fused RMSNorm prologue, rounded to the operand type); each 64-lane
// wavefront owns ROWS weight rows and streams them with 16-byte loads, lane l
// covering elements l*VEC + i*64*VEC, so one wavefront instruction reads 1 KiB
// of contiguous row. Several rows and two K strides per iteration keep enough
// loads in flight to cover HBM latency.
#include "common.hpp"
#include "internal.hpp"

namespace vlm {

template <class T> struct GvTraits { static constexpr int VEC = 16 / sizeof(T); };

// Fills vs[0..K) with the operand row: RMSNorm of fp32 x with gain g (rounded
// to T), or a plain T vector widened to float.
template <class T, Pro PRO>
__device__ __forceinline__ void load_vec(const GemvArgs& a, float* vs, float* red) {
    const int K = a.K;
    if constexpr (PRO == Pro::RmsNorm) {
        const float* x = (const float*)a.vec;
        float ss = 0.f;
        for (int k = threadIdx.x; k < K; k += 256) {
            const float v = x[k];
            ss += v * v;
        }
        const float r = rsqrtf(block_sum<256>(ss, red) / (float)K + a.eps);
        const T* g = (const T*)a.gain;
        for (int k = threadIdx.x; k < K; k += 256) vs[k] = Elt<T>::rnd(x[k] * r * Elt<T>::ld(g, k));
    } else {
        const T* v = (const T*)a.vec;
        for (int k = threadIdx.x; k < K; k += 256) vs[k] = Elt<T>::ld(v, k);
    }
    __syncthreads();
}

// Dot products of NR weight rows with vs; every lane returns the full sums.
template <class T, int NR>
__device__ __forceinline__ void rows_dot(const T* W, const int* rows, int K, const float* vs, float* acc) {
    constexpr int VEC = GvTraits<T>::VEC, STEP = kWave * VEC;
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int r = 0; r < NR; r++) acc[r] = 0.f;
    int k = lane * VEC;
    for (; k + STEP < K; k += 2 * STEP) {
        float w0[NR][VEC], w1[NR][VEC];
#pragma unroll
        for (int r = 0; r < NR; r++) {
            ld16(W + (size_t)rows[r] * K + k, w0[r]);
            ld16(W + (size_t)rows[r] * K + k + STEP, w1[r]);
        }
#pragma unroll
        for (int i = 0; i < VEC; i++) {
            const float v0 = vs[k + i], v1 = vs[k + STEP + i];
#pragma unroll
            for (int r = 0; r < NR; r++) acc[r] = fmaf(w0[r][i], v0, fmaf(w1[r][i], v1, acc[r]));
        }
    }
    if (k < K) {
        float w0[NR][VEC];
#pragma unroll
        for (int r = 0; r < NR; r++) ld16(W + (size_t)rows[r] * K + k, w0[r]);
#pragma unroll
        for (int i = 0; i < VEC; i++) {
            const float v0 = vs[k + i];
#pragma unroll
            for (int r = 0; r < NR; r++) acc[r] = fmaf(w0[r][i], v0, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < NR; r++) acc[r] = wave_sum(acc[r]);
}

template <class T, Pro PRO, Epi EPI, int ROWS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    extern __shared__ float vs[];
    __shared__ float red[4];
    load_vec<T, PRO>(a, vs, red);
    const int wave = blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const T* W = (const T*)a.W;
    if constexpr (EPI == Epi::SwiGLU) {
        // output features o = wave*ROWS + r: gate row 64*(o/32) + o%32, up row +32
        const int nout = a.N / 2;
        int rows[2 * ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            int o = wave * ROWS + r;
            o = o < nout ? o : nout - 1;
            rows[r] = 64 * (o / 32) + (o % 32);
            rows[ROWS + r] = rows[r] + 32;
        }
        float acc[2 * ROWS];
        rows_dot<T, 2 * ROWS>(W, rows, a.K, vs, acc);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int o = wave * ROWS + r;
            if (lane == r && o < nout) Elt<T>::st((T*)a.out, o, silu_f(acc[r]) * acc[ROWS + r]);
        }
    } else {
        int rows[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int n = wave * ROWS + r;
            rows[r] = n < a.N ? n : a.N - 1;
        }
        float acc[ROWS];
        rows_dot<T, ROWS>(W, rows, a.K, vs, acc);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int n = wave * ROWS + r;
            if (lane == r && n < a.N) {
                float* o = (float*)a.out;
                if constexpr (EPI == Epi::Resid)
                    o[n] += acc[r];
                else
                    o[n] = acc[r];
            }
        }
    }
}

template <class T, Pro PRO, Epi EPI, int ROWS>
static hipError_t run_gemv(const GemvArgs& a, hipStream_t st) {
    const int nrows = EPI == Epi::SwiGLU ? a.N / 2 : a.N;
    const int waves = (nrows + ROWS - 1) / ROWS;
    const int blocks = (waves + 3) / 4;
    const size_t smem = (size_t)a.K * sizeof(float);  // <= 64 KiB: K <= 16384 is checked by the caller
    gemv_kernel<T, PRO, EPI, ROWS><<<blocks, 256, smem, st>>>(a);
    return hipGetLastError();
}

template <class T, Pro PRO, Epi EPI>
static hipError_t pick_rows(const GemvArgs& a, hipStream_t st) {
    const int nrows = EPI == Epi::SwiGLU ? a.N / 2 : a.N;
    if (nrows >= 8192) return run_gemv<T, PRO, EPI, 4>(a, st);
    if (nrows >= 4096) return run_gemv<T, PRO, EPI, 2>(a, st);
    return run_gemv<T, PRO, EPI, 1>(a, st);
}

template <class T>
static hipError_t gemv_dispatch(Pro pro, Epi epi, const GemvArgs& a, hipStream_t st) {
    if (pro == Pro::RmsNorm) {
        if (epi == Epi::StoreF32) return pick_rows<T, Pro::RmsNorm, Epi::StoreF32>(a, st);
        if (epi == Epi::SwiGLU) return pick_rows<T, Pro::RmsNorm, Epi::SwiGLU>(a, st);
    } else {
        if (epi == Epi::Resid) return pick_rows<T, Pro::Plain, Epi::Resid>(a, st);
        if (epi == Epi::StoreF32) return pick_rows<T, Pro::Plain, Epi::StoreF32>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int dtype, Pro pro, Epi epi, const GemvArgs& a, hipStream_t st) {
    if (a.N <= 0) return hipSuccess;
    return dtype == 1 ? gemv_dispatch<bf16_t>(pro, epi, a, st) : gemv_dispatch<float>(pro, epi, a, st);
}

// ---------------------------------------------------------------- lm_head + argmax
// Argmax key: (ordered(logit) << 32) | (0xffffffff - index), so the u64
// maximum is the largest logit with the lowest index; any non-finite logit
// makes the block key all-ones, which the final reduction reports as -1.
constexpr int kLmRows = 4;  // rows per wavefront

template <class T>
__global__ __launch_bounds__(256) void lmhead_kernel(const T* __restrict__ table, const float* __restrict__ x,
                                                     const T* __restrict__ gain, float eps, int V, int K,
                                                     unsigned long long* __restrict__ partials,
                                                     float* __restrict__ logits) {
    extern __shared__ float vs[];
    __shared__ float red[4];
    __shared__ unsigned long long bk[4];
    GemvArgs a;
    a.vec = x; a.gain = gain; a.eps = eps; a.K = K;
    load_vec<T, Pro::RmsNorm>(a, vs, red);
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wave = blockIdx.x * 4 + w;
    int rows[kLmRows];
#pragma unroll
    for (int r = 0; r < kLmRows; r++) {
        const int n = wave * kLmRows + r;
        rows[r] = n < V ? n : V - 1;
    }
    float acc[kLmRows];
    rows_dot<T, kLmRows>(table, rows, K, vs, acc);
    unsigned long long best = 0ull;
#pragma unroll
    for (int r = 0; r < kLmRows; r++) {
        const int n = wave * kLmRows + r;
        if (n < V) {
            const float v = acc[r];
            const unsigned long long key = isfinite(v)
                ? (((unsigned long long)ordered_key(v)) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n)
                : ~0ull;
            best = key > best ? key : best;
            if (logits && lane == r) logits[n] = v;
        }
    }
    if (lane == 0) bk[w] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long b = bk[0];
        for (int i = 1; i < 4; i++) b = bk[i] > b ? bk[i] : b;
        partials[blockIdx.x] = b;
    }
}

__global__ __launch_bounds__(1024) void argmax_final_kernel(const unsigned long long* __restrict__ partials, int n,
                                                            int32_t* token_out, int32_t* hist, int32_t* kv_len) {
    __shared__ unsigned long long sm[1024];
    unsigned long long b = 0ull;
    for (int i = threadIdx.x; i < n; i += 1024) b = partials[i] > b ? partials[i] : b;
    sm[threadIdx.x] = b;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s && sm[threadIdx.x + s] > sm[threadIdx.x]) sm[threadIdx.x] = sm[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const unsigned long long best = sm[0];
        const int32_t tok = best == ~0ull ? -1 : (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        token_out[0] = tok;
        if (kv_len) {
            const int t = kv_len[0];
            if (hist) hist[t + 1] = tok;
            kv_len[0] = t + 1;
        }
    }
}

int lmhead_blocks(int V) { return (V + 4 * kLmRows - 1) / (4 * kLmRows); }

hipError_t launch_lmhead(int dtype, const void* table, const float* x, const void* gain, float eps, int V, int K,
                         unsigned long long* partials, float* logits, hipStream_t st) {
    const int blocks = lmhead_blocks(V);
    const size_t smem = (size_t)K * sizeof(float);
    if (dtype == 1)
        lmhead_kernel<bf16_t><<<blocks, 256, smem, st>>>((const bf16_t*)table, x, (const bf16_t*)gain, eps, V, K,
                                                         partials, logits);
    else
        lmhead_kernel<float><<<blocks, 256, smem, st>>>((const float*)table, x, (const float*)gain, eps, V, K,
                                                        partials, logits);
    return hipGetLastError();
}

hipError_t launch_argmax_final(const unsigned long long* partials, int nblocks, int32_t* token_out, int32_t* hist,
                               int32_t* kv_len, hipStream_t st) {
    argmax_final_kernel<<<1, 1024, 0, st>>>(partials, nblocks, token_out, hist, kv_len);
    return hipGetLastError();
}

}  // namespace vlm
