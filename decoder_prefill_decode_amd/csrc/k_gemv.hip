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
#include <stdlib.h>

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

// Latency-hiding variant used when K fits the register plan. Lane l of a
// wavefront owns the elements k = l*VEC + c*64*VEC (+0..VEC-1) of every row
// it reads. Requests go out in the order operand vector, weights, old output
// (for a residual update); vector-memory loads complete in issue order, so
// the operand is prepared while the weight stream is still in flight.
//  * Plain operand (a bf16/fp32 row): each lane loads the vector at its own
//    positions, so the wavefront needs no LDS and no barrier.
//  * RMSNorm operand (fp32 x and a gain): the block loads x once, reduces the
//    sum of squares and writes the normalised, rounded row into LDS (a
//    per-lane copy would cost 12 registers per chunk and halve occupancy).
// Every load is unconditional (indices are clamped into range, out-of-range
// lanes are masked afterwards) and raw data is converted only after the last
// request: a load under a branch, or arithmetic between loads, makes the
// compiler wait for a memory round trip before the next request.

// Four gain values in their storage type, raw.
template <class T> struct Raw4;
template <> struct Raw4<float> {
    u32x4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ float get(int e) const { return __uint_as_float(v[e]); }
};
template <> struct Raw4<bf16_t> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = e < 2 ? v.x : v.y;
        return __uint_as_float(e % 2 ? (w & 0xffff0000u) : (w << 16));
    }
};

//  * PlainLds operand: a plain vector staged once per block into LDS (raw
//    16-byte chunks), so the four wavefronts of a block share one read of it;
//    with long rows a per-lane copy would double the L2 traffic of the GEMV.
//  * NW wavefronts per block (4, or 5 where that gives every CU the same
//    number of blocks).
template <class T, Pro PRO, Epi EPI, int NR, int KCH, int NW>
__global__ __launch_bounds__(NW * 64) void gemv2_kernel(GemvArgs a) {
    constexpr int VEC = 16 / sizeof(T), STEP = kWave * VEC, BT = NW * kWave;
    constexpr bool NORM = PRO == Pro::RmsNorm, SHARE = PRO == Pro::PlainLds, STAGED = NORM || SHARE;
    constexpr int VCH = NORM ? (KCH * STEP / 4 + BT - 1) / BT : 1;  // 4-float chunks of x per thread
    constexpr int SCH = SHARE ? (KCH * kWave + BT - 1) / BT : 1;     // 16-byte operand chunks per thread
    extern __shared__ __attribute__((aligned(16))) float vs[];  // 16-byte aligned: PlainLds reads u32x4
    __shared__ float red[NW];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = blockIdx.x * NW + tid / kWave;
    const int K = a.K;
    const T* W = (const T*)a.W;

    // (1) operand: RMSNorm -> this thread's chunks of x and gain; Plain -> this lane's slice;
    // PlainLds -> this thread's share of the vector
    u32x4 xr[NORM ? VCH : (SHARE ? SCH : KCH)];
    Raw4<T> gr[VCH];
    if constexpr (SHARE) {
        const int nch = K / VEC;
#pragma unroll
        for (int i = 0; i < SCH; i++)
            xr[i] = *reinterpret_cast<const u32x4*>((const T*)a.vec + VEC * min(tid + BT * i, nch - 1));
    } else if constexpr (NORM) {
        const int nx = K / 4;
#pragma unroll
        for (int i = 0; i < VCH; i++) {
            const int c = min(tid + BT * i, nx - 1);
            xr[i] = *reinterpret_cast<const u32x4*>((const float*)a.vec + 4 * c);
            gr[i].load((const T*)a.gain + 4 * c);
        }
    } else {
#pragma unroll
        for (int c = 0; c < KCH; c++) {
            const int k = lane * VEC + c * STEP;
            xr[c] = *reinterpret_cast<const u32x4*>((const T*)a.vec + (k < K ? k : 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the operand requests ahead of the weight stream
    // (2) weight rows of this wavefront
    int rows[NR];
    if constexpr (EPI == Epi::SwiGLU) {
        const int nout = a.N / 2;
#pragma unroll
        for (int r = 0; r < NR / 2; r++) {
            int o = wave * (NR / 2) + r;
            o = o < nout ? o : nout - 1;
            rows[r] = 64 * (o / 32) + (o % 32);
            rows[NR / 2 + r] = rows[r] + 32;
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int n = wave * NR + r;
            rows[r] = n < a.N ? n : a.N - 1;
        }
    }
    u32x4 wr[NR][KCH];
#pragma unroll
    for (int c = 0; c < KCH; c++) {
        const int k = lane * VEC + c * STEP;
        const int kk = k < K ? k : 0;
#pragma unroll
        for (int r = 0; r < NR; r++) wr[r][c] = *reinterpret_cast<const u32x4*>(W + (size_t)rows[r] * K + kk);
    }
    // (2b) the value a residual update adds to: lane r holds row wave*NR + r
    float old = 0.f;
    if constexpr (EPI == Epi::Resid) {
        const int n = min(wave * NR + min(lane, NR - 1), a.N - 1);
        old = ((const float*)a.out)[n];
    }
    __builtin_amdgcn_sched_barrier(0);  // no arithmetic is hoisted between the requests
    // (3) RMSNorm: normalised, rounded row into LDS
    if constexpr (NORM) {
        const int nx = K / 4;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < VCH; i++)
            if (tid + BT * i < nx)
#pragma unroll
                for (int e = 0; e < 4; e++) ss += __uint_as_float(xr[i][e]) * __uint_as_float(xr[i][e]);
        const float rs = rsqrtf(block_sum<BT>(ss, red) / (float)K + a.eps);
#pragma unroll
        for (int i = 0; i < VCH; i++) {
            const int c = tid + BT * i;
            if (c < nx)
#pragma unroll
                for (int e = 0; e < 4; e++) vs[4 * c + e] = Elt<T>::rnd(__uint_as_float(xr[i][e]) * rs * gr[i].get(e));
        }
        __syncthreads();
    } else if constexpr (SHARE) {
        u32x4* vq = reinterpret_cast<u32x4*>(vs);
        const int nch = K / VEC;
#pragma unroll
        for (int i = 0; i < SCH; i++)
            if (tid + BT * i < nch) vq[tid + BT * i] = xr[i];
        __syncthreads();
    }
    // (4) dot products
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; r++) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; c++) {
        const int k = lane * VEC + c * STEP;
        if (k < K) {
            float h[VEC];
            if constexpr (NORM) {
#pragma unroll
                for (int e = 0; e < VEC; e++) h[e] = vs[k + e];
            } else if constexpr (SHARE) {
                unpack16(reinterpret_cast<const u32x4*>(vs)[k / VEC], (const T*)nullptr, h);
            } else {
                unpack16(xr[c], (const T*)nullptr, h);
            }
#pragma unroll
            for (int r = 0; r < NR; r++) {
                float wf[VEC];
                unpack16(wr[r][c], (const T*)nullptr, wf);
#pragma unroll
                for (int e = 0; e < VEC; e++) acc[r] = fmaf(wf[e], h[e], acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; r++) acc[r] = wave_sum(acc[r]);
    // (5) epilogue: lane r stores row r
    if constexpr (EPI == Epi::Argmax) {
        __shared__ unsigned long long bk[NW];
        unsigned long long best = 0ull;
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int n = wave * NR + r;
            if (n < a.N) {
                const float v = acc[r];
                const unsigned long long key = isfinite(v)
                    ? (((unsigned long long)ordered_key(v)) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n)
                    : ~0ull;
                best = key > best ? key : best;
                if (a.out && lane == r) ((float*)a.out)[n] = v;
            }
        }
        if (lane == 0) bk[tid / kWave] = best;
        __syncthreads();
        if (tid == 0) {
            unsigned long long b = bk[0];
            for (int i = 1; i < NW; i++) b = bk[i] > b ? bk[i] : b;
            a.partials[blockIdx.x] = b;
        }
    } else if constexpr (EPI == Epi::SwiGLU) {
#pragma unroll
        for (int r = 0; r < NR / 2; r++) {
            const int o = wave * (NR / 2) + r;
            if (lane == r && o < a.N / 2) Elt<T>::st((T*)a.out, o, silu_f(acc[r]) * acc[NR / 2 + r]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int n = wave * NR + r;
            if (lane == r && n < a.N) {
                float* o = (float*)a.out;
                if constexpr (EPI == Epi::Resid)
                    o[n] = old + acc[r];
                else
                    o[n] = acc[r];
            }
        }
    }
}

static int device_cus() {
    static int v = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 256;
        return n > 0 ? n : 256;
    }();
    return v;
}

// Share of the CU slots the busiest CU's blocks fill: blocks / (cus * ceil(blocks / cus)).
static double cu_balance(int blocks, int cus) {
    const int rounds = (blocks + cus - 1) / cus;
    return rounds > 0 ? (double)blocks / ((double)rounds * cus) : 0.0;
}

// VLM_GEMV_WAVES (4 or 5) fixes the wavefronts per block of the plain-operand
// projections, for tuning; unset or 0 lets the balance decide.
static int gemv_waves_override() {
    static int v = [] {
        const char* e = getenv("VLM_GEMV_WAVES");
        return e ? atoi(e) : 0;
    }();
    return v;
}

template <class T, Pro PRO, Epi EPI, int NR, int KCH, int NW>
static hipError_t launch_gemv2(const GemvArgs& a, int waves, hipStream_t st) {
    const int blocks = (waves + NW - 1) / NW;
    const size_t smem = PRO == Pro::RmsNorm ? (size_t)a.K * sizeof(float)
                        : (PRO == Pro::PlainLds ? (size_t)a.K * sizeof(T) : 0);
    gemv2_kernel<T, PRO, EPI, NR, KCH, NW><<<blocks, NW * kWave, smem, st>>>(a);
    return hipGetLastError();
}

// Blocks of 4 wavefronts, or of 5 for the plain-operand row projections when
// that spreads the blocks evenly over the CUs (a CU holding one block more
// than the others streams that block's rows after the rest have finished).
// The argmax head keeps 4 (its block partials are counted in 4-wavefront
// blocks) and the RMSNorm prologues keep 4 (the block sum's order).
template <class T, Pro PRO, Epi EPI, int NR, int KCH>
static hipError_t run_gemv2(const GemvArgs& a, hipStream_t st) {
    const int nrows = a.N;  // SwiGLU: NR counts gate + up rows
    const int waves = (nrows + NR - 1) / NR;
    if constexpr (PRO != Pro::RmsNorm && (EPI == Epi::Resid || EPI == Epi::StoreF32)) {
        const int cus = device_cus(), ov = gemv_waves_override();
        const bool five = ov ? ov == 5
                             : cu_balance((waves + 4) / 5, cus) > cu_balance((waves + 3) / 4, cus) + 0.05;
        if (five) return launch_gemv2<T, PRO, EPI, NR, KCH, 5>(a, waves, st);
    }
    return launch_gemv2<T, PRO, EPI, NR, KCH, 4>(a, waves, st);
}

// VLM_GEMV_ROWS (1, 2, 4 or 8) fixes the rows per wavefront of the decode
// projections, for tuning; unset or 0 keeps the choice below.
// Plain operands of at least this many 16-byte chunks per lane are staged in
// LDS (Pro::PlainLds); VLM_GEMV_SHARE overrides it for tuning (0 = never).
// Measured: the 36-layer stack's down projection (19 chunks) 11.7 -> 10.8 us,
// the 28-layer stack's O projection (4 chunks) 3.2 -> 3.0 us.
static int share_min_chunks() {
    static int v = [] {
        const char* e = getenv("VLM_GEMV_SHARE");
        return e ? atoi(e) : 4;
    }();
    return v;
}

static int gemv_rows_override() {
    static int v = [] {
        const char* e = getenv("VLM_GEMV_ROWS");
        return e ? atoi(e) : 0;
    }();
    return v;
}

// Rows per wavefront: as many as the register plan allows (NR*KCH <= 24 chunks)
// while keeping >= 1024 wavefronts in flight.
template <class T, Pro PRO, Epi EPI, int KCH>
static hipError_t pick_nr(const GemvArgs& a, hipStream_t st) {
    // the RMSNorm operand is staged with at most 12 chunks per thread: wider rows take the generic path
    if constexpr (PRO == Pro::RmsNorm && KCH > 12) {
        return hipErrorNotSupported;
    } else {
        if constexpr (PRO == Pro::Plain)
            if (share_min_chunks() > 0 && KCH >= share_min_chunks()) return pick_nr<T, Pro::PlainLds, EPI, KCH>(a, st);
        constexpr int cap = 24 / KCH;
        const int n = a.N;
        switch (gemv_rows_override()) {  // tuning override: rows per wavefront, if the plan allows it
            case 8: if constexpr (cap >= 8) return run_gemv2<T, PRO, EPI, 8, KCH>(a, st); break;
            case 4: if constexpr (cap >= 4) return run_gemv2<T, PRO, EPI, 4, KCH>(a, st); break;
            case 2: if constexpr (cap >= 2) return run_gemv2<T, PRO, EPI, 2, KCH>(a, st); break;
            case 1: if constexpr (EPI != Epi::SwiGLU) return run_gemv2<T, PRO, EPI, 1, KCH>(a, st); break;
        }
        // SwiGLU: one gate and one up row per wavefront (the 36-layer stack's gate/up 18.1 -> 17.8 us
        // against two of each; decode 451.4 -> 448.6 ms per 256 tokens)
        if constexpr (EPI == Epi::SwiGLU && cap >= 2) return run_gemv2<T, PRO, EPI, 2, KCH>(a, st);
        if constexpr (cap >= 8) if (n / 8 >= 1024) return run_gemv2<T, PRO, EPI, 8, KCH>(a, st);
        if constexpr (cap >= 4) if (n / 4 >= 1024) return run_gemv2<T, PRO, EPI, 4, KCH>(a, st);
        if constexpr (cap >= 2) if (n / 2 >= 1024) return run_gemv2<T, PRO, EPI, 2, KCH>(a, st);
        if constexpr (EPI != Epi::SwiGLU) return run_gemv2<T, PRO, EPI, 1, KCH>(a, st);
        return hipErrorNotSupported;
    }
}

// Returns hipErrorNotSupported when K has no register plan (caller falls back).
template <class T, Pro PRO, Epi EPI>
static hipError_t try_gemv2(const GemvArgs& a, hipStream_t st) {
    constexpr int VEC = 16 / sizeof(T);
    const int kch = (a.K + kWave * VEC - 1) / (kWave * VEC);
    switch (kch) {
        case 1: return pick_nr<T, PRO, EPI, 1>(a, st);
        case 2: return pick_nr<T, PRO, EPI, 2>(a, st);
        case 3: return pick_nr<T, PRO, EPI, 3>(a, st);
        case 4: return pick_nr<T, PRO, EPI, 4>(a, st);
        case 5: return pick_nr<T, PRO, EPI, 5>(a, st);
        case 6: return pick_nr<T, PRO, EPI, 6>(a, st);
        case 8: return pick_nr<T, PRO, EPI, 8>(a, st);
        case 12: return pick_nr<T, PRO, EPI, 12>(a, st);
        case 19: return pick_nr<T, PRO, EPI, 19>(a, st);
        case 20: return pick_nr<T, PRO, EPI, 20>(a, st);
    }
    return hipErrorNotSupported;
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
    {
        const hipError_t e = try_gemv2<T, PRO, EPI>(a, st);
        if (e != hipErrorNotSupported) return e;
    }
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
        if (kv_len) {  // kv_len: the cache header (word 0 length, 1 non-finite flag, 2 its first position)
            const int t = kv_len[0];
            if (tok >= 0) {
                if (hist) hist[t + 1] = tok;
                kv_len[0] = t + 1;
            } else if (kv_len[1] == 0) {  // not committed: the length stays at t
                kv_len[1] = 1;
                kv_len[2] = t;
            }
        }
    }
}

// Row-wise argmax of a logits matrix (the multi-token verify head) in two launches, with the
// u64 keys of the lm_head (largest logit, lowest index; ~0 for a non-finite value, which wins and
// gives -1): block (b, r) scans piece b of row r, `piece` consecutive entries (a multiple of 4),
// and writes its best key to part[r * gridDim.x + b]; one wavefront per row then takes the
// largest of the row's keys. (One block per row left 8 CUs to scan a 128256-entry row each:
// 16.6 us for 8 rows.) Each thread requests U 16-byte chunks (indices clamped) before it
// compares any of them.
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
    return isfinite(v) ? (((unsigned long long)ordered_key(v)) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n)
                       : ~0ull;
}

__global__ __launch_bounds__(256) void argmax_rows_part_kernel(const float* __restrict__ logits, int V, int ld,
                                                               int piece, unsigned long long* __restrict__ part) {
    constexpr int U = 4, NT = 256;
    __shared__ unsigned long long sm[NT / kWave];
    const float* row = logits + (size_t)blockIdx.y * ld;
    const int tid = threadIdx.x, n0 = blockIdx.x * piece, n1 = min(V, n0 + piece);
    unsigned long long best = 0ull;  // below every key
    int tail = n0;                   // first element the scalar loop covers
    if (n1 > n0 && (reinterpret_cast<uintptr_t>(row + n0) & 15) == 0) {
        const int nv = (n1 - n0) / 4;
        const float* base = row + n0;
        for (int c0 = 0; c0 < nv; c0 += NT * U) {
            f32x4 r[U];
#pragma unroll
            for (int u = 0; u < U; u++)
                r[u] = *reinterpret_cast<const f32x4*>(base + 4 * (size_t)min(c0 + tid + NT * u, nv - 1));
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = c0 + tid + NT * u;
                if (c < nv)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const unsigned long long key = argmax_key(r[u][e], n0 + 4 * c + e);
                        best = key > best ? key : best;
                    }
            }
        }
        tail = n0 + 4 * nv;
    }
    for (int n = tail + tid; n < n1; n += NT) {
        const unsigned long long key = argmax_key(row[n], n);
        best = key > best ? key : best;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off);
        best = o > best ? o : best;
    }
    if (tid % kWave == 0) sm[tid / kWave] = best;
    __syncthreads();
    if (tid == 0) {
        unsigned long long b = sm[0];
#pragma unroll
        for (int i = 1; i < NT / kWave; i++) b = sm[i] > b ? sm[i] : b;
        part[(size_t)blockIdx.y * gridDim.x + blockIdx.x] = b;
    }
}

__global__ __launch_bounds__(64) void argmax_rows_final_kernel(const unsigned long long* __restrict__ part, int nb,
                                                               int32_t* __restrict__ out) {
    const int lane = threadIdx.x;
    unsigned long long best = lane < nb ? part[(size_t)blockIdx.x * nb + lane] : 0ull;
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off);
        best = o > best ? o : best;
    }
    if (lane == 0) out[blockIdx.x] = best == ~0ull ? -1 : (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
}

int argmax_rows_pieces(int V) { return V / 2048 < 1 ? 1 : (V / 2048 > 32 ? 32 : V / 2048); }

hipError_t launch_argmax_rows(const float* logits, int S, int V, int ld, int32_t* out, unsigned long long* part,
                              hipStream_t st) {
    if (S <= 0) return hipSuccess;
    const int nb = argmax_rows_pieces(V);
    const int piece = 4 * ((V + 4 * nb - 1) / (4 * nb));
    argmax_rows_part_kernel<<<dim3(nb, S), 256, 0, st>>>(logits, V, ld, piece, part);
    argmax_rows_final_kernel<<<S, kWave, 0, st>>>(part, nb, out);
    return hipGetLastError();
}

int lmhead_blocks(int V) { return (V + 4 * kLmRows - 1) / (4 * kLmRows); }

template <class T, int NR, int KCH>
static hipError_t run_lm2(const GemvArgs& a, int* nblocks, hipStream_t st) {
    *nblocks = (((a.N + NR - 1) / NR) + 3) / 4;
    return run_gemv2<T, Pro::RmsNorm, Epi::Argmax, NR, KCH>(a, st);
}

// lm_head on the latency-hiding GEMV; hipErrorNotSupported when K has no register plan.
template <class T>
static hipError_t lm2_dispatch(const GemvArgs& a, int* nb, hipStream_t st) {
    constexpr int VEC = 16 / sizeof(T);
    const int kch = (a.K + kWave * VEC - 1) / (kWave * VEC);
    // rows per wavefront (measured: the 28-layer stack's 151936 x 1024 table 48.7 -> 47.8 us with 4
    // rows instead of 8; the 36-layer stack's 128256 x 2560 table gains nothing in the decode from 2)
    switch (kch) {
        case 1: return run_lm2<T, 8, 1>(a, nb, st);
        case 2: return run_lm2<T, 4, 2>(a, nb, st);
        case 3: return run_lm2<T, 8, 3>(a, nb, st);
        case 4: return run_lm2<T, 4, 4>(a, nb, st);
        case 5: return run_lm2<T, 4, 5>(a, nb, st);
        case 6: return run_lm2<T, 4, 6>(a, nb, st);
        case 8: return run_lm2<T, 2, 8>(a, nb, st);
        case 12: return run_lm2<T, 2, 12>(a, nb, st);
    }
    return hipErrorNotSupported;
}

int lmhead_partials_max(int V) { return (V + 3) / 4 + 1; }

hipError_t launch_lmhead_argmax(int dtype, const void* table, const float* x, const void* gain, float eps, int V,
                                int K, unsigned long long* partials, float* logits, int32_t* token_out, int32_t* hist,
                                int32_t* kv_len, hipStream_t st) {
    GemvArgs a{};
    a.W = table; a.vec = x; a.gain = gain; a.eps = eps; a.out = logits; a.N = V; a.K = K; a.partials = partials;
    int nb = 0;
    hipError_t e = dtype == 1 ? lm2_dispatch<bf16_t>(a, &nb, st) : lm2_dispatch<float>(a, &nb, st);
    if (e == hipErrorNotSupported) {
        e = launch_lmhead(dtype, table, x, gain, eps, V, K, partials, logits, st);
        nb = lmhead_blocks(V);
    }
    if (e != hipSuccess) return e;
    if (token_out) return launch_argmax_final(partials, nb, token_out, hist, kv_len, st);
    return hipSuccess;
}

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
