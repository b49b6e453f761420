// Prefill projections on the matrix cores: C[M][N] = A[M][K] * W[N][K]^T with
// fused epilogues (residual add, SwiGLU over 32-row interleaved gate/up
// groups, bias + GELU, bias + row-remapped store). These are the decoder
// matmuls that dominate prefill (MNN llm_demo Omni article §5.3; HunyuanOCR
// v1.5 ncnn port §5).
//
// gfx950 tiling: 256 threads = 4 wavefronts in a 2x2 grid, each owning a
// (BM/2) x (BN/2) sub-tile built from 32x32 MFMA blocks:
//   bf16: v_mfma_f32_32x32x16_bf16, 64-element K stage;
//   f32:  v_mfma_f32_32x32x2f32,   32-element K stage.
// Both operands are K-contiguous, so every lane feeds the MFMA from one
// 16-byte LDS read (bf16) or one 4-byte read (f32). LDS is double-buffered
// and the next stage's global loads are in flight during the current stage's
// MFMAs. Blocks are remapped so that consecutive output tiles (which share a
// weight panel) land on the same XCD and its L2.
#include <stdlib.h>

#include "common.hpp"
#include "internal.hpp"

namespace vlm {

template <class T> struct GemmTraits;
template <> struct GemmTraits<bf16_t> { static constexpr int BK = 64, VEC = 8, PAD = 8; };
template <> struct GemmTraits<float>  { static constexpr int BK = 32, VEC = 4, PAD = 4; };

__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int q = n / 8;
    if (b < 8 * q) return (b % 8) * q + b / 8;
    return b;
}

template <class T, int BM, int BN, Epi EPI, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    using Tr = GemmTraits<T>;
    constexpr int BK = Tr::BK, VEC = Tr::VEC, LDK = BK + Tr::PAD;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int CPR = BK / VEC;                    // 16-byte chunks per tile row
    constexpr int ACH = BM * CPR / 256, BCH = BN * CPR / 256;
    static_assert(ACH >= 1 && BCH >= 1, "tile too small");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* smem = reinterpret_cast<T*>(smem_raw);
    T* As[2] = {smem, smem + (BM + BN) * LDK};
    T* Bs[2] = {smem + BM * LDK, smem + (BM + BN) * LDK + BM * LDK};

    const int M = a.M, N = a.N, K = a.K;
    const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
    const int tile = xcd_remap(blockIdx.x, mt * nt);
    const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int wm = w / 2, wn = w % 2, h = lane / 32, l32 = lane % 32;
    const T* A = (const T*)a.A;
    const T* B = (const T*)a.B;

    u32x4 ra[ACH], rb[BCH];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < ACH; i++) {
            const int c = tid + 256 * i, r = c / CPR, k = k0 + (c % CPR) * VEC;
            const int gm = m0 + r;
            ra[i] = (gm < M && k < K) ? *reinterpret_cast<const u32x4*>(A + (size_t)gm * K + k) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < BCH; i++) {
            const int c = tid + 256 * i, r = c / CPR, k = k0 + (c % CPR) * VEC;
            const int gn = n0 + r;
            rb[i] = (gn < N && k < K) ? *reinterpret_cast<const u32x4*>(B + (size_t)gn * K + k) : u32x4{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH; i++) {
            const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
            *reinterpret_cast<u32x4*>(As[buf] + r * LDK + kc) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; i++) {
            const int c = tid + 256 * i, r = c / CPR, kc = (c % CPR) * VEC;
            *reinterpret_cast<u32x4*>(Bs[buf] + r * LDK + kc) = rb[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // split-K: blockIdx.y selects a contiguous range of K stages
    int kt0 = 0, nk = (K + BK - 1) / BK;
    if constexpr (SPLIT) {
        const int per = (nk + gridDim.y - 1) / gridDim.y;
        kt0 = blockIdx.y * per;
        nk = max(0, min(nk, kt0 + per) - kt0);
    }
    gload(kt0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt0 + kt + 1);
        const T* as = As[cur] + (wm * WM + l32) * LDK;
        const T* bs = Bs[cur] + (wn * WN + l32) * LDK;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; i++)
                    fa[i] = *reinterpret_cast<const bf16x8*>(as + i * 32 * LDK + kk * 16 + h * 8);
#pragma unroll
                for (int j = 0; j < TN; j++)
                    fb[j] = *reinterpret_cast<const bf16x8*>(bs + j * 32 * LDK + kk * 16 + h * 8);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 2; kk++) {
                float fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; i++) fa[i] = as[i * 32 * LDK + kk * 2 + h];
#pragma unroll
                for (int j = 0; j < TN; j++) fb[j] = bs[j * 32 * LDK + kk * 2 + h];
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue. C layout of a 32x32 block: lane owns column l32 and rows
    // (r/4)*8 + h*4 + r%4, r = 0..15.
    const T* bias = (const T*)a.bias;
    if constexpr (SPLIT) {  // raw partial sums; splitk_reduce_kernel applies the epilogue
        float* part = a.part + (size_t)blockIdx.y * M * N;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = n0 + wn * WN + j * 32 + l32;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
                    if (m < M) part[(size_t)m * N + n] = acc[i][j][r];
                }
        }
    } else if constexpr (EPI == Epi::SwiGLU) {
        static_assert(TN == 2, "SwiGLU needs a 64-column wave tile (gate block, up block)");
        const int ncol = (n0 + wn * WN) / 2 + l32;
        T* out = (T*)a.out;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
                if (m < M && n0 + wn * WN < N) {  // N = 2F is a multiple of 64: whole groups
                    const float gt = acc[i][0][r], up = acc[i][1][r];
                    Elt<T>::st(out, (size_t)m * a.ldo + ncol, silu_f(gt) * up);
                }
            }
    } else {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = n0 + wn * WN + j * 32 + l32;
            if (n >= N) continue;
            const float bn = bias ? Elt<T>::ld(bias, n) : 0.f;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
                    if (m >= M) continue;
                    const float v = acc[i][j][r] + bn;
                    if constexpr (EPI == Epi::StoreF32) {
                        ((float*)a.out)[(size_t)m * a.ldo + n] = v;
                    } else if constexpr (EPI == Epi::Resid) {
                        float* x = (float*)a.out + (size_t)m * a.ldo + n;
                        *x = *x + v;
                    } else if constexpr (EPI == Epi::Gelu) {
                        Elt<T>::st((T*)a.out, (size_t)m * a.ldo + n, gelu_tanh_f(v));
                    } else {  // StoreRowMap
                        ((float*)a.out)[(size_t)a.rowmap[m] * a.ldo + n] = v;
                    }
                }
        }
    }
}

// Sums the split partials in split order (deterministic) and applies the epilogue.
template <class T, Epi EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, int splits) {
    const int M = a.M, N = a.N;
    const size_t MN = (size_t)M * N;
    const T* bias = (const T*)a.bias;
    const int nout = EPI == Epi::SwiGLU ? N / 2 : N;
    const size_t total = (size_t)M * nout;
    for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (size_t)gridDim.x * 256) {
        const int m = (int)(idx / nout), o = (int)(idx % nout);
        if constexpr (EPI == Epi::SwiGLU) {
            const int ng = 64 * (o / 32) + (o % 32);
            float gt = 0.f, up = 0.f;
            for (int s = 0; s < splits; s++) {
                gt += a.part[s * MN + (size_t)m * N + ng];
                up += a.part[s * MN + (size_t)m * N + ng + 32];
            }
            Elt<T>::st((T*)a.out, (size_t)m * a.ldo + o, silu_f(gt) * up);
        } else {
            float v = 0.f;
            for (int s = 0; s < splits; s++) v += a.part[s * MN + (size_t)m * N + o];
            if (bias) v += Elt<T>::ld(bias, o);
            if constexpr (EPI == Epi::StoreF32) {
                ((float*)a.out)[(size_t)m * a.ldo + o] = v;
            } else if constexpr (EPI == Epi::Resid) {
                float* x = (float*)a.out + (size_t)m * a.ldo + o;
                *x = *x + v;
            } else if constexpr (EPI == Epi::Gelu) {
                Elt<T>::st((T*)a.out, (size_t)m * a.ldo + o, gelu_tanh_f(v));
            } else {
                ((float*)a.out)[(size_t)a.rowmap[m] * a.ldo + o] = v;
            }
        }
    }
}

template <class T, int BM, int BN, Epi EPI, bool SPLIT>
static hipError_t run_gemm(const GemmArgs& a, int splits, hipStream_t st) {
    using Tr = GemmTraits<T>;
    const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
    const size_t smem = 2 * (size_t)(BM + BN) * (Tr::BK + Tr::PAD) * sizeof(T);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<T, BM, BN, EPI, SPLIT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_kernel<T, BM, BN, EPI, SPLIT><<<dim3(mt * nt, SPLIT ? splits : 1), 256, smem, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    const size_t total = (size_t)a.M * (EPI == Epi::SwiGLU ? a.N / 2 : a.N);
    int blocks = (int)((total + 255) / 256);
    blocks = blocks > 4096 ? 4096 : blocks;
    splitk_reduce_kernel<T, EPI><<<blocks, 256, 0, st>>>(a, splits);
    return hipGetLastError();
}

// Blocks a prefill GEMM aims for before it splits K (several blocks per CU
// keep more loads in flight; the GEMMs here are latency-bound, not MFMA-bound).
// VLM_GEMM_TARGET_BLOCKS overrides it for tuning.
static int target_blocks() {
    static int v = [] {
        const char* e = getenv("VLM_GEMM_TARGET_BLOCKS");
        const int t = e ? atoi(e) : 0;
        return t > 0 ? t : 512;
    }();
    return v;
}

// Tile choice: the largest tile that still gives >= 256 blocks (one per CU),
// else the smallest; then a K split (2-4 ways, >= 4 stages each) up to the
// target block count when the caller provided split-K scratch.
template <class T, Epi EPI>
static hipError_t pick_tile(const GemmArgs& a, hipStream_t st) {
    auto tiles = [&](int bm, int bn) { return (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    const int nk = (a.K + GemmTraits<T>::BK - 1) / GemmTraits<T>::BK;
    auto splits_for = [&](long t) {
        if (!a.part) return 1;
        int sp = (int)(target_blocks() / t);
        sp = sp > 4 ? 4 : sp;
        while (sp > 1 && (nk / sp < 4 || (size_t)sp * a.M * a.N > a.part_cap)) sp--;
        return sp < 1 ? 1 : sp;
    };
    if (tiles(128, 128) >= 256) {
        const int sp = splits_for(tiles(128, 128));
        return sp > 1 ? run_gemm<T, 128, 128, EPI, true>(a, sp, st) : run_gemm<T, 128, 128, EPI, false>(a, 1, st);
    }
    if (tiles(64, 128) >= 256 || EPI == Epi::SwiGLU) {
        const int sp = splits_for(tiles(64, 128));
        return sp > 1 ? run_gemm<T, 64, 128, EPI, true>(a, sp, st) : run_gemm<T, 64, 128, EPI, false>(a, 1, st);
    }
    if constexpr (EPI != Epi::SwiGLU) {
        const int sp = splits_for(tiles(64, 64));
        return sp > 1 ? run_gemm<T, 64, 64, EPI, true>(a, sp, st) : run_gemm<T, 64, 64, EPI, false>(a, 1, st);
    }
    return hipErrorInvalidValue;
}

template <class T>
static hipError_t dispatch_epi(Epi epi, const GemmArgs& a, hipStream_t st) {
    switch (epi) {
        case Epi::StoreF32: return pick_tile<T, Epi::StoreF32>(a, st);
        case Epi::Resid: return pick_tile<T, Epi::Resid>(a, st);
        case Epi::SwiGLU: return pick_tile<T, Epi::SwiGLU>(a, st);
        case Epi::Gelu: return pick_tile<T, Epi::Gelu>(a, st);
        case Epi::StoreRowMap: return pick_tile<T, Epi::StoreRowMap>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    return dtype == 1 ? dispatch_epi<bf16_t>(epi, a, st) : dispatch_epi<float>(epi, a, st);
}

}  // namespace vlm
