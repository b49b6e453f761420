// Projections of a few rows (bf16, M <= 16): the multi-token verify block and
// short chunked prefills (HunyuanOCR v1.5 ncnn port §3.8: the target model
// scores a drafted block in one causal forward, so every projection of the
// stack sees a handful of rows).
//
// With M <= 16 a projection streams its weights like the decode GEMV and
// reuses each weight load for every row; the prefill GEMM's 64-row MFMA tiles
// would run at most a quarter full. The layout is that of the decode GEMV
// (gemv2_kernel), widened to MR operand rows:
//   * the block's M rows of the split's K range go straight from global
//     memory into LDS (global_load_lds_dwordx4, 1 KiB per instruction; rows
//     past M repeat row M - 1 and their sums are never stored);
//   * each of the 4 wavefronts owns NR weight rows; lane l owns the 16-byte
//     chunks k = l * 8 + c * 512 of every row, so one load instruction reads
//     1 KiB of contiguous row, and requests all of them before its first
//     product (one memory round trip);
//   * each weight chunk is multiplied with the MR operand chunks at the same
//     k (read from LDS, four rows at a time) by v_dot2_f32_bf16, two products
//     per instruction accumulated in fp32;
//   * a wavefront sum per (row, operand row) gives every lane the NR x MR
//     results; lane r * MR + m writes (row r, operand row m).
// Long rows are split over blocks (grid y, at most 6 chunks per lane each):
// the blocks write fp32 partials and the split reduction of the prefill GEMM
// sums them in split order, adding into the residual rows and writing the
// next RMSNorm where asked (a residual projection always takes this route,
// with one split when K fits). The order of every sum is fixed, so results
// are deterministic.
#include <stdlib.h>

#include "common.hpp"
#include "internal.hpp"

namespace vlm {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kRowsNW = 4;         // wavefronts per block
constexpr int kRowsMaxChunks = 6;  // 16-byte chunks per lane and row (split K beyond)
constexpr int kRowsMaxM = 16;

// (Each dword goes through a scalar first: a bit cast of the vector element itself compiled to the
// first dword for every e.)
__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t we = w[e], xe = x[e];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, we), __builtin_bit_cast(bf16x2, xe), acc,
                                              false);
    }
    return acc;
}

// SWIGLU: rows are NR / 2 (gate, up) pairs and out is the model-type [M][ldo] activation; otherwise
// out is fp32 [M][ldo] (the projection, or split y's partial block when a.part is used).
template <bool SWIGLU, int NR, int KCH, int MR>
__global__ __launch_bounds__(kRowsNW * 64) void gemv_rows_kernel(GemmArgs a, int kspan, float* out, int ldo) {
    constexpr int NW = kRowsNW, XI = MR * KCH / NW;  // operand load instructions per wavefront
    static_assert(MR % 4 == 0 && (MR * KCH) % NW == 0, "operand rows");
    extern __shared__ __attribute__((aligned(16))) u32x4 xs[];  // [MR][KCH * 64] chunks of the operand rows
    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int k0 = blockIdx.y * kspan, k1 = min(K, k0 + kspan);
    const bf16_t* A = (const bf16_t*)a.A;
    const bf16_t* W = (const bf16_t*)a.B;
    out += (size_t)blockIdx.y * M * ldo;  // split y's partial block (one split when writing the result)

    // (1) operand rows of the split into LDS: instruction q fills 64 chunks of row q / KCH
#pragma unroll
    for (int i = 0; i < XI; i++) {
        const int q = w + NW * i, m = q / KCH, j = q % KCH;
        const int k = min(k0 + (64 * j + lane) * 8, k1 - 8);
        __builtin_amdgcn_global_load_lds((const void*)(A + (size_t)min(m, M - 1) * K + k),
                                         (lds_void*)(xs + (size_t)m * KCH * 64 + 64 * j), 16, 0, 0);
    }
    // the operand loads stay ahead of the weight loads: the wait below counts on their issue order
    __builtin_amdgcn_sched_barrier(0);
    // (2) this wavefront's weight rows
    const int wave = blockIdx.x * NW + w;
    int rows[NR];
    if constexpr (SWIGLU) {
        constexpr int P = NR / 2;
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int o = min(wave * P + p, N / 2 - 1);
            rows[p] = 64 * (o / 32) + (o % 32);
            rows[P + p] = rows[p] + 32;
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; r++) rows[r] = min(wave * NR + r, N - 1);
    }
    u32x4 wr[NR][KCH];
#pragma unroll
    for (int c = 0; c < KCH; c++) {
        const int k = min(k0 + (64 * c + lane) * 8, k1 - 8);
#pragma unroll
        for (int r = 0; r < NR; r++) wr[r][c] = *reinterpret_cast<const u32x4*>(W + (size_t)rows[r] * K + k);
    }
    wait_vm<NR * KCH>();               // this wavefront's operand loads have landed ...
    __builtin_amdgcn_s_barrier();      // ... and every wavefront's
    __builtin_amdgcn_sched_barrier(0);

    // (3) products: chunk c of every weight row against chunk c of the operand rows
    float acc[NR][MR];
#pragma unroll
    for (int r = 0; r < NR; r++)
#pragma unroll
        for (int m = 0; m < MR; m++) acc[r][m] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; c++) {
        if (k0 + (64 * c + lane) * 8 < k1) {
#pragma unroll
            for (int m4 = 0; m4 < MR; m4 += 4) {
                u32x4 xv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) xv[i] = xs[(size_t)(m4 + i) * KCH * 64 + 64 * c + lane];
#pragma unroll
                for (int r = 0; r < NR; r++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[r][m4 + i] = dot8(wr[r][c], xv[i], acc[r][m4 + i]);
            }
        }
    }
    // (4) wavefront sums; lane r * MR + m keeps (row r, operand row m)
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < NR; r++)
#pragma unroll
        for (int m = 0; m < MR; m++) {
            const float v = wave_sum(acc[r][m]);
            if (lane == r * MR + m) mine = v;
        }
    if constexpr (SWIGLU) {
        constexpr int P = NR / 2;
        // the up sum of pair p sits in lane (P + p) * MR + m: fetch it into lane p * MR + m
        const float up = __shfl_down(mine, P * MR);
        const int p = lane / MR, m = lane % MR, o = wave * P + p;
        if (p < P && m < M && o < N / 2)
            Elt<bf16_t>::st((bf16_t*)out, (size_t)m * ldo + o, silu_f(mine) * up);
    } else {
        const int r = lane / MR, m = lane % MR, n = wave * NR + r;
        if (r < NR && m < M && n < N) out[(size_t)m * ldo + n] = mine;
    }
}

struct RowsPlan { int splits, kspan, kch, mr; };
static RowsPlan rows_plan(const GemmArgs& a) {
    RowsPlan p;
    p.splits = (a.K + kRowsMaxChunks * 512 - 1) / (kRowsMaxChunks * 512);
    p.kspan = ((a.K + p.splits - 1) / p.splits + 7) / 8 * 8;
    p.kch = (p.kspan + 511) / 512;
    p.mr = a.M <= 4 ? 4 : (a.M <= 8 ? 8 : 16);
    return p;
}

bool gemm_small_fits(int dtype, Epi epi, const GemmArgs& a) {
    // VLM_FEW_ROWS (read per call): bit 0 = these projections, bit 1 = the few-row attention
    // launch; unset = both, 0 = the prefill kernels for every row count
    const char* e = getenv("VLM_FEW_ROWS");
    if (e && !(atoi(e) & 1)) return false;
    if (dtype != 1 || a.M < 1 || a.M > kRowsMaxM || a.K < 8 || a.K % 8 != 0) return false;
    if (a.bias || a.rowmap) return false;
    if (epi != Epi::StoreF32 && epi != Epi::Resid && epi != Epi::SwiGLU) return false;
    if (epi == Epi::SwiGLU && a.N % 64 != 0) return false;
    const RowsPlan p = rows_plan(a);
    const bool split = epi == Epi::Resid || p.splits > 1;
    return !split || (a.part && (size_t)p.splits * a.M * a.N <= a.part_cap);
}

template <bool SWIGLU, int NR, int KCH, int MR>
static hipError_t rows_launch(const GemmArgs& a, const RowsPlan& p, float* out, int ldo, hipStream_t st) {
    constexpr int rows_per_block = kRowsNW * (SWIGLU ? NR / 2 : NR);
    const int nout = SWIGLU ? a.N / 2 : a.N;
    const size_t smem = (size_t)MR * KCH * 64 * sizeof(u32x4);
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void*)gemv_rows_kernel<SWIGLU, NR, KCH, MR>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 grid((nout + rows_per_block - 1) / rows_per_block, p.splits);
    gemv_rows_kernel<SWIGLU, NR, KCH, MR><<<grid, kRowsNW * 64, smem, st>>>(a, p.kspan, out, ldo);
    return hipGetLastError();
}

// Rows per wavefront: 2, or 4 with 16 operand rows or at least kRowsWideN rows (a block restages
// its M operand rows for every 4 * NR weight rows, so wide projections such as the verify head's
// table pass keep those L2 reads below the weight bytes); SwiGLU two (gate, up) pairs.
constexpr int kRowsWideN = 16384;
template <bool SWIGLU, int KCH>
static hipError_t rows_mr(const GemmArgs& a, const RowsPlan& p, float* out, int ldo, hipStream_t st) {
    const bool wide = SWIGLU || a.N >= kRowsWideN;
    switch (p.mr) {
        case 4: return wide ? rows_launch<SWIGLU, 4, KCH, 4>(a, p, out, ldo, st)
                            : rows_launch<SWIGLU, 2, KCH, 4>(a, p, out, ldo, st);
        case 8: return wide ? rows_launch<SWIGLU, 4, KCH, 8>(a, p, out, ldo, st)
                            : rows_launch<SWIGLU, 2, KCH, 8>(a, p, out, ldo, st);
        default: return rows_launch<SWIGLU, 4, KCH, 16>(a, p, out, ldo, st);
    }
}

template <bool SWIGLU>
static hipError_t rows_kch(const GemmArgs& a, const RowsPlan& p, float* out, int ldo, hipStream_t st) {
    switch (p.kch) {
        case 1: return rows_mr<SWIGLU, 1>(a, p, out, ldo, st);
        case 2: return rows_mr<SWIGLU, 2>(a, p, out, ldo, st);
        case 3: return rows_mr<SWIGLU, 3>(a, p, out, ldo, st);
        case 4: return rows_mr<SWIGLU, 4>(a, p, out, ldo, st);
        case 5: return rows_mr<SWIGLU, 5>(a, p, out, ldo, st);
        default: return rows_mr<SWIGLU, 6>(a, p, out, ldo, st);
    }
}

hipError_t launch_gemm_small(Epi epi, const GemmArgs& a, hipStream_t st) {
    const RowsPlan p = rows_plan(a);
    if (epi != Epi::Resid && p.splits == 1) {
        if (epi == Epi::SwiGLU) return rows_kch<true>(a, p, (float*)a.out, a.ldo, st);
        return rows_kch<false>(a, p, (float*)a.out, a.ldo, st);
    }
    // partials [split][M][N] (the SwiGLU partials are the raw gate/up rows), then the split reduction
    const hipError_t e = rows_kch<false>(a, p, a.part, a.N, st);
    if (e != hipSuccess) return e;
    return launch_split_reduce(epi, a, p.splits, st);
}

}  // namespace vlm
