// Prefill projections on the matrix cores: C[M][N] = A[M][K] * W[N][K]^T with
// fused epilogues (residual add, SwiGLU over 32-row interleaved gate/up
// groups, bias + GELU, bias + row-remapped store). These are the decoder
// matmuls that dominate prefill (MNN llm_demo Omni article §5.3; HunyuanOCR
// v1.5 ncnn port §5).
//
// Register-staged kernel (fp32, and bf16 rows with K % 8 != 0): 256 threads =
// 4 wavefronts in a 2x2 grid, each owning a (BM/2) x (BN/2) sub-tile built
// from 32x32 MFMA blocks:
//   bf16: v_mfma_f32_32x32x16_bf16, 64-element K stage;
//   f32:  v_mfma_f32_32x32x2f32,   32-element K stage.
// Both operands are K-contiguous, so every lane feeds the MFMA from one
// 16-byte LDS read (bf16: one 16-wide step; f32: four 2-wide steps of a quad
// of 8 columns). LDS is double-buffered and the next stage's global loads are
// in flight during the current stage's MFMAs. The bf16 prefill shapes use the
// direct-to-LDS kernel further down (its own wavefront grids and tile plan).
// Blocks are remapped so that consecutive output tiles (which share a weight
// panel) land on the same XCD and its L2.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

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

// (tile, K split) of this block: the remap runs over the whole grid (blocks are dealt to the XCDs
// in launch order, x fastest), so each XCD takes a contiguous run of (tile, split) work with the
// tiles of one split together: the M tiles that read the same weight columns share an L2. (With
// the split taken from blockIdx.y the M tiles of one column block fell on different XCDs and the
// split down projection fetched 2.7x its weight bytes from memory.) Any bijection is correct.
__device__ __forceinline__ void gemm_work(int ntiles, int* tile, int* split) {
    const int w = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    *tile = w % ntiles;
    *split = w / ntiles;
}

// Epilogue of one wavefront's (TM*32) x (TN*32) accumulator tile at output
// rows m0 + wm*WM, columns n0 + wn*WN. C layout of a 32x32 block: lane owns
// column l32 and rows (r/4)*8 + h*4 + r%4, r = 0..15.
template <class T, int WM, int WN, int TM, int TN, Epi EPI, bool SPLIT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, f32x16 (&acc)[TM][TN], int m0, int n0, int wm,
                                              int wn, int h, int l32, int split) {
    const int M = a.M, N = a.N;
    const T* bias = (const T*)a.bias;
    if constexpr (SPLIT) {  // raw partial sums; splitk_reduce_kernel applies the epilogue
        float* part = a.part + (size_t)split * M * N;
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
        static_assert(TN % 2 == 0, "SwiGLU needs whole 64-column (gate block, up block) pairs per wave tile");
        T* out = (T*)a.out;
#pragma unroll
        for (int jp = 0; jp < TN / 2; jp++) {
            const int nb = n0 + wn * WN + jp * 64, ncol = nb / 2 + l32;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
                    if (m < M && nb < N) {  // N = 2F is a multiple of 64: whole groups
                        const float gt = acc[i][2 * jp][r], up = acc[i][2 * jp + 1][r];
                        Elt<T>::st(out, (size_t)m * a.ldo + ncol, silu_f(gt) * up);
                    }
                }
        }
    } else if constexpr (EPI == Epi::Resid) {
        // The 16 old residual values of a 32x32 block are all requested before its first store:
        // with load, add and store per element, the compiler cannot prove the rows apart, so each
        // load waited behind the previous store, a chain of L2 round trips (64x128 tiles: 32 per
        // lane, ~7 us of a 21 us projection; now one per 32x32 block, with 16 registers more).
        // Indices are clamped so that the loads are unconditional; the sums are the same.
        float* x = (float*)a.out;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int nj = n0 + wn * WN + j * 32 + l32, nc = min(nj, N - 1);
            const float bn = bias ? Elt<T>::ld(bias, nc) : 0.f;
#pragma unroll
            for (int i = 0; i < TM; i++) {
                float old[16];
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = min(m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4), M - 1);
                    old[r] = x[(size_t)m * a.ldo + nc];
                }
                if (nj >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + wm * WM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
                    if (m < M) x[(size_t)m * a.ldo + nj] = old[r] + (acc[i][j][r] + bn);
                }
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
                    } else if constexpr (EPI == Epi::Gelu) {
                        Elt<T>::st((T*)a.out, (size_t)m * a.ldo + n, gelu_tanh_f(v));
                    } else {  // StoreRowMap
                        ((float*)a.out)[(size_t)a.rowmap[m] * a.ldo + n] = v;
                    }
                }
        }
    }
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
    int tile, split;
    gemm_work(mt * nt, &tile, &split);
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

    // split-K: the block's split selects a contiguous range of K stages
    int kt0 = 0, nk = (K + BK - 1) / BK;
    if constexpr (SPLIT) {
        const int per = (nk + gridDim.y - 1) / gridDim.y;
        kt0 = split * per;
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
            // K is taken in quads of 8 columns: in MFMA step e of quad q the lanes of half h
            // contribute column 8q + 4h + e, so one 16-byte LDS read per operand and half feeds
            // four steps (the same permutation on A and B leaves the contraction unchanged)
#pragma unroll
            for (int kq = 0; kq < BK / 8; kq++) {
                f32x4 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; i++) fa[i] = *reinterpret_cast<const f32x4*>(as + i * 32 * LDK + kq * 8 + h * 4);
#pragma unroll
                for (int j = 0; j < TN; j++) fb[j] = *reinterpret_cast<const f32x4*>(bs + j * 32 * LDK + kq * 8 + h * 4);
#pragma unroll
                for (int e = 0; e < 4; e++)
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][e], fb[j][e], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    gemm_epilogue<T, WM, WN, TM, TN, EPI, SPLIT>(a, acc, m0, n0, wm, wn, h, l32, split);
}

// ------------------------------------------------- bf16, direct-to-LDS pipeline
// The prefill shapes (M ~ 500 rows) give each block little MFMA work per K
// stage, so a stage is bound by the global-load round trip unless several
// stages are in flight. Here the operands go straight from global memory into
// a ring of P LDS stages (global_load_lds_dwordx4: lane L's 16 bytes land at
// the wave-uniform base + 16*L), P-1 stages ahead of the MFMAs, with no
// register staging. A stage holds BK (64 or 32) bf16 of each tile row; one
// load instruction fills 1 KiB, i.e. 8 rows of 64 or 16 rows of 32. Chunk c
// (16 bytes) of row r is stored at chunk position c ^ swz(r) of that row, so
// the MFMA operand reads (32 rows, one chunk) spread over the LDS banks
// (lds_swz below). Lane L of load instruction i therefore fetches tile row
// i * RPI + L / CPR and chunk (L % CPR) ^ swz(that row) (CPR = chunks per
// row). Requires K % 8 == 0:
// when K is not a multiple of BK, the last stage's loads past K are clamped to
// the row's last chunk and those columns are zeroed in LDS (A and B rows)
// before any wavefront reads the stage.
__device__ __forceinline__ void wait_lgkm0() {  // s_waitcnt lgkmcnt(0), other counters untouched
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// Waits until at most k * LPS of this wave's loads are outstanding, k in [0, KMAX] (wave-uniform).
template <int LPS, int KMAX>
__device__ __forceinline__ void wait_stages(int k) {
    if constexpr (KMAX > 0) {
        if (k >= KMAX) {
            wait_vm<KMAX * LPS>();
            return;
        }
        wait_stages<LPS, KMAX - 1>(k);
    } else {
        wait_vm<0>();
    }
}

// The LDS of gfx950 serves a 16-byte read of 16 lanes at once from 64 four-byte banks (256 bytes),
// so the 16 rows of one chunk column must cover every bank: with 128-byte rows, even and odd rows
// fall in opposite bank halves and (r >> 1) & 7 spreads each half's 8 rows over its 8 chunk slots;
// with 64-byte rows, r % 4 picks the bank quarter and (r >> 2) & 3 the slot. (r & 7 on 128-byte
// rows put rows r and r + 8 on the same banks: half of the GEMMs' LDS cycles were conflict stalls.)
// Both have a period of 16 rows.
template <int CPR>
__device__ __forceinline__ int lds_swz(int r) { return CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }

// WGM x WGN wavefronts per block, each owning a (BM/WGM) x (BN/WGN) sub-tile.
// T = float: a stage holds 32 floats of each row (the same 128 bytes as 64 bf16); each 16-byte
// operand read feeds four v_mfma_f32_32x32x2f32 steps, in which the lanes of half h contribute
// column 8q + 4h + e (step e of column quad q; the same permutation on A and B leaves the
// contraction unchanged).
template <class T, int BM, int BN, int P, int WGM, int WGN, Epi EPI, bool SPLIT, int BK, bool TAIL>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_lds_kernel(GemmArgs a) {
    constexpr int VEC = 16 / sizeof(T), LDI = 1024 / sizeof(T);  // elements per 16-byte chunk / load instruction
    static_assert(BK * sizeof(T) == 128 || BK * sizeof(T) == 64, "stage depth: 128- or 64-byte rows");
    constexpr int NW = WGM * WGN, WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
    constexpr int CPR = BK / VEC, RPI = 64 / CPR;  // 16-byte chunks per row, rows per load instruction
    constexpr int AI = BM / (RPI * NW), BI = BN / (RPI * NW);  // load instructions per wave per stage
    static_assert(AI * RPI * NW == BM && BI * RPI * NW == BN && TM >= 1 && TN >= 1, "tile / wavefront grid");
    constexpr int LPS = AI + BI, STAGE = (BM + BN) * BK;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* smem = reinterpret_cast<T*>(smem_raw);

    const int M = a.M, N = a.N, K = a.K;
    const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
    int tile, split;
    gemm_work(mt * nt, &tile, &split);
    const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int wm = w / WGN, wn = w % WGN, h = lane / 32, l32 = lane % 32;
    const T* A = (const T*)a.A;
    const T* B = (const T*)a.B;

    // this lane's source row/chunk in each of the wave's load instructions (rows past M / N are clamped:
    // their products land in output rows / columns the epilogue never stores)
    // (the chunk depends on the tile row, whose swizzle has a period of 16 rows: with 8-row load
    // instructions it alternates between instructions)
    const int lr = lane / CPR;
    const T* ga[AI];
    const T* gb[BI];
    int lca[AI], lcb[BI];
#pragma unroll
    for (int i = 0; i < AI; i++) {
        ga[i] = A + (size_t)min(m0 + (w * AI + i) * RPI + lr, M - 1) * K;
        lca[i] = (lane % CPR) ^ lds_swz<CPR>((w * AI + i) * RPI + lr);
    }
#pragma unroll
    for (int i = 0; i < BI; i++) {
        gb[i] = B + (size_t)min(n0 + (w * BI + i) * RPI + lr, N - 1) * K;
        lcb[i] = (lane % CPR) ^ lds_swz<CPR>((w * BI + i) * RPI + lr);
    }
    const int kmax = K - VEC;  // last 16-byte chunk of a row: loads of the tail stage are clamped to it

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    const int nk_all = (K + BK - 1) / BK, ktail = K - (nk_all - 1) * BK;  // columns of the last stage
    int kt0 = 0, nk = nk_all;
    if constexpr (SPLIT) {
        const int per = (nk + gridDim.y - 1) / gridDim.y;
        kt0 = split * per;
        nk = max(0, min(nk, kt0 + per) - kt0);
    }
    // one K stage of both tiles into LDS stage ST: instruction i of wavefront w fills RPI rows (1 KiB).
    // (The source pointer is passed as const void*: the host pass silently drops the kernel otherwise.)
#define VLM_LDS_KC(KOFF, LC) (TAIL ? min((KOFF) + (LC) * VEC, kmax) : (KOFF) + (LC) * VEC)
#define VLM_LDS_STAGE(KOFF, ST)                                                                              \
    do {                                                                                                     \
        _Pragma("unroll") for (int i = 0; i < AI; i++) __builtin_amdgcn_global_load_lds(                     \
            (const void*)(ga[i] + VLM_LDS_KC(KOFF, lca[i])), (lds_void*)((ST) + (w * AI + i) * LDI), 16, 0, 0); \
        _Pragma("unroll") for (int i = 0; i < BI; i++) __builtin_amdgcn_global_load_lds(                     \
            (const void*)(gb[i] + VLM_LDS_KC(KOFF, lcb[i])), (lds_void*)((ST) + BM * BK + (w * BI + i) * LDI), \
            16, 0, 0);                                                                                       \
    } while (0)
    // the last stage (global index nk_all - 1) of a K that is not a multiple of BK: zero its columns
    // ktail..BK-1 in every A and B row once they have landed (callers hold a barrier on both sides)
    auto zero_tail = [&](int kt_local, T* st) {
        if (!TAIL || ktail == BK || kt0 + kt_local != nk_all - 1) return;  // uniform
        const int c0 = ktail / VEC;
        for (int idx = tid; idx < (BM + BN) * CPR; idx += NW * kWave) {
            const int r = idx / CPR, c = idx % CPR;
            if (c >= c0) *reinterpret_cast<u32x4*>(st + r * BK + ((c ^ lds_swz<CPR>(r)) * VEC)) = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
    };
#pragma unroll
    for (int s = 0; s < P - 1; s++)
        if (s < nk) VLM_LDS_STAGE((kt0 + s) * BK, smem + s * STAGE);
    // operand rows of this lane inside a stage; chunk c of row r sits at r*BK + ((c ^ swz(r)) * 8)
    int ra[TM], rb[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) ra[i] = wm * WM + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < TN; j++) rb[j] = BM + wn * WN + j * 32 + l32;
    constexpr int KS = BK / (2 * VEC);  // fragment steps per stage (one 16-byte read per operand row and half)
    using Frag = typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type;
    auto read_frags = [&](const T* st, int kk, Frag* fa, Frag* fb) {
        const int c = kk * 2 + h;
#pragma unroll
        for (int i = 0; i < TM; i++)
            fa[i] = *reinterpret_cast<const Frag*>(st + ra[i] * BK + ((c ^ lds_swz<CPR>(ra[i])) * VEC));
#pragma unroll
        for (int j = 0; j < TN; j++)
            fb[j] = *reinterpret_cast<const Frag*>(st + rb[j] * BK + ((c ^ lds_swz<CPR>(rb[j])) * VEC));
    };
    // a wavefront issuing its MFMA burst runs at raised priority, so the arbiter favours it over the
    // other wavefronts' load issue and LDS reads (prefill 0.9% faster over 5 A/B pairs on the 36-layer
    // stack, results unchanged)
    auto mfmas = [&](const Frag* fa, const Frag* fb) {
        __builtin_amdgcn_s_setprio(1);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++)
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][e], fb[j][e], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Software pipeline: the fragments of step kk+1 are read while the MFMAs of step kk run, and
    // the first step of stage kt+1 is read (after its wait and barrier) before the last MFMAs of
    // stage kt, so LDS reads overlap the matrix cores within each wavefront. (Reading a whole
    // stage's fragments before its first MFMA measured 5-12% slower on the prefill shapes.)
    {
        Frag fa[2][TM], fb[2][TN];
        if (nk > 0) {
            wait_stages<LPS, P - 2>(nk - 1);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (TAIL) zero_tail(0, smem);
            if (P - 1 < nk) VLM_LDS_STAGE((kt0 + P - 1) * BK, smem + (P - 1) * STAGE);
            read_frags(smem, 0, fa[0], fb[0]);
        }
        for (int kt = 0; kt < nk; kt++) {
            const T* st = smem + (kt % P) * STAGE;
#pragma unroll
            for (int kk = 0; kk < KS - 1; kk++) {
                read_frags(st, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                mfmas(fa[kk & 1], fb[kk & 1]);
            }
            if (kt + 1 < nk) {
                wait_stages<LPS, P - 2>(nk - 2 - kt);  // stage kt+1 has landed (this lane)
                wait_lgkm0();                          // this wave's reads of stage kt have returned
                __builtin_amdgcn_s_barrier();          // ... every wave's; stage kt's slot may be refilled
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (TAIL) zero_tail(kt + 1, smem + ((kt + 1) % P) * STAGE);
                if (kt + P < nk) VLM_LDS_STAGE((kt0 + kt + P) * BK, smem + (kt % P) * STAGE);
                read_frags(smem + ((kt + 1) % P) * STAGE, 0, fa[0], fb[0]);
            }
            mfmas(fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
        }
    }
#undef VLM_LDS_STAGE
#undef VLM_LDS_KC
    gemm_epilogue<T, WM, WN, TM, TN, EPI, SPLIT>(a, acc, m0, n0, wm, wn, h, l32, split);
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

// Split-K reduction of a residual GEMM fused with the row norm that follows it:
// one block per row, thread t owns columns t + 256 i (the column split and the
// summation order of norm_rows_reg_kernel, so the normalised row is bitwise the
// one a separate norm launch would write). x[m] += sum of the partials (split
// order) + bias, then norm_out[m] = norm(x[m]).
// SM >= splits partial planes and NPT >= N / 256 columns per thread are requested (clamped indices),
// so both are sized to the launch: with 8 planes and 8 columns for a 4-split, 1152-column row, 96
// loads per thread went out for 20 distinct values (vision tower fc2 reduction 15.4 us).
constexpr int kReduceNormMaxSplits = 8;
template <class T, bool LAYER, int NPT, int SM>
__global__ __launch_bounds__(256) void splitk_reduce_norm_kernel(GemmArgs a, int splits) {
    __shared__ float red[4];
    const int m = blockIdx.x, N = a.N, tid = threadIdx.x;
    const size_t MN = (size_t)a.M * N;
    const T* bias = (const T*)a.bias;
    const T* gn = (const T*)a.norm_gain;
    const T* sh = (const T*)a.norm_shift;
    float* x = (float*)a.out + (size_t)m * a.ldo;
    const float* pr = a.part + (size_t)m * N;
    // every load of the row is requested before the first sum (split and column indices clamped)
    float pv[SM][NPT], xv[NPT], gv[NPT], bv[NPT], cb[NPT];
#pragma unroll
    for (int sp = 0; sp < SM; sp++)
#pragma unroll
        for (int i = 0; i < NPT; i++) pv[sp][i] = pr[(size_t)min(sp, splits - 1) * MN + min(tid + 256 * i, N - 1)];
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const int j = min(tid + 256 * i, N - 1);
        xv[i] = x[j];
        cb[i] = bias ? Elt<T>::ld(bias, j) : 0.f;
        gv[i] = Elt<T>::ld(gn, j);
        bv[i] = (LAYER && sh) ? Elt<T>::ld(sh, j) : 0.f;
    }
    float v[NPT];
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        float acc = 0.f;
#pragma unroll
        for (int sp = 0; sp < SM; sp++)
            if (sp < splits) acc += pv[sp][i];
        if (bias) acc += cb[i];
        v[i] = xv[i] + acc;
    }
#pragma unroll
    for (int i = 0; i < NPT; i++)
        if (tid + 256 * i < N) x[tid + 256 * i] = v[i];
    float mu = 0.f;
    if (LAYER) {
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < NPT; i++) sm += tid + 256 * i < N ? v[i] : 0.f;
        mu = block_sum<256>(sm, red) / (float)N;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const float c = v[i] - mu;
        ss += tid + 256 * i < N ? c * c : 0.f;
    }
    const float r = rsqrtf(block_sum<256>(ss, red) / (float)N + a.norm_eps);
    T* o = (T*)a.norm_out + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < NPT; i++) {
        const int j = tid + 256 * i;
        if (j < N) Elt<T>::st(o, j, (v[i] - mu) * r * gv[i] + bv[i]);
    }
}

// The reduction of a split residual GEMM: fused with the following row norm when the caller asked
// for it and the row fits the register form (N <= 4096), else the plain reduction.
template <class T, Epi EPI>
static hipError_t run_reduce(const GemmArgs& a, int splits, hipStream_t st) {
    if constexpr (EPI == Epi::Resid) {
        if (a.norm_out && a.norm_gain && a.N <= 4096 && splits <= kReduceNormMaxSplits) {
            const int npt = (a.N + 255) / 256;
#define VLM_RED_NORM_S(NPT_, SM_)                                                                              \
    do {                                                                                                       \
        if (a.norm_layer) splitk_reduce_norm_kernel<T, true, NPT_, SM_><<<a.M, 256, 0, st>>>(a, splits);       \
        else splitk_reduce_norm_kernel<T, false, NPT_, SM_><<<a.M, 256, 0, st>>>(a, splits);                   \
    } while (0)
#define VLM_RED_NORM(NPT_)                                  \
    do {                                                    \
        if (splits <= 2) VLM_RED_NORM_S(NPT_, 2);           \
        else if (splits <= 4) VLM_RED_NORM_S(NPT_, 4);      \
        else VLM_RED_NORM_S(NPT_, kReduceNormMaxSplits);    \
    } while (0)
            if (npt <= 2) VLM_RED_NORM(2);
            else if (npt <= 4) VLM_RED_NORM(4);
            else if (npt <= 5) VLM_RED_NORM(5);
            else if (npt <= 8) VLM_RED_NORM(8);
            else if (npt <= 10) VLM_RED_NORM(10);
            else if (npt <= 12) VLM_RED_NORM(12);
            else VLM_RED_NORM(16);
#undef VLM_RED_NORM
#undef VLM_RED_NORM_S
            const hipError_t e = hipGetLastError();
            if (e == hipSuccess && a.fused_norm) *a.fused_norm = 1;
            return e;
        }
    }
    const size_t total = (size_t)a.M * (EPI == Epi::SwiGLU ? a.N / 2 : a.N);
    int blocks = (int)((total + 255) / 256);
    blocks = blocks > 4096 ? 4096 : blocks;
    splitk_reduce_kernel<T, EPI><<<blocks, 256, 0, st>>>(a, splits);
    return hipGetLastError();
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
    return run_reduce<T, EPI>(a, splits, st);
}

template <class T, int BM, int BN, int P, int WGM, int WGN, Epi EPI, bool SPLIT, int BK, bool TAIL>
static hipError_t run_gemm_lds(const GemmArgs& a, int splits, hipStream_t st) {
    const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
    const size_t smem = (size_t)P * (BM + BN) * BK * sizeof(T);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_lds_kernel<T, BM, BN, P, WGM, WGN, EPI, SPLIT, BK, TAIL>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_lds_kernel<T, BM, BN, P, WGM, WGN, EPI, SPLIT, BK, TAIL><<<dim3(mt * nt, SPLIT ? splits : 1), WGM * WGN * 64, smem, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    return run_reduce<T, EPI>(a, splits, st);
}

// Tile and K-split choice of the direct-to-LDS kernel from a per-CU feed model.
// On these shapes a block's time is set by how fast its CU pulls operand
// stages out of L2 rather than by the matrix cores: an estimate is
//   3 us + q * stages * stage_bytes / feed,   q = ceil(blocks / 256),
// with feed the measured per-CU rate of the tile shape (bytes/us, "one" for a
// lone block per CU, "two" when two blocks share it), plus, for a K split,
// 3 us and the fp32 partials written and re-read by the reduce (~4 GB/ms).
// The constants come from timing every candidate on the decoder prefill
// shapes (M 512-560; K 1024-9728) with two-stage rings for the 128-row tiles
// and three for 64x128; the model picks within ~6% of the fastest.
// The 256x192 SwiGLU tile (eight 32x192 wavefront tiles, so each wavefront
// holds whole gate/up pairs) covers N = 19456 in 204 blocks instead of 152:
// gate/up of the 36-layer stack 78.5 -> 71.7 us (four 64x192 wavefront tiles,
// one wavefront per SIMD: 77.8 us). It is planned for SwiGLU only, where it
// was measured.
struct LdsPlan { int bm, bn, sp; };
static LdsPlan plan_lds(const GemmArgs& a, bool swiglu) {
    // {BM, BN, blocks per CU that fit the LDS ring, feed with one block per CU, feed with two}
    static const int cand[6][5] = {{256, 256, 1, 37000, 37000}, {256, 192, 1, 33400, 33400},
                                   {128, 256, 1, 46500, 46500}, {128, 128, 2, 43000, 52000},
                                   {64, 128, 2, 44000, 62000},  {64, 64, 2, 40000, 55000}};
    static const int splits[6] = {1, 2, 3, 4, 6, 8};
    const int nk = (a.K + 63) / 64;
    double best = 1e30;
    LdsPlan bp{64, 128, 1};
    for (const auto& c : cand) {
        if (swiglu && c[1] < 128) continue;  // SwiGLU pairs a 32-column gate block with its up block
        if (!swiglu && c[1] == 192) continue;
        const long tiles = (long)((a.M + c[0] - 1) / c[0]) * ((a.N + c[1] - 1) / c[1]);
        for (int sp : splits) {
            if (sp > 1 && (!a.part || nk / sp < 4 || (size_t)sp * a.M * a.N > a.part_cap)) continue;
            const long q = (tiles * sp + 255) / 256;  // blocks per CU
            const double feed = (c[2] >= 2 && q >= 2) ? c[4] : c[3];
            const double stages = (double)((nk + sp - 1) / sp);
            double t = 3.0 + (double)q * stages * (c[0] + c[1]) * 128.0 / feed;  // us
            if (sp > 1) t += 3.0 + (double)sp * a.M * a.N * 8.0 / 4.0e6;
            if (t < best) {
                best = t;
                bp = {c[0], c[1], sp};
            }
        }
    }
    return bp;
}

// Tile and K split: the direct-to-LDS kernel for bf16 with K % 8 == 0 (plan_lds), else the
// register-staged kernel planned by the work model below.
template <class T, Epi EPI>
static hipError_t pick_tile(const GemmArgs& a, hipStream_t st) {
    auto tiles = [&](int bm, int bn) { return (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    const int nk = (a.K + GemmTraits<T>::BK - 1) / GemmTraits<T>::BK;
    if constexpr (sizeof(T) == 2) {
        if (a.K % 8 == 0 && a.K >= 64) {  // direct-to-LDS pipeline; rings of at most 144 KiB (one block per CU)
            const LdsPlan pl = plan_lds(a, EPI == Epi::SwiGLU);
#define VLM_RUN_LDS_T(BM_, BN_, P_, GM_, GN_, BK_, T_)                                            \
    return pl.sp > 1 ? run_gemm_lds<bf16_t, BM_, BN_, P_, GM_, GN_, EPI, true, BK_, T_>(a, pl.sp, st)     \
                     : run_gemm_lds<bf16_t, BM_, BN_, P_, GM_, GN_, EPI, false, BK_, T_>(a, 1, st)
#define VLM_RUN_LDS(BM_, BN_, P_, GM_, GN_, BK_)                                                   \
    do {                                                                                          \
        if (a.K % BK_ != 0) VLM_RUN_LDS_T(BM_, BN_, P_, GM_, GN_, BK_, true);                     \
        VLM_RUN_LDS_T(BM_, BN_, P_, GM_, GN_, BK_, false);                                        \
    } while (0)
            // The 128-row tiles keep 2 stages in flight instead of 1 (a ring of 3), 64x128 tiles 4
            // instead of 2 (a ring of 5): on M 512-1288 a stage waits on the L2 round trip, not on the
            // matrix cores, so more bytes in flight feed the CU faster. bf16 vision tower 4.70 -> 4.46 ms
            // per pass, prefill of the 36-layer stack 6.83 -> 6.57 ms, of the 28-layer stack 2.82 ->
            // 2.66 ms; one stage more again (128x128 in 4, 64x128 in 6) gained nothing. Only the depth
            // of the ring differs, so the products are bitwise those of the shallow ring, which
            // VLM_LDS_DEEP=0 selects (read per call, for comparison).
            const char* dv = getenv("VLM_LDS_DEEP");
            const bool deep = !(dv && atoi(dv) == 0);
            if constexpr (EPI == Epi::SwiGLU)
                if (pl.bm == 256 && pl.bn == 192) VLM_RUN_LDS(256, 192, 2, 8, 1, 64);
            // an unsplit 128x256 plan whose blocks fit one round as 128x192 tiles takes those (eight
            // 32x96 wavefront tiles; three 32-column blocks per wavefront, so not for SwiGLU): the
            // vision tower's fc1 (N 4304: 187 -> 253 blocks) and QKV (N 3456: 154 -> 198), bf16 tower
            // 5.05 -> 4.83 ms per pass (a four-wavefront 64x96 form: 5.07 ms)
            if constexpr (EPI != Epi::SwiGLU)
                if (pl.bm == 128 && pl.bn == 256 && pl.sp == 1 && tiles(128, 192) <= 256) {
                    if (deep) VLM_RUN_LDS(128, 192, 3, 4, 2, 64);
                    VLM_RUN_LDS(128, 192, 2, 4, 2, 64);
                }
            if (pl.bm == 256) VLM_RUN_LDS(256, 256, 2, 4, 2, 64);
            if (pl.bm == 128 && pl.bn == 256) {
                if (deep) VLM_RUN_LDS(128, 256, 3, 2, 4, 64);
                VLM_RUN_LDS(128, 256, 2, 2, 4, 64);
            }
            if (pl.bm == 128) {
                if (deep) VLM_RUN_LDS(128, 128, 3, 2, 2, 64);
                VLM_RUN_LDS(128, 128, 2, 2, 2, 64);
            }
            if (pl.bn == 128) {
                if (deep) VLM_RUN_LDS(64, 128, 5, 2, 2, 64);
                VLM_RUN_LDS(64, 128, 3, 2, 2, 64);
            }
            if constexpr (EPI != Epi::SwiGLU) VLM_RUN_LDS(64, 64, 4, 2, 2, 64);
#undef VLM_RUN_LDS
#undef VLM_RUN_LDS_T
        }
    }
    // fp32 rows of 16-byte chunks (K % 4 == 0): the direct-to-LDS ring of 32-float stages with 64x64
    // tiles in 4 stages (64x128 in 3 for SwiGLU, whose wavefront tiles hold whole gate/up column
    // pairs; four wavefronts of 2 x 2), one block per tile and no K split. Measured on the vision
    // tower (M 1288; N 1152-4304; K 1152-4304), ms per pass: 16.4 (4 or 3 stages; 2: 16.5), with a
    // K split of up to 2 16.8, with the register-staged plan's tiles 17.6 (its splits too: 18.0),
    // 64x128 18.1, 128x128 24.0; the register-staged kernel 20.8. VLM_F32_LDS=0 keeps the
    // register-staged kernel (read per call, for comparison).
    if constexpr (sizeof(T) == 4) {
        const char* ev = getenv("VLM_F32_LDS");
        if (a.K % 4 == 0 && a.K >= 32 && !(ev && atoi(ev) == 0)) {
            constexpr int BN32 = EPI == Epi::SwiGLU ? 128 : 64, P32 = EPI == Epi::SwiGLU ? 3 : 4;
            if (a.K % 32 != 0) return run_gemm_lds<float, 64, BN32, P32, 2, 2, EPI, false, 32, true>(a, 1, st);
            return run_gemm_lds<float, 64, BN32, P32, 2, 2, EPI, false, 32, false>(a, 1, st);
        }
    }
    // register-staged kernel (f32, or bf16 with K % 8 != 0): tile and K split from a per-CU work
    // model fitted on the vision tower's shapes (M 322-1288, N 1152-4608, K 1152-4608, f32):
    // a CU runs ceil(blocks / 256) blocks one after another at a rate set by the tile shape, and a
    // split adds its reduction (the fp32 partials written and read back, ~4 GB/ms, plus 3 us); a
    // 128x128 tile does 6.7 ns of work per 1000 MACs-columns unit, smaller tiles 0.8x / 0.74x that
    // rate. The model reproduces the measured times within ~10% and picks within ~5% of the fastest.
    struct Cand { int bm, bn; double eff; };
    static const Cand cand[3] = {{128, 128, 1.0}, {64, 128, 0.8}, {64, 64, 0.74}};
    static const int splits[4] = {1, 2, 3, 4};
    double best = 1e30;
    int bbm = 64, bbn = 128, bsp = 1;
    for (const auto& c : cand) {
        if (EPI == Epi::SwiGLU && c.bn < 128) continue;  // a wave tile holds whole (gate, up) 64-column pairs
        const long t = tiles(c.bm, c.bn);
        for (int sp : splits) {
            if (sp > 1 && (!a.part || nk / sp < 4 || (size_t)sp * a.M * a.N > a.part_cap)) continue;
            const double per = (double)c.bm * c.bn * ((nk + sp - 1) / sp) * GemmTraits<T>::BK;
            double us = (double)((t * sp + 255) / 256) * per * 6.7e-6 / c.eff;
            if (sp > 1) us += 3.0 + (double)(sp + 1) * a.M * a.N * 4.0 / 4.0e6;
            if (us < best) {
                best = us;
                bbm = c.bm;
                bbn = c.bn;
                bsp = sp;
            }
        }
    }
#define VLM_RUN_REG(BM_, BN_)                                                                  \
    return bsp > 1 ? run_gemm<T, BM_, BN_, EPI, true>(a, bsp, st) : run_gemm<T, BM_, BN_, EPI, false>(a, 1, st)
    if (bbm == 128) VLM_RUN_REG(128, 128);
    if (bbn == 128) VLM_RUN_REG(64, 128);
    if constexpr (EPI != Epi::SwiGLU) VLM_RUN_REG(64, 64);
#undef VLM_RUN_REG
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
        default: break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(Epi epi, const GemmArgs& a, int splits, hipStream_t st) {
    switch (epi) {
        case Epi::StoreF32: return run_reduce<bf16_t, Epi::StoreF32>(a, splits, st);
        case Epi::Resid: return run_reduce<bf16_t, Epi::Resid>(a, splits, st);
        case Epi::SwiGLU: return run_reduce<bf16_t, Epi::SwiGLU>(a, splits, st);
        default: break;
    }
    return hipErrorNotSupported;
}

hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (gemm_small_fits(dtype, epi, a)) return launch_gemm_small(epi, a, st);
    return dtype == 1 ? dispatch_epi<bf16_t>(epi, a, st) : dispatch_epi<float>(epi, a, st);
}

}  // namespace vlm
