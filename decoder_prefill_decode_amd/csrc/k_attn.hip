// Attention kernels.
//
// Prefill: fused (flash-style) attention — scores, mask, softmax and the
// product with V in one kernel with the intermediates in registers and LDS
// (MNN llm_demo Omni article §5.1), over the KV cache the same call just wrote
// (Youtu-VL-4B ncnn port, 实现流程 §7). GQA: query head h reads KV head
// h / (nq/nkv) (Penguin-VL ncnn port §3). Softmax as max, subtract, exp, sum,
// divide (Youtu-VL-4B ncnn port, 实现难点 §3), done online per key tile.
//
// gfx950 mapping of the prefill kernel: one block = one query head x 128
// query rows, 4 wavefronts x 32 rows; 64-key K/V tiles staged in LDS.
// Each wavefront computes S^T = K Q^T with 32x32 MFMAs, so a lane holds all
// scores of ONE query (column) and the row max / sum need a single cross-half
// shuffle; P^T is then already in the B-operand layout of O^T = V^T P^T, and
// the rescaling of O^T by the running max is lane-local. The 32-key MFMA
// block permutes keys inside a 16-key step the same way for P and V, which
// leaves the contraction unchanged. bf16 uses 32x32x16 (V transposed in LDS
// so each lane reads two 8-byte runs) and feeds P as a hi + lo pair of bf16
// values; f32 uses 32x32x2.
//
// Decode: split-K over the valid slots 0..t of the fixed window (Youtu-VL-4B
// ncnn port, 实现流程 §7: slots beyond t carry -1e9 in the mask, i.e. they
// are skipped), each block covering one KV head and a slice of slots for all
// query heads of its group; 16 lanes share a key row (coalesced 16-byte
// loads), softmax statistics merge across lanes, wavefronts and blocks by
// log-sum-exp.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace vlm {

constexpr float kLog2e = 1.4426950408889634f;

// Key tiles a query block has to visit under a segment (window) mask: a tile
// can hold a visible key only if some key in it has a segment id within
// [min, max] of the block's query segments, so every other tile is skipped
// (exact for any id assignment; with windows laid out contiguously, as the
// vision tower does, a block visits only the tiles of its own windows instead
// of the whole sequence). Writes the visited tiles in order to list and
// returns their count; all threads of the block take part.
// Under a segment mask: true when every query row of this wavefront (lane % 32 -> row q0 + lane % 32)
// and every key of the tile [key0, key0 + BKEY) lie in one and the same segment, so the tile needs no
// per-element test. `sg` holds the tile's segment ids, staged in LDS with its K/V. Wavefront-uniform.
template <int BKEY>
__device__ __forceinline__ bool segment_tile_full(const int* sg, int seg_q, bool row_ok, int key0, int nkeys) {
    const int s0 = __builtin_amdgcn_readfirstlane(seg_q);
    const int kl = (threadIdx.x % kWave) % BKEY;
    const bool key_ok = key0 + kl < nkeys && sg[kl] == s0;
    return __all(row_ok && seg_q == s0 && key_ok);
}

// The ids of the block's query rows and of up to NT * kSegKeysPerThread keys are requested in one
// round trip (indices clamped, no load under a branch); longer key ranges read the rest in a loop.
constexpr int kSegMaxTiles = 512, kSegKeysPerThread = 8;
template <int NT, int BKEY>
__device__ int segment_tiles(const int32_t* seg, int row0, int nrows, int S, int nkeys, int nkt, short* list,
                             unsigned char* flag, int* lohi) {
    const int tid = threadIdx.x;
    const int rv = seg[min(row0 + min(tid, nrows - 1), S - 1)];
    int kv[kSegKeysPerThread];
#pragma unroll
    for (int i = 0; i < kSegKeysPerThread; i++) kv[i] = seg[min(tid + NT * i, nkeys - 1)];
    if (tid == 0) {
        lohi[0] = 0x7fffffff;
        lohi[1] = (int)0x80000000;
    }
    for (int t = tid; t < nkt; t += NT) flag[t] = 0;
    __syncthreads();
    if (tid < nrows && row0 + tid < S) {
        atomicMin(lohi, rv);
        atomicMax(lohi + 1, rv);
    }
    for (int r = tid + NT; r < nrows; r += NT)  // blocks of more than NT rows
        if (row0 + r < S) {
            const int sv = seg[row0 + r];
            atomicMin(lohi, sv);
            atomicMax(lohi + 1, sv);
        }
    __syncthreads();
    const int lo = lohi[0], hi = lohi[1];
#pragma unroll
    for (int i = 0; i < kSegKeysPerThread; i++) {
        const int k = tid + NT * i;
        if (k < nkeys && kv[i] >= lo && kv[i] <= hi) flag[k / BKEY] = 1;
    }
    for (int k = tid + NT * kSegKeysPerThread; k < nkeys; k += NT) {
        const int sv = seg[k];
        if (sv >= lo && sv <= hi) flag[k / BKEY] = 1;
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        for (int t = 0; t < nkt; t++)
            if (flag[t]) list[n++] = (short)t;
        lohi[2] = n;
    }
    __syncthreads();
    return lohi[2];
}

// ============================================================== prefill, bf16
// A block covers 64 query rows of one head with 2 * KP wavefronts: wavefronts
// w, w + 2, ... own the same 32 rows and take every KP-th 64-key tile (KP
// tiles are staged per iteration), which divides the sequential key chain of
// the longest (last, causal) row block by KP; their (m, l, O) merge through
// LDS at the end. KP = 2 (4 wavefronts, two blocks per CU for heads up to 80
// wide) or KP = 4 (8 wavefronts, one block per CU: used when the grid has no
// more blocks than CUs, where two blocks per CU would leave half the wavefront
// slots empty).
// DQ: width of q and k rows, DV: width of v and output rows (equal except for expanded MLA).
// PACK (a few query rows, causal or no mask): the block's 64 rows are the (query head, row) pairs
// of one KV head (blockIdx.y), row r = local head r / S, row r % S, so the KV head's keys are read
// once for all its query heads; blockIdx.x takes a.split_tiles key tiles, and the block writes
// unnormalised (o, m, l) partials [(row * nq + head) * gridDim.x + split][DV + 4] to a.part for
// the decode merge kernel.
template <int DQ, int DV, int MASK, int KP, bool PACK = false>
__global__ __launch_bounds__(128 * KP, (DQ <= 80 && KP == 2) ? 2 : 1) void attn_prefill_bf16(AttnArgs a) {
    constexpr int BQ = 64, BKEY = 64, NT = 128 * KP;
    // a q/k width that is not a multiple of 16 (72) is zero-padded to DK * 16 in the K tile and
    // the q fragments, which leaves every dot product unchanged
    constexpr int DK = (DQ + 15) / 16, NB = (DV + 31) / 32, DP = NB * 32, DQP = DK * 16;
    constexpr int LDK = DQP + 8, LDV = BKEY + 8;
    constexpr int CH = DQ / 8, CHV = DV / 8;  // 16-byte chunks per key / value row
    constexpr int KSZ = BKEY * LDK, VSZ = DP * LDV;                 // elements of one K / V^T tile
    constexpr int MRG = NB * 16 + 2;                                // floats per lane in the final merge
    constexpr int TILE_BYTES = KP * (KSZ + VSZ) * 2, MRG_BYTES = (KP - 1) * 2 * 64 * MRG * 4;
    __shared__ __attribute__((aligned(16))) unsigned char sm[TILE_BYTES > MRG_BYTES ? TILE_BYTES : MRG_BYTES];
    bf16_t* const Ks = reinterpret_cast<bf16_t*>(sm);   // [KP][KSZ]
    bf16_t* const Vt = Ks + KP * KSZ;                    // [KP][VSZ]

    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, hh = lane / 32, l32 = lane % 32;
    const int rg = w & 1, kpar = w >> 1;  // row group, key-tile parity
    const int S = a.S, G = a.nq / a.nkv;
    // PACK: lane row r = q0 + l32 is query row r % S of head g * G + r / S (valid below G * S)
    const int hq = PACK ? blockIdx.y * G + min((rg * 32 + l32) / S, G - 1) : blockIdx.y, g = hq / G;
    const int q0 = PACK ? rg * 32 : blockIdx.x * BQ + rg * 32;
    const int qrow = PACK ? (q0 + l32) % S : q0 + l32;  // the lane's query row (position pos0 + qrow)
    const bool qvalid = PACK ? q0 + l32 < G * S : qrow < S;
    const bf16_t* Q = (const bf16_t*)a.q + (size_t)hq * a.ldq * DQ;
    const bf16_t* Kg = (const bf16_t*)a.k + (size_t)g * a.ldkv * DQ;
    const bf16_t* Vg = (const bf16_t*)a.v + (size_t)g * a.ldkv * DV;

    for (int i = tid; i < (DP - DV) * LDV; i += NT)
#pragma unroll
        for (int b = 0; b < KP; b++) Vt[b * VSZ + DV * LDV + i] = 0;
    if constexpr (DQP > DQ) {  // pad columns of every K tile (the stages write columns < DQ only)
        for (int i = tid; i < BKEY * (DQP - DQ); i += NT) {
            const int r = i / (DQP - DQ), c = DQ + i % (DQP - DQ);
#pragma unroll
            for (int b = 0; b < KP; b++) Ks[b * KSZ + r * LDK + c] = 0;
        }
    }

    bf16x8 Qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; kk++) {
        if (qvalid && kk * 16 + hh * 8 < DQ) {
            Qf[kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)qrow * DQ + kk * 16 + hh * 8);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) Qf[kk][i] = (__bf16)0.0f;
        }
    }
    f32x16 oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[nb][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float scale = kLog2e / sqrtf((float)DQ);

    int kend = a.nkeys;
    if (MASK == VLM_MASK_CAUSAL_ID && !PACK) {
        const int last = min(S, (int)(blockIdx.x + 1) * BQ) - 1;
        kend = min(kend, a.pos0 + last + 1);
    }
    const int seg_q = (MASK == VLM_MASK_SEGMENT_ID && qrow < S) ? a.seg[qrow] : 0;
    const int nkt = (kend + BKEY - 1) / BKEY;
    // tiles visited, in order: all of them, or under a segment mask those that can hold a visible key
    // (PACK: this block's a.split_tiles tiles)
    const int tfirst = PACK ? (int)blockIdx.x * a.split_tiles : 0;
    int nvis = PACK ? max(0, min(nkt, tfirst + a.split_tiles) - tfirst) : nkt;
    __shared__ short tlist[MASK == VLM_MASK_SEGMENT_ID ? kSegMaxTiles : 1];
    __shared__ unsigned char tflag[MASK == VLM_MASK_SEGMENT_ID ? kSegMaxTiles : 1];
    __shared__ int tlohi[3];
    const bool listed = MASK == VLM_MASK_SEGMENT_ID && nkt <= kSegMaxTiles;
    if constexpr (MASK == VLM_MASK_SEGMENT_ID)
        if (listed) nvis = segment_tiles<NT, BKEY>(a.seg, blockIdx.x * BQ, BQ, S, a.nkeys, nkt, tlist, tflag, tlohi);
    auto tile_at = [&](int i) { return listed ? (int)tlist[i] : tfirst + i; };

    // K/V tile kt+1 is requested into registers (unconditional, key index clamped; keys past nkeys
    // are zeroed when stored) while tile kt runs on the matrix cores. K chunks are spread along rows
    // (coalesced 16-byte row pieces into the row-major K tile); V is fetched as key pairs so that
    // each transposed LDS store writes two keys of one dimension as a dword, 32 lanes to 32
    // consecutive dwords.
    constexpr int TCH = (BKEY * CH + NT - 1) / NT;        // 16-byte chunks of the K tile per thread
    constexpr int NVP = (BKEY / 2) * CHV, VP = (NVP + NT - 1) / NT;  // (key pair, chunk) items of the V tile
    // the segment ids of a tile's keys travel with its K/V: requested with them (every thread, key
    // tid % BKEY), stored to LDS by the first BKEY threads
    __shared__ int segs[MASK == VLM_MASK_SEGMENT_ID ? KP : 1][MASK == VLM_MASK_SEGMENT_ID ? BKEY : 1];
    auto request = [&](int kt, u32x4 (&kreg)[TCH], u32x4 (&vreg)[VP][2], int& sreg) {
        if constexpr (MASK == VLM_MASK_SEGMENT_ID) sreg = a.seg[min(kt * BKEY + tid % BKEY, a.nkeys - 1)];
#pragma unroll
        for (int i = 0; i < TCH; i++) {
            const int c = min(tid + NT * i, BKEY * CH - 1), r = c / CH, d0 = (c % CH) * 8;
            const int key = min(kt * BKEY + r, a.nkeys - 1);
            kreg[i] = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * DQ + d0);
        }
#pragma unroll
        for (int i = 0; i < VP; i++) {
            const int pi = min(tid + NT * i, NVP - 1), kp = pi % (BKEY / 2), d0 = (pi / (BKEY / 2)) * 8;
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int key = min(kt * BKEY + 2 * kp + u, a.nkeys - 1);
                vreg[i][u] = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * DV + d0);
            }
        }
    };
    auto stage = [&](int kt, int buf, const u32x4 (&kreg)[TCH], const u32x4 (&vreg)[VP][2], int sreg) {
        const int key0 = kt * BKEY;
        if constexpr (MASK == VLM_MASK_SEGMENT_ID)
            if (tid < BKEY) segs[buf][tid] = sreg;
        bf16_t* kd = Ks + buf * KSZ;
        bf16_t* vd = Vt + buf * VSZ;
#pragma unroll
        for (int i = 0; i < TCH; i++) {
            const int c = tid + NT * i;
            if (c < BKEY * CH) {
                const int r = c / CH, d0 = (c % CH) * 8;
                *reinterpret_cast<u32x4*>(kd + r * LDK + d0) = key0 + r < a.nkeys ? kreg[i] : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < VP; i++) {
            const int pi = tid + NT * i, kp = pi % (BKEY / 2), d0 = (pi / (BKEY / 2)) * 8;
            if (pi >= NVP) break;
            const u32x4 v0 = key0 + 2 * kp < a.nkeys ? vreg[i][0] : u32x4{0, 0, 0, 0};
            const u32x4 v1 = key0 + 2 * kp + 1 < a.nkeys ? vreg[i][1] : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                uint32_t* row0 = reinterpret_cast<uint32_t*>(vd + (d0 + 2 * e) * LDV + 2 * kp);
                uint32_t* row1 = reinterpret_cast<uint32_t*>(vd + (d0 + 2 * e + 1) * LDV + 2 * kp);
                *row0 = (v0[e] & 0xffffu) | (v1[e] << 16);
                *row1 = (v0[e] >> 16) | (v1[e] & 0xffff0000u);
            }
        }
    };
    u32x4 kr[KP][TCH], vr[KP][VP][2];
    int sr[KP];
#pragma unroll
    for (int b = 0; b < KP; b++) {
        sr[b] = 0;
        if (b < nvis) request(tile_at(b), kr[b], vr[b], sr[b]);
    }
    for (int kt2 = 0; kt2 < nvis; kt2 += KP) {
#pragma unroll
        for (int b = 0; b < KP; b++)
            if (kt2 + b < nvis) stage(tile_at(kt2 + b), b, kr[b], vr[b], sr[b]);
        __syncthreads();
        // the next KP tiles are in flight during these tiles' MFMAs
#pragma unroll
        for (int b = 0; b < KP; b++)
            if (kt2 + KP + b < nvis) request(tile_at(kt2 + KP + b), kr[b], vr[b], sr[b]);
        const int kv = kt2 + kpar;  // position in the visit order
        const int key0 = (kv < nvis ? tile_at(kv) : 0) * BKEY;
        const bf16_t* const Kw = Ks + kpar * KSZ;
        const bf16_t* const Vw = Vt + kpar * VSZ;
        bool active = kv < nvis;
        // the row group's lowest and highest query rows (PACK: rows 0 .. S - 1 of each head)
        const int qlo = PACK ? 0 : q0, qhi = PACK ? S - 1 : q0 + 31;
        if (PACK) active = active && q0 < G * S;
        if (MASK == VLM_MASK_CAUSAL_ID) active = active && key0 <= a.pos0 + qhi;
        if (active) {
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) sacc[kb][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < DK; kk++) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kw + (kb * 32 + l32) * LDK + kk * 16 + hh * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, Qf[kk], sacc[kb], 0, 0, 0);
                }
            }
            // a tile every key of which is visible to every query row of this wavefront skips the mask
            bool full = (MASK == VLM_MASK_NONE_ID ||
                         (MASK == VLM_MASK_CAUSAL_ID && key0 + BKEY - 1 <= a.pos0 + qlo)) &&
                        key0 + BKEY <= a.nkeys;
            if constexpr (MASK == VLM_MASK_SEGMENT_ID)
                full = segment_tile_full<BKEY>(segs[kpar], seg_q, qrow < S, key0, a.nkeys);
            float mt = -INFINITY;
            // wavefront-uniform: one scalar branch per tile (the segment mask keeps the test per
            // element: its two loop bodies together would spill)
            if (MASK != VLM_MASK_SEGMENT_ID && __builtin_amdgcn_readfirstlane((int)full)) {
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        sacc[kb][r] *= scale;
                        mt = fmaxf(mt, sacc[kb][r]);
                    }
            } else {
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = key0 + kb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                    float s = sacc[kb][r] * scale;
                    if (MASK == VLM_MASK_SEGMENT_ID && full) {
                        sacc[kb][r] = s;
                        mt = fmaxf(mt, s);
                        continue;
                    }
                    bool vis = key < a.nkeys;
                    if (MASK == VLM_MASK_CAUSAL_ID) vis = vis && key <= a.pos0 + qrow;
                    if (MASK == VLM_MASK_SEGMENT_ID) vis = vis && qrow < S && segs[kpar][key - key0] == seg_q;
                    if (MASK == VLM_MASK_ADDITIVE_ID && vis && qrow < S)
                        s += a.add[(size_t)qrow * a.ld_add + key] * kLog2e;
                    s = vis ? s : -INFINITY;
                    sacc[kb][r] = s;
                    mt = fmaxf(mt, s);
                }
            }
            {
                const LanePair h2 = swap32(mt);
                mt = fmaxf(h2.lo, h2.hi);
            }
            const float mn = fmaxf(m, mt);
            const float mu = mn == -INFINITY ? 0.f : mn;
            // arguments are <= 0 (or -inf): the bare v_exp_f32 needs no range reduction
            const float alpha = __builtin_amdgcn_exp2f(m - mu);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float p = __builtin_amdgcn_exp2f(sacc[kb][r] - mu);
                    sacc[kb][r] = p;
                    rs += p;
                }
            {
                const LanePair h2 = swap32(rs);
                rs = h2.lo + h2.hi;
            }
            l = l * alpha + rs;
            m = mn;
            if (!__all(alpha == 1.f)) {  // the running max moved for some row of this wavefront
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[nb][r] *= alpha;
            }
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int hs = 0; hs < 2; hs++) {
                    // P = hi + lo with both parts bf16: the product with V keeps ~16
                    // significant bits of P instead of 8.
                    bf16x8 phi, plo;
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const float p = sacc[kb][hs * 8 + i];
                        const bf16_t b = f2bf(p);
                        phi[i] = __builtin_bit_cast(__bf16, b);
                        plo[i] = __builtin_bit_cast(__bf16, f2bf(p - bf2f(b)));
                    }
                    const int kofs = kb * 32 + hs * 16 + hh * 4;
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const bf16_t* vp = Vw + (nb * 32 + l32) * LDV + kofs;
                        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
                        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
                        u32x4 raw = {lo.x, lo.y, hi.x, hi.y};
                        const bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
                        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi, oacc[nb], 0, 0, 0);
                        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo, oacc[nb], 0, 0, 0);
                    }
                }
        }
        __syncthreads();
    }
    // merge the KP key parities of each row group: wavefronts 2, 3, ... hand (m, l, O) to 0, 1
    float* const mbase = reinterpret_cast<float*>(sm);
    if (kpar > 0) {
        float* mb = mbase + (size_t)(((kpar - 1) * 2 + rg) * 64 + lane) * MRG;
        mb[0] = m;
        mb[1] = l;
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) mb[2 + nb * 16 + r] = oacc[nb][r];
    }
    __syncthreads();
    if (kpar > 0) return;
#pragma unroll
    for (int pp = 1; pp < KP; pp++) {
        const float* mb = mbase + (size_t)(((pp - 1) * 2 + rg) * 64 + lane) * MRG;
        const float m2 = mb[0], l2 = mb[1];
        const float mn = fmaxf(m, m2);
        const float fa = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float fb = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
        l = l * fa + l2 * fb;
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) oacc[nb][r] = oacc[nb][r] * fa + mb[2 + nb * 16 + r] * fb;
        m = mn;
    }
    if constexpr (PACK) {
        if (qvalid) {
            float* pr = a.part + ((size_t)(qrow * a.nq + hq) * gridDim.x + blockIdx.x) * (DV + 4);
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int n = nb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                    if (n < DV) pr[n] = oacc[nb][r];
                }
            if (hh == 0) {
                pr[DV] = m;
                pr[DV + 1] = l;
            }
        }
        return;
    }
    if (qrow < S) {
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        bf16_t* O = (bf16_t*)a.out + (size_t)qrow * a.nq * DV + (size_t)hq * DV;
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int n = nb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                if (n < DV) O[n] = f2bf(oacc[nb][r] * inv);
            }
    }
}

// ============================================================== prefill, f32
template <int DQ, int DV, int MASK>
__global__ __launch_bounds__(256) void attn_prefill_f32(AttnArgs a) {
    constexpr int BQ = 128, KB = DQ >= 128 ? 1 : 2, BKEY = 32 * KB;
    constexpr int NB = (DV + 31) / 32, DP = NB * 32;
    constexpr int LDK = DQ + 4, LDV = DP + 4;
    constexpr int CH = DQ / 4, CHV = DV / 4;
    // two K / V tile buffers: tile kv + 1 is requested into registers while tile kv runs on the
    // matrix cores, and stored into the other buffer after it (one barrier per tile)
    __shared__ __attribute__((aligned(16))) float Ks[2][BKEY * LDK];
    __shared__ __attribute__((aligned(16))) float Vs[2][BKEY * LDV];

    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, hh = lane / 32, l32 = lane % 32;
    const int hq = blockIdx.y, g = hq / (a.nq / a.nkv);
    const int q0 = blockIdx.x * BQ + w * 32;
    const int qrow = q0 + l32;
    const int S = a.S;
    const float* Q = (const float*)a.q + (size_t)hq * a.ldq * DQ;
    const float* Kg = (const float*)a.k + (size_t)g * a.ldkv * DQ;
    const float* Vg = (const float*)a.v + (size_t)g * a.ldkv * DV;

    if constexpr (DP > DV) {
        for (int i = tid; i < BKEY * (DP - DV); i += 256)
#pragma unroll
            for (int b = 0; b < 2; b++) Vs[b][(i / (DP - DV)) * LDV + DV + i % (DP - DV)] = 0.f;
    }

    float Qf[DQ / 2];
#pragma unroll
    for (int kk = 0; kk < DQ / 2; kk++) Qf[kk] = qrow < S ? Q[(size_t)qrow * DQ + kk * 2 + hh] : 0.f;
    f32x16 oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[nb][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float scale = kLog2e / sqrtf((float)DQ);

    int kend = a.nkeys;
    if (MASK == VLM_MASK_CAUSAL_ID) {
        const int last = min(S, (int)(blockIdx.x + 1) * BQ) - 1;
        kend = min(kend, a.pos0 + last + 1);
    }
    const int seg_q = (MASK == VLM_MASK_SEGMENT_ID && qrow < S) ? a.seg[qrow] : 0;
    const int nkt = (kend + BKEY - 1) / BKEY;
    // tiles visited, in order: all of them, or under a segment mask those that can hold a visible key
    int nvis = nkt;
    __shared__ short tlist[MASK == VLM_MASK_SEGMENT_ID ? kSegMaxTiles : 1];
    __shared__ unsigned char tflag[MASK == VLM_MASK_SEGMENT_ID ? kSegMaxTiles : 1];
    __shared__ int tlohi[3];
    const bool listed = MASK == VLM_MASK_SEGMENT_ID && nkt <= kSegMaxTiles;
    if constexpr (MASK == VLM_MASK_SEGMENT_ID)
        if (listed) nvis = segment_tiles<256, BKEY>(a.seg, blockIdx.x * BQ, BQ, S, a.nkeys, nkt, tlist, tflag, tlohi);

    __shared__ int segs[2][MASK == VLM_MASK_SEGMENT_ID ? BKEY : 1];  // the tiles' segment ids
    auto tile_at = [&](int i) { return listed ? (int)tlist[i] : i; };
    // K / V chunks of a tile: requested unconditionally (indices clamped), keys past nkeys zeroed when
    // stored; the segment ids travel with them
    constexpr int KCH = (BKEY * CH + 255) / 256, VCH = (BKEY * CHV + 255) / 256;
    f32x4 kreg[KCH], vreg[VCH];
    int sreg = 0;
    auto request = [&](int kt) {
        const int key0 = kt * BKEY;
        if constexpr (MASK == VLM_MASK_SEGMENT_ID) sreg = a.seg[min(key0 + tid % BKEY, a.nkeys - 1)];
#pragma unroll
        for (int i = 0; i < KCH; i++) {
            const int c = min(tid + 256 * i, BKEY * CH - 1), r = c / CH, d0 = (c % CH) * 4;
            kreg[i] = *reinterpret_cast<const f32x4*>(Kg + (size_t)min(key0 + r, a.nkeys - 1) * DQ + d0);
        }
#pragma unroll
        for (int i = 0; i < VCH; i++) {
            const int c = min(tid + 256 * i, BKEY * CHV - 1), r = c / CHV, d0 = (c % CHV) * 4;
            vreg[i] = *reinterpret_cast<const f32x4*>(Vg + (size_t)min(key0 + r, a.nkeys - 1) * DV + d0);
        }
    };
    auto stage = [&](int kt, int buf) {
        const int key0 = kt * BKEY;
        if constexpr (MASK == VLM_MASK_SEGMENT_ID)
            if (tid < BKEY) segs[buf][tid] = sreg;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KCH; i++) {
            const int c = tid + 256 * i, r = c / CH, d0 = (c % CH) * 4;
            if (c < BKEY * CH) *reinterpret_cast<f32x4*>(&Ks[buf][r * LDK + d0]) = key0 + r < a.nkeys ? kreg[i] : zero;
        }
#pragma unroll
        for (int i = 0; i < VCH; i++) {
            const int c = tid + 256 * i, r = c / CHV, d0 = (c % CHV) * 4;
            if (c < BKEY * CHV) *reinterpret_cast<f32x4*>(&Vs[buf][r * LDV + d0]) = key0 + r < a.nkeys ? vreg[i] : zero;
        }
    };
    if (nvis > 0) {
        request(tile_at(0));
        stage(tile_at(0), 0);
    }
    __syncthreads();
    for (int kv = 0; kv < nvis; kv++) {
        const int buf = kv & 1;
        const int key0 = tile_at(kv) * BKEY;
        if (kv + 1 < nvis) request(tile_at(kv + 1));
        const float* const Kb = Ks[buf];
        const float* const Vb = Vs[buf];
        bool active = true;
        if (MASK == VLM_MASK_CAUSAL_ID) active = key0 <= a.pos0 + q0 + 31;
        if (active) {
            f32x16 sacc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; kb++) {
#pragma unroll
                for (int r = 0; r < 16; r++) sacc[kb][r] = 0.f;
                const float* kr = Kb + (kb * 32 + l32) * LDK + hh;
#pragma unroll
                for (int kk = 0; kk < DQ / 2; kk++)
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[kk * 2], Qf[kk], sacc[kb], 0, 0, 0);
            }
            bool full = false;  // segment mask: the whole tile lies in this wavefront's one segment
            if constexpr (MASK == VLM_MASK_SEGMENT_ID)
                full = segment_tile_full<BKEY>(segs[buf], seg_q, qrow < S, key0, a.nkeys);
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = key0 + kb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                    float s = sacc[kb][r] * scale;
                    bool vis = key < a.nkeys;
                    if (MASK == VLM_MASK_CAUSAL_ID) vis = vis && key <= a.pos0 + qrow;
                    if (MASK == VLM_MASK_SEGMENT_ID) vis = full || (vis && qrow < S && segs[buf][key - key0] == seg_q);
                    if (MASK == VLM_MASK_ADDITIVE_ID && vis && qrow < S)
                        s += a.add[(size_t)qrow * a.ld_add + key] * kLog2e;
                    s = vis ? s : -INFINITY;
                    sacc[kb][r] = s;
                    mt = fmaxf(mt, s);
                }
            {
                const LanePair h2 = swap32(mt);
                mt = fmaxf(h2.lo, h2.hi);
            }
            const float mn = fmaxf(m, mt);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float alpha = exp2f(m - mu);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float p = exp2f(sacc[kb][r] - mu);
                    sacc[kb][r] = p;
                    rs += p;
                }
            {
                const LanePair h2 = swap32(rs);
                rs = h2.lo + h2.hi;
            }
            l = l * alpha + rs;
            m = mn;
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
#pragma unroll
                for (int r = 0; r < 16; r++) oacc[nb][r] *= alpha;
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int kl = kb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                    const float* vr = Vb + kl * LDV + l32;
#pragma unroll
                    for (int nb = 0; nb < NB; nb++)
                        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[nb * 32], sacc[kb][r], oacc[nb], 0, 0, 0);
                }
        }
        // the other buffer was last read in the previous iteration, before its closing barrier
        if (kv + 1 < nvis) stage(tile_at(kv + 1), buf ^ 1);
        __syncthreads();
    }
    if (qrow < S) {
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float* O = (float*)a.out + (size_t)qrow * a.nq * DV + (size_t)hq * DV;
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int n = nb * 32 + (r / 4) * 8 + hh * 4 + (r % 4);
                if (n < DV) O[n] = oacc[nb][r] * inv;
            }
    }
}

static int attn_cus() {
    static const int v = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        return n;
    }();
    return v;
}

// A few query rows (bf16, causal or no mask, the rows of all query heads of a KV head in one
// 64-row tile): blocks over (key-tile range, KV head) writing partials, then the decode merge
// kernel (partial row (row, head) = decode "head" row * nq + head, so it writes [S][nq][DV]).
// The row-tiled launch would give each query head its own block reading the KV head's keys, with
// at most S of its 64 rows in use. Returns hipErrorNotSupported when the launch does not apply.
template <int DQ, int DV, int MASK>
static hipError_t run_prefill_few(const AttnArgs& a, hipStream_t st) {
    if constexpr ((MASK == VLM_MASK_CAUSAL_ID || MASK == VLM_MASK_NONE_ID) && DQ % 8 == 0 && DV % 8 == 0 &&
                  (DV == 64 || DV == 80 || DV == 128)) {
        const char* e = getenv("VLM_FEW_ROWS");  // bit 1 clear: the row-tiled kernel for every row count
        if ((e && !(atoi(e) & 2)) || !a.part || a.nkv < 1 || a.nq % a.nkv != 0) return hipErrorNotSupported;
        if ((a.nq / a.nkv) * a.S > 64) return hipErrorNotSupported;
        const int ntiles = (a.nkeys + 63) / 64;
        if (ntiles < 1) return hipErrorNotSupported;
        const int tps = std::max(2, (ntiles + kDecMaxSplits - 1) / kDecMaxSplits);
        const int nsplit = (ntiles + tps - 1) / tps;
        if ((size_t)a.S * a.nq * nsplit * (DV + 4) > a.part_cap) return hipErrorNotSupported;
        AttnArgs b = a;
        b.split_tiles = tps;
        attn_prefill_bf16<DQ, DV, MASK, 2, true><<<dim3(nsplit, a.nkv), 256, 0, st>>>(b);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        return launch_attn_combine(1, a.part, a.S * a.nq, nsplit, DV, a.out, st);
    } else {
        return hipErrorNotSupported;
    }
}

template <int DQ, int DV, int MASK>
static hipError_t run_prefill(int dtype, const AttnArgs& a, hipStream_t st) {
    dim3 grid((a.S + 127) / 128, a.nq);
    if (dtype == 1) {
        const hipError_t fe = run_prefill_few<DQ, DV, MASK>(a, st);
        if (fe != hipErrorNotSupported) return fe;
        if constexpr (DQ % 8 == 0 && DV % 8 == 0) {
            const dim3 g64((a.S + 63) / 64, a.nq);
            bool kp4 = false;  // one block per CU anyway: 8 wavefronts, 4 key parities (LDS: heads up to 128)
            if constexpr (DQ <= 128) kp4 = (int)(g64.x * g64.y) <= attn_cus();
            if constexpr (DQ <= 128)
                if (kp4) attn_prefill_bf16<DQ, DV, MASK, 4><<<g64, 512, 0, st>>>(a);
            if (!kp4) attn_prefill_bf16<DQ, DV, MASK, 2><<<g64, 256, 0, st>>>(a);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        attn_prefill_f32<DQ, DV, MASK><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

template <int DQ, int DV>
static hipError_t prefill_mask(int dtype, const AttnArgs& a, hipStream_t st) {
    switch (a.mask_kind) {
        case VLM_MASK_CAUSAL_ID: return run_prefill<DQ, DV, VLM_MASK_CAUSAL_ID>(dtype, a, st);
        case VLM_MASK_NONE_ID: return run_prefill<DQ, DV, VLM_MASK_NONE_ID>(dtype, a, st);
        case VLM_MASK_ADDITIVE_ID: return run_prefill<DQ, DV, VLM_MASK_ADDITIVE_ID>(dtype, a, st);
        case VLM_MASK_SEGMENT_ID: return run_prefill<DQ, DV, VLM_MASK_SEGMENT_ID>(dtype, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_prefill(int dtype, const AttnArgs& a, hipStream_t st) {
    if (a.S <= 0) return hipSuccess;
    const int dv = a.dv > 0 ? a.dv : a.d;
    if (dv != a.d) {  // expanded MLA heads: keys 192 wide (128 + 64 rotated), values 128
        if (a.d == 192 && dv == 128 && (a.mask_kind == VLM_MASK_CAUSAL_ID || a.mask_kind == VLM_MASK_ADDITIVE_ID))
            return a.mask_kind == VLM_MASK_CAUSAL_ID ? run_prefill<192, 128, VLM_MASK_CAUSAL_ID>(dtype, a, st)
                                                     : run_prefill<192, 128, VLM_MASK_ADDITIVE_ID>(dtype, a, st);
        return hipErrorInvalidValue;
    }
    switch (a.d) {
        case 64: return prefill_mask<64, 64>(dtype, a, st);
        case 72: return prefill_mask<72, 72>(dtype, a, st);
        case 80: return prefill_mask<80, 80>(dtype, a, st);
        case 128: return prefill_mask<128, 128>(dtype, a, st);
    }
    return hipErrorInvalidValue;
}

// ============================================================== decode, fused
// One block of kDecWaves wavefronts per (KV head g, split sp); split sp owns the
// slots [sp*chunk, (sp+1)*chunk) of the window, of which those below T = t+1
// are valid. The host sizes the splits for the band of positions it decodes
// (attn_decode_plan); the device length t is read by the kernel. Each 16-lane
// quarter of a wavefront scores
// one key per step (a step covers 4 keys per wavefront). Phases:
//  1. the block's K/V rows, the projections it rotates (q heads of g, the
//     new k and v), their norm gains and the RoPE row of position t (staged
//     once per token by the embed kernel) are requested first: none of these
//     addresses depends on the device length t, so no request waits for it;
//  2. QK-Norm + RoPE run while K/V are in flight; with t known, the block
//     owning slot t writes the new k and v into the cache;
//  3. softmax over the block's valid slots, one max/rescale per batch of
//     steps, merged across the quarters and wavefronts into one (o, m, l)
//     partial per query head; attn_combine_fast_kernel merges the splits.
// Loads are unconditional within a step that exists (indices clamped into
// range) and raw data is converted only after the batch is requested.
constexpr int kDecWaves = 4;  // wavefronts per block
constexpr int kDecSteps = 8;  // key steps requested in one batch (fewer for 4 or 8 heads per KV head)

// Splits: slots [0, tb) of a band in up to kDecMaxSplits splits of a
// multiple of 16 slots (the keys a block scores per step). A block streams at
// most ~50 GB/s, so the KV read wants >= ~128 blocks in flight; fewer, longer
// splits lengthen each block's serial scoring chain. (Measured on the 28-layer
// stack's shape at 624 valid slots: 4 wavefronts x 32 splits 5.1 us,
// 8 x 16 5.6 us, 2 x 64 5.8 us.)
// VLM_DEC_SPLITS (1..kDecMaxSplits) caps the splits, for tuning. Measured on
// the 36-layer stack (positions 512..767), vector-ALU form: a cap of 32 gives
// 465.8 ms per 256-token decode, 16 467.1 ms, 48 and 64 (with a 64-split
// maximum) 473.5 ms; matrix-core form (one box): 32 454.6 ms, 16 453.9 ms,
// 8 458.9 ms, 4 466.9 ms.
// Read at every plan, so a process can compare plans (a graph keeps the plan it was captured with).
static int dec_split_cap() {
    const char* e = getenv("VLM_DEC_SPLITS");
    const int n = e ? atoi(e) : 32;
    return n < 1 ? 1 : (n > kDecMaxSplits ? kDecMaxSplits : n);
}

DecSplitPlan attn_decode_plan(int capacity, int t) {
    constexpr int unit = kDecWaves * 4;
    const int cap = dec_split_cap();
    DecSplitPlan p;
    p.band = (t < 0 ? 0 : t) / kDecBand;
    const int tb = std::max(1, std::min(capacity, (p.band + 1) * kDecBand));
    p.chunk = unit * ((tb + unit * cap - 1) / (unit * cap));
    p.nsplit = (tb + p.chunk - 1) / p.chunk;
    return p;
}

// The rotation phase of a decode attention block for KV head g, shared by both
// forms: wavefront w takes the items w, w + NW, ... of (the G q heads of the
// group, the new k, the new v); lane i < D/2 holds rotation pair i. load()
// requests the projections, norm gains and the RoPE row of position t (staged
// once per token by the embed kernel): no address depends on the device
// length, so nothing waits for it. apply() runs QK-Norm + RoPE, leaves the
// rounded q heads in qs and, in the block owning slot t, the new k / v in
// knew / vnew and in the cache.
template <class T, int D, int G, int NW>
struct DecRotation {
    static constexpr int NI = (G + 2 + NW - 1) / NW;  // items per wavefront
    float x0[NI], x1[NI], g0[NI], g1[NI];
    float c0, c1, s0, s1;
    int i0, i1;
    bool on;

    __device__ __forceinline__ void load(const DecAttnArgs& a, int g, int w, int lane) {
        const int half = D / 2, sd = D / a.segments, sh = sd / 2;
        on = lane < half;
        const int lp = on ? lane : 0;
        i0 = (lp / sh) * sd + lp % sh;
        i1 = i0 + sh;
        // inputs of a rotated head: the adjacent pair for interleaved RoPE (V keeps i0, i1)
        const int r0 = a.interleave ? (lp / sh) * sd + 2 * (lp % sh) : i0, r1 = a.interleave ? r0 + 1 : i1;
        // gain index: input order if the norm runs before the rotation, output order after it
        const int n0 = a.norm_after ? i0 : r0, n1 = a.norm_after ? i1 : r1;
#pragma unroll
        for (int ii = 0; ii < NI; ii++) {
            const int it = min(w + ii * NW, G + 1);
            const bool isq = it < G, isk = it == G;
            const int row = isq ? g * G + it : (isk ? a.nq + g : a.nq + a.nkv + g);
            const float* src = a.qkv + (size_t)row * D;
            const T* gn = (const T*)(isq ? a.qn : a.kn);
            const T* gp = (it <= G && gn) ? gn : (const T*)a.kc;  // any valid address when unused
            x0[ii] = src[it <= G ? r0 : i0];
            x1[ii] = src[it <= G ? r1 : i1];
            g0[ii] = Elt<T>::ld(gp, n0);
            g1[ii] = Elt<T>::ld(gp, n1);
        }
        c0 = a.rope[i0];
        c1 = a.rope[i1];
        s0 = a.rope[D + i0];
        s1 = a.rope[D + i1];
    }

    __device__ __forceinline__ void apply(const DecAttnArgs& a, int g, int w, int t, bool own, float (*qs)[D],
                                          T* knew, T* vnew) {
#pragma unroll
        for (int ii = 0; ii < NI; ii++) {
            const int it = w + ii * NW;
            if (it >= G + (own ? 2 : 0)) continue;  // uniform per wavefront
            const bool isq = it < G, isk = it == G;
            const bool rot = isq || isk, norm = rot && (isq ? a.qn : a.kn) != nullptr;
            float y0 = on ? x0[ii] : 0.f, y1 = on ? x1[ii] : 0.f;
            if (norm && !a.norm_after) {
                const float r = rsqrtf(wave_sum(y0 * y0 + y1 * y1) / (float)D + a.eps);
                y0 = y0 * r * g0[ii];
                y1 = y1 * r * g1[ii];
            }
            if (rot) {
                const float z0 = y0 * c0 - y1 * s0;
                const float z1 = y1 * c1 + y0 * s1;
                y0 = z0;
                y1 = z1;
            }
            if (norm && a.norm_after) {
                const float r = rsqrtf(wave_sum(y0 * y0 + y1 * y1) / (float)D + a.eps);
                y0 = y0 * r * g0[ii];
                y1 = y1 * r * g1[ii];
            }
            if (!on) continue;
            if (isq) {
                qs[it][i0] = Elt<T>::rnd(y0);
                qs[it][i1] = Elt<T>::rnd(y1);
            } else {
                T* cache = (T*)(isk ? a.kc : a.vc) + ((size_t)g * a.W + t) * D;
                T* lds = isk ? knew : vnew;
                Elt<T>::st(lds, i0, y0);
                Elt<T>::st(lds, i1, y1);
                Elt<T>::st(cache, i0, y0);
                Elt<T>::st(cache, i1, y1);
            }
        }
    }
};

template <class T, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_fused_kernel(DecAttnArgs a) {
    constexpr int VEC = 16 / sizeof(T), CH = D / VEC, CPL = (CH + 15) / 16, KSTEP = NW * 4;
    constexpr int PS = D + 4;  // partial row: o[D], m, l, pad
    constexpr int NB = G <= 2 ? kDecSteps : (G == 4 ? kDecSteps / 2 : kDecSteps / 4);  // steps per batch
    __shared__ float qs[G][D];
    __shared__ __attribute__((aligned(16))) T knew[D];
    __shared__ __attribute__((aligned(16))) T vnew[D];
    // LDS merge: one (m, l, o) partial per 16-lane quarter (NQ = NW * 4 of them) for groups of 4+
    // query heads whose partials fit (the register merge there costs 2 * G * 8 permlane swaps per
    // lane); otherwise the quarters merge in registers first and one partial per wavefront is stored
    constexpr bool QMERGE = G >= 4 && NW * 4 * G * D * 4 <= 48 * 1024;
    constexpr int NQ = QMERGE ? NW * 4 : NW;
    __shared__ float sm_m[NQ][G], sm_l[NQ][G];
    __shared__ float sm_o[NQ][G][D];
    const int g = blockIdx.x, sp = blockIdx.y;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, sub = lane % 16, kq = lane / 16;
    const int chunk = a.chunk;
    const int k0 = sp * chunk, kend = min(a.W, k0 + chunk);
    const int nst = kend > k0 ? (kend - k0 + KSTEP - 1) / KSTEP : 0;  // key steps of the slot range
    const T* Kg = (const T*)a.kc + (size_t)g * a.W * D;
    const T* Vg = (const T*)a.vc + (size_t)g * a.W * D;
    const int jl = max(kend - 1, 0);  // a valid slot for clamped requests

    // (1) K/V rows of the first batch, then the projections to rotate
    u32x4 kr[NB][CPL], vr[NB][CPL];
    const int jw = k0 + w * 4 + kq;  // this quarter's key in step 0
    auto request = [&](int s0) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            if (s0 + b < nst) {  // uniform over the block
                const int j = min(jw + (s0 + b) * KSTEP, jl);
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    const int ch = min(sub + 16 * c, CH - 1);
                    kr[b][c] = *reinterpret_cast<const u32x4*>(Kg + (size_t)j * D + ch * VEC);
                    vr[b][c] = *reinterpret_cast<const u32x4*>(Vg + (size_t)j * D + ch * VEC);
                }
            }
        }
    };
    request(0);
    DecRotation<T, D, G, NW> rot;
    rot.load(a, g, w, lane);
    __builtin_amdgcn_sched_barrier(0);

    // (2) the valid range, then QK-Norm + RoPE of q (G heads) and of the owner's new k / v
    const int t = a.len[0];
    const int k1 = min(t + 1, kend);
    const bool own = k0 <= t && t < kend;
    rot.apply(a, g, w, t, own, qs, knew, vnew);
    __syncthreads();

    float qf[G][CPL][VEC];
#pragma unroll
    for (int gg = 0; gg < G; gg++)
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            const int ch = min(sub + 16 * c, CH - 1);
#pragma unroll
            for (int i = 0; i < VEC; i++) qf[gg][c][i] = sub + 16 * c < CH ? qs[gg][ch * VEC + i] : 0.f;
        }
    const float scale = kLog2e / sqrtf((float)D);
    float mrun[G], lrun[G], o[G][CPL][VEC];
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
        mrun[gg] = -INFINITY;
        lrun[gg] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; c++)
#pragma unroll
            for (int i = 0; i < VEC; i++) o[gg][c][i] = 0.f;
    }
    // (3) softmax over this block's slots, one batch of steps at a time; K/V
    // stay packed in registers and are widened at use
    for (int s0 = 0; s0 < nst; s0 += NB) {
        if (s0 > 0) request(s0);
        float sc[G][NB];
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int j = jw + (s0 + b) * KSTEP;
            const bool valid = s0 + b < nst && j < k1;
            if (s0 + b >= nst) {  // uniform: a step past the slot range
#pragma unroll
                for (int gg = 0; gg < G; gg++) sc[gg][b] = -INFINITY;
#pragma unroll
                for (int c = 0; c < CPL; c++) vr[b][c] = u32x4{0, 0, 0, 0};
                continue;
            }
            float kf[CPL][VEC];
#pragma unroll
            for (int c = 0; c < CPL; c++) unpack16(kr[b][c], (const T*)nullptr, kf[c]);
            if (j == t) {  // the new slot: this token's rotated k and v
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    const int ch = min(sub + 16 * c, CH - 1);
                    ld16(knew + ch * VEC, kf[c]);
                    vr[b][c] = *reinterpret_cast<const u32x4*>(vnew + ch * VEC);
                }
            }
            if (!valid) {  // clamped or unrequested rows hold arbitrary bits: weight 0 must not meet NaN
#pragma unroll
                for (int c = 0; c < CPL; c++) vr[b][c] = u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int gg = 0; gg < G; gg++) {
                float sv = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; c++)
#pragma unroll
                    for (int i = 0; i < VEC; i++) sv = fmaf(qf[gg][c][i], kf[c][i], sv);
                sv = row16_sum(sv);  // the 16 lanes of this quarter hold one key row
                sc[gg][b] = valid ? sv * scale : -INFINITY;
            }
        }
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
            float mb = sc[gg][0];
#pragma unroll
            for (int b = 1; b < NB; b++)
                if (s0 + b < nst) mb = fmaxf(mb, sc[gg][b]);
            if (mb == -INFINITY) continue;  // no valid key of this quarter in the batch
            const float mn = fmaxf(mrun[gg], mb);
            const float alpha = exp2f(mrun[gg] - mn);
            lrun[gg] *= alpha;
            mrun[gg] = mn;
#pragma unroll
            for (int c = 0; c < CPL; c++)
#pragma unroll
                for (int i = 0; i < VEC; i++) o[gg][c][i] *= alpha;
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (s0 + b >= nst) break;  // uniform
                const float pb = exp2f(sc[gg][b] - mn);
                lrun[gg] += pb;
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    float vf[VEC];
                    unpack16(vr[b][c], (const T*)nullptr, vf);
#pragma unroll
                    for (int i = 0; i < VEC; i++) o[gg][c][i] = fmaf(pb, vf[i], o[gg][c][i]);
                }
            }
        }
    }
    if constexpr (QMERGE) {
        // every quarter stores its partial; the block merges the NQ partials of each head below
        const int slot = w * 4 + kq;
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const int ch = sub + 16 * c;
                if (ch < CH)
#pragma unroll
                    for (int i = 0; i < VEC; i++) sm_o[slot][gg][ch * VEC + i] = o[gg][c][i];
            }
            if (sub == 0) {
                sm_m[slot][gg] = mrun[gg];
                sm_l[slot][gg] = lrun[gg];
            }
        }
    } else {
    // merge the four 16-lane quarters of the wavefront (lane pairs l, l^16 then
    // l, l^32; each pair computes the same symmetric merge), then the wavefronts
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
#pragma unroll
        for (int lvl = 0; lvl < 2; lvl++) {
            const LanePair m2 = lvl ? swap32(mrun[gg]) : swap16(mrun[gg]);
            const LanePair l2 = lvl ? swap32(lrun[gg]) : swap16(lrun[gg]);
            const float mn = fmaxf(m2.lo, m2.hi);
            const float fa = mn == -INFINITY ? 0.f : exp2f(m2.lo - mn);
            const float fb = mn == -INFINITY ? 0.f : exp2f(m2.hi - mn);
            lrun[gg] = l2.lo * fa + l2.hi * fb;
#pragma unroll
            for (int c = 0; c < CPL; c++)
#pragma unroll
                for (int i = 0; i < VEC; i++) {
                    const LanePair o2 = lvl ? swap32(o[gg][c][i]) : swap16(o[gg][c][i]);
                    o[gg][c][i] = o2.lo * fa + o2.hi * fb;
                }
            mrun[gg] = mn;
        }
        if (kq == 0) {
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const int ch = sub + 16 * c;
                if (ch < CH)
#pragma unroll
                    for (int i = 0; i < VEC; i++) sm_o[w][gg][ch * VEC + i] = o[gg][c][i];
            }
            if (sub == 0) {
                sm_m[w][gg] = mrun[gg];
                sm_l[w][gg] = lrun[gg];
            }
        }
    }
    }
    __syncthreads();
    for (int idx = tid; idx < G * (D + 2); idx += NW * kWave) {
        const int gg = idx / (D + 2), e = idx % (D + 2);
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < NQ; q++) mx = fmaxf(mx, sm_m[q][gg]);
        float v = 0.f;
        if (e == D) {
            v = mx;
        } else {
#pragma unroll
            for (int q = 0; q < NQ; q++) {
                const float f = mx == -INFINITY ? 0.f : exp2f(sm_m[q][gg] - mx);
                v += f * (e < D ? sm_o[q][gg][e] : sm_l[q][gg]);
            }
        }
        a.partial[((size_t)(g * G + gg) * a.nsplit + sp) * PS + e] = v;
    }
}

// ============================================================== decode, bf16 on the matrix cores
// The work of attn_decode_fused_kernel<bf16_t, D, G, 4> (one block per (KV
// head g, split sp): rotation of the group's q heads and of the new k / v,
// the owner's write of slot t, one (o, m, l) partial per query head), in
// blocks of NW wavefronts, with the products of each 16-key tile on the matrix
// cores. The
// group's query heads are the 16 columns of the products (G of them used):
//   S^T[16 keys][16 heads] = K tile . q^T      v_mfma_f32_16x16x32_bf16, ceil(D/32) steps;
//   V tile in the operand layout of P . V: the product of the tile with 0/1
//     columns of the identity, exact in fp32   v_mfma_f32_16x16x32_bf16, one per 16 dims;
//   O[16 heads][16 dims] += P . V               v_mfma_f32_16x16x16bf16_1k, P = hi + lo in bf16.
// In these 16x16 layouts lane l holds column l % 16 and rows 4 (l / 16) .. +3
// of a result, and row l % 16 with contraction indices 8 (l / 16) .. +7 (x32)
// or 4 (l / 16) .. +3 (x16) of an operand, so the rows of S^T a lane holds (4
// keys for the lane's head) are already the lane's part of the P operand.
// Wavefront w scores the tiles w, w + NW, ... of the split, NT at a time,
// with an online softmax across its batches; the wavefronts merge through LDS
// as in the other form.
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, int G, int NW, int NT>
__global__ __launch_bounds__(NW * 64) void attn_decode_mfma_kernel(DecAttnArgs a) {
    typedef bf16_t T;
    constexpr int KS = (D + 31) / 32, DB = D / 16, PS = D + 4;
    static_assert(D % 16 == 0 && G <= 16, "16-dim blocks, at most 16 query heads per KV head");
    __shared__ float qs[G][D];
    __shared__ __attribute__((aligned(16))) T knew[D];
    __shared__ __attribute__((aligned(16))) T vnew[D];
    __shared__ float sm_m[NW][G], sm_l[NW][G];
    __shared__ float sm_o[NW][G][D];
    const int g = blockIdx.x, sp = blockIdx.y;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, l16 = lane % 16, grp = lane / 16;
    const int chunk = a.chunk;
    const int k0 = sp * chunk, kend = min(a.W, k0 + chunk);
    const int ntile = kend > k0 ? (kend - k0 + 15) / 16 : 0;
    const int nmine = ntile > w ? (ntile - w + NW - 1) / NW : 0;  // this wavefront's tiles (uniform)
    const T* Kg = (const T*)a.kc + (size_t)g * a.W * D;
    const T* Vg = (const T*)a.vc + (size_t)g * a.W * D;
    const int jl = max(kend - 1, 0);  // a valid slot for clamped requests

    // (1) K/V rows of the first batch: lane l loads key l % 16 of a tile, dims
    // 32 ks + 8 (l / 16) .. +7 (clamped to the last 8 dims past D: those lanes'
    // products meet zero q entries and zero identity entries)
    u32x4 kr[NT][KS], vr[NT][KS];
    auto request = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NT; b++) {
            if (i0 + b < nmine) {  // uniform over the wavefront
                const int j = min(k0 + (w + NW * (i0 + b)) * 16 + l16, jl);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int d = min(32 * ks + 8 * grp, D - 8);
                    kr[b][ks] = *reinterpret_cast<const u32x4*>(Kg + (size_t)j * D + d);
                    vr[b][ks] = *reinterpret_cast<const u32x4*>(Vg + (size_t)j * D + d);
                }
            }
        }
    };
    request(0);
    DecRotation<T, D, G, NW> rot;
    rot.load(a, g, w, lane);
    __builtin_amdgcn_sched_barrier(0);

    // (2) the valid range, then QK-Norm + RoPE of q (G heads) and of the owner's new k / v
    const int t = a.len[0];
    const int k1 = min(t + 1, kend);
    const bool own = k0 <= t && t < kend;
    rot.apply(a, g, w, t, own, qs, knew, vnew);
    __syncthreads();

    // q^T operand (lane l: head l % 16, dims 32 ks + 8 (l / 16) .. +7; zero past G or D)
    // and the two identity operands (column j of half h selects dim 16 h + j of a 32-dim step)
    bf16x8 qb[KS], ib[2];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int d = 32 * ks + 8 * grp + e;
            const float v = (l16 < G && d < D) ? qs[l16 < G ? l16 : 0][d < D ? d : 0] : 0.f;
            qb[ks][e] = __builtin_bit_cast(__bf16, f2bf(v));
        }
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int e = 0; e < 8; e++)
            ib[h][e] = __builtin_bit_cast(__bf16, (bf16_t)(8 * grp + e == l16 + 16 * h ? 0x3f80 : 0));
    const float scale = kLog2e / sqrtf((float)D);
    float mrun = -INFINITY, lpart = 0.f;  // per head l % 16 (replicated over the four lanes of a head)
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // (3) this wavefront's tiles, NT per batch
    for (int b0 = 0; b0 < nmine; b0 += NT) {
        if (b0 > 0) request(b0);
        float s[NT][4];
#pragma unroll
        for (int b = 0; b < NT; b++) {
#pragma unroll
            for (int r = 0; r < 4; r++) s[b][r] = -INFINITY;
            if (b0 + b >= nmine) continue;  // uniform
            const int kt = k0 + (w + NW * (b0 + b)) * 16;
            const int ka = kt + l16;  // the key this lane loaded
            if (ka == t) {  // the new slot: this token's rotated k and v
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int d = min(32 * ks + 8 * grp, D - 8);
                    kr[b][ks] = *reinterpret_cast<const u32x4*>(knew + d);
                    vr[b][ks] = *reinterpret_cast<const u32x4*>(vnew + d);
                }
            }
            if (ka >= k1) {  // clamped or past t: arbitrary bits; weight 0 must not meet NaN
#pragma unroll
                for (int ks = 0; ks < KS; ks++) vr[b][ks] = u32x4{0, 0, 0, 0};
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[b][ks]), qb[ks], acc, 0,
                                                              0, 0);
#pragma unroll
            for (int r = 0; r < 4; r++) s[b][r] = kt + 4 * grp + r < k1 ? acc[r] * scale : -INFINITY;
        }
        float mb = -INFINITY;
#pragma unroll
        for (int b = 0; b < NT; b++)
#pragma unroll
            for (int r = 0; r < 4; r++) mb = fmaxf(mb, s[b][r]);
        {
            const LanePair p16 = swap16(mb);
            mb = fmaxf(p16.lo, p16.hi);
            const LanePair p32 = swap32(mb);
            mb = fmaxf(p32.lo, p32.hi);
        }
        const float mn = fmaxf(mrun, mb);
        const float mu = mn == -INFINITY ? 0.f : mn;
        // arguments are <= 0 (or -inf): the bare v_exp_f32 needs no range reduction
        const float alpha = __builtin_amdgcn_exp2f(mrun - mu);
        mrun = mn;
        lpart *= alpha;
        if (b0 > 0) {  // rows of oacc are heads 4 (l / 16) + r: their factors from lanes 4 (l / 16) + r
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float f = __shfl(alpha, 4 * grp + r);
#pragma unroll
                for (int db = 0; db < DB; db++) oacc[db][r] *= f;
            }
        }
#pragma unroll
        for (int b = 0; b < NT; b++) {
            if (b0 + b >= nmine) continue;  // uniform
            s16x4 phi, plo;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float p = __builtin_amdgcn_exp2f(s[b][r] - mu);
                lpart += p;
                const bf16_t h = f2bf(p);
                phi[r] = (short)h;
                plo[r] = (short)f2bf(p - bf2f(h));
            }
#pragma unroll
            for (int db = 0; db < DB; db++) {
                const f32x4 vt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, vr[b][db / 2]), ib[db % 2], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                s16x4 vb;
#pragma unroll
                for (int r = 0; r < 4; r++) vb[r] = (short)(__float_as_uint(vt[r]) >> 16);  // exact: bf16 values
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, oacc[db], 0, 0, 0);
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, oacc[db], 0, 0, 0);
            }
        }
    }
    {
        const LanePair p16 = swap16(lpart);
        lpart = p16.lo + p16.hi;
        const LanePair p32 = swap32(lpart);
        lpart = p32.lo + p32.hi;
    }
    if (grp == 0 && l16 < G) {
        sm_m[w][l16] = mrun;
        sm_l[w][l16] = lpart;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int hd = 4 * grp + r;
        if (hd < G)
#pragma unroll
            for (int db = 0; db < DB; db++) sm_o[w][hd][16 * db + l16] = oacc[db][r];
    }
    __syncthreads();
    for (int idx = tid; idx < G * (D + 2); idx += NW * kWave) {
        const int gg = idx / (D + 2), e = idx % (D + 2);
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < NW; q++) mx = fmaxf(mx, sm_m[q][gg]);
        float v = 0.f;
        if (e == D) {
            v = mx;
        } else {
#pragma unroll
            for (int q = 0; q < NW; q++) {
                const float f = mx == -INFINITY ? 0.f : exp2f(sm_m[q][gg] - mx);
                v += f * (e < D ? sm_o[q][gg][e] : sm_l[q][gg]);
            }
        }
        a.partial[((size_t)(g * G + gg) * a.nsplit + sp) * PS + e] = v;
    }
}

// Merge of the split partials: one single-wavefront block per 64 columns of a
// query head's output row. Lane s holds the statistics (m, l) of split
// s; every lane requests its column of the NS >= nsplit launched splits' o rows
// up front (indices clamped, unconditional: at most 32 + 2 loads, within the
// 63 a wavefront keeps in flight, so the merge is one memory round trip),
// then the split weights f_s = exp2(m_s - max m) are broadcast with readlane.
template <class T, int D, int NS>
__global__ __launch_bounds__(64) void attn_combine_fast_kernel(const float* __restrict__ partial, int nsplit,
                                                               T* __restrict__ out) {
    constexpr int PS = D + 4, NSL = (D + 63) / 64;
    static_assert(NS <= 64, "one lane per split");
    // block b: columns 64 (b % NSL) .. +63 of head b / NSL
    const int h = blockIdx.x / NSL, lane = threadIdx.x, e = (blockIdx.x % NSL) * kWave + lane;
    const float* p = partial + (size_t)h * nsplit * PS;
    const int sl = min(lane, nsplit - 1);
    const float ms = p[sl * PS + D], ls = p[sl * PS + D + 1];
    const int ec = min(e, D - 1);
    float ov[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) ov[s] = p[min(s, nsplit - 1) * PS + ec];
    __builtin_amdgcn_sched_barrier(0);
    const float m = lane < nsplit ? ms : -INFINITY;
    const float mx = wave_max(m);
    const float f = (lane < nsplit && m != -INFINITY) ? exp2f(m - mx) : 0.f;
    const float lsum = wave_sum(f * (lane < nsplit ? ls : 0.f));
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < NS; s++) {
        const float fsv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), s));
        v = fmaf(fsv, ov[s], v);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    v *= inv;
    asm volatile("" ::"v"(v));  // computed here: keeps the loads from sinking into the store branch
    if (e < D) Elt<T>::st(out, (size_t)h * D + e, v);
}

// VLM_DEC_MFMA=0 keeps bf16 decode attention on the vector-ALU form (for comparison; read at
// every launch, a captured graph keeps the form it was captured with).
static bool dec_mfma_on() {
    const char* e = getenv("VLM_DEC_MFMA");
    return !(e && atoi(e) == 0);
}

template <class T, int D>
static hipError_t fused_group(const DecAttnArgs& a, hipStream_t st) {
    const dim3 grid(a.nkv, a.nsplit);
    if constexpr (std::is_same<T, bf16_t>::value && D % 16 == 0) {
        const int G = a.nq / a.nkv;
        // for 1-2 heads per KV head the vector-ALU form is faster; eight wavefronts rotate the q, k,
        // v rows one each (36-layer stack: 2 wavefronts 454.3, 4 453.5, 8 452.4 ms per 256 tokens)
        if (dec_mfma_on() && G >= 4) {
            switch (G) {
                case 4: attn_decode_mfma_kernel<D, 4, 8, 2><<<grid, 512, 0, st>>>(a); return hipGetLastError();
                case 8: attn_decode_mfma_kernel<D, 8, 8, 2><<<grid, 512, 0, st>>>(a); return hipGetLastError();
                default: break;
            }
        }
    }
    switch (a.nq / a.nkv) {
        case 1: attn_decode_fused_kernel<T, D, 1, kDecWaves><<<grid, kDecWaves * 64, 0, st>>>(a); break;
        case 2: attn_decode_fused_kernel<T, D, 2, kDecWaves><<<grid, kDecWaves * 64, 0, st>>>(a); break;
        case 4: attn_decode_fused_kernel<T, D, 4, kDecWaves><<<grid, kDecWaves * 64, 0, st>>>(a); break;
        case 8: attn_decode_fused_kernel<T, D, 8, kDecWaves><<<grid, kDecWaves * 64, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ============================================================== decode, expanded MLA
// Keys DQ wide, values DV wide, one KV head per query head. The assembly
// kernel (launch_mla_rope) has already written this token's rotated q into
// a.qrot and its key and value into slot t, so this kernel only reads: one
// block of NW wavefronts per (head, split) as in attn_decode_fused_kernel,
// each 16-lane quarter scoring one key per step, partial rows of DV + 4
// floats merged by attn_combine_fast_kernel.
template <class T, int DQ, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_mla_kernel(DecAttnArgs a) {
    constexpr int VEC = 16 / sizeof(T), CHK = DQ / VEC, CHV = DV / VEC;
    constexpr int CPK = (CHK + 15) / 16, CPV = (CHV + 15) / 16, KSTEP = NW * 4, NB = kDecSteps;
    constexpr int PS = DV + 4;
    __shared__ float qs[DQ];
    __shared__ float sm_m[NW], sm_l[NW];
    __shared__ float sm_o[NW][DV];
    const int g = blockIdx.x, sp = blockIdx.y;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave, sub = lane % 16, kq = lane / 16;
    const int chunk = a.chunk;
    const int k0 = sp * chunk, kend = min(a.W, k0 + chunk);
    const int nst = kend > k0 ? (kend - k0 + KSTEP - 1) / KSTEP : 0;
    const T* Kg = (const T*)a.kc + (size_t)g * a.W * DQ;
    const T* Vg = (const T*)a.vc + (size_t)g * a.W * DV;
    const int jl = max(kend - 1, 0);
    u32x4 kr[NB][CPK], vr[NB][CPV];
    const int jw = k0 + w * 4 + kq;
    auto request = [&](int s0) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            if (s0 + b < nst) {  // uniform over the block
                const int j = min(jw + (s0 + b) * KSTEP, jl);
#pragma unroll
                for (int c = 0; c < CPK; c++)
                    kr[b][c] = *reinterpret_cast<const u32x4*>(Kg + (size_t)j * DQ + min(sub + 16 * c, CHK - 1) * VEC);
#pragma unroll
                for (int c = 0; c < CPV; c++)
                    vr[b][c] = *reinterpret_cast<const u32x4*>(Vg + (size_t)j * DV + min(sub + 16 * c, CHV - 1) * VEC);
            }
        }
    };
    request(0);
    const T* qh = (const T*)a.qrot + (size_t)g * DQ;
    for (int e = tid; e < DQ; e += NW * kWave) qs[e] = Elt<T>::ld(qh, e);
    const int t = a.len[0];
    const int k1 = min(t + 1, kend);
    __syncthreads();
    float qf[CPK][VEC];
#pragma unroll
    for (int c = 0; c < CPK; c++) {
        const int ch = min(sub + 16 * c, CHK - 1);
#pragma unroll
        for (int i = 0; i < VEC; i++) qf[c][i] = sub + 16 * c < CHK ? qs[ch * VEC + i] : 0.f;
    }
    const float scale = kLog2e / sqrtf((float)DQ);
    float mrun = -INFINITY, lrun = 0.f, o[CPV][VEC];
#pragma unroll
    for (int c = 0; c < CPV; c++)
#pragma unroll
        for (int i = 0; i < VEC; i++) o[c][i] = 0.f;
    for (int s0 = 0; s0 < nst; s0 += NB) {
        if (s0 > 0) request(s0);
        float sc[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int j = jw + (s0 + b) * KSTEP;
            const bool valid = s0 + b < nst && j < k1;
            if (s0 + b >= nst) {  // uniform: a step past the slot range
                sc[b] = -INFINITY;
#pragma unroll
                for (int c = 0; c < CPV; c++) vr[b][c] = u32x4{0, 0, 0, 0};
                continue;
            }
            if (!valid) {  // clamped rows hold arbitrary bits: weight 0 must not meet NaN
#pragma unroll
                for (int c = 0; c < CPV; c++) vr[b][c] = u32x4{0, 0, 0, 0};
            }
            float sv = 0.f;
#pragma unroll
            for (int c = 0; c < CPK; c++) {
                float kf[VEC];
                unpack16(kr[b][c], (const T*)nullptr, kf);
#pragma unroll
                for (int i = 0; i < VEC; i++) sv = fmaf(qf[c][i], kf[i], sv);
            }
            sv = row16_sum(sv);
            sc[b] = valid ? sv * scale : -INFINITY;
        }
        float mb = sc[0];
#pragma unroll
        for (int b = 1; b < NB; b++)
            if (s0 + b < nst) mb = fmaxf(mb, sc[b]);
        if (mb == -INFINITY) continue;
        const float mn = fmaxf(mrun, mb);
        const float alpha = exp2f(mrun - mn);
        lrun *= alpha;
        mrun = mn;
#pragma unroll
        for (int c = 0; c < CPV; c++)
#pragma unroll
            for (int i = 0; i < VEC; i++) o[c][i] *= alpha;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            if (s0 + b >= nst) break;  // uniform
            const float pb = exp2f(sc[b] - mn);
            lrun += pb;
#pragma unroll
            for (int c = 0; c < CPV; c++) {
                float vf[VEC];
                unpack16(vr[b][c], (const T*)nullptr, vf);
#pragma unroll
                for (int i = 0; i < VEC; i++) o[c][i] = fmaf(pb, vf[i], o[c][i]);
            }
        }
    }
    // merge the quarters (l, l^16 then l, l^32), then the wavefronts
#pragma unroll
    for (int lvl = 0; lvl < 2; lvl++) {
        const LanePair m2 = lvl ? swap32(mrun) : swap16(mrun);
        const LanePair l2 = lvl ? swap32(lrun) : swap16(lrun);
        const float mn = fmaxf(m2.lo, m2.hi);
        const float fa = mn == -INFINITY ? 0.f : exp2f(m2.lo - mn);
        const float fb = mn == -INFINITY ? 0.f : exp2f(m2.hi - mn);
        lrun = l2.lo * fa + l2.hi * fb;
#pragma unroll
        for (int c = 0; c < CPV; c++)
#pragma unroll
            for (int i = 0; i < VEC; i++) {
                const LanePair o2 = lvl ? swap32(o[c][i]) : swap16(o[c][i]);
                o[c][i] = o2.lo * fa + o2.hi * fb;
            }
        mrun = mn;
    }
    if (kq == 0) {
#pragma unroll
        for (int c = 0; c < CPV; c++) {
            const int ch = sub + 16 * c;
            if (ch < CHV)
#pragma unroll
                for (int i = 0; i < VEC; i++) sm_o[w][ch * VEC + i] = o[c][i];
        }
        if (sub == 0) {
            sm_m[w] = mrun;
            sm_l[w] = lrun;
        }
    }
    __syncthreads();
    for (int e = tid; e < DV + 2; e += NW * kWave) {
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ww++) mx = fmaxf(mx, sm_m[ww]);
        float v = 0.f;
        if (e == DV) {
            v = mx;
        } else {
#pragma unroll
            for (int ww = 0; ww < NW; ww++) {
                const float f = mx == -INFINITY ? 0.f : exp2f(sm_m[ww] - mx);
                v += f * (e < DV ? sm_o[ww][e] : sm_l[ww]);
            }
        }
        a.partial[((size_t)g * a.nsplit + sp) * PS + e] = v;
    }
}

hipError_t launch_attn_decode_mla(int dtype, const DecAttnArgs& a, hipStream_t st) {
    if (a.d != 192 || a.dv != 128 || a.nq != a.nkv || !a.qrot) return hipErrorInvalidValue;
    const dim3 grid(a.nkv, a.nsplit);
    if (dtype == 1)
        attn_decode_mla_kernel<bf16_t, 192, 128, 4><<<grid, 4 * 64, 0, st>>>(a);
    else
        attn_decode_mla_kernel<float, 192, 128, 4><<<grid, 4 * 64, 0, st>>>(a);
    return hipGetLastError();
}

// Loads per lane follow the launched splits: 8, 16 or 32 rows requested.
template <class T, int D>
static void combine_ns(const float* partial, int nq, int nsplit, void* out, hipStream_t st) {
    // one wavefront per block, a block per (head, 64-column slice): on the 36-layer stack's decode
    // 452.3 against 453.0 ms per 256 tokens for one two-wavefront block per head
    const int blocks = nq * ((D + 63) / 64);
    if (nsplit <= 8)
        attn_combine_fast_kernel<T, D, 8><<<blocks, kWave, 0, st>>>(partial, nsplit, (T*)out);
    else if (nsplit <= 16)
        attn_combine_fast_kernel<T, D, 16><<<blocks, kWave, 0, st>>>(partial, nsplit, (T*)out);
    else
        attn_combine_fast_kernel<T, D, kDecMaxSplits><<<blocks, kWave, 0, st>>>(partial, nsplit, (T*)out);
}

template <class T>
static hipError_t combine_dim(const float* partial, int nq, int nsplit, int d, void* out, hipStream_t st) {
    switch (d) {
        case 64: combine_ns<T, 64>(partial, nq, nsplit, out, st); break;
        case 72: combine_ns<T, 72>(partial, nq, nsplit, out, st); break;
        case 80: combine_ns<T, 80>(partial, nq, nsplit, out, st); break;
        case 128: combine_ns<T, 128>(partial, nq, nsplit, out, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_combine(int dtype, const float* partial, int nq, int nsplit, int d, void* out,
                               hipStream_t st) {
    if (nsplit < 1 || nsplit > kDecMaxSplits) return hipErrorInvalidValue;
    return dtype == 1 ? combine_dim<bf16_t>(partial, nq, nsplit, d, out, st)
                      : combine_dim<float>(partial, nq, nsplit, d, out, st);
}

template <class T>
static hipError_t fused_dim(const DecAttnArgs& a, hipStream_t st) {
    switch (a.d) {
        case 64: return fused_group<T, 64>(a, st);
        case 72: return fused_group<T, 72>(a, st);
        case 80: return fused_group<T, 80>(a, st);
        case 128: return fused_group<T, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_decode_fused(int dtype, const DecAttnArgs& a, hipStream_t st) {
    return dtype == 1 ? fused_dim<bf16_t>(a, st) : fused_dim<float>(a, st);
}

}  // namespace vlm
