// Next-token sampling on the logits row: repetition penalty, temperature,
// top-k, top-p, softmax and an inverse-CDF draw with a caller-supplied
// uniform number (MNN llm_demo Omni article §4.1; HunyuanOCR v1.5 ncnn port
// §3.6 for the generation options).
//
// One block of 1024 threads; the vocabulary streams from L2 two to four times:
//  1. the context ids become a bitmap in LDS (membership in one read);
//  2. for top-k up to 256, a threshold from the threads' maxima (step (2)
//     below): two passes (maxima, gather) when the values at or above it
//     fit the candidate slots, as they do for ordinary logits;
//  2'. else radix select on order-preserving 32-bit keys with 11-, 11- and
//     10-bit digits (LDS histograms of 2048 bins, a parallel suffix scan
//     finds the bin holding the k-th largest): as soon as every value at or
//     above that bin's lower bound fits the 2048 candidate slots they are
//     gathered, else the next digit is resolved. (One 8-bit top digit would
//     put nearly every logit in one or two bins, and their LDS atomics would
//     serialise on one address.)
//  3. the candidates are sorted by (value descending, id ascending) with a
//     bitonic sort; those at or above the k-th value are kept (ties kept);
//  4. softmax over the kept candidates, a block scan gives the cumulative
//     sums: top-p keeps the prefix whose preceding mass is below top_p * Z,
//     and the draw takes the first kept token whose cumulative sum exceeds
//     u times the kept mass.
// Processed value of id i: x = logits[i]; x = x > 0 ? x / r : x * r when i is
// in the context; x /= temperature (fp32 throughout).
#include <stdint.h>

#include "common.hpp"
#include "internal.hpp"

namespace vlm {

constexpr int kSampleThreads = 1024;
constexpr int kSampleCand = 2 * kSampleMaxK;  // candidate slots (ties at the k-th value included)
constexpr int kSampleBins = 2048;             // histogram bins of an 11-bit digit
constexpr int kSampleBatch = 8;               // logits each thread requests together
constexpr int kSamplePreK = 256;              // top-k up to which the threshold of step (2) is tried

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Decode-step form (kv_len != null, the cache header): position t = kv_len[0]; the context is
// ctx[0..t] (the token history: prompt ids, then every token fed so far), the draw uptr[t + 1];
// the token goes to out[0] and ctx[t + 1] and the length becomes t + 1; a step with no token
// (-1) is not committed and sets the header's non-finite flag, as the greedy head does.
__device__ __forceinline__ void sample_commit(int32_t tok, int32_t* out, int32_t* hist, int32_t* kv_len) {
    out[0] = tok;
    if (!kv_len) return;
    const int t = kv_len[0];
    if (tok >= 0) {
        hist[t + 1] = tok;
        kv_len[0] = t + 1;
    } else if (kv_len[1] == 0) {
        kv_len[1] = 1;
        kv_len[2] = t;
    }
}

__global__ __launch_bounds__(kSampleThreads) void sample_logits_kernel(const float* __restrict__ logits, int V,
                                                                       SampleParams sp, int32_t* ctx, int nctx,
                                                                       const float* __restrict__ uptr,
                                                                       int32_t* __restrict__ out, int32_t* kv_len) {
    __shared__ uint32_t bits[kSampleVocabMax / 32];
    __shared__ uint32_t hist[kSampleBins];
    __shared__ uint32_t ckey[kSampleCand];
    __shared__ int32_t cidx[kSampleCand];
    __shared__ float cval[kSampleCand];
    __shared__ float red[kSampleThreads / kWave];
    __shared__ uint32_t redu[kSampleThreads / kWave];
    __shared__ uint32_t s_prefix, s_krem, s_count, s_bad, s_bin, s_above, s_inbin;
    const int tid = threadIdx.x;
    const int nw = (V + 31) / 32;
    if (kv_len) {  // decode-step form: context and draw follow the device length
        const int t = kv_len[0];
        nctx = t + 1;
        uptr += t + 1;
    }
    for (int i = tid; i < nw; i += kSampleThreads) bits[i] = 0u;
    if (tid == 0) {
        s_prefix = 0u;
        s_krem = (uint32_t)min(sp.top_k, V);
        s_count = 0u;
        s_bad = 0u;
    }
    __syncthreads();
    for (int i = tid; i < nctx; i += kSampleThreads) {
        const int id = ctx[i];
        if (id >= 0 && id < V) atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    const float inv_t = 1.0f / sp.temperature, r = sp.penalty;

    // One pass over the row: f(i, key) for every value, key = the order-preserving bits of the value
    // after the penalty (context ids) and the temperature. A lane takes 4 consecutive values per load
    // (they share one context-bitmap word) and requests kSampleBatch loads together; values are
    // bounds-checked per 4 and a non-finite value sets s_bad once per thread (one CU does all the
    // arithmetic of the row, so the instructions per value set the pass time). A row that is not
    // 16-byte aligned, and the last V % 4 values, take one value per load.
    const int nv = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 ? V / 4 : 0;
    auto for_keys = [&](auto&& f, auto&& stop) __attribute__((always_inline)) {
        bool bad = false;
        auto proc = [&](int i, float x, uint32_t in_ctx) __attribute__((always_inline)) {
            if (in_ctx) x = x > 0.f ? x / r : x * r;
            x *= inv_t;
            bad |= !isfinite(x);
            f(i, ordered_key(x));
        };
        for (int c0 = tid; c0 < nv; c0 += kSampleThreads * kSampleBatch) {
            if (stop()) break;  // a gather past its slots: the pass's result is discarded anyway
            f32x4 xv[kSampleBatch];
#pragma unroll
            for (int u = 0; u < kSampleBatch; u++)
                xv[u] = *reinterpret_cast<const f32x4*>(logits + 4 * (size_t)min(c0 + u * kSampleThreads, nv - 1));
#pragma unroll
            for (int u = 0; u < kSampleBatch; u++) {
                const int c = c0 + u * kSampleThreads;
                if (c < nv) {
                    const uint32_t word = bits[c >> 3] >> ((4 * c) & 31);
#pragma unroll
                    for (int e = 0; e < 4; e++) proc(4 * c + e, xv[u][e], (word >> e) & 1u);
                }
            }
        }
        for (int i = 4 * nv + tid; i < V; i += kSampleThreads) proc(i, logits[i], (bits[i >> 5] >> (i & 31)) & 1u);
        if (bad) s_bad = 1u;
    };
    // suffix scan over the bins of `hist` (highest first) for the bin holding the need-th largest:
    // thread t holds bins top - 2t and top - 2t - 1; the result goes to s_bin, s_above, s_inbin
    auto scan_bins = [&](uint32_t need, int top) __attribute__((always_inline)) {
        const int j0 = top - 2 * tid, j1 = j0 - 1;
        const uint32_t c0 = j0 >= 0 ? hist[j0] : 0u, c1 = j1 >= 0 ? hist[j1] : 0u;
        const uint32_t pair = c0 + c1;
        const int lane = tid % kWave, w = tid / kWave;
        uint32_t sc = pair;
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t o = __shfl_up(sc, off, kWave);
            if (lane >= off) sc += o;
        }
        if (lane == kWave - 1) redu[w] = sc;
        __syncthreads();
        uint32_t base = 0u;
        for (int q = 0; q < w; q++) base += redu[q];
        const uint32_t excl = base + sc - pair;
        if (j0 >= 0 && excl < need && need <= excl + c0) {
            s_bin = (uint32_t)j0;
            s_above = excl;
            s_inbin = c0;
        } else if (j1 >= 0 && excl + c0 < need && need <= excl + pair) {
            s_bin = (uint32_t)j1;
            s_above = excl + c0;
            s_inbin = c1;
        }
        __syncthreads();
    };
    // gather the values with key >= lower into the candidate slots (s_count may end above the slots)
    auto gather = [&](uint32_t lower) __attribute__((always_inline)) {
        for_keys([&](int i, uint32_t k) __attribute__((always_inline)) {
            if (k >= lower) {
                const uint32_t slot = atomicAdd(&s_count, 1u);
                if (slot < (uint32_t)kSampleCand) {
                    ckey[slot] = k;
                    cidx[slot] = i;
                }
            }
        }, [&]() __attribute__((always_inline)) { return *(volatile uint32_t*)&s_count > (uint32_t)kSampleCand; });
        __syncthreads();
    };
    const uint32_t need0 = s_krem;
    bool gathered = false;

    // (2) a threshold from the threads' maxima: thread t's largest key over the values it reads is a
    // value of the row, so the lower bound of the (11-bit top digit) bin holding the need0-th largest
    // of those maxima has at least need0 values at or above it. When those fit the candidate slots
    // (an ordinary top-k of logits: a few dozen to a few hundred values) one pass computing the maxima
    // and one gathering replace the histogram passes below, whose LDS atomics collide on the few bins
    // that hold most logits.
    if (need0 <= (uint32_t)kSamplePreK) {
        uint32_t kmax = 0u;
        bool owns = false;
        for_keys([&](int, uint32_t k) __attribute__((always_inline)) {
            kmax = max(kmax, k);
            owns = true;
        }, []() { return false; });
        for (int b = tid; b < kSampleBins; b += kSampleThreads) hist[b] = 0u;
        if (tid == 0) s_above = 0u;  // here: the number of maxima
        __syncthreads();
        if (owns) {
            atomicAdd(&hist[kmax >> 21], 1u);
            atomicAdd(&s_above, 1u);
        }
        __syncthreads();
        if (need0 <= s_above && !s_bad) {  // uniform
            scan_bins(need0, kSampleBins - 1);
            gather(s_bin << 21);
            gathered = s_count <= (uint32_t)kSampleCand;
            __syncthreads();
            if (!gathered && tid == 0) s_count = 0u;  // too many at or above the threshold: select below
            __syncthreads();
        }
    }

    // (2') radix select: digits of 11, 11 and 10 bits, most significant first. The prefix of the
    // resolved digits is `prefix` under `mask`; `above` values lie strictly above the prefix bin.
    uint32_t prefix = 0u, mask = 0u, above = 0u, lower = 0u;
    bool resolved = gathered;
    for (int pass = 0; pass < 3 && !resolved && !s_bad; pass++) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 1023u : 2047u;
        for (int b = tid; b < kSampleBins; b += kSampleThreads) hist[b] = 0u;
        __syncthreads();
        for_keys([&](int, uint32_t k) __attribute__((always_inline)) {
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
        }, []() { return false; });
        __syncthreads();
        if (s_bad) break;
        scan_bins(need0 - above, (int)dmask);
        prefix |= s_bin << shift;
        mask |= dmask << shift;
        above += s_above;
        lower = prefix;  // keys >= lower: every value above the prefix bin and the bin itself
        resolved = above + s_inbin <= (uint32_t)kSampleCand || pass == 2;
        __syncthreads();
    }
    if (s_bad) {  // a non-finite logit: no token (the argmax path reports it the same way)
        if (tid == 0) sample_commit(-1, out, ctx, kv_len);
        return;
    }

    // (3) gather the values with key >= lower (the k-th largest is among them) unless the threshold
    // of (2) already did, sort by (value desc, id asc), keep those >= the k-th value (ties kept)
    if (!gathered) gather(lower);
    const int ngath = (int)s_count;
    if (ngath > kSampleCand) {  // more ties at the k-th value than slots
        if (tid == 0) sample_commit(-1, out, ctx, kv_len);
        return;
    }
    int np2 = 1;
    while (np2 < ngath) np2 <<= 1;
    for (int i = ngath + tid; i < np2; i += kSampleThreads) {
        ckey[i] = 0u;
        cidx[i] = 0x7fffffff;
    }
    __syncthreads();
    // "a before b": larger key, or equal key and smaller id
    for (int size = 2; size <= np2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < np2 / 2; t += kSampleThreads) {
                const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
                const bool up = (lo & size) == 0;  // this run is sorted "before-first"
                const uint32_t ka = ckey[lo], kb = ckey[hi];
                const int ia = cidx[lo], ib = cidx[hi];
                const bool b_first = kb > ka || (kb == ka && ib < ia);
                if (b_first == up) {
                    ckey[lo] = kb;
                    ckey[hi] = ka;
                    cidx[lo] = ib;
                    cidx[hi] = ia;
                }
            }
            __syncthreads();
        }
    }
    // the k-th largest key is ckey[need0 - 1]; the kept candidates are the prefix of keys >= it
    const uint32_t kth = ckey[need0 - 1];
    if (tid == 0) s_count = (uint32_t)ngath;
    __syncthreads();
    for (int i = tid; i < ngath; i += kSampleThreads)
        if (ckey[i] < kth) atomicMin(&s_count, (uint32_t)i);
    __syncthreads();
    const int n = (int)s_count;

    // (4) softmax over the sorted candidates; inclusive scan of the weights
    const float m = key_to_float(ckey[0]);
    for (int i = tid; i < n; i += kSampleThreads) cval[i] = __expf(key_to_float(ckey[i]) - m);
    __syncthreads();
    // two elements per thread (n <= 2048): sequential pair, then a block scan of the pair sums
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const float a0 = i0 < n ? cval[i0] : 0.f, a1 = i1 < n ? cval[i1] : 0.f;
    const float pair = a0 + a1;
    // inclusive scan of `pair` across the block: wavefront scan by shuffles, then the wave totals
    const int lane = tid % kWave, w = tid / kWave;
    float sc = pair;
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(sc, off, kWave);
        if (lane >= off) sc += o;
    }
    if (lane == kWave - 1) red[w] = sc;
    __syncthreads();
    float base = 0.f;
    for (int j = 0; j < w; j++) base += red[j];
    float Z = 0.f;
    for (int j = 0; j < kSampleThreads / kWave; j++) Z += red[j];
    const float incl1 = base + sc, incl0 = incl1 - a1, excl0 = incl0 - a0;
    __syncthreads();
    // cumulative sums back into cval: cval[i] = inclusive sum up to i
    if (i0 < n) cval[i0] = incl0;
    if (i1 < n) cval[i1] = incl1;
    if (tid == 0) s_count = (uint32_t)n;  // kept count, reduced below
    __syncthreads();
    // top-p: candidate i is kept iff the mass before it is < top_p * Z; kept ones form a prefix
    if (sp.top_p < 1.f) {
        const float thr = sp.top_p * Z;
        const float before0 = excl0, before1 = incl0;
        if (i0 < n && before0 >= thr) atomicMin(&s_count, (uint32_t)i0);
        if (i1 < n && before1 >= thr) atomicMin(&s_count, (uint32_t)i1);
        __syncthreads();
    }
    const int nk = max((int)s_count, 1);
    const float total = cval[nk - 1];
    const float target = uptr[0] * total;
    // the first kept candidate whose inclusive sum exceeds target (the last kept one if none does)
    if (tid == 0) s_prefix = (uint32_t)(nk - 1);
    __syncthreads();
    for (int i = tid; i < nk; i += kSampleThreads) {
        const float before = i == 0 ? 0.f : cval[i - 1];
        if (cval[i] > target && before <= target) atomicMin(&s_prefix, (uint32_t)i);
    }
    __syncthreads();
    if (tid == 0) sample_commit(cidx[s_prefix], out, ctx, kv_len);
}

hipError_t launch_sample_logits(const float* logits, int V, const SampleParams& p, const int32_t* ctx, int nctx,
                                const float* u, int32_t* out, hipStream_t st) {
    sample_logits_kernel<<<1, kSampleThreads, 0, st>>>(logits, V, p, const_cast<int32_t*>(ctx), nctx, u, out,
                                                       nullptr);
    return hipGetLastError();
}

hipError_t launch_sample_step(const float* logits, int V, const SampleParams& p, int32_t* hist, const float* u,
                              int32_t* out, int32_t* kv_len, hipStream_t st) {
    sample_logits_kernel<<<1, kSampleThreads, 0, st>>>(logits, V, p, hist, 0, u, out, kv_len);
    return hipGetLastError();
}

}  // namespace vlm
