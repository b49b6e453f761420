// Next-token sampling on the logits row: repetition penalty, temperature,
// top-k, top-p, softmax and an inverse-CDF draw with a caller-supplied
// uniform number (MNN llm_demo Omni article §4.1; HunyuanOCR v1.5 ncnn port
// §3.6 for the generation options).
//
// One block of 1024 threads; the vocabulary streams from L2 two to four times:
//  1. the context ids become a bitmap in LDS (membership in one read);
//  2. radix select on order-preserving 32-bit keys with 11-, 11- and 10-bit
//     digits (LDS histograms of 2048 bins, a parallel suffix scan finds the
//     bin holding the k-th largest): as soon as every value at or above that
//     bin's lower bound fits the 2048 candidate slots they are gathered (one
//     or two histogram passes for ordinary logits), else the next digit is
//     resolved. (One 8-bit top digit would put nearly every logit in one or
//     two bins, and their LDS atomics would serialise on one address.)
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

    // (2) radix select: digits of 11, 11 and 10 bits, most significant first. The prefix of the
    // resolved digits is `prefix` under `mask`; `above` values lie strictly above the prefix bin.
    const uint32_t need0 = s_krem;
    uint32_t prefix = 0u, mask = 0u, above = 0u, lower = 0u;
    bool gathered = false;
    for (int pass = 0; pass < 3 && !gathered; pass++) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 1023u : 2047u;
        for (int b = tid; b < kSampleBins; b += kSampleThreads) hist[b] = 0u;
        __syncthreads();
        // values in batches of kSampleBatch per thread, requested together (indices clamped)
        for (int i0 = tid; i0 < V; i0 += kSampleThreads * kSampleBatch) {
            float xv[kSampleBatch];
#pragma unroll
            for (int u = 0; u < kSampleBatch; u++) xv[u] = logits[min(i0 + u * kSampleThreads, V - 1)];
#pragma unroll
            for (int u = 0; u < kSampleBatch; u++) {
                const int i = i0 + u * kSampleThreads;
                if (i >= V) break;
                float x = xv[u];
                if ((bits[i >> 5] >> (i & 31)) & 1u) x = x > 0.f ? x / r : x * r;
                x *= inv_t;
                if (pass == 0 && !isfinite(x)) s_bad = 1u;
                const uint32_t k = ordered_key(x);
                if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        // suffix scan over the bins (highest first): thread t holds bins top - 2t and top - 2t - 1
        const uint32_t need = need0 - above;
        const int top = (int)dmask;
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
        if (s_bad) break;
        prefix |= s_bin << shift;
        mask |= dmask << shift;
        above += s_above;
        lower = prefix;  // keys >= lower: every value above the prefix bin and the bin itself
        gathered = above + s_inbin <= (uint32_t)kSampleCand || pass == 2;
        __syncthreads();
    }
    if (s_bad) {  // a non-finite logit: no token (the argmax path reports it the same way)
        if (tid == 0) sample_commit(-1, out, ctx, kv_len);
        return;
    }

    // (3) gather the values with key >= lower (the k-th largest is among them), sort by (value desc,
    // id asc), keep those >= the k-th value (ties kept)
    for (int i0 = tid; i0 < V; i0 += kSampleThreads * kSampleBatch) {
        float xv[kSampleBatch];
#pragma unroll
        for (int u = 0; u < kSampleBatch; u++) xv[u] = logits[min(i0 + u * kSampleThreads, V - 1)];
#pragma unroll
        for (int u = 0; u < kSampleBatch; u++) {
            const int i = i0 + u * kSampleThreads;
            if (i >= V) break;
            float x = xv[u];
            if ((bits[i >> 5] >> (i & 31)) & 1u) x = x > 0.f ? x / r : x * r;
            const uint32_t k = ordered_key(x * inv_t);
            if (k >= lower) {
                const uint32_t slot = atomicAdd(&s_count, 1u);
                if (slot < (uint32_t)kSampleCand) {
                    ckey[slot] = k;
                    cidx[slot] = i;
                }
            }
        }
    }
    __syncthreads();
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
