// C ABI of the decoder hot path: argument validation, workspace carving, the
// KV-cache handle, the per-layer launch sequences of prefill and decode, and
// the HIP-graph decode loop. All checks run before anything is enqueued, so a
// failed call changes nothing (HunyuanOCR v1.5 ncnn port §3.6 and §3.7: strict
// checks at load, the cache committed only after success).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"
#include "vlm.h"

using namespace vlm;

namespace {

thread_local std::string g_err;

vlm_status fail(vlm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

vlm_status ok() {
    g_err.clear();
    return VLM_OK;
}

#define HIP_TRY(expr)                                                                   \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) return fail(VLM_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// KV buffer header (int32 words): [0] length; [1] set when a decode step's
// argmax saw a non-finite logit, [2] that step's position; the rest is zeroed
// at bind time and reserved.
constexpr size_t kHeader = 256;
constexpr int kHdrWords = 64;

size_t esize(int dtype) { return dtype == VLM_BF16 ? 2 : 4; }
size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

vlm_status check_desc(const vlm_model_desc* d) {
    if (!d) return fail(VLM_ERR_ARG, "desc is NULL");
    if (d->block_kind != VLM_BLOCK_DECODER && d->block_kind != VLM_BLOCK_VIT && d->block_kind != VLM_BLOCK_MLA)
        return fail(VLM_ERR_ARG, "block_kind %d invalid", d->block_kind);
    if (d->block_kind == VLM_BLOCK_MLA) {
        if (d->n_kv_heads != d->n_q_heads) return fail(VLM_ERR_SHAPE, "MLA needs n_kv_heads == n_q_heads");
        if (d->head_dim != 192 || d->qk_rope_dim != 64 || d->v_head_dim != 128)
            return fail(VLM_ERR_UNSUPPORTED, "MLA kernels exist for head_dim 192, qk_rope_dim 64, v_head_dim 128");
        if (d->q_lora_rank < 8 || d->q_lora_rank % 8 || d->kv_lora_rank < 8 || d->kv_lora_rank % 8 ||
            d->q_lora_rank > 16384 || d->kv_lora_rank > 16384)
            return fail(VLM_ERR_SHAPE, "MLA ranks must be positive multiples of 8 up to 16384");
        if (d->qk_norm || d->rope_segments != 1) return fail(VLM_ERR_UNSUPPORTED, "MLA takes no QK-Norm, one RoPE segment");
    } else if (d->q_lora_rank || d->kv_lora_rank || d->qk_rope_dim || d->v_head_dim) {
        return fail(VLM_ERR_ARG, "MLA fields must be 0 for block_kind %d", d->block_kind);
    }
    if (d->dtype != VLM_F32 && d->dtype != VLM_BF16) return fail(VLM_ERR_DTYPE, "dtype %d invalid", d->dtype);
    if (d->n_layers < 1) return fail(VLM_ERR_SHAPE, "n_layers %d < 1", d->n_layers);
    if (d->hidden < 8 || d->hidden % 8) return fail(VLM_ERR_SHAPE, "hidden %d must be a positive multiple of 8", d->hidden);
    if (d->hidden > 16384) return fail(VLM_ERR_UNSUPPORTED, "hidden %d > 16384", d->hidden);
    if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads)
        return fail(VLM_ERR_SHAPE, "n_q_heads %d must be a multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
    const int grp = d->n_q_heads / d->n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
        return fail(VLM_ERR_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}", grp);
    if (d->block_kind != VLM_BLOCK_MLA && d->head_dim != 64 && d->head_dim != 72 && d->head_dim != 80 &&
        d->head_dim != 128)
        return fail(VLM_ERR_UNSUPPORTED, "head_dim %d not in {64,72,80,128}", d->head_dim);
    if (d->rope_segments != 1 && d->rope_segments != 2) return fail(VLM_ERR_ARG, "rope_segments %d", d->rope_segments);
    if ((d->head_dim / d->rope_segments) % 2) return fail(VLM_ERR_SHAPE, "rope segment length must be even");
    if (d->qk_norm < 0 || d->qk_norm > 2) return fail(VLM_ERR_ARG, "qk_norm %d not in {0,1,2}", d->qk_norm);
    if (d->rope_interleave != 0 && d->rope_interleave != 1)
        return fail(VLM_ERR_ARG, "rope_interleave %d not in {0,1}", d->rope_interleave);
    if (d->ffn < 8 || d->ffn % 8) return fail(VLM_ERR_SHAPE, "ffn %d must be a positive multiple of 8", d->ffn);
    if (d->ffn > 16384) return fail(VLM_ERR_UNSUPPORTED, "ffn %d > 16384", d->ffn);
    if (d->block_kind != VLM_BLOCK_VIT && d->ffn % 32)
        return fail(VLM_ERR_SHAPE, "decoder ffn %d must be a multiple of 32 (gate/up groups)", d->ffn);
    if (d->n_q_heads * d->head_dim > 16384) return fail(VLM_ERR_UNSUPPORTED, "n_q_heads*head_dim too large");
    if (d->vocab < 0) return fail(VLM_ERR_SHAPE, "vocab %d < 0", d->vocab);
    if (!(d->norm_eps >= 0.f)) return fail(VLM_ERR_ARG, "norm_eps must be >= 0");
    if (d->block_kind == VLM_BLOCK_VIT && (d->n_kv_heads != d->n_q_heads || d->qk_norm))
        return fail(VLM_ERR_UNSUPPORTED, "ViT blocks need n_kv_heads == n_q_heads and no QK-Norm");
    return VLM_OK;
}

bool is_mla(const vlm_model_desc* d) { return d->block_kind == VLM_BLOCK_MLA; }
int vdim(const vlm_model_desc* d) { return is_mla(d) ? d->v_head_dim : d->head_dim; }
// Width of the projections' fp32 output per row: q, k, v of the fused QKV GEMM, or for MLA the
// q_b output [nq*d] followed by the kv_b output [nq*(dn + dv)].
int qkv_rows(const vlm_model_desc* d) {
    if (is_mla(d)) return d->n_q_heads * (2 * d->head_dim - d->qk_rope_dim + d->v_head_dim);
    return (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
}
// MLA: columns of the shared down-projection output [q latent qr | kv latent r | rotated key dr].
int mla_a_cols(const vlm_model_desc* d) { return is_mla(d) ? d->q_lora_rank + d->kv_lora_rank + d->qk_rope_dim : 0; }

struct Ws {
    size_t h, qkv, q, kv, o, a, gpart, gpart_floats, xrow, qkvrow, qrow, part, orow, arow, rope, lm;
    size_t ma, mqa, mc, marow;  // MLA: down-projection output, normed q / kv latents (rows), its decode row
    size_t logits;              // decode step's logits row for the sampler (vocab floats)
    size_t total;
};

Ws ws_layout(const vlm_model_desc* d, int max_rows) {
    const size_t E = esize(d->dtype), R = std::max(max_rows, 1);
    const size_t H = d->hidden, F = d->ffn, nq = d->n_q_heads, nkv = d->n_kv_heads, hd = d->head_dim;
    Ws w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += al256(bytes);
        return o;
    };
    w.h = take(R * H * E);
    w.qkv = take(R * qkv_rows(d) * 4);
    w.q = take(nq * R * hd * E);
    w.kv = d->block_kind == VLM_BLOCK_VIT ? take(2 * nkv * R * hd * E) : off;
    w.o = take(R * nq * hd * E);
    w.a = take(R * F * E);
    // split-K partials of the narrow prefill GEMMs: up to 4 splits of [R][max(N)] fp32
    w.gpart_floats = 4 * R * std::max({(size_t)qkv_rows(d), H, 2 * F, (size_t)mla_a_cols(d)});
    w.gpart = take(w.gpart_floats * 4);
    w.xrow = take(H * 4);
    w.qkvrow = take(qkv_rows(d) * 4);
    w.qrow = take(nq * hd * E);
    w.part = take(nq * kDecMaxSplits * (hd + 4) * 4);
    w.orow = take(nq * hd * E);
    w.arow = take(F * E);
    w.rope = take(2 * hd * 4);  // cos/sin row of the decode position
    w.lm = take(d->vocab > 0 ? (size_t)lmhead_partials_max(d->vocab) * 8 : 8);
    w.ma = take(R * mla_a_cols(d) * 4);
    w.mqa = take(is_mla(d) ? R * d->q_lora_rank * E : 0);
    w.mc = take(is_mla(d) ? R * d->kv_lora_rank * E : 0);
    w.marow = take((size_t)mla_a_cols(d) * 4);
    w.logits = take(d->vocab > 0 ? (size_t)d->vocab * 4 : 0);
    w.total = off;
    return w;
}

vlm_status check_ws(const vlm_model_desc* d, int rows, const void* ws, size_t bytes, Ws* out) {
    if (!ws) return fail(VLM_ERR_ARG, "workspace is NULL");
    if ((uintptr_t)ws & 255) return fail(VLM_ERR_ARG, "workspace must be 256-byte aligned");
    *out = ws_layout(d, rows);
    if (bytes < out->total)
        return fail(VLM_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", bytes, out->total);
    return VLM_OK;
}

char* P(void* base, size_t off) { return (char*)base + off; }

vlm_status need(const void* p, const char* name, int layer) {
    if (!p) return fail(VLM_ERR_ARG, "layer %d: %s is NULL", layer, name);
    if (!aligned16(p)) return fail(VLM_ERR_ARG, "layer %d: %s not 16-byte aligned", layer, name);
    return VLM_OK;
}

vlm_status check_layers(const vlm_model_desc* d, const vlm_layer* L) {
    if (!L) return fail(VLM_ERR_ARG, "layers is NULL");
    for (int l = 0; l < d->n_layers; l++) {
        const vlm_layer& y = L[l];
        vlm_status s;
        if ((s = need(y.attn_norm, "attn_norm", l)) || (s = need(y.wo, "wo", l)) ||
            (s = need(y.mlp_norm, "mlp_norm", l)) || (s = need(y.w1, "w1", l)) || (s = need(y.w2, "w2", l)))
            return s;
        if (is_mla(d)) {
            if ((s = need(y.w_a, "w_a", l)) || (s = need(y.q_a_norm, "q_a_norm", l)) || (s = need(y.q_b, "q_b", l)) ||
                (s = need(y.kv_a_norm, "kv_a_norm", l)) || (s = need(y.kv_b, "kv_b", l)))
                return s;
            continue;
        }
        if ((s = need(y.wqkv, "wqkv", l))) return s;
        if (d->qk_norm && ((s = need(y.q_norm, "q_norm", l)) || (s = need(y.k_norm, "k_norm", l)))) return s;
        if (d->block_kind == VLM_BLOCK_VIT) {
            if ((s = need(y.attn_norm_b, "attn_norm_b", l)) || (s = need(y.bqkv, "bqkv", l)) ||
                (s = need(y.bo, "bo", l)) || (s = need(y.mlp_norm_b, "mlp_norm_b", l)) || (s = need(y.b1, "b1", l)) ||
                (s = need(y.b2, "b2", l)))
                return s;
        }
    }
    return VLM_OK;
}

}  // namespace

// =============================================================================== KV cache
struct GraphKey {
    vlm_model_desc desc;
    std::vector<vlm_layer> layers;
    const void *embed, *fnorm, *table;
    int32_t* tok;
    const float *cos, *sin;
    int table_rows;
    int32_t* hist;
    void* ws;
    size_t ws_bytes;
    bool sampled = false;  // the sampler instead of the argmax ends each step
    SampleParams sp{};
    const float* uniform = nullptr;
    int steps = 1;  // decode steps in a band's multi-step graph
    bool operator==(const GraphKey& o) const {
        return memcmp(&desc, &o.desc, sizeof(desc)) == 0 && layers.size() == o.layers.size() &&
               memcmp(layers.data(), o.layers.data(), layers.size() * sizeof(vlm_layer)) == 0 && embed == o.embed &&
               fnorm == o.fnorm && table == o.table && tok == o.tok && cos == o.cos && sin == o.sin &&
               table_rows == o.table_rows && hist == o.hist && ws == o.ws && ws_bytes == o.ws_bytes &&
               sampled == o.sampled && uniform == o.uniform && sp.temperature == o.sp.temperature &&
               sp.top_k == o.sp.top_k && sp.top_p == o.sp.top_p && sp.penalty == o.sp.penalty && steps == o.steps;
    }
};

struct vlm_kv {
    vlm_model_desc desc;
    int capacity;
    void* buf;
    size_t bytes;
    int len;  // host mirror
    hipStream_t cap_stream = nullptr;
    // per band of positions (the attention split plan changes from band to band): a graph of one
    // decode step (graph, exec) and one of kDecGraphSteps steps (graphk, execk)
    std::vector<hipGraph_t> graph, graphk;
    std::vector<hipGraphExec_t> exec, execk;
    bool has_key = false;
    GraphKey key;
    int32_t* dlen() const { return (int32_t*)buf; }
    size_t k_bytes() const { return (size_t)desc.n_kv_heads * capacity * desc.head_dim * esize(desc.dtype); }
    size_t layer_bytes() const { return k_bytes() + (size_t)desc.n_kv_heads * capacity * vdim(&desc) * esize(desc.dtype); }
    char* kptr(int l) const { return (char*)buf + kHeader + (size_t)l * layer_bytes(); }
    char* vptr(int l) const { return kptr(l) + k_bytes(); }
    void drop_graph() {
        for (auto* v : {&exec, &execk})
            for (hipGraphExec_t e : *v)
                if (e) hipGraphExecDestroy(e);
        for (auto* v : {&graph, &graphk})
            for (hipGraph_t g : *v)
                if (g) hipGraphDestroy(g);
        exec.clear();
        execk.clear();
        graph.clear();
        graphk.clear();
        has_key = false;
    }
};

extern "C" {

const char* vlm_last_error(void) { return g_err.c_str(); }

vlm_status vlm_kv_bytes(const vlm_model_desc* desc, int32_t capacity, size_t* bytes) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->block_kind == VLM_BLOCK_VIT) return fail(VLM_ERR_ARG, "KV cache is for decoder stacks");
    if (capacity < 1) return fail(VLM_ERR_SHAPE, "capacity %d < 1", capacity);
    if (!bytes) return fail(VLM_ERR_ARG, "bytes is NULL");
    *bytes = kHeader + (size_t)desc->n_layers * desc->n_kv_heads * capacity * (desc->head_dim + vdim(desc)) *
                           esize(desc->dtype);
    return ok();
}

vlm_status vlm_kv_alloc(const vlm_model_desc* desc, int32_t capacity, void* d_buf, size_t bytes, hipStream_t stream,
                        vlm_kv** out) {
    size_t need_b = 0;
    vlm_status s = vlm_kv_bytes(desc, capacity, &need_b);
    if (s) return s;
    if (!out) return fail(VLM_ERR_ARG, "out is NULL");
    if (!d_buf || ((uintptr_t)d_buf & 255)) return fail(VLM_ERR_ARG, "KV buffer NULL or not 256-byte aligned");
    if (bytes < need_b) return fail(VLM_ERR_CAPACITY, "KV buffer %zu bytes < %zu needed", bytes, need_b);
    HIP_TRY(launch_zero_i32((int32_t*)d_buf, kHdrWords, stream));
    vlm_kv* kv = new vlm_kv();
    kv->desc = *desc;
    kv->capacity = capacity;
    kv->buf = d_buf;
    kv->bytes = bytes;
    kv->len = 0;
    *out = kv;
    return ok();
}

vlm_status vlm_kv_free(vlm_kv* kv) {
    if (!kv) return fail(VLM_ERR_ARG, "kv is NULL");
    kv->drop_graph();
    if (kv->cap_stream) hipStreamDestroy(kv->cap_stream);
    delete kv;
    return ok();
}

vlm_status vlm_kv_len(const vlm_kv* kv, int32_t* len) {
    if (!kv || !len) return fail(VLM_ERR_ARG, "NULL argument");
    *len = kv->len;
    return ok();
}

vlm_status vlm_kv_truncate(vlm_kv* kv, int32_t new_len, hipStream_t stream) {
    if (!kv) return fail(VLM_ERR_ARG, "kv is NULL");
    if (new_len < 0 || new_len > kv->len)
        return fail(VLM_ERR_CAPACITY, "new length %d outside [0, %d]", new_len, kv->len);
    HIP_TRY(launch_set_len(kv->dlen(), new_len, stream));
    kv->len = new_len;
    return ok();
}

vlm_status vlm_kv_status(vlm_kv* kv, hipStream_t stream, int32_t* h_pos) {
    if (!kv) return fail(VLM_ERR_ARG, "kv is NULL");
    int32_t hdr[3] = {0, 0, 0};
    HIP_TRY(hipStreamSynchronize(stream));
    HIP_TRY(hipMemcpy(hdr, kv->buf, sizeof(hdr), hipMemcpyDeviceToHost));
    if (h_pos) *h_pos = hdr[1] ? hdr[2] : -1;
    if (!hdr[1]) return ok();
    kv->len = hdr[0];  // the failed steps did not advance the device length
    HIP_TRY(launch_zero_i32((int32_t*)kv->buf + 1, 2, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    return fail(VLM_ERR_NONFINITE, "non-finite logits at decode position %d; the cache length stays %d", hdr[2],
                hdr[0]);
}

vlm_status vlm_token_status(const int32_t* d_token, hipStream_t stream, int32_t* h_token) {
    if (!d_token) return fail(VLM_ERR_ARG, "d_token is NULL");
    int32_t tok = 0;
    HIP_TRY(hipStreamSynchronize(stream));
    HIP_TRY(hipMemcpy(&tok, d_token, sizeof(tok), hipMemcpyDeviceToHost));
    if (h_token) *h_token = tok;
    if (tok == -1) return fail(VLM_ERR_NONFINITE, "the token was taken over non-finite logits");
    return ok();
}

vlm_status vlm_workspace_bytes(const vlm_model_desc* desc, int32_t max_rows, size_t* bytes) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (max_rows < 0) return fail(VLM_ERR_SHAPE, "max_rows %d < 0", max_rows);
    if (!bytes) return fail(VLM_ERR_ARG, "bytes is NULL");
    *bytes = ws_layout(desc, max_rows).total;
    return ok();
}

// =============================================================================== packing
vlm_status vlm_pack_qkv(const void* d_wq, const void* d_wk, const void* d_wv, int32_t q_rows, int32_t kv_rows,
                        int32_t hidden, int32_t dtype, void* d_out, hipStream_t stream) {
    if (!d_wq || !d_wk || !d_wv || !d_out) return fail(VLM_ERR_ARG, "NULL pointer");
    if (dtype != VLM_F32 && dtype != VLM_BF16) return fail(VLM_ERR_DTYPE, "dtype %d", dtype);
    if (q_rows < 1 || kv_rows < 1 || hidden < 1) return fail(VLM_ERR_SHAPE, "bad sizes");
    const size_t E = esize(dtype), qb = (size_t)q_rows * hidden * E, kb = (size_t)kv_rows * hidden * E;
    HIP_TRY(hipMemcpyAsync(d_out, d_wq, qb, hipMemcpyDeviceToDevice, stream));
    HIP_TRY(hipMemcpyAsync((char*)d_out + qb, d_wk, kb, hipMemcpyDeviceToDevice, stream));
    HIP_TRY(hipMemcpyAsync((char*)d_out + qb + kb, d_wv, kb, hipMemcpyDeviceToDevice, stream));
    return ok();
}

vlm_status vlm_pack_gate_up(const void* d_wg, const void* d_wu, int32_t ffn, int32_t hidden, int32_t dtype,
                            void* d_out, hipStream_t stream) {
    if (!d_wg || !d_wu || !d_out) return fail(VLM_ERR_ARG, "NULL pointer");
    if (dtype != VLM_F32 && dtype != VLM_BF16) return fail(VLM_ERR_DTYPE, "dtype %d", dtype);
    if (ffn < 32 || ffn % 32 || hidden < 1) return fail(VLM_ERR_SHAPE, "ffn must be a positive multiple of 32");
    HIP_TRY(launch_pack_gate_up(dtype, d_wg, d_wu, ffn, hidden, d_out, stream));
    return ok();
}

// =============================================================================== RoPE table
vlm_status vlm_rope_table(const int32_t* d_pos, int32_t n_axes, int32_t n_rows, const int32_t* h_axis_of_pair,
                          int32_t rope_segments, int32_t head_dim, double theta, float* d_cos, float* d_sin,
                          hipStream_t stream) {
    if (!d_pos || !h_axis_of_pair || !d_cos || !d_sin) return fail(VLM_ERR_ARG, "NULL pointer");
    if (n_axes < 1 || n_rows < 0) return fail(VLM_ERR_SHAPE, "n_axes %d / n_rows %d", n_axes, n_rows);
    if (head_dim < 2 || head_dim > 128) return fail(VLM_ERR_UNSUPPORTED, "head_dim %d not in [2, 128]", head_dim);
    if (rope_segments != 1 && rope_segments != 2) return fail(VLM_ERR_ARG, "rope_segments %d", rope_segments);
    if (head_dim % (2 * rope_segments)) return fail(VLM_ERR_SHAPE, "segment length must be even");
    if (!(theta > 0.0)) return fail(VLM_ERR_ARG, "theta must be > 0");
    for (int i = 0; i < head_dim / 2; i++)
        if (h_axis_of_pair[i] < 0 || h_axis_of_pair[i] >= n_axes)
            return fail(VLM_ERR_ARG, "axis_of_pair[%d] = %d outside [0, %d)", i, h_axis_of_pair[i], n_axes);
    HIP_TRY(launch_rope_table(d_pos, n_axes, n_rows, h_axis_of_pair, rope_segments, head_dim, theta, d_cos, d_sin, stream));
    return ok();
}

vlm_status vlm_rope_alpha_base(double theta, double alpha, int32_t head_dim, double* base) {
    if (!base) return fail(VLM_ERR_ARG, "NULL pointer");
    if (!(theta > 0.0) || !(alpha > 0.0) || head_dim <= 2)
        return fail(VLM_ERR_ARG, "need theta > 0, alpha > 0, head_dim > 2 (got %g, %g, %d)", theta, alpha, head_dim);
    *base = theta * pow(alpha, (double)head_dim / (double)(head_dim - 2));
    return ok();
}

// =============================================================================== embed / inject
vlm_status vlm_embed(const vlm_model_desc* desc, const void* d_embed, const int32_t* d_ids, int32_t S, float* d_x,
                     hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->vocab < 1) return fail(VLM_ERR_SHAPE, "model has no embedding table (vocab 0)");
    if (S < 0) return fail(VLM_ERR_SHAPE, "S %d < 0", S);
    if (S == 0) return ok();
    if (!d_embed || !d_ids || !d_x) return fail(VLM_ERR_ARG, "NULL pointer");
    HIP_TRY(launch_embed(desc->dtype, d_embed, desc->vocab, desc->hidden, d_ids, S, d_x, stream));
    return ok();
}

vlm_status vlm_inject_image_embeds(const vlm_model_desc* desc, float* d_x, int32_t S, const int32_t* h_ids,
                                   const int32_t* d_ids, int32_t placeholder_id, const void* d_img, int32_t n_img,
                                   int32_t img_dtype, hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (S < 0 || n_img < 0) return fail(VLM_ERR_SHAPE, "S %d / n_img %d negative", S, n_img);
    if (img_dtype != VLM_F32 && img_dtype != VLM_BF16) return fail(VLM_ERR_DTYPE, "img_dtype %d", img_dtype);
    if (S > 0 && (!h_ids || !d_ids || !d_x)) return fail(VLM_ERR_ARG, "NULL pointer");
    if (n_img > 0 && !d_img) return fail(VLM_ERR_ARG, "d_img is NULL");
    int count = 0;
    for (int i = 0; i < S; i++) count += h_ids[i] == placeholder_id;
    if (count != n_img)
        return fail(VLM_ERR_COUNT_MISMATCH, "%d placeholder rows (id %d) but %d image rows", count, placeholder_id, n_img);
    if (n_img == 0) return ok();
    HIP_TRY(launch_inject(img_dtype, d_x, S, desc->hidden, d_ids, placeholder_id, d_img, n_img, stream));
    return ok();
}

// =============================================================================== prefill
vlm_status vlm_prefill(const vlm_model_desc* desc, const vlm_layer* h_layers, float* d_x, int32_t S, int32_t pos0,
                       const float* d_cos, const float* d_sin, int32_t table_rows, const vlm_mask* h_masks,
                       int32_t n_masks, vlm_kv* kv, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    const bool vit = desc->block_kind == VLM_BLOCK_VIT;
    if (S < 0 || pos0 < 0) return fail(VLM_ERR_SHAPE, "S %d / pos0 %d negative", S, pos0);
    if (vit) {
        if (kv) return fail(VLM_ERR_ARG, "ViT prefill takes no KV cache");
        if (pos0 != 0) return fail(VLM_ERR_ARG, "ViT prefill needs pos0 == 0");
    } else {
        if (!kv) return fail(VLM_ERR_ARG, "decoder prefill needs a KV cache");
        if (memcmp(&kv->desc, desc, sizeof(*desc)) != 0) return fail(VLM_ERR_ARG, "KV cache bound to another model desc");
        if (pos0 > kv->len) return fail(VLM_ERR_CAPACITY, "pos0 %d beyond the cache length %d", pos0, kv->len);
        if ((long)pos0 + S > kv->capacity)
            return fail(VLM_ERR_CAPACITY, "sequence end %d exceeds the KV window %d", pos0 + S, kv->capacity);
    }
    if ((long)pos0 + S > table_rows)
        return fail(VLM_ERR_CAPACITY, "sequence end %d exceeds the RoPE table rows %d", pos0 + S, table_rows);
    if (!d_x || !aligned16(d_x) || !d_cos || !d_sin) return fail(VLM_ERR_ARG, "x/cos/sin NULL or x misaligned");
    if ((s = check_layers(desc, h_layers))) return s;
    if (!h_masks || (n_masks != 1 && n_masks != desc->n_layers))
        return fail(VLM_ERR_ARG, "masks: need 1 or n_layers entries (got %d)", n_masks);
    for (int i = 0; i < n_masks; i++) {
        const vlm_mask& m = h_masks[i];
        if (m.kind < VLM_MASK_CAUSAL || m.kind > VLM_MASK_SEGMENT) return fail(VLM_ERR_ARG, "mask %d kind %d", i, m.kind);
        if (m.kind == VLM_MASK_ADDITIVE && (!m.add || m.ld_add < pos0 + S))
            return fail(VLM_ERR_ARG, "mask %d: additive mask NULL or ld_add %d < %d", i, m.ld_add, pos0 + S);
        if (m.kind == VLM_MASK_SEGMENT && (!m.seg || pos0 != 0))
            return fail(VLM_ERR_ARG, "mask %d: segment mask needs seg ids and pos0 == 0", i);
        if (is_mla(desc) && m.kind != VLM_MASK_CAUSAL && m.kind != VLM_MASK_ADDITIVE)
            return fail(VLM_ERR_UNSUPPORTED, "mask %d: MLA prefill takes CAUSAL or ADDITIVE masks", i);
    }
    Ws w;
    if ((s = check_ws(desc, S, d_ws, ws_bytes, &w))) return s;
    if (S == 0) {
        if (!vit && kv->len != pos0) {
            HIP_TRY(launch_set_len(kv->dlen(), pos0, stream));
            kv->len = pos0;
        }
        return ok();
    }

    const int dt = desc->dtype, H = desc->hidden, F = desc->ffn, nq = desc->n_q_heads, nkv = desc->n_kv_heads;
    const int hd = desc->head_dim, dv = vdim(desc), QKV = qkv_rows(desc);
    const bool mla = is_mla(desc);
    const size_t E = esize(dt);
    void* hbuf = P(d_ws, w.h);
    float* qkv = (float*)P(d_ws, w.qkv);
    void* qb = P(d_ws, w.q);
    void* ob = P(d_ws, w.o);
    void* ab = P(d_ws, w.a);
    bool normed = false;  // hbuf already holds this layer's input norm (written by the previous reduction)
    for (int l = 0; l < desc->n_layers; l++) {
        const vlm_layer& y = h_layers[l];
        const vlm_mask& mk = h_masks[n_masks == 1 ? 0 : l];
        void *kd, *vd;
        int ldkv;
        if (vit) {
            kd = P(d_ws, w.kv);
            vd = (char*)kd + (size_t)nkv * S * hd * E;
            ldkv = S;
        } else {
            kd = kv->kptr(l);
            vd = kv->vptr(l);
            ldkv = kv->capacity;
        }
        if (!normed)
            HIP_TRY(launch_norm_rows(dt, vit, d_x, S, H, y.attn_norm, y.attn_norm_b, desc->norm_eps, hbuf, stream));
        float* gpart = (float*)P(d_ws, w.gpart);
        GemmArgs g{};
        if (mla) {
            // down-projections of q and kv in one GEMM, their latents normed, then the per-head expansions
            const int AC = mla_a_cols(desc), qr = desc->q_lora_rank, rk = desc->kv_lora_rank;
            float* ma = (float*)P(d_ws, w.ma);
            void* mqa = P(d_ws, w.mqa);
            void* mc = P(d_ws, w.mc);
            float* mkv = qkv + (size_t)S * nq * hd;
            g.A = hbuf; g.B = y.w_a; g.out = ma; g.M = S; g.N = AC; g.K = H; g.ldo = AC;
            g.part = gpart; g.part_cap = w.gpart_floats;
            HIP_TRY(launch_gemm(dt, Epi::StoreF32, g, stream));
            HIP_TRY(launch_norm_rows(dt, false, ma, S, qr, y.q_a_norm, nullptr, desc->norm_eps, mqa, stream, AC));
            HIP_TRY(launch_norm_rows(dt, false, ma + qr, S, rk, y.kv_a_norm, nullptr, desc->norm_eps, mc, stream, AC));
            g = GemmArgs{};
            g.A = mqa; g.B = y.q_b; g.out = qkv; g.M = S; g.N = nq * hd; g.K = qr; g.ldo = nq * hd;
            g.part = gpart; g.part_cap = w.gpart_floats;
            HIP_TRY(launch_gemm(dt, Epi::StoreF32, g, stream));
            const int KVC = nq * (hd - desc->qk_rope_dim + dv);
            g = GemmArgs{};
            g.A = mc; g.B = y.kv_b; g.out = mkv; g.M = S; g.N = KVC; g.K = rk; g.ldo = KVC;
            g.part = gpart; g.part_cap = w.gpart_floats;
            HIP_TRY(launch_gemm(dt, Epi::StoreF32, g, stream));
            MlaRopeArgs r{};
            r.q = qkv; r.kv = mkv; r.ka = ma; r.lda = AC; r.kcol = qr + rk;
            r.S = S; r.nq = nq; r.d = hd; r.dr = desc->qk_rope_dim; r.dv = dv; r.interleave = desc->rope_interleave;
            r.cos = d_cos; r.sin = d_sin; r.qout = qb; r.ldq = S; r.kdst = kd; r.vdst = vd; r.ldkv = ldkv;
            r.pos0 = pos0; r.pos_dev = nullptr;
            HIP_TRY(launch_mla_rope(dt, r, stream));
        } else {
            g.A = hbuf; g.B = y.wqkv; g.bias = vit ? y.bqkv : nullptr; g.out = qkv; g.M = S; g.N = QKV; g.K = H;
            g.ldo = QKV; g.part = gpart; g.part_cap = w.gpart_floats;
            HIP_TRY(launch_gemm(dt, Epi::StoreF32, g, stream));
            RopeArgs r{};
            r.qkv = qkv; r.S = S; r.nq = nq; r.nkv = nkv; r.d = hd; r.segments = desc->rope_segments;
            r.interleave = desc->rope_interleave; r.norm_after = desc->qk_norm == 2;
            r.qn = desc->qk_norm ? y.q_norm : nullptr; r.kn = desc->qk_norm ? y.k_norm : nullptr;
            r.eps = desc->norm_eps;
            r.cos = d_cos; r.sin = d_sin; r.q = qb; r.ldq = S; r.kdst = kd; r.vdst = vd; r.ldkv = ldkv;
            r.pos0 = pos0; r.pos_dev = nullptr;
            HIP_TRY(launch_rope_qkv(dt, r, stream));
        }
        AttnArgs at{};
        at.q = qb; at.ldq = S; at.k = kd; at.v = vd; at.ldkv = ldkv; at.out = ob;
        at.S = S; at.nq = nq; at.nkv = nkv; at.d = hd; at.dv = dv; at.pos0 = pos0; at.nkeys = pos0 + S;
        at.mask_kind = mk.kind; at.add = mk.add; at.ld_add = mk.ld_add; at.seg = mk.seg;
        at.part = gpart; at.part_cap = w.gpart_floats;  // free between the QKV and O projections
        HIP_TRY(launch_attn_prefill(dt, at, stream));
        // O projection + residual; a split-K reduction also writes the post-attention norm of the rows
        int fused = 0;
        g = GemmArgs{};
        g.A = ob; g.B = y.wo; g.bias = vit ? y.bo : nullptr; g.out = d_x; g.M = S; g.N = H; g.K = nq * dv; g.ldo = H;
        g.part = gpart; g.part_cap = w.gpart_floats;
        g.norm_gain = y.mlp_norm; g.norm_shift = vit ? y.mlp_norm_b : nullptr; g.norm_eps = desc->norm_eps;
        g.norm_layer = vit; g.norm_out = hbuf; g.fused_norm = &fused;
        HIP_TRY(launch_gemm(dt, Epi::Resid, g, stream));
        if (!fused)
            HIP_TRY(launch_norm_rows(dt, vit, d_x, S, H, y.mlp_norm, y.mlp_norm_b, desc->norm_eps, hbuf, stream));
        g = GemmArgs{};
        g.A = hbuf; g.B = y.w1; g.out = ab; g.M = S; g.K = H; g.ldo = F;
        g.part = gpart; g.part_cap = w.gpart_floats;
        if (vit) {
            g.bias = y.b1; g.N = F;
            HIP_TRY(launch_gemm(dt, Epi::Gelu, g, stream));
        } else {
            g.N = 2 * F;
            HIP_TRY(launch_gemm(dt, Epi::SwiGLU, g, stream));
        }
        // down projection + residual; a split-K reduction also writes the next layer's input norm
        fused = 0;
        g = GemmArgs{};
        g.A = ab; g.B = y.w2; g.bias = vit ? y.b2 : nullptr; g.out = d_x; g.M = S; g.N = H; g.K = F; g.ldo = H;
        g.part = gpart; g.part_cap = w.gpart_floats;
        if (l + 1 < desc->n_layers) {
            const vlm_layer& yn = h_layers[l + 1];
            g.norm_gain = yn.attn_norm; g.norm_shift = vit ? yn.attn_norm_b : nullptr; g.norm_eps = desc->norm_eps;
            g.norm_layer = vit; g.norm_out = hbuf; g.fused_norm = &fused;
        }
        HIP_TRY(launch_gemm(dt, Epi::Resid, g, stream));
        normed = fused != 0;
    }
    if (!vit) {
        HIP_TRY(launch_set_len(kv->dlen(), pos0 + S, stream));
        kv->len = pos0 + S;
    }
    return ok();
}

// =============================================================================== head
vlm_status vlm_lmhead_argmax(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                             const float* d_x_row, int32_t* d_token_out, float* d_logits, void* d_ws, size_t ws_bytes,
                             hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->vocab < 1) return fail(VLM_ERR_SHAPE, "model has no lm_head table (vocab 0)");
    if (!d_final_norm || !d_table || !aligned16(d_table) || !d_x_row || !d_token_out)
        return fail(VLM_ERR_ARG, "NULL or misaligned pointer");
    Ws w;
    if ((s = check_ws(desc, 0, d_ws, ws_bytes, &w))) return s;
    auto* part = (unsigned long long*)P(d_ws, w.lm);
    HIP_TRY(launch_lmhead_argmax(desc->dtype, d_table, d_x_row, d_final_norm, desc->norm_eps, desc->vocab,
                                 desc->hidden, part, d_logits, d_token_out, nullptr, nullptr, stream));
    return ok();
}

// Allocation-free lm_head argmax: the block partials of the argmax live in a
// file-scope device array (one copy per GPU, held until the process ends)
// instead of the caller's workspace. Host code never passes `scratch` itself
// (in host code the name is a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
constexpr int kNoAllocPartials = 65536;  // u64 argmax keys: vocabularies up to 262137 rows
static __device__ __align__(256) unsigned long long scratch[kNoAllocPartials];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static unsigned long long* g_scratch_ptr[kMaxDevices] = {};

static vlm_status scratch_for_current_device(unsigned long long** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(VLM_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(VLM_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
        g_scratch_ptr[dev] = (unsigned long long*)p;
    }
    *out = g_scratch_ptr[dev];
    return VLM_OK;
}

vlm_status vlm_lmhead_argmax_noalloc(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                                     const float* d_x_row, int32_t* d_token_out, float* d_logits,
                                     hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->vocab < 1) return fail(VLM_ERR_SHAPE, "model has no lm_head table (vocab 0)");
    if (lmhead_partials_max(desc->vocab) > kNoAllocPartials)
        return fail(VLM_ERR_UNSUPPORTED, "vocab %d needs %d argmax partials; the allocation-free scratch holds %d",
                    desc->vocab, lmhead_partials_max(desc->vocab), kNoAllocPartials);
    if (!d_final_norm || !d_table || !aligned16(d_table) || !d_x_row || !d_token_out)
        return fail(VLM_ERR_ARG, "NULL or misaligned pointer");
    unsigned long long* part = nullptr;
    if ((s = scratch_for_current_device(&part))) return s;
    HIP_TRY(launch_lmhead_argmax(desc->dtype, d_table, d_x_row, d_final_norm, desc->norm_eps, desc->vocab,
                                 desc->hidden, part, d_logits, d_token_out, nullptr, nullptr, stream));
    return ok();
}

vlm_status vlm_lmhead_argmax_rows(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                                  const float* d_x, int32_t S, int32_t* d_tokens_out, float* d_logits, void* d_ws,
                                  size_t ws_bytes, hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->vocab < 1) return fail(VLM_ERR_SHAPE, "model has no lm_head table (vocab 0)");
    if (S < 0) return fail(VLM_ERR_SHAPE, "S %d < 0", S);
    if (!d_final_norm || !d_table || !aligned16(d_table) || !d_x || !aligned16(d_x) || !d_tokens_out)
        return fail(VLM_ERR_ARG, "NULL or misaligned pointer");
    Ws w;
    if ((s = check_ws(desc, S, d_ws, ws_bytes, &w))) return s;
    // after the S normalised rows (the only other regions this call uses): the logits when the caller
    // passes none, then the row argmax's partial keys
    float* logits = d_logits;
    size_t off = w.h + al256((size_t)S * desc->hidden * esize(desc->dtype));
    if (!logits) {
        logits = (float*)P(d_ws, off);
        off += al256((size_t)S * desc->vocab * 4);
    }
    const size_t need = off + (size_t)S * argmax_rows_pieces(desc->vocab) * 8;
    if (need > ws_bytes)
        return fail(VLM_ERR_WORKSPACE, "%d rows x vocab %d %sneed %zu workspace bytes, got %zu%s", S, desc->vocab,
                    d_logits ? "argmax keys " : "logits and argmax keys ", need, ws_bytes,
                    d_logits ? "" : "; pass d_logits");
    auto* keys = (unsigned long long*)P(d_ws, off);
    if (S == 0) return ok();
    const int dt = desc->dtype, H = desc->hidden;
    void* hbuf = P(d_ws, w.h);
    HIP_TRY(launch_norm_rows(dt, false, d_x, S, H, d_final_norm, nullptr, desc->norm_eps, hbuf, stream));
    GemmArgs g{};
    g.A = hbuf; g.B = d_table; g.out = logits; g.M = S; g.N = desc->vocab; g.K = H; g.ldo = desc->vocab;
    HIP_TRY(launch_gemm(dt, Epi::StoreF32, g, stream));
    HIP_TRY(launch_argmax_rows(logits, S, desc->vocab, desc->vocab, d_tokens_out, keys, stream));
    return ok();
}

vlm_status vlm_verify_commit(vlm_kv* kv, int32_t pos0, const int32_t* h_draft, int32_t k, const int32_t* d_pred,
                             hipStream_t stream, int32_t* h_n_accept, int32_t* h_next) {
    if (!kv || !h_draft || !d_pred || !h_n_accept || !h_next) return fail(VLM_ERR_ARG, "NULL argument");
    if (k < 1 || k > 4096) return fail(VLM_ERR_SHAPE, "block length %d not in [1, 4096]", k);
    if (pos0 < 0 || (long)pos0 + k != kv->len)
        return fail(VLM_ERR_CAPACITY, "the verified block [%d, %d) must end at the cache length %d", pos0, pos0 + k,
                    kv->len);
    std::vector<int32_t> pred(k);
    HIP_TRY(hipStreamSynchronize(stream));
    HIP_TRY(hipMemcpy(pred.data(), d_pred, k * sizeof(int32_t), hipMemcpyDeviceToHost));
    for (int i = 0; i < k; i++)
        if (pred[i] < 0) return fail(VLM_ERR_NONFINITE, "non-finite logits at verified row %d", i);
    int a = 0;
    while (a + 1 < k && h_draft[a + 1] == pred[a]) a++;
    HIP_TRY(launch_set_len(kv->dlen(), pos0 + a + 1, stream));
    kv->len = pos0 + a + 1;
    *h_n_accept = a;
    *h_next = pred[a];
    return ok();
}

// =============================================================================== sampling
static vlm_status check_sampling(const vlm_sampling* h_params, int vocab, SampleParams* out) {
    if (!h_params) return fail(VLM_ERR_ARG, "sampling parameters NULL");
    if (vocab < 1 || vocab > kSampleVocabMax) return fail(VLM_ERR_SHAPE, "vocab %d not in [1, %d]", vocab, kSampleVocabMax);
    const vlm_sampling& p = *h_params;
    if (!(p.temperature > 0.f) || !std::isfinite(p.temperature))
        return fail(VLM_ERR_ARG, "temperature must be > 0 (greedy decoding is vlm_lmhead_argmax)");
    if (p.top_k < 1 || p.top_k > kSampleMaxK) return fail(VLM_ERR_UNSUPPORTED, "top_k %d not in [1, %d]", p.top_k, kSampleMaxK);
    if (!(p.top_p > 0.f && p.top_p <= 1.f)) return fail(VLM_ERR_ARG, "top_p must be in (0, 1]");
    if (!(p.repetition_penalty > 0.f) || !std::isfinite(p.repetition_penalty))
        return fail(VLM_ERR_ARG, "repetition_penalty must be > 0");
    *out = SampleParams{p.temperature, p.top_k, p.top_p, p.repetition_penalty};
    return VLM_OK;
}

vlm_status vlm_sample_logits(const float* d_logits, int32_t vocab, const vlm_sampling* h_params,
                             const int32_t* d_context_ids, int32_t n_context, const float* d_uniform,
                             int32_t* d_token_out, hipStream_t stream) {
    if (!h_params || !d_logits || !d_uniform || !d_token_out) return fail(VLM_ERR_ARG, "NULL pointer");
    SampleParams sp;
    vlm_status s = check_sampling(h_params, vocab, &sp);
    if (s) return s;
    if (n_context < 0 || (n_context > 0 && !d_context_ids)) return fail(VLM_ERR_ARG, "context ids");
    HIP_TRY(launch_sample_logits(d_logits, vocab, sp, d_context_ids, n_context, d_uniform, d_token_out, stream));
    return ok();
}

// =============================================================================== decode
static vlm_status enqueue_decode(const vlm_model_desc* desc, const vlm_layer* L, const void* embed, const void* fnorm,
                                 const void* table, vlm_kv* kv, const int32_t* tok_in, const float* x_in,
                                 const float* cosv, const float* sinv, int32_t* tok_out, float* x_out, int32_t* hist,
                                 void* ws, const Ws& w, const DecSplitPlan& plan, hipStream_t st,
                                 const SampleParams* samp = nullptr, const float* uniform = nullptr) {
    const int dt = desc->dtype, H = desc->hidden, F = desc->ffn, nq = desc->n_q_heads, nkv = desc->n_kv_heads;
    const int hd = desc->head_dim, dv = vdim(desc), QKV = qkv_rows(desc), W = kv->capacity;
    const bool mla = is_mla(desc);
    float* x = (float*)P(ws, w.xrow);
    void* qrow = P(ws, w.qrow);
    float* qkv = (float*)P(ws, w.qkvrow);
    float* part = (float*)P(ws, w.part);
    void* orow = P(ws, w.orow);
    void* arow = P(ws, w.arow);
    const int nsplit = plan.nsplit;
    float* rope = (float*)P(ws, w.rope);
    HIP_TRY(launch_embed_or_copy(dt, embed, desc->vocab, H, tok_in, x_in, x, kv->dlen(), cosv, sinv,
                                 mla ? desc->qk_rope_dim : hd, rope, st));
    for (int l = 0; l < desc->n_layers; l++) {
        const vlm_layer& y = L[l];
        GemvArgs g{};
        if (mla) {
            // q / kv down-projections of the normed row, the latents' norms fused into the expansions
            const int AC = mla_a_cols(desc), qr = desc->q_lora_rank, rk = desc->kv_lora_rank;
            float* ma = (float*)P(ws, w.marow);
            float* mkv = qkv + (size_t)nq * hd;
            g.W = y.w_a; g.vec = x; g.gain = y.attn_norm; g.eps = desc->norm_eps; g.out = ma; g.N = AC; g.K = H;
            HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::StoreF32, g, st));
            g = GemvArgs{};
            g.W = y.q_b; g.vec = ma; g.gain = y.q_a_norm; g.eps = desc->norm_eps; g.out = qkv; g.N = nq * hd; g.K = qr;
            HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::StoreF32, g, st));
            g = GemvArgs{};
            g.W = y.kv_b; g.vec = ma + qr; g.gain = y.kv_a_norm; g.eps = desc->norm_eps; g.out = mkv;
            g.N = nq * (hd - desc->qk_rope_dim + dv); g.K = rk;
            HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::StoreF32, g, st));
            MlaRopeArgs r{};
            r.q = qkv; r.kv = mkv; r.ka = ma; r.lda = AC; r.kcol = qr + rk;
            r.S = 1; r.nq = nq; r.d = hd; r.dr = desc->qk_rope_dim; r.dv = dv; r.interleave = desc->rope_interleave;
            r.cos = cosv; r.sin = sinv; r.qout = qrow; r.ldq = 1; r.kdst = kv->kptr(l); r.vdst = kv->vptr(l);
            r.ldkv = W; r.pos0 = 0; r.pos_dev = kv->dlen();
            HIP_TRY(launch_mla_rope(dt, r, st));
            DecAttnArgs at{};
            at.qrot = qrow; at.kc = kv->kptr(l); at.vc = kv->vptr(l); at.W = W; at.nq = nq; at.nkv = nkv; at.d = hd;
            at.dv = dv; at.len = kv->dlen(); at.nsplit = nsplit; at.chunk = plan.chunk; at.partial = part;
            HIP_TRY(launch_attn_decode_mla(dt, at, st));
            HIP_TRY(launch_attn_combine(dt, part, nq, nsplit, dv, orow, st));
            g = GemvArgs{};
            g.W = y.wo; g.vec = orow; g.out = x; g.N = H; g.K = nq * dv;
            HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, st));
            g = GemvArgs{};
            g.W = y.w1; g.vec = x; g.gain = y.mlp_norm; g.eps = desc->norm_eps; g.out = arow; g.N = 2 * F; g.K = H;
            HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::SwiGLU, g, st));
            g = GemvArgs{};
            g.W = y.w2; g.vec = arow; g.out = x; g.N = H; g.K = F;
            HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, st));
            continue;
        }
        g.W = y.wqkv; g.vec = x; g.gain = y.attn_norm; g.eps = desc->norm_eps; g.out = qkv; g.N = QKV; g.K = H;
        HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::StoreF32, g, st));
        DecAttnArgs at{};
        at.qkv = qkv; at.qn = desc->qk_norm ? y.q_norm : nullptr; at.kn = desc->qk_norm ? y.k_norm : nullptr;
        at.eps = desc->norm_eps; at.rope = rope; at.segments = desc->rope_segments;
        at.interleave = desc->rope_interleave; at.norm_after = desc->qk_norm == 2;
        at.kc = kv->kptr(l); at.vc = kv->vptr(l); at.W = W; at.nq = nq; at.nkv = nkv; at.d = hd;
        at.len = kv->dlen(); at.nsplit = nsplit; at.chunk = plan.chunk; at.partial = part;
        HIP_TRY(launch_attn_decode_fused(dt, at, st));
        HIP_TRY(launch_attn_combine(dt, part, nq, nsplit, hd, orow, st));
        g = GemvArgs{};
        g.W = y.wo; g.vec = orow; g.out = x; g.N = H; g.K = nq * hd;
        HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, st));
        g = GemvArgs{};
        g.W = y.w1; g.vec = x; g.gain = y.mlp_norm; g.eps = desc->norm_eps; g.out = arow; g.N = 2 * F; g.K = H;
        HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::SwiGLU, g, st));
        g = GemvArgs{};
        g.W = y.w2; g.vec = arow; g.out = x; g.N = H; g.K = F;
        HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, st));
    }
    if (x_out) HIP_TRY(launch_copy_f32(x, x_out, H, st));
    if (table && samp) {  // logits row, then the sampler commits the token (context: the history)
        auto* lm = (unsigned long long*)P(ws, w.lm);
        float* lg = (float*)P(ws, w.logits);
        HIP_TRY(launch_lmhead_argmax(dt, table, x, fnorm, desc->norm_eps, desc->vocab, H, lm, lg, nullptr, nullptr,
                                     nullptr, st));
        HIP_TRY(launch_sample_step(lg, desc->vocab, *samp, hist, uniform, tok_out, kv->dlen(), st));
    } else if (table) {
        auto* lm = (unsigned long long*)P(ws, w.lm);
        HIP_TRY(launch_lmhead_argmax(dt, table, x, fnorm, desc->norm_eps, desc->vocab, H, lm, nullptr, tok_out, hist,
                                     kv->dlen(), st));
    } else {
        HIP_TRY(launch_inc_len(kv->dlen(), st));
    }
    return VLM_OK;
}

static vlm_status check_decode(const vlm_model_desc* desc, const vlm_layer* L, const void* embed, const void* fnorm,
                               const void* table, vlm_kv* kv, const int32_t* tok_in, const float* x_in,
                               const float* cosv, const float* sinv, int32_t table_rows, const int32_t* tok_out,
                               void* ws, size_t ws_bytes, int steps, Ws* w) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->block_kind == VLM_BLOCK_VIT) return fail(VLM_ERR_ARG, "decode needs a decoder stack");
    if (!kv) return fail(VLM_ERR_ARG, "kv is NULL");
    if (memcmp(&kv->desc, desc, sizeof(*desc)) != 0) return fail(VLM_ERR_ARG, "KV cache bound to another model desc");
    if ((long)kv->len + steps > kv->capacity)
        return fail(VLM_ERR_CAPACITY, "decode to length %d exceeds the KV window %d", kv->len + steps, kv->capacity);
    if ((long)kv->len + steps > table_rows)
        return fail(VLM_ERR_CAPACITY, "decode to length %d exceeds the RoPE table rows %d", kv->len + steps, table_rows);
    if (!cosv || !sinv) return fail(VLM_ERR_ARG, "cos/sin NULL");
    if ((s = check_layers(desc, L))) return s;
    if (!x_in) {
        if (desc->vocab < 1 || !embed || !aligned16(embed) || !tok_in)
            return fail(VLM_ERR_ARG, "token input needs an embedding table and d_token_in");
    }
    if (table) {
        if (desc->vocab < 1 || !aligned16(table) || !fnorm || !tok_out)
            return fail(VLM_ERR_ARG, "lm_head needs vocab > 0, final norm and d_token_out");
    }
    return check_ws(desc, 1, ws, ws_bytes, w);
}

vlm_status vlm_decode_step(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                           const void* d_final_norm, const void* d_table, vlm_kv* kv, const int32_t* d_token_in,
                           const float* d_x_in, const float* d_cos, const float* d_sin, int32_t table_rows,
                           int32_t* d_token_out, float* d_x_out, int32_t* d_token_hist, void* d_ws, size_t ws_bytes,
                           hipStream_t stream) {
    Ws w;
    vlm_status s = check_decode(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_in, d_x_in, d_cos, d_sin,
                                table_rows, d_token_out, d_ws, ws_bytes, 1, &w);
    if (s) return s;
    if ((s = enqueue_decode(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_in, d_x_in, d_cos, d_sin,
                            d_token_out, d_x_out, d_token_hist, d_ws, w, attn_decode_plan(kv->capacity, kv->len),
                            stream)))
        return s;
    kv->len += 1;
    return ok();
}

// Decode steps captured into one graph for the launches inside a band (VLM_DEC_GRAPH_STEPS, read per
// call; 1 = one step per launch). Each graph launch costs the GPU a few microseconds more than a
// kernel boundary inside a graph: 8 steps per launch took the 36-layer stack's 256-token decode
// 451.9 -> 450.7 ms (4: 450.9) and the 28-layer stack's 128 tokens 88.0 -> 87.2 ms.
static int dec_graph_steps() {
    const char* e = getenv("VLM_DEC_GRAPH_STEPS");
    const int n = e ? atoi(e) : 8;
    return n < 1 ? 1 : (n > kDecBand ? kDecBand : n);
}

// Captures the steps of each band of positions into HIP graphs (before any launch: one step, and
// dec_graph_steps() steps) and launches n_steps of them; samp == nullptr: greedy argmax head, else
// the sampler with draws `uniform`.
static vlm_status decode_loop_impl(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                                   const void* d_final_norm, const void* d_table, vlm_kv* kv, int32_t* d_token_io,
                                   const float* d_cos, const float* d_sin, int32_t table_rows, int32_t* d_token_hist,
                                   int32_t n_steps, void* d_ws, size_t ws_bytes, const Ws& w, const SampleParams* samp,
                                   const float* uniform, hipStream_t stream) {
    if (n_steps == 0) return ok();
    GraphKey key;
    key.desc = *desc;
    key.layers.assign(h_layers, h_layers + desc->n_layers);
    key.embed = d_embed; key.fnorm = d_final_norm; key.table = d_table; key.tok = d_token_io;
    key.cos = d_cos; key.sin = d_sin; key.table_rows = table_rows; key.hist = d_token_hist;
    key.ws = d_ws; key.ws_bytes = ws_bytes;
    key.sampled = samp != nullptr;
    if (samp) key.sp = *samp;
    key.uniform = uniform;
    const int K = dec_graph_steps();
    key.steps = K;
    if (!kv->has_key || !(kv->key == key)) {
        kv->drop_graph();
        kv->key = key;
        kv->has_key = true;
    }
    // the graphs of the bands the steps pass through, captured before any launch
    vlm_status s = VLM_OK;
    const int b0 = attn_decode_plan(kv->capacity, kv->len).band;
    const int b1 = attn_decode_plan(kv->capacity, kv->len + n_steps - 1).band;
    if ((int)kv->exec.size() <= b1) {
        kv->exec.resize(b1 + 1, nullptr);
        kv->graph.resize(b1 + 1, nullptr);
        kv->execk.resize(b1 + 1, nullptr);
        kv->graphk.resize(b1 + 1, nullptr);
    }
    auto capture = [&](int b, int steps, hipGraph_t* g_out, hipGraphExec_t* e_out) -> vlm_status {
        const DecSplitPlan plan = attn_decode_plan(kv->capacity, b * kDecBand);
        if (!kv->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&kv->cap_stream, hipStreamNonBlocking));
        HIP_TRY(hipStreamBeginCapture(kv->cap_stream, hipStreamCaptureModeThreadLocal));
        vlm_status es = VLM_OK;
        for (int i = 0; i < steps && !es; i++)  // each step reads the length the one before it advanced
            es = enqueue_decode(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_io, nullptr, d_cos, d_sin,
                                d_token_io, nullptr, d_token_hist, d_ws, w, plan, kv->cap_stream, samp, uniform);
        hipGraph_t graph = nullptr;
        hipError_t ee = hipStreamEndCapture(kv->cap_stream, &graph);
        if (es) {
            if (graph) hipGraphDestroy(graph);
            return es;
        }
        if (ee != hipSuccess) return fail(VLM_ERR_HIP, "graph capture: %s", hipGetErrorString(ee));
        hipGraphExec_t exec = nullptr;
        hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        if (ie != hipSuccess) {
            hipGraphDestroy(graph);
            return fail(VLM_ERR_HIP, "graph instantiate: %s", hipGetErrorString(ie));
        }
        *g_out = graph;
        *e_out = exec;
        return VLM_OK;
    };
    for (int b = b0; b <= b1; b++) {
        if (!kv->exec[b] && (s = capture(b, 1, &kv->graph[b], &kv->exec[b]))) return s;
        if (K > 1 && !kv->execk[b] && (s = capture(b, K, &kv->graphk[b], &kv->execk[b]))) return s;
    }
    for (int i = 0; i < n_steps;) {
        const int band = attn_decode_plan(kv->capacity, kv->len).band;
        // K steps in one launch when they all stay in this band (one split plan)
        const bool many = K > 1 && n_steps - i >= K && kv->len % kDecBand + K <= kDecBand;
        const hipError_t le = hipGraphLaunch(many ? kv->execk[band] : kv->exec[band], stream);
        if (le != hipSuccess) return fail(VLM_ERR_HIP, "graph launch at position %d: %s", kv->len, hipGetErrorString(le));
        const int adv = many ? K : 1;
        kv->len += adv;  // the launched steps advance the device length
        i += adv;
    }
    return ok();
}

vlm_status vlm_decode_loop(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                           const void* d_final_norm, const void* d_table, vlm_kv* kv, int32_t* d_token_io,
                           const float* d_cos, const float* d_sin, int32_t table_rows, int32_t* d_token_hist,
                           int32_t n_steps, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    if (n_steps < 0) return fail(VLM_ERR_SHAPE, "n_steps %d < 0", n_steps);
    Ws w;
    vlm_status s = check_decode(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_io, nullptr, d_cos, d_sin,
                                table_rows, d_token_io, d_ws, ws_bytes, n_steps, &w);
    if (s) return s;
    if (!d_table) return fail(VLM_ERR_ARG, "decode loop needs the lm_head table");
    return decode_loop_impl(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_io, d_cos, d_sin, table_rows,
                            d_token_hist, n_steps, d_ws, ws_bytes, w, nullptr, nullptr, stream);
}

vlm_status vlm_decode_loop_sampled(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                                   const void* d_final_norm, const void* d_table, vlm_kv* kv, int32_t* d_token_io,
                                   const float* d_cos, const float* d_sin, int32_t table_rows, int32_t* d_token_hist,
                                   const vlm_sampling* h_params, const float* d_uniform, int32_t n_steps, void* d_ws,
                                   size_t ws_bytes, hipStream_t stream) {
    if (n_steps < 0) return fail(VLM_ERR_SHAPE, "n_steps %d < 0", n_steps);
    Ws w;
    vlm_status s = check_decode(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_io, nullptr, d_cos, d_sin,
                                table_rows, d_token_io, d_ws, ws_bytes, n_steps, &w);
    if (s) return s;
    if (!d_table) return fail(VLM_ERR_ARG, "decode loop needs the lm_head table");
    if (!d_token_hist || !d_uniform) return fail(VLM_ERR_ARG, "the sampled loop needs the token history and draws");
    SampleParams sp;
    if ((s = check_sampling(h_params, desc->vocab, &sp))) return s;
    return decode_loop_impl(desc, h_layers, d_embed, d_final_norm, d_table, kv, d_token_io, d_cos, d_sin, table_rows,
                            d_token_hist, n_steps, d_ws, ws_bytes, w, &sp, d_uniform, stream);
}

// =============================================================================== vision helpers
vlm_status vlm_vit_window_index(int32_t grid_h, int32_t grid_w, int32_t merge, int32_t window, int32_t* h_unit_perm,
                                int32_t* h_row_perm, int32_t* h_row_seg, int32_t* h_pos) {
    if (grid_h < 1 || grid_w < 1 || merge < 1 || window < 1) return fail(VLM_ERR_SHAPE, "sizes must be positive");
    if (grid_h % merge || grid_w % merge) return fail(VLM_ERR_SHAPE, "grid not divisible by merge");
    const int gh = grid_h / merge, gw = grid_w / merge, m2 = merge * merge, n_rows = grid_h * grid_w;
    int p = 0, wid = 0;
    for (int wr = 0; wr < gh; wr += window)
        for (int wc = 0; wc < gw; wc += window, wid++)
            for (int r = wr; r < std::min(wr + window, gh); r++)
                for (int c = wc; c < std::min(wc + window, gw); c++, p++) {
                    const int u = r * gw + c;
                    if (h_unit_perm) h_unit_perm[p] = u;
                    for (int sI = 0; sI < m2; sI++) {
                        const int row = p * m2 + sI;
                        if (h_row_perm) h_row_perm[row] = u * m2 + sI;
                        if (h_row_seg) h_row_seg[row] = wid;
                        if (h_pos) {
                            h_pos[row] = r * merge + sI / merge;
                            h_pos[n_rows + row] = c * merge + sI % merge;
                        }
                    }
                }
    return ok();
}

vlm_status vlm_gather_rows(const float* d_src, int32_t n_src, const int32_t* d_idx, int32_t n_rows, int32_t row_len,
                           float* d_dst, hipStream_t stream) {
    if (n_rows < 0 || row_len < 0 || n_src < 0) return fail(VLM_ERR_SHAPE, "negative size");
    if (n_rows == 0) return ok();
    if (!d_src || !d_idx || !d_dst) return fail(VLM_ERR_ARG, "NULL pointer");
    HIP_TRY(launch_gather_rows(d_src, n_src, d_idx, n_rows, row_len, d_dst, stream));
    return ok();
}

static vlm_status check_merger(const vlm_merger* m, int N) {
    if (!m) return fail(VLM_ERR_ARG, "merger desc NULL");
    if (m->dtype != VLM_F32 && m->dtype != VLM_BF16) return fail(VLM_ERR_DTYPE, "dtype %d", m->dtype);
    if (m->hidden < 8 || m->hidden % 8 || m->merge < 1 || m->merger_hidden < 8 || m->merger_hidden % 8 ||
        m->out_dim < 1)
        return fail(VLM_ERR_SHAPE, "merger sizes invalid");
    if (N < 0 || N % (m->merge * m->merge)) return fail(VLM_ERR_SHAPE, "N %d not a multiple of merge^2", N);
    if (!m->post_ln || !m->post_ln_b || !m->w1 || !m->b1 || !m->w2 || !m->b2) return fail(VLM_ERR_ARG, "NULL weight");
    if (!aligned16(m->w1) || !aligned16(m->w2)) return fail(VLM_ERR_ARG, "weights not 16-byte aligned");
    return VLM_OK;
}

static size_t merger_ws(const vlm_merger* m, int N, size_t* z_off) {
    const size_t E = esize(m->dtype);
    const size_t a = al256((size_t)N * m->hidden * E);
    *z_off = a;
    return a + al256((size_t)(N / (m->merge * m->merge)) * m->merger_hidden * E);
}

vlm_status vlm_vit_merger_workspace_bytes(const vlm_merger* m, int32_t N, size_t* bytes) {
    vlm_status s = check_merger(m, N);
    if (s) return s;
    if (!bytes) return fail(VLM_ERR_ARG, "bytes NULL");
    size_t z;
    *bytes = merger_ws(m, N, &z);
    return ok();
}

vlm_status vlm_vit_merger(const vlm_merger* m, const float* d_x, int32_t N, const int32_t* d_unit_perm, float* d_out,
                          void* d_ws, size_t ws_bytes, hipStream_t stream) {
    vlm_status s = check_merger(m, N);
    if (s) return s;
    if (!d_x || !d_unit_perm || !d_out || !d_ws || ((uintptr_t)d_ws & 255)) return fail(VLM_ERR_ARG, "NULL pointer");
    size_t zoff;
    const size_t need_b = merger_ws(m, N, &zoff);
    if (ws_bytes < need_b) return fail(VLM_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, need_b);
    if (N == 0) return ok();
    const int m2 = m->merge * m->merge, U = N / m2;
    void* hp = d_ws;
    void* z = P(d_ws, zoff);
    HIP_TRY(launch_norm_rows(m->dtype, true, d_x, N, m->hidden, m->post_ln, m->post_ln_b, m->norm_eps, hp, stream));
    GemmArgs g{};
    g.A = hp; g.B = m->w1; g.bias = m->b1; g.out = z; g.M = U; g.N = m->merger_hidden; g.K = m2 * m->hidden;
    g.ldo = m->merger_hidden;
    HIP_TRY(launch_gemm(m->dtype, Epi::Gelu, g, stream));
    g = GemmArgs{};
    g.A = z; g.B = m->w2; g.bias = m->b2; g.out = d_out; g.rowmap = d_unit_perm; g.M = U; g.N = m->out_dim;
    g.K = m->merger_hidden; g.ldo = m->out_dim;
    HIP_TRY(launch_gemm(m->dtype, Epi::StoreRowMap, g, stream));
    return ok();
}

// =============================================================================== measurement
vlm_status vlm_decode_split_plan(int32_t capacity, int32_t t, int32_t* nsplit, int32_t* chunk) {
    if (!nsplit || !chunk) return fail(VLM_ERR_ARG, "NULL pointer");
    if (capacity < 1 || t < 0 || t >= capacity) return fail(VLM_ERR_SHAPE, "t %d outside [0, %d)", t, capacity);
    const DecSplitPlan p = attn_decode_plan(capacity, t);
    *nsplit = p.nsplit;
    *chunk = p.chunk;
    return ok();
}

vlm_status vlm_launch_kernel(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_final_norm,
                             const void* d_table, vlm_kv* kv, const float* d_cos, const float* d_sin,
                             int32_t table_rows, int32_t which, int32_t n_launches, const float* d_x_row, void* d_ws,
                             size_t ws_bytes, hipStream_t stream) {
    vlm_status s = check_desc(desc);
    if (s) return s;
    if (desc->block_kind != VLM_BLOCK_DECODER) return fail(VLM_ERR_ARG, "decoder (GQA) kernels only");
    if (which < VLM_KERNEL_LMHEAD || which > VLM_KERNEL_ATTN) return fail(VLM_ERR_ARG, "which %d", which);
    if (n_launches < 0) return fail(VLM_ERR_SHAPE, "n_launches < 0");
    if (!d_x_row) return fail(VLM_ERR_ARG, "d_x_row is NULL");
    if (which == VLM_KERNEL_LMHEAD) {
        if (desc->vocab < 1 || !d_table || !aligned16(d_table) || !d_final_norm)
            return fail(VLM_ERR_ARG, "lm_head needs vocab > 0, table and final norm");
    } else if ((s = check_layers(desc, h_layers))) {
        return s;
    }
    if (which == VLM_KERNEL_ATTN) {
        if (!kv || !d_cos || !d_sin) return fail(VLM_ERR_ARG, "attention needs the KV cache and RoPE tables");
        if (memcmp(&kv->desc, desc, sizeof(*desc)) != 0) return fail(VLM_ERR_ARG, "KV cache bound to another model");
        if (kv->len >= kv->capacity) return fail(VLM_ERR_CAPACITY, "cache full");
        if (kv->len >= table_rows)
            return fail(VLM_ERR_CAPACITY, "position %d beyond the RoPE table rows %d", kv->len, table_rows);
    }
    Ws w;
    if ((s = check_ws(desc, 1, d_ws, ws_bytes, &w))) return s;
    const int dt = desc->dtype, H = desc->hidden, F = desc->ffn, nq = desc->n_q_heads, hd = desc->head_dim;
    float* x = (float*)P(d_ws, w.xrow);
    float* rope = (float*)P(d_ws, w.rope);
    if (which == VLM_KERNEL_ATTN)  // the row copy also stages the RoPE row, as a decode step's embed kernel does
        HIP_TRY(launch_embed_or_copy(desc->dtype, nullptr, 0, H, nullptr, d_x_row, x, kv->dlen(), d_cos, d_sin, hd,
                                     rope, stream));
    else
        HIP_TRY(launch_copy_f32(d_x_row, x, H, stream));
    for (int i = 0; i < n_launches; i++) {
        const int l = i % desc->n_layers;
        const vlm_layer& y = h_layers ? h_layers[l] : vlm_layer{};
        GemvArgs g{};
        switch (which) {
            case VLM_KERNEL_LMHEAD:
                HIP_TRY(launch_lmhead_argmax(dt, d_table, x, d_final_norm, desc->norm_eps, desc->vocab, H,
                                             (unsigned long long*)P(d_ws, w.lm), nullptr, nullptr, nullptr, nullptr,
                                             stream));
                break;
            case VLM_KERNEL_QKV:
                g.W = y.wqkv; g.vec = x; g.gain = y.attn_norm; g.eps = desc->norm_eps; g.out = P(d_ws, w.qkvrow);
                g.N = qkv_rows(desc); g.K = H;
                HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::StoreF32, g, stream));
                break;
            case VLM_KERNEL_O:
                g.W = y.wo; g.vec = P(d_ws, w.orow); g.out = P(d_ws, w.qkvrow); g.N = H; g.K = nq * hd;
                HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, stream));
                break;
            case VLM_KERNEL_GATE_UP:
                g.W = y.w1; g.vec = x; g.gain = y.mlp_norm; g.eps = desc->norm_eps; g.out = P(d_ws, w.arow);
                g.N = 2 * F; g.K = H;
                HIP_TRY(launch_gemv(dt, Pro::RmsNorm, Epi::SwiGLU, g, stream));
                break;
            case VLM_KERNEL_DOWN:
                g.W = y.w2; g.vec = P(d_ws, w.arow); g.out = P(d_ws, w.qkvrow); g.N = H; g.K = F;
                HIP_TRY(launch_gemv(dt, Pro::Plain, Epi::Resid, g, stream));
                break;
            default: {
                DecAttnArgs at{};
                at.qkv = (const float*)P(d_ws, w.qkvrow); at.qn = desc->qk_norm ? y.q_norm : nullptr;
                at.kn = desc->qk_norm ? y.k_norm : nullptr; at.eps = desc->norm_eps; at.rope = rope;
                at.segments = desc->rope_segments; at.kc = kv->kptr(l); at.vc = kv->vptr(l); at.W = kv->capacity;
                at.interleave = desc->rope_interleave; at.norm_after = desc->qk_norm == 2;
                at.nq = nq; at.nkv = desc->n_kv_heads; at.d = hd; at.len = kv->dlen();
                const DecSplitPlan plan = attn_decode_plan(kv->capacity, kv->len);
                at.nsplit = plan.nsplit; at.chunk = plan.chunk;
                at.partial = (float*)P(d_ws, w.part);
                HIP_TRY(launch_attn_decode_fused(dt, at, stream));
                break;
            }
        }
    }
    return ok();
}

}  // extern "C"
