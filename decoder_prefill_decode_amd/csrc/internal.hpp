// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Launchers enqueue on `st` and return the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vlm {

// vlm_mask_kind values of the C ABI
constexpr int VLM_MASK_CAUSAL_ID = 0, VLM_MASK_NONE_ID = 1, VLM_MASK_ADDITIVE_ID = 2, VLM_MASK_SEGMENT_ID = 3;

enum class Epi : int {
    StoreF32 = 0,    // out_f32[m][n] = acc (+ bias[n])
    Resid = 1,       // x[m][n] += acc (+ bias[n])
    SwiGLU = 2,      // out_T[m][n/2] = silu(gate) * up over 32-row interleaved groups
    Gelu = 3,        // out_T[m][n] = gelu_tanh(acc + bias[n])
    StoreRowMap = 4, // out_f32[rowmap[m]][n] = acc + bias[n]
    Argmax = 5       // GEMV only: per-block argmax key of the row results (+ optional logits)
};

struct GemmArgs {
    const void* A;     // [M][K] operand rows, element type of the model (bf16 or f32)
    const void* B;     // [N][K] weights
    const void* bias;  // [N] or null (model element type)
    void* out;         // epilogue target
    const int32_t* rowmap;
    int M, N, K;
    int ldo;           // row stride of `out` in elements
    float* part = nullptr;  // split-K scratch (fp32 [splits][M][N]); null: no split-K
    size_t part_cap = 0;    // floats available at `part`
    // Epi::Resid with norm_out set: when the GEMM splits K (and N <= 4096), the reduction that adds
    // the partials into the residual rows also writes their RMSNorm (LayerNorm when norm_layer)
    // with norm_gain / norm_shift to norm_out ([M][N], model type) and sets *fused_norm = 1.
    // Bitwise the same rows as a separate launch_norm_rows over the updated x.
    const void* norm_gain = nullptr;
    const void* norm_shift = nullptr;
    float norm_eps = 0.f;
    bool norm_layer = false;
    void* norm_out = nullptr;
    int* fused_norm = nullptr;  // host flag
};

// dtype: 0 = f32, 1 = bf16 (vlm_dtype values)
hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t st);
// bf16 projections of M <= 16 rows (StoreF32, Resid, SwiGLU; no bias or row map, K % 8 == 0):
// a weight stream reusing each load for every row; launch_gemm takes it whenever
// gemm_small_fits() (a residual or a split projection needs a.part for its fp32 partials).
bool gemm_small_fits(int dtype, Epi epi, const GemmArgs& a);
hipError_t launch_gemm_small(Epi epi, const GemmArgs& a, hipStream_t st);
// The split-K reduction of a bf16 GEMM whose fp32 partials [splits][M][N] are in a.part (Resid with
// a.norm_out also writes the row norm when it fits, as the prefill GEMM's reduction does).
hipError_t launch_split_reduce(Epi epi, const GemmArgs& a, int splits, hipStream_t st);

// Operand of a decode projection: RMSNorm of fp32 x, or a plain model-type vector (PlainLds: the
// same operand, staged once per block in LDS; chosen inside launch_gemv for long rows).
enum class Pro : int { RmsNorm = 0, Plain = 1, PlainLds = 2 };
struct GemvArgs {
    const void* W;          // [N][K]
    const void* vec;        // Pro::RmsNorm: fp32 x [K]; Pro::Plain: model-type vector [K]
    const void* gain;       // RmsNorm gain [K] (model type)
    float eps;
    void* out;              // StoreF32: f32 [N]; Resid: f32 x [N]; SwiGLU: model type [N/2]; Argmax: f32 logits or null
    int N, K;
    unsigned long long* partials = nullptr;  // Argmax only: one key per block
};
hipError_t launch_gemv(int dtype, Pro pro, Epi epi, const GemvArgs& a, hipStream_t st);

// lm_head: logits of final-normed x against table [V][K]; block partials of the argmax
// into `partials` (u64 per block), optional logits; then a final reduction.
int lmhead_blocks(int V);
hipError_t launch_lmhead(int dtype, const void* table, const float* x, const void* gain, float eps, int V, int K,
                         unsigned long long* partials, float* logits, hipStream_t st);
// token_out[0] = argmax (or -1); when kv_len != null (the cache header): hist[len+1] = token (if hist),
// *kv_len += 1; for -1 instead the length stays and header words 1, 2 record the first such position.
hipError_t launch_argmax_final(const unsigned long long* partials, int nblocks, int32_t* token_out, int32_t* hist,
                               int32_t* kv_len, hipStream_t st);

// out[r] = argmax of logits row r (r < S, row stride ld; lowest index on ties, -1 for a non-finite row).
// Row argmax of S logits rows (row r at logits + r * ld): argmax_rows_pieces(V) blocks per row write
// partial keys to part [S][argmax_rows_pieces(V)], then one wavefront per row reduces them.
int argmax_rows_pieces(int V);
hipError_t launch_argmax_rows(const float* logits, int S, int V, int ld, int32_t* out, unsigned long long* part,
                              hipStream_t st);

// Row norms producing the GEMM operand (model type): RMSNorm (shift == null, layer == false)
// or LayerNorm (layer == true, shift may be null).
hipError_t launch_norm_rows(int dtype, bool layer, const float* x, int R, int H, const void* gain, const void* shift,
                            float eps, void* out, hipStream_t st, int ldx = 0);  // ldx: row stride of x (0: H)

// qkv fp32 [S][(nq+2nkv)*d] -> q' [nq][ldq][d] (model type), K/V rows written to
// kdst/vdst [nkv][ldkv][d] at slot base+s, base = pos_dev ? *pos_dev : pos0.
// cos/sin rows base+s. Optional per-head RMSNorm (qn/kn gains) before RoPE
// (norm_after == 0) or after it (norm_after == 1). interleave: each segment's
// adjacent pairs (2j, 2j+1) rotate together and land at j and j + segment/2.
struct RopeArgs {
    const float* qkv;
    int S, nq, nkv, d, segments, interleave, norm_after;
    const void* qn; const void* kn; float eps;
    const float* cos; const float* sin;
    void* q; int ldq;
    void* kdst; void* vdst; int ldkv;
    int pos0; const int32_t* pos_dev;
};
hipError_t launch_rope_qkv(int dtype, const RopeArgs& a, hipStream_t st);

// Expanded MLA heads: q [S][nq*d] and kv [S][nq*(dn + dv)] fp32 projections (per head
// [q_nope | q_rope] and [k_nope | v]), the shared rotated key at column kcol of ka [S][lda];
// writes q' [nq][ldq][d] (model type) and the K [nq][ldkv][d] / V [nq][ldkv][dv] cache rows of
// slot base+s, k = [k_nope | RoPE(k_rope)]. cos/sin rows are dr wide.
struct MlaRopeArgs {
    const float* q; const float* kv; const float* ka;
    int lda, kcol;
    int S, nq, d, dr, dv, interleave;
    const float* cos; const float* sin;
    void* qout; int ldq;
    void* kdst; void* vdst; int ldkv;
    int pos0; const int32_t* pos_dev;
};
hipError_t launch_mla_rope(int dtype, const MlaRopeArgs& a, hipStream_t st);

// Prefill flash attention. q [nq][ldq][d], k [nkv][ldkv][d], v [nkv][ldkv][dv]; keys
// 0..nkeys-1; query row s has position pos0+s; out [S][nq*dv] (model type). dv = 0 means d.
struct AttnArgs {
    const void* q; int ldq;
    const void* k; const void* v; int ldkv;
    void* out;
    int S, nq, nkv, d, pos0, nkeys;
    int mask_kind; const float* add; int ld_add; const int32_t* seg;
    int dv = 0;
    // fp32 scratch for a few-row launch (bf16, causal or no mask, nq/nkv * S <= 64): the key tiles
    // split over blocks, each writing (o, m, l) partials that the decode merge kernel combines.
    // Null (or too small): the row-tiled kernel runs instead.
    float* part = nullptr;
    size_t part_cap = 0;  // floats at part
    int split_tiles = 0;  // set by the launcher: 64-key tiles per block of the few-row launch
};
hipError_t launch_attn_prefill(int dtype, const AttnArgs& a, hipStream_t st);

// Decode attention over slots 0..*len (inclusive) of k/v [nkv][W][d]; q [nq][d].
// Decode attention splits the valid slots over at most this many blocks per KV
// head; each writes one partial row of d + 4 floats (o[d], m, l, pad) per query head.
constexpr int kDecMaxSplits = 32;
// Split plan of the decode attention at position t (0-based): the positions
// come in bands of kDecBand; a band's launches cover slots [0, tb), tb the
// band's end (at most the capacity), with nsplit <= kDecMaxSplits splits of
// `chunk` slots (a multiple of the 16 keys a block scores per step). The
// split layout lives only between one attention launch and its merge, so it
// may change from band to band; the decode graphs are kept per band.
constexpr int kDecBand = 64;
struct DecSplitPlan {
    int nsplit, chunk, band;
};
DecSplitPlan attn_decode_plan(int capacity, int t);

// Decode attention of one layer: QK-Norm + RoPE of the new token's q and k
// (position t = *len), K/V written into slot t, split-K attention over slots
// 0..t into `partial`; launch_attn_combine merges the splits into `out`.
struct DecAttnArgs {
    const float* qkv;  // [nq + 2*nkv][d] fp32 projections of the token
    const void* qn; const void* kn; float eps;
    const float* rope; int segments;  // cos[d] then sin[d] of position len (staged by the embed kernel)
    int interleave, norm_after;       // as in RopeArgs
    const void* qrot = nullptr;       // expanded MLA: the rotated q [nq][d] (model type), k/v already in slot t
    int dv = 0;                       // expanded MLA: value width (partial rows dv + 4)
    void* kc; void* vc;  // layer K and V, [nkv][W][d]
    int W, nq, nkv, d;
    const int32_t* len;
    int nsplit, chunk;   // launched splits; split sp scores slots [sp*chunk, (sp+1)*chunk) below t + 1
    float* partial;      // [nq][nsplit][d + 4]
};
hipError_t launch_attn_decode_fused(int dtype, const DecAttnArgs& a, hipStream_t st);
// Expanded MLA decode attention (d 192, dv 128, nq == nkv): reads a.qrot and the cache only.
hipError_t launch_attn_decode_mla(int dtype, const DecAttnArgs& a, hipStream_t st);
hipError_t launch_attn_combine(int dtype, const float* partial, int nq, int nsplit, int d, void* out,
                               hipStream_t st);

// Next-token sampler over one logits row (one block): penalty on context ids,
// temperature, top-k (1..kSampleMaxK), top-p, inverse-CDF draw with *u.
constexpr int kSampleMaxK = 1024;
constexpr int kSampleVocabMax = 1 << 19;
struct SampleParams { float temperature; int top_k; float top_p; float penalty; };
hipError_t launch_sample_logits(const float* logits, int V, const SampleParams& p, const int32_t* ctx, int nctx,
                                const float* u, int32_t* out, hipStream_t st);
// The sampler as the last kernel of a decode step at position t = kv_len[0] (the cache header):
// context hist[0..t], draw u[t + 1]; the token goes to out[0] and hist[t + 1], the length to t + 1
// (a step with no token is not committed and flags the header, as launch_argmax_final does).
hipError_t launch_sample_step(const float* logits, int V, const SampleParams& p, int32_t* hist, const float* u,
                              int32_t* out, int32_t* kv_len, hipStream_t st);

// Final RMSNorm + lm_head GEMV + argmax. Writes per-block argmax keys to
// `partials` (lmhead_partials_max(V) entries) and the logits when non-null.
// token_out == null: partials only; otherwise a second kernel reduces the
// token, then hist[len+1] = token (if hist) and *kv_len += 1 (if kv_len; a non-finite step is not
// committed: the length stays and header words 1, 2 flag it, see launch_argmax_final).
int lmhead_partials_max(int V);
hipError_t launch_lmhead_argmax(int dtype, const void* table, const float* x, const void* gain, float eps, int V,
                                int K, unsigned long long* partials, float* logits, int32_t* token_out, int32_t* hist,
                                int32_t* kv_len, hipStream_t st);

hipError_t launch_embed(int dtype, const void* table, int V, int H, const int32_t* ids, int S, float* x,
                        hipStream_t st);
// Decode input row: embedding of *tok (or a copy of xin); with rope != NULL also
// stages the RoPE row of position *len: rope[0..D) = cos, rope[D..2D) = sin.
hipError_t launch_embed_or_copy(int dtype, const void* table, int V, int H, const int32_t* tok, const float* xin,
                                float* x, const int32_t* len, const float* cosv, const float* sinv, int D, float* rope,
                                hipStream_t st);
hipError_t launch_inject(int img_dtype, float* x, int S, int H, const int32_t* ids, int pid, const void* img,
                         int n_img, hipStream_t st);
hipError_t launch_set_len(int32_t* len, int value, hipStream_t st);
hipError_t launch_inc_len(int32_t* len, hipStream_t st);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st);
hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t st);
hipError_t launch_rope_table(const int32_t* pos, int n_axes, int n_rows, const int32_t* axis_of_pair, int segments,
                             int d, double theta, float* cos, float* sin, hipStream_t st);
hipError_t launch_gather_rows(const float* src, int n_src, const int32_t* idx, int n_rows, int row_len, float* dst,
                              hipStream_t st);
hipError_t launch_pack_gate_up(int dtype, const void* wg, const void* wu, int F, int H, void* out, hipStream_t st);

}  // namespace vlm
