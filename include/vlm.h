/*
 * vlm.h — C ABI of the MI355X (gfx950) VLM decoder hot path.
 *
 * The library runs, on one GPU, the decoder stack that a vision-language
 * model executes after its vision tower: embedding lookup, injection of
 * projected image rows into the placeholder positions, parallel causal
 * prefill that fills a per-layer fixed-window KV cache, one-token KV-cache
 * decode, final RMSNorm, lm_head and greedy argmax; plus the window/full
 * attention ViT stack with its 2x2 patch merger.
 *
 * Sources (page title, section) cited below:
 *   [Youtu]   Youtu-VL-4B ncnn port (ncnn discussion #6850)
 *   [Penguin] Penguin-VL ncnn port (ncnn discussion #6868)
 *   [HyOCR15] HunyuanOCR v1.5 ncnn port, technical report (ncnn discussion #6846)
 *   [HyOCR10] HunyuanOCR v1.0 ncnn port (ncnn discussion #6847)
 *   [MNN]     MNN llm_demo Omni article (hmyw.cn news 148174)
 *
 * Conventions for every entry point:
 *   - Pointers prefixed d_ are device pointers, h_ are host pointers. Every
 *     device buffer belongs to the caller; the library never allocates or
 *     frees device memory. Pointers are borrowed: they must stay valid until
 *     the work enqueued on `stream` has completed. Host arrays are read during
 *     the call only.
 *   - All device work is enqueued asynchronously on the caller's `stream`.
 *   - Every argument, shape, count and capacity check runs before anything is
 *     enqueued, so a call that returns an error has changed nothing (the KV
 *     length included). A HIP launch failure returns VLM_ERR_HIP; faults of
 *     earlier asynchronous work surface at the caller's next synchronisation.
 *   - vlm_last_error() returns a thread-local description of the last error.
 *   - A vlm_kv handle and a workspace must not be used by two streams at once.
 *   - Weight element type: desc->dtype (VLM_F32 -> float, VLM_BF16 -> bfloat16
 *     bits). All matrices are row-major, [out_features][in_features].
 */
#ifndef VLM_H
#define VLM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VLM_OK = 0,
    VLM_ERR_ARG = -1,            /* NULL / misaligned pointer, bad enum value */
    VLM_ERR_SHAPE = -2,          /* sizes inconsistent or unsupported by the kernels */
    VLM_ERR_CAPACITY = -3,       /* sequence would exceed the KV window or the RoPE table */
    VLM_ERR_COUNT_MISMATCH = -4, /* placeholder count != image rows */
    VLM_ERR_DTYPE = -5,          /* dtype not valid for this call */
    VLM_ERR_NONFINITE = -6,      /* an argmax saw a non-finite logit (vlm_kv_status, vlm_token_status) */
    VLM_ERR_HIP = -7,            /* a HIP runtime call failed */
    VLM_ERR_UNSUPPORTED = -8,    /* valid request that this build has no kernel for */
    VLM_ERR_WORKSPACE = -9       /* workspace too small */
} vlm_status;

typedef enum { VLM_F32 = 0, VLM_BF16 = 1 } vlm_dtype;
/* DECODER: Qwen3/Llama-style GQA layer. VIT: pre-LayerNorm vision layer.
 * MLA: multi-head latent attention in the expanded form of [Youtu] 实现流程 §6
 * (no latent absorption: kv_b expands the compressed KV into per-head keys and
 * values, which the cache stores; n_kv_heads == n_q_heads). */
typedef enum { VLM_BLOCK_DECODER = 0, VLM_BLOCK_VIT = 1, VLM_BLOCK_MLA = 2 } vlm_block_kind;

/* Attention masks of the prefill ([Youtu] 实现流程 §3 and §7; [HyOCR10] 五.6).
 * CAUSAL:   query row s (position pos0+s) sees cache slots 0..pos0+s.
 * NONE:     every query row sees slots 0..pos0+S-1.
 * ADDITIVE: every query row sees slots 0..pos0+S-1 and add[s*ld_add + j] is
 *           added to the scaled score of slot j (the pages' finite 0 / -1e9
 *           form; any finite values are allowed).
 * SEGMENT:  non-causal, pos0 must be 0: row s sees row j iff seg[s] == seg[j]
 *           (the block-diagonal window mask of the vision tower). */
typedef enum { VLM_MASK_CAUSAL = 0, VLM_MASK_NONE = 1, VLM_MASK_ADDITIVE = 2, VLM_MASK_SEGMENT = 3 } vlm_mask_kind;

typedef struct {
    int32_t kind;          /* vlm_mask_kind */
    int32_t ld_add;        /* ADDITIVE: row stride of add in floats, >= pos0+S */
    const float* add;      /* ADDITIVE: d_ [S][ld_add] fp32; else NULL */
    const int32_t* seg;    /* SEGMENT: d_ [S] segment ids; else NULL */
} vlm_mask;

/* Model shape ([Penguin] §2.1 for the Qwen3 fields; [Youtu] 实现流程 §3 for the ViT).
 * Kernels exist for head_dim in {64, 72, 80, 128}; hidden, ffn and
 * n_q_heads*head_dim must be multiples of 8; a decoder's ffn a multiple of 32;
 * n_q_heads a multiple of n_kv_heads (GQA: query head h reads KV head
 * h / (n_q_heads / n_kv_heads), [Penguin] §3). */
typedef struct {
    int32_t block_kind;    /* vlm_block_kind */
    int32_t n_layers;
    int32_t hidden;        /* H */
    int32_t n_q_heads;     /* nq */
    int32_t n_kv_heads;    /* nkv (ViT: equal to nq) */
    int32_t head_dim;      /* d */
    int32_t ffn;           /* F */
    int32_t vocab;         /* V rows of the embedding / lm_head table; 0 = none */
    int32_t dtype;         /* vlm_dtype of weights, gains, table, KV cache and GEMM operands */
    int32_t qk_norm;       /* per-head RMSNorm of q and k with gains q_norm / k_norm: 0 none;
                              1 before RoPE (Qwen3 order, [Penguin] §5.4); 2 after RoPE, so the
                              cache holds the normalised k (HunyuanOCR order, [HyOCR10] 五.2) */
    int32_t rope_segments; /* 1: rotate-half over the whole head; 2: each half rotated on its own (2D vision RoPE, [Penguin] §2.3) */
    float norm_eps;        /* RMSNorm / LayerNorm epsilon (1e-6) */
    int32_t rope_interleave; /* 0: rotate-half pairs (j, j + seg/2) of each RoPE segment; 1: adjacent
                              pairs (2j, 2j+1) rotate (at the frequency of pair j) and are stored at
                              j and j + seg/2, i.e. the head is de-interleaved before rotate-half
                              ([Youtu] 实现难点 §2); q and the cached k keep that order, v does not
                              move. The cos/sin tables are the same for both. */
    /* VLM_BLOCK_MLA only (0 for the other kinds). head_dim is the q/k head width
     * dn + dr, where the last dr = qk_rope_dim elements rotate; v_head_dim the
     * value width; the RoPE tables are dr wide. Kernels exist for head_dim 192,
     * qk_rope_dim 64, v_head_dim 128 (the pages' K 192 / V 128), q_lora_rank and
     * kv_lora_rank multiples of 8; qk_norm 0, rope_segments 1. */
    int32_t q_lora_rank;   /* qr: rank of the q down-projection */
    int32_t kv_lora_rank;  /* r: width of the compressed KV (512 on the pages) */
    int32_t qk_rope_dim;   /* dr */
    int32_t v_head_dim;    /* dv */
} vlm_model_desc;

/* Per-layer weights (device pointers, element type desc->dtype).
 * Expanded MLA (block_kind MLA; wqkv, q_norm, k_norm unused): attn_norm,
 *   mlp_norm [H]; w_a [qr + r + dr][H] = the q down-projection rows, then the
 *   kv down-projection rows (r latent rows, then dr rows of the shared rotated
 *   key); q_a_norm [qr], kv_a_norm [r] RMSNorm gains; q_b [nq*(dn+dr)][qr]
 *   (per head: dn rows, then dr rows to rotate); kv_b [nq*(dn+dv)][r] (per
 *   head: dn key rows, then dv value rows); wo [H][nq*dv]; w1, w2 as for the
 *   decoder. Order: h = RMSNorm(x); q = RMSNorm(h q_a^T) q_b^T;
 *   [c | k_rope] = h kv_a^T; [k_nope | v] = RMSNorm(c) kv_b^T; q and k are
 *   [nope | RoPE(rope part)], the rotated key shared by all heads; attention
 *   scale 1/sqrt(dn + dr).
 * Decoder ([Penguin] §2.1, §4.2): RMSNorm gains attn_norm, mlp_norm [H];
 *   wqkv [(nq+2*nkv)*d][H] = rows of Wq, then Wk, then Wv (see vlm_pack_qkv);
 *   q_norm, k_norm [d] (qk_norm only); wo [H][nq*d];
 *   w1 [2F][H] = gate and up rows interleaved in groups of 32 rows: rows
 *   64g..64g+31 are gate rows 32g..32g+31 and rows 64g+32..64g+63 the up rows
 *   32g..32g+31 (see vlm_pack_gate_up); w2 = down [H][F]. Biases NULL.
 * ViT ([Youtu] 实现流程 §3): LayerNorm gain/shift attn_norm/attn_norm_b and
 *   mlp_norm/mlp_norm_b [H]; wqkv [3*nq*d][H] + bqkv; wo [H][nq*d] + bo;
 *   w1 = fc1 [F][H] + b1; w2 = fc2 [H][F] + b2. GELU (tanh form) after fc1. */
typedef struct {
    const void* attn_norm;
    const void* attn_norm_b;
    const void* wqkv;
    const void* bqkv;
    const void* q_norm;
    const void* k_norm;
    const void* wo;
    const void* bo;
    const void* mlp_norm;
    const void* mlp_norm_b;
    const void* w1;
    const void* b1;
    const void* w2;
    const void* b2;
    const void* w_a;        /* MLA only (see above); NULL otherwise */
    const void* q_a_norm;
    const void* q_b;
    const void* kv_a_norm;
    const void* kv_b;
} vlm_layer;

/* ------------------------------------------------------------------------- */
/* KV cache ([Youtu] 实现流程 §7: fixed window per layer, runtime-owned slots;
 * [HyOCR15] §3.7: cache stays resident on the device).
 * The caller provides one device buffer of vlm_kv_bytes() bytes. Layout:
 *   bytes [0, 256): device header (int32 length at offset 0, rest reserved);
 *   then per layer the K elements [nkv][W][d], then the V elements
 *   [nkv][W][dv] (type desc->dtype; dv = v_head_dim for MLA, else d; the
 *   last index contiguous), so one decode split reads a contiguous run of
 *   slots of one KV head.
 * The handle keeps a host mirror of the length; kernels use the device copy,
 * which lets a captured decode step replay unchanged. */
typedef struct vlm_kv vlm_kv;

/* Bytes needed for a cache of `capacity` slots per layer. */
vlm_status vlm_kv_bytes(const vlm_model_desc* desc, int32_t capacity, size_t* bytes);
/* Binds caller memory (256-byte aligned, >= vlm_kv_bytes) to a new host
 * handle and enqueues a kernel that sets the device length to 0. */
vlm_status vlm_kv_alloc(const vlm_model_desc* desc, int32_t capacity, void* d_buf, size_t bytes,
                        hipStream_t stream, vlm_kv** out);
/* Frees the host handle (and its cached decode graphs), not the device memory. */
vlm_status vlm_kv_free(vlm_kv* kv);
/* Host mirror of the number of valid slots. */
vlm_status vlm_kv_len(const vlm_kv* kv, int32_t* len);
/* Shrinks the valid length to new_len <= current length (host mirror and,
 * through an enqueued kernel, the device copy); slots >= new_len are then
 * treated as empty. Used to commit only an accepted prefix after a
 * multi-token verify ([HyOCR15] §3.8). */
vlm_status vlm_kv_truncate(vlm_kv* kv, int32_t new_len, hipStream_t stream);

/* Non-finite results ([Penguin] §4.1: a mismatch that silently produced token 0
 * is the failure to avoid; an explicit error instead). A decode step whose
 * argmax sees a NaN or infinite logit writes -1 as its token, does not advance
 * the device length (the step is not committed: slots 0..t-1 and the length
 * stay as they were) and sets a flag in the cache header with its position t;
 * later steps of a loop then read token -1, whose embedding row is NaN, and
 * fail the same way, so the cache stays at t.
 * vlm_kv_status synchronizes `stream`, reads the header and returns
 * VLM_ERR_NONFINITE with *h_pos = t (the first failed position) when the flag
 * is set; it then sets the host length mirror to the device length and clears
 * the flag. Otherwise VLM_OK and *h_pos = -1 (h_pos may be NULL).
 * vlm_token_status synchronizes `stream` and reads d_token[0] (the output of
 * vlm_lmhead_argmax or vlm_sample_logits): VLM_ERR_NONFINITE when it is -1,
 * else VLM_OK; *h_token receives the value (h_token may be NULL). */
vlm_status vlm_kv_status(vlm_kv* kv, hipStream_t stream, int32_t* h_pos);
vlm_status vlm_token_status(const int32_t* d_token, hipStream_t stream, int32_t* h_token);

/* Bytes of scratch needed by vlm_prefill (S <= max_rows), vlm_decode_step,
 * vlm_decode_loop and vlm_lmhead_argmax for this model. */
vlm_status vlm_workspace_bytes(const vlm_model_desc* desc, int32_t max_rows, size_t* bytes);

/* ------------------------------------------------------------------------- */
/* Weight packing (device to device copies, element type dtype).
 * vlm_pack_qkv: out [(nq+2nkv)*d][H] = concat(wq [nq*d][H], wk [nkv*d][H], wv [nkv*d][H]).
 * vlm_pack_gate_up: out [2F][H] interleaved in 32-row groups as vlm_layer.w1 states; F % 32 == 0. */
vlm_status vlm_pack_qkv(const void* d_wq, const void* d_wk, const void* d_wv, int32_t q_rows, int32_t kv_rows,
                        int32_t hidden, int32_t dtype, void* d_out, hipStream_t stream);
vlm_status vlm_pack_gate_up(const void* d_wg, const void* d_wu, int32_t ffn, int32_t hidden, int32_t dtype,
                            void* d_out, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* RoPE tables ([Youtu] 实现难点 §2 and 实现流程 §6: q*cos + rotate_half(q)*sin
 * with cos/sin fed from the runtime; [Penguin] §2.3: 2D split of the head;
 * [HyOCR15] §3.3: several position-id axes select frequencies).
 * d_pos: [n_axes][n_rows] int32 positions. The head is split into
 * rope_segments segments of length s = head_dim/rope_segments; rotation pair j
 * of segment g (elements g*s+j and g*s+j+s/2) turns by
 * pos[h_axis_of_pair[g*s/2 + j]][row] * theta^(-2j/s), computed in float64 and
 * rounded to float. Writes d_cos, d_sin [n_rows][head_dim] fp32. */
vlm_status vlm_rope_table(const int32_t* d_pos, int32_t n_axes, int32_t n_rows, const int32_t* h_axis_of_pair,
                          int32_t rope_segments, int32_t head_dim, double theta, float* d_cos, float* d_sin,
                          hipStream_t stream);

/* Effective base of the alpha-scaled multi-axis RoPE ([HyOCR10] 二 and 五.1):
 * *base = theta * alpha^(head_dim / (head_dim - 2)), the value to pass as
 * vlm_rope_table's theta. Host arithmetic in float64, no device work.
 * VLM_ERR_ARG unless theta > 0, alpha > 0, head_dim > 2 and base != NULL. */
vlm_status vlm_rope_alpha_base(double theta, double alpha, int32_t head_dim, double* base);

/* ------------------------------------------------------------------------- */
/* Embedding lookup ([Youtu] 实现流程 §5 and §6: tied [V][H] table, looked up
 * by the runtime). d_x[s][:] = float(d_embed[d_ids[s]][:]) for s < S.
 * An id outside [0, V) is not read: its row is written as NaN, which a later
 * argmax reports as non-finite. */
vlm_status vlm_embed(const vlm_model_desc* desc, const void* d_embed, const int32_t* d_ids, int32_t S,
                     float* d_x, hipStream_t stream);

/* Image-row injection ([Youtu] 实现流程 §5; [HyOCR15] §3.2): the rows whose
 * id equals placeholder_id are, in increasing position order, overwritten by
 * d_img rows 0..n_img-1 (exact copies, img_dtype VLM_F32 or VLM_BF16).
 * The count of placeholders in h_ids (host copy of the ids) must equal n_img,
 * else VLM_ERR_COUNT_MISMATCH and nothing is enqueued. d_ids is the device
 * copy of the same ids, which the kernel ranks; a placeholder whose rank is
 * >= n_img (ids differing from h_ids) is skipped, so no read goes out of bounds. */
vlm_status vlm_inject_image_embeds(const vlm_model_desc* desc, float* d_x, int32_t S, const int32_t* h_ids,
                                   const int32_t* d_ids, int32_t placeholder_id, const void* d_img, int32_t n_img,
                                   int32_t img_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Parallel prefill over all layers ([Youtu] 实现流程 §6-§7; [HyOCR10] 四.3:
 * per layer (x, cos, sin, mask) -> hidden and K/V for the cache).
 * d_x [S][H] fp32: input rows on entry, hidden state after the last layer
 * (before the final norm) on return. Row s has position pos0+s and uses row
 * pos0+s of d_cos/d_sin ([table_rows][d] fp32; for MLA the rows are
 * qk_rope_dim wide, and only CAUSAL and ADDITIVE masks are supported).
 * masks: n_masks == 1 (same mask for every layer) or n_layers.
 * Decoder: kv must be bound; requires pos0 <= current length and
 *   pos0+S <= capacity (else VLM_ERR_CAPACITY: an over-long sequence is
 *   rejected, [Youtu] 已知限制); K/V of the rows go to slots pos0..pos0+S-1;
 *   afterwards the length is pos0+S. A CAUSAL prefill with pos0 > 0 is a
 *   chunked prefill / multi-token verify over the existing cache.
 * ViT: kv must be NULL, pos0 == 0; K/V live in the workspace.
 * Workspace: d_ws of ws_bytes >= vlm_workspace_bytes(desc, S). */
vlm_status vlm_prefill(const vlm_model_desc* desc, const vlm_layer* h_layers, float* d_x, int32_t S, int32_t pos0,
                       const float* d_cos, const float* d_sin, int32_t table_rows, const vlm_mask* h_masks,
                       int32_t n_masks, vlm_kv* kv, void* d_ws, size_t ws_bytes, hipStream_t stream);

/* Final RMSNorm + lm_head + greedy argmax of one row ([Youtu] 实现流程 §6 and
 * 解码与采样说明; [HyOCR15] §3.4: a single [V][H] table, one weight copy).
 * d_token_out[0] = index of the largest logit (lowest index on ties); -1 if any
 * logit is NaN or infinite (vlm_token_status reports it). d_logits ([V] fp32) receives the logits when
 * non-NULL. The table may alias the embedding (tied weights). */
vlm_status vlm_lmhead_argmax(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                             const float* d_x_row, int32_t* d_token_out, float* d_logits, void* d_ws,
                             size_t ws_bytes, hipStream_t stream);

/* vlm_lmhead_argmax without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, kernels and results as
 * vlm_lmhead_argmax; the argmax block partials live in a library-owned device
 * array of 65536 u64 keys (512 KiB per GPU the library runs on, held until the
 * process ends), so the vocabulary is limited to 262137 rows
 * (VLM_ERR_UNSUPPORTED beyond, nothing enqueued). No hipMalloc, hipFree or
 * other allocating call is made. Every call on one GPU shares that array:
 * calls that overlap on one GPU (other streams or threads) race and must be
 * serialized by the caller. The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) with that device current. */
vlm_status vlm_lmhead_argmax_noalloc(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                                     const float* d_x_row, int32_t* d_token_out, float* d_logits,
                                     hipStream_t stream);

/* Multi-token verify head ([HyOCR15] §3.8: the target model checks a drafted
 * block in one causal forward). Rows d_x [S][H] fp32 (hidden rows after the
 * last layer, e.g. of a vlm_prefill over the block at pos0 = cache length):
 * final RMSNorm of each row, logits against the [V][H] table in one pass over
 * the table (an MFMA GEMM), then d_tokens_out[r] = argmax of row r (lowest
 * index on ties; -1 for a non-finite row). d_logits [S][V] fp32 receives the
 * logits when non-NULL; with NULL they live in the workspace after the S
 * normalised rows. The argmax then keeps S * P u64 partial keys after that,
 * P = min(32, max(1, V / 2048)) pieces per row. The workspace must hold
 * 256-aligned S * H * dtype-size bytes, then (without d_logits) 256-aligned
 * S * V * 4 bytes, then the keys (else VLM_ERR_WORKSPACE, nothing enqueued);
 * the workspace of vlm_workspace_bytes(desc, max_rows >= S) is required in
 * any case. */
vlm_status vlm_lmhead_argmax_rows(const vlm_model_desc* desc, const void* d_final_norm, const void* d_table,
                                  const float* d_x, int32_t S, int32_t* d_tokens_out, float* d_logits, void* d_ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Accept and commit a verified block ([HyOCR15] §3.8: keep the longest prefix
 * of drafted tokens the target agrees with, plus the target's first
 * correction, then trim the cache). The block h_draft[0..k) (host; h_draft[0]
 * is the last committed token, h_draft[1..k) the drafted ones) occupies cache
 * slots [pos0, pos0 + k), which must end at the current length, and d_pred
 * [k] holds the verify head's picks (d_pred[i] = the target's token after
 * h_draft[0..i]). Synchronizes `stream`, finds the largest a < k with
 * h_draft[i + 1] == d_pred[i] for all i < a, sets the cache length to
 * pos0 + a + 1 (slots of the accepted rows stay, the rest are dropped) and
 * returns *h_n_accept = a (drafted tokens accepted) and *h_next = d_pred[a]
 * (the correction, or the next token when every draft matched): the a + 1
 * tokens h_draft[1..a], *h_next are what greedy one-token decoding gives.
 * VLM_ERR_NONFINITE (nothing changed) if a verified row was non-finite. */
vlm_status vlm_verify_commit(vlm_kv* kv, int32_t pos0, const int32_t* h_draft, int32_t k, const int32_t* d_pred,
                             hipStream_t stream, int32_t* h_n_accept, int32_t* h_next);

/* One-token decode step ([Youtu] 实现流程 §8; [HyOCR10] 四.4: q/k/v of the new
 * token, K/V written into slot t, attention over the window with slots > t
 * masked; [HyOCR15] §3.7: one submission per token, cache committed on success).
 * t = device length. The input row is d_x_in ([H] fp32) when non-NULL, else
 * the embedding row of d_token_in[0]. Runs every layer at position t (RoPE row
 * t), then, when d_table is non-NULL, final norm + lm_head + argmax into
 * d_token_out[0] (may alias d_token_in) and, when d_token_hist is non-NULL,
 * into d_token_hist[t+1] (array of capacity+1 ints). d_x_out ([H]) receives the
 * hidden row after the last layer when non-NULL. Device length becomes t+1.
 * Requires host length < capacity and < table_rows. */
vlm_status vlm_decode_step(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                           const void* d_final_norm, const void* d_table, vlm_kv* kv, const int32_t* d_token_in,
                           const float* d_x_in, const float* d_cos, const float* d_sin, int32_t table_rows,
                           int32_t* d_token_out, float* d_x_out, int32_t* d_token_hist, void* d_ws,
                           size_t ws_bytes, hipStream_t stream);

/* n_steps greedy decode steps with each step's token feeding the next
 * (d_token_io is read and written by every step). Per band of 64 positions
 * (the decode attention's split layout follows the band) one step and 8
 * consecutive steps are captured into HIP graphs, before the first launch of
 * the call; the graphs are cached on the kv handle and dropped when any
 * argument changes. Eight steps that stay inside one band are one graph launch
 * on `stream`, the others one launch each, and the host never synchronises
 * inside the loop. Requires vocab > 0 and length + n_steps <= min(capacity,
 * table_rows). */
vlm_status vlm_decode_loop(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                           const void* d_final_norm, const void* d_table, vlm_kv* kv, int32_t* d_token_io,
                           const float* d_cos, const float* d_sin, int32_t table_rows, int32_t* d_token_hist,
                           int32_t n_steps, void* d_ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Vision tower helpers ([Youtu] 实现流程 §3: window grouping is a permutation
 * built by the runtime, the mask block-diagonal, 2x2 neighbours concatenated).
 * Input rows are 2x2-group-major: rows 4u..4u+3 are the merge*merge patches of
 * merge unit u (units in raster order of the merged grid, patches in raster
 * order inside the unit). Windows tile the merged grid in window x window
 * cells; units are permuted window by window (raster inside a window).
 * Host-only; writes h_unit_perm [n_units] (raster unit at permuted slot p),
 * h_row_perm [n_rows] (input row at permuted row r), h_row_seg [n_rows]
 * (window id of permuted row r) and h_pos [2][n_rows] (patch row h, then patch
 * column w, of permuted row r). Any output pointer may be NULL. */
vlm_status vlm_vit_window_index(int32_t grid_h, int32_t grid_w, int32_t merge, int32_t window,
                                int32_t* h_unit_perm, int32_t* h_row_perm, int32_t* h_row_seg, int32_t* h_pos);

/* d_dst[r][:] = d_src[d_idx[r]][:] for r < n_rows (fp32 rows of row_len);
 * an index outside [0, n_src) yields a NaN row. */
vlm_status vlm_gather_rows(const float* d_src, int32_t n_src, const int32_t* d_idx, int32_t n_rows,
                           int32_t row_len, float* d_dst, hipStream_t stream);

typedef struct {
    int32_t hidden;        /* H of the tower */
    int32_t merge;         /* 2: 2x2 neighbours */
    int32_t merger_hidden; /* width of the first merger layer */
    int32_t out_dim;       /* language-model width */
    int32_t dtype;         /* vlm_dtype (VLM_F32) */
    float norm_eps;
    const void* post_ln;   /* [H] */
    const void* post_ln_b; /* [H] */
    const void* w1;        /* [merger_hidden][merge*merge*H] */
    const void* b1;
    const void* w2;        /* [out_dim][merger_hidden] */
    const void* b2;
} vlm_merger;

/* post_layernorm -> view [N/m^2][m^2*H] (2x2 concat of the permuted rows) ->
 * Linear + GELU -> Linear -> rows written in raster unit order:
 * d_out[d_unit_perm[p]][:] = result row p. d_x [N][H] fp32 (permuted order). */
vlm_status vlm_vit_merger(const vlm_merger* m, const float* d_x, int32_t N, const int32_t* d_unit_perm,
                          float* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream);
vlm_status vlm_vit_merger_workspace_bytes(const vlm_merger* m, int32_t N, size_t* bytes);

/* ------------------------------------------------------------------------- */
/* Sampling instead of the greedy argmax ([MNN] §4.1: temperature, top_k,
 * top_p, softmax, draw; repeat penalty on tokens already in the context;
 * [HyOCR15] §3.6 generation options). On one fp32 logits row d_logits [vocab]
 * (e.g. the d_logits output of vlm_lmhead_argmax), in this order:
 *   x_i = logits_i; for i in the context: x_i = x_i > 0 ? x_i / r : x_i * r;
 *   x_i /= temperature; keep the x_i >= the top_k-th largest (ties kept);
 *   order the kept ids by (x desc, id asc), p = softmax(x) over them;
 *   top_p < 1 keeps the prefix whose preceding mass is < top_p * sum p;
 *   the token is the first kept id whose cumulative p exceeds u * (kept mass),
 *   u = d_uniform[0] in [0, 1) supplied by the caller (the random draw is an
 *   input; a fixed u makes the call deterministic).
 * fp32 throughout; d_token_out[0] = the id, or -1 for a non-finite logit or
 * more than 2048 values tied at the top_k-th. d_context_ids [n_context]
 * (repeats allowed, ids outside [0, vocab) ignored; NULL if n_context == 0).
 * Greedy decoding (temperature 0) is vlm_lmhead_argmax.
 * Errors (nothing enqueued): vocab not in [1, 524288], temperature not > 0,
 * top_k not in [1, 1024], top_p not in (0, 1], repetition_penalty not > 0. */
typedef struct {
    float temperature;
    int32_t top_k;
    float top_p;
    float repetition_penalty;
} vlm_sampling;
vlm_status vlm_sample_logits(const float* d_logits, int32_t vocab, const vlm_sampling* h_params,
                             const int32_t* d_context_ids, int32_t n_context, const float* d_uniform,
                             int32_t* d_token_out, hipStream_t stream);

/* vlm_decode_loop with the sampler in place of the greedy argmax ([MNN] §4.1;
 * [HyOCR15] §3.6 generation options): every captured step ends with the
 * lm_head logits row (workspace) and the sampler above, whose context is the
 * token history d_token_hist[0..t] and whose draw is d_uniform[t + 1], t the
 * step's position (the device length), so the graphs replay unchanged from
 * step to step. Before the call the caller fills d_token_hist[0..len) with the
 * ids of the cached positions (the prompt; the penalty treats them as context)
 * and d_token_hist[len] = d_token_io[0] (the token fed first); each step writes
 * its token to d_token_io[0] and d_token_hist[t + 1]. d_uniform holds at least
 * len + n_steps + 1 draws in [0, 1). A step whose sampler returns no token
 * (non-finite logits, or more than 2048 values tied at the top_k-th) writes -1
 * and is not committed (vlm_kv_status reports it). Parameter checks as in
 * vlm_sample_logits; the other requirements as in vlm_decode_loop. */
vlm_status vlm_decode_loop_sampled(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_embed,
                                   const void* d_final_norm, const void* d_table, vlm_kv* kv, int32_t* d_token_io,
                                   const float* d_cos, const float* d_sin, int32_t table_rows, int32_t* d_token_hist,
                                   const vlm_sampling* h_params, const float* d_uniform, int32_t n_steps, void* d_ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Host-only: the split plan of the decode attention at position t in a window
 * of `capacity` slots, as vlm_decode_step launches it (the slots [0, tb) of
 * t's band of 64 positions, tb the band's end or the capacity, in *nsplit
 * splits of *chunk slots; *nsplit <= 32). For accounting (bytes a launch
 * reads) and tests; no device work. */
vlm_status vlm_decode_split_plan(int32_t capacity, int32_t t, int32_t* nsplit, int32_t* chunk);

/* Measurement helper: enqueues n_launches back-to-back launches of one kernel
 * of the decode step, exactly as vlm_decode_step launches it, cycling over the
 * layers so that consecutive launches read different weights. Inputs come from
 * d_x_row ([H] fp32, copied into the workspace first) and the workspace;
 * outputs go to the workspace only, except VLM_KERNEL_ATTN, which (like a
 * decode step) writes the new token's K/V into slot t = current length of
 * `kv` and reads slots 0..t; the length does not change. `kv`, d_cos and
 * d_sin ([table_rows][d]) are needed for VLM_KERNEL_ATTN only, which requires
 * length < table_rows (else VLM_ERR_CAPACITY); otherwise they may be NULL.
 * Used to time one kernel with events on `stream`, and under a profiler,
 * without the rest of the step. */
typedef enum {
    VLM_KERNEL_LMHEAD = 0,   /* final RMSNorm + lm_head GEMV + block argmax partials */
    VLM_KERNEL_QKV = 1,      /* RMSNorm + fused QKV GEMV */
    VLM_KERNEL_O = 2,        /* O-projection GEMV + residual */
    VLM_KERNEL_GATE_UP = 3,  /* RMSNorm + gate/up GEMV + SwiGLU */
    VLM_KERNEL_DOWN = 4,     /* down GEMV + residual */
    VLM_KERNEL_ATTN = 5      /* QK-Norm + RoPE + slot write + split-K attention (without the split merge) */
} vlm_kernel_id;
vlm_status vlm_launch_kernel(const vlm_model_desc* desc, const vlm_layer* h_layers, const void* d_final_norm,
                             const void* d_table, vlm_kv* kv, const float* d_cos, const float* d_sin,
                             int32_t table_rows, int32_t which, int32_t n_launches, const float* d_x_row,
                             void* d_ws, size_t ws_bytes, hipStream_t stream);

/* Thread-local description of the last error. */
const char* vlm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* VLM_H */
