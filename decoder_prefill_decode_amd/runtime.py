"""Device-memory plumbing around the C ABI.

PyTorch provides device buffers and the current stream; every step of the
decoder path runs in libvlm's kernels, called through `native`. The classes
here only upload weights, keep buffers alive, and pass pointers.
"""
import ctypes as C

import numpy as np
import torch

from . import native as N

TORCH_DT = {N.VLM_F32: torch.float32, N.VLM_BF16: torch.bfloat16}
DTYPES = {"f32": N.VLM_F32, "bf16": N.VLM_BF16}


def ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def to_device(a, dtype: int) -> torch.Tensor:
    """Upload float32 host values; bf16 models receive values that are already
    bf16-exact, so the cast is exact."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == N.VLM_BF16 else t


class Model:
    """Model description + per-layer weights resident in HBM."""

    def __init__(self, *, n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab=0, dtype="f32",
                 qk_norm=0, rope_segments=1, eps=1e-6, block_kind=N.VLM_BLOCK_DECODER, rope_interleave=False,
                 q_lora_rank=0, kv_lora_rank=0, qk_rope_dim=0, v_head_dim=0):
        """qk_norm: 0 none, 1 (or True) before RoPE, 2 after RoPE. The last four sizes describe an
        expanded MLA stack (block_kind VLM_BLOCK_MLA) and are 0 otherwise."""
        self.dtype = DTYPES[dtype] if isinstance(dtype, str) else dtype
        self.desc = N.ModelDesc(block_kind, n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab,
                                self.dtype, int(qk_norm), rope_segments, eps, int(bool(rope_interleave)),
                                q_lora_rank, kv_lora_rank, qk_rope_dim, v_head_dim)
        self.layers = (N.Layer * n_layers)()
        self._keep = [dict() for _ in range(n_layers)]
        self.embed = None
        self.final_norm = None

    @property
    def tdtype(self):
        return TORCH_DT[self.dtype]

    def _dev(self, a):
        return to_device(a, self.dtype)

    def set_decoder_layer(self, l, w):
        """w: natural-form weights (wq, wk, wv, wo, wg, wu, wd, attn_norm, mlp_norm, q_norm, k_norm)."""
        d = self.desc
        st = stream()
        wq, wk, wv = self._dev(w["wq"]), self._dev(w["wk"]), self._dev(w["wv"])
        wqkv = torch.empty(((d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, d.hidden), dtype=self.tdtype, device="cuda")
        N.call("vlm_pack_qkv", ptr(wq), ptr(wk), ptr(wv), d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim,
               d.hidden, self.dtype, ptr(wqkv), st)
        wg, wu = self._dev(w["wg"]), self._dev(w["wu"])
        w1 = torch.empty((2 * d.ffn, d.hidden), dtype=self.tdtype, device="cuda")
        N.call("vlm_pack_gate_up", ptr(wg), ptr(wu), d.ffn, d.hidden, self.dtype, ptr(w1), st)
        keep = {"wqkv": wqkv, "w1": w1, "wo": self._dev(w["wo"]), "w2": self._dev(w["wd"]),
                "attn_norm": self._dev(w["attn_norm"]), "mlp_norm": self._dev(w["mlp_norm"])}
        if d.qk_norm:
            keep["q_norm"] = self._dev(w["q_norm"])
            keep["k_norm"] = self._dev(w["k_norm"])
        self._bind(l, keep)

    def set_mla_layer(self, l, w):
        """w: natural-form expanded-MLA weights (wq_a, q_a_norm, wq_b, wkv_a, kv_a_norm, wkv_b, wo, norms,
        wg, wu, wd); the two down-projections are stacked into w_a as the header lays out."""
        d = self.desc
        st = stream()
        wg, wu = self._dev(w["wg"]), self._dev(w["wu"])
        w1 = torch.empty((2 * d.ffn, d.hidden), dtype=self.tdtype, device="cuda")
        N.call("vlm_pack_gate_up", ptr(wg), ptr(wu), d.ffn, d.hidden, self.dtype, ptr(w1), st)
        keep = {"w_a": self._dev(np.concatenate([w["wq_a"], w["wkv_a"]], axis=0)),
                "q_a_norm": self._dev(w["q_a_norm"]), "q_b": self._dev(w["wq_b"]),
                "kv_a_norm": self._dev(w["kv_a_norm"]), "kv_b": self._dev(w["wkv_b"]),
                "w1": w1, "wo": self._dev(w["wo"]), "w2": self._dev(w["wd"]),
                "attn_norm": self._dev(w["attn_norm"]), "mlp_norm": self._dev(w["mlp_norm"])}
        self._bind(l, keep)

    def set_vit_layer(self, l, w):
        """w: natural-form ViT weights (wq/wk/wv + biases, wo/bo, w1/b1, w2/b2, LayerNorm gains/shifts)."""
        keep = {"wqkv": self._dev(np.concatenate([w["wq"], w["wk"], w["wv"]], axis=0)),
                "bqkv": self._dev(np.concatenate([w["bq"], w["bk"], w["bv"]])),
                "wo": self._dev(w["wo"]), "bo": self._dev(w["bo"]), "w1": self._dev(w["w1"]),
                "b1": self._dev(w["b1"]), "w2": self._dev(w["w2"]), "b2": self._dev(w["b2"]),
                "attn_norm": self._dev(w["attn_norm"]), "attn_norm_b": self._dev(w["attn_norm_b"]),
                "mlp_norm": self._dev(w["mlp_norm"]), "mlp_norm_b": self._dev(w["mlp_norm_b"])}
        self._bind(l, keep)

    def _bind(self, l, keep):
        self._keep[l] = keep
        lay = self.layers[l]
        for name, _ in N.Layer._fields_:
            setattr(lay, name, keep[name].data_ptr() if name in keep else None)

    def set_table(self, embed, final_norm):
        self.embed = self._dev(embed)
        self.final_norm = self._dev(final_norm)

    def workspace(self, max_rows: int) -> torch.Tensor:
        n = C.c_size_t()
        N.call("vlm_workspace_bytes", C.byref(self.desc), max_rows, C.byref(n))
        return torch.empty(n.value, dtype=torch.uint8, device="cuda")

    # ---- thin calls -------------------------------------------------------
    def embed_ids(self, ids_dev: torch.Tensor, x: torch.Tensor):
        N.call("vlm_embed", C.byref(self.desc), ptr(self.embed), ptr(ids_dev), ids_dev.numel(), ptr(x), stream())

    def inject(self, x, ids_host: np.ndarray, ids_dev, placeholder_id, img: torch.Tensor):
        ids_host = np.ascontiguousarray(ids_host, dtype=np.int32)
        n_img = 0 if img is None else img.shape[0]
        img_dt = N.VLM_BF16 if (img is not None and img.dtype == torch.bfloat16) else N.VLM_F32
        N.call("vlm_inject_image_embeds", C.byref(self.desc), ptr(x), x.shape[0],
               ids_host.ctypes.data_as(C.POINTER(C.c_int32)), ptr(ids_dev), placeholder_id, ptr(img), n_img, img_dt,
               stream())

    def prefill(self, x, pos0, cos, sin, masks, kv, ws):
        masks = masks if isinstance(masks, (list, tuple)) else [masks]
        arr = (N.Mask * len(masks))(*masks)
        N.call("vlm_prefill", C.byref(self.desc), self.layers, ptr(x), x.shape[0], pos0, ptr(cos), ptr(sin),
               cos.shape[0], arr, len(masks), None if kv is None else kv.handle, ptr(ws), ws.numel(), stream())

    def lmhead_argmax(self, x_row, token_out, ws, logits=None):
        N.call("vlm_lmhead_argmax", C.byref(self.desc), ptr(self.final_norm), ptr(self.embed), ptr(x_row),
               ptr(token_out), ptr(logits), ptr(ws), ws.numel(), stream())

    def lmhead_argmax_rows(self, x_rows, tokens_out, ws, logits=None):
        N.call("vlm_lmhead_argmax_rows", C.byref(self.desc), ptr(self.final_norm), ptr(self.embed), ptr(x_rows),
               x_rows.shape[0], ptr(tokens_out), ptr(logits), ptr(ws), ws.numel(), stream())

    def decode_step(self, kv, cos, sin, ws, token_in=None, x_in=None, token_out=None, x_out=None, hist=None,
                    with_head=True):
        table = self.embed if (with_head and self.desc.vocab > 0) else None
        N.call("vlm_decode_step", C.byref(self.desc), self.layers, ptr(self.embed), ptr(self.final_norm),
               ptr(table), kv.handle, ptr(token_in), ptr(x_in), ptr(cos), ptr(sin), cos.shape[0], ptr(token_out),
               ptr(x_out), ptr(hist), ptr(ws), ws.numel(), stream())

    def decode_loop(self, kv, cos, sin, ws, token_io, n_steps, hist=None):
        N.call("vlm_decode_loop", C.byref(self.desc), self.layers, ptr(self.embed), ptr(self.final_norm),
               ptr(self.embed), kv.handle, ptr(token_io), ptr(cos), ptr(sin), cos.shape[0], ptr(hist), n_steps,
               ptr(ws), ws.numel(), stream())


def decode_loop_sampled(model, kv, cos, sin, ws, token_io, n_steps, hist, params, uniform):
    """vlm_decode_loop_sampled: n_steps graph-captured steps ending in the sampler (params: N.Sampling)."""
    N.call("vlm_decode_loop_sampled", C.byref(model.desc), model.layers, ptr(model.embed), ptr(model.final_norm),
           ptr(model.embed), kv.handle, ptr(token_io), ptr(cos), ptr(sin), cos.shape[0], ptr(hist), C.byref(params),
           ptr(uniform), n_steps, ptr(ws), ws.numel(), stream())


class KVCache:
    """Caller-owned KV buffer bound to a library handle."""

    def __init__(self, model: Model, capacity: int):
        n = C.c_size_t()
        N.call("vlm_kv_bytes", C.byref(model.desc), capacity, C.byref(n))
        self.model = model
        self.capacity = capacity
        self.buf = torch.empty(n.value, dtype=torch.uint8, device="cuda")
        h = C.c_void_p()
        N.call("vlm_kv_alloc", C.byref(model.desc), capacity, ptr(self.buf), n.value, stream(), C.byref(h))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                N.lib().vlm_kv_free(h)
            except Exception:
                pass
            self.handle = None

    def len(self) -> int:
        v = C.c_int32()
        N.call("vlm_kv_len", self.handle, C.byref(v))
        return v.value

    def truncate(self, new_len: int):
        N.call("vlm_kv_truncate", self.handle, new_len, stream())

    def verify_commit(self, pos0: int, draft, pred: torch.Tensor):
        """vlm_verify_commit: (drafted tokens accepted, next token); the cache keeps the accepted rows."""
        d = np.ascontiguousarray(draft, dtype=np.int32)
        na, nx = C.c_int32(), C.c_int32()
        N.call("vlm_verify_commit", self.handle, pos0, d.ctypes.data_as(C.POINTER(C.c_int32)), len(d), ptr(pred),
               stream(), C.byref(na), C.byref(nx))
        return na.value, nx.value

    def status(self) -> int:
        """vlm_kv_status: synchronizes the stream; raises VlmError (VLM_ERR_NONFINITE) when a decode
        step's argmax saw a non-finite logit (the cache then stays at that step's position)."""
        pos = C.c_int32()
        N.call("vlm_kv_status", self.handle, stream(), C.byref(pos))
        return pos.value

    def device_len(self) -> torch.Tensor:
        return self.buf[:4].view(torch.int32)

    def kv(self, layer: int):
        """(K, V) views [nkv][W][d] and [nkv][W][dv] of one layer (dv = v_head_dim for MLA, else d)."""
        d = self.model.desc
        e = 2 if d.dtype == N.VLM_BF16 else 4
        dv = d.v_head_dim if d.block_kind == N.VLM_BLOCK_MLA else d.head_dim
        pk, pv = d.n_kv_heads * self.capacity * d.head_dim, d.n_kv_heads * self.capacity * dv
        off = N.KV_HEADER_BYTES + layer * (pk + pv) * e
        k = self.buf[off:off + pk * e].view(self.model.tdtype).view(d.n_kv_heads, self.capacity, d.head_dim)
        v = self.buf[off + pk * e:off + (pk + pv) * e].view(self.model.tdtype).view(d.n_kv_heads, self.capacity, dv)
        return k, v


def token_status(token: torch.Tensor) -> int:
    """vlm_token_status: synchronizes the stream and returns the device token; raises VlmError
    (VLM_ERR_NONFINITE) when it is -1 (the argmax or sampler saw a non-finite logit)."""
    tok = C.c_int32()
    N.call("vlm_token_status", ptr(token), stream(), C.byref(tok))
    return tok.value


def rope_table(positions: np.ndarray, axis_of_pair, segments: int, head_dim: int, theta: float):
    """cos, sin [n_rows][head_dim] fp32 on the device from int positions [n_axes][n_rows]."""
    pos = np.ascontiguousarray(np.atleast_2d(positions), dtype=np.int32)
    n_axes, n_rows = pos.shape
    dpos = torch.from_numpy(pos).to("cuda")
    axes = np.ascontiguousarray(axis_of_pair, dtype=np.int32)
    cos = torch.empty((n_rows, head_dim), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    N.call("vlm_rope_table", ptr(dpos), n_axes, n_rows, axes.ctypes.data_as(C.POINTER(C.c_int32)), segments,
           head_dim, float(theta), ptr(cos), ptr(sin), stream())
    torch.cuda.current_stream().synchronize()
    return cos, sin


def sample_logits(logits: torch.Tensor, temperature: float, top_k: int, top_p: float, penalty: float,
                  context: torch.Tensor, u: torch.Tensor, out: torch.Tensor):
    """vlm_sample_logits on a device fp32 logits row; context: device int32 ids (may be empty);
    u: device float32 [1] uniform draw; out: device int32 [1]."""
    prm = N.Sampling(temperature, top_k, top_p, penalty)
    N.call("vlm_sample_logits", ptr(logits), logits.numel(), C.byref(prm), ptr(context) if context.numel() else None,
           context.numel(), ptr(u), ptr(out), stream())


def rope_alpha_base(theta: float, alpha: float, head_dim: int) -> float:
    """vlm_rope_alpha_base: the effective base of the alpha-scaled multi-axis RoPE."""
    out = C.c_double()
    N.call("vlm_rope_alpha_base", C.c_double(theta), C.c_double(alpha), head_dim, C.byref(out))
    return out.value


def text_rope(n_rows: int, head_dim: int, theta: float):
    return rope_table(np.arange(n_rows)[None, :], np.zeros(head_dim // 2, np.int32), 1, head_dim, theta)


def causal_mask():
    return N.Mask(N.VLM_MASK_CAUSAL, 0, None, None)


def none_mask():
    return N.Mask(N.VLM_MASK_NONE, 0, None, None)


def additive_mask(add: torch.Tensor):
    return N.Mask(N.VLM_MASK_ADDITIVE, add.shape[1], add.data_ptr(), None)


def segment_mask(seg: torch.Tensor):
    return N.Mask(N.VLM_MASK_SEGMENT, 0, None, seg.data_ptr())
