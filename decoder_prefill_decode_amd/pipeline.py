"""End-to-end drivers of the decoder and vision paths on one GPU.

A config object needs the attributes n_layers, hidden, n_q_heads, n_kv_heads,
head_dim, ffn, vocab, seq, capacity, dtype ("f32"/"bf16"), qk_norm, theta,
eps, placeholder_id (decoder) or the vision fields (ViT). Weights and inputs
are plain host arrays; all arithmetic runs in libvlm's kernels.
"""
import numpy as np
import torch

from . import native as N
from .runtime import (KVCache, Model, causal_mask, none_mask, ptr, rope_table, segment_mask, stream, text_rope,
                      to_device, token_status)


class DecoderRun:
    """Model + KV cache + workspace + RoPE tables for one decoder workload.

    The prompt follows the pages' runtime order: embedding lookup, image-row
    injection, parallel causal prefill filling the cache, lm_head argmax on the
    last row, then one-token decode steps.
    """

    def __init__(self, cfg, layer_weights, glob):
        self.cfg = cfg
        mla = getattr(cfg, "kv_lora_rank", 0) > 0
        m = Model(n_layers=cfg.n_layers, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                  head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, dtype=cfg.dtype, qk_norm=int(cfg.qk_norm),
                  eps=cfg.eps, rope_interleave=getattr(cfg, "rope_interleave", False),
                  block_kind=N.VLM_BLOCK_MLA if mla else N.VLM_BLOCK_DECODER,
                  q_lora_rank=cfg.q_lora_rank if mla else 0, kv_lora_rank=cfg.kv_lora_rank if mla else 0,
                  qk_rope_dim=cfg.qk_rope_dim if mla else 0, v_head_dim=cfg.v_head_dim if mla else 0)
        for l in range(cfg.n_layers):
            (m.set_mla_layer if mla else m.set_decoder_layer)(l, layer_weights(l))
        if cfg.vocab > 0:
            m.set_table(glob["embed"], glob["final_norm"])
        self.model = m
        self.kv = KVCache(m, cfg.capacity)
        self.ws = m.workspace(cfg.seq)
        self.cos, self.sin = text_rope(cfg.capacity, cfg.qk_rope_dim if mla else cfg.head_dim, cfg.theta)
        self.glob = glob
        H = cfg.hidden
        self.x = torch.empty((cfg.seq, H), dtype=torch.float32, device="cuda")
        if cfg.vocab > 0:
            self.ids_host = np.ascontiguousarray(glob["ids"], np.int32)
            self.ids_dev = torch.from_numpy(self.ids_host).to("cuda")
            self.img = torch.from_numpy(np.ascontiguousarray(glob["img"], np.float32)).to("cuda") \
                if glob.get("img") is not None else None
        else:
            self.x_in = torch.from_numpy(np.ascontiguousarray(glob["x"], np.float32)).to("cuda")
            self.dec_x = torch.from_numpy(np.ascontiguousarray(glob["decode_x"], np.float32)).to("cuda")
        self.tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.hist = torch.full((cfg.capacity + 1,), -2, dtype=torch.int32, device="cuda")
        self.x_row = torch.empty(H, dtype=torch.float32, device="cuda")

    def reset(self):
        self.kv.truncate(0)

    def embed_inject(self):
        if self.cfg.vocab > 0:
            self.model.embed_ids(self.ids_dev, self.x)
            self.model.inject(self.x, self.ids_host, self.ids_dev, self.cfg.placeholder_id, self.img)
        else:
            self.x.copy_(self.x_in)

    def prefill(self, S=None, pos0=0, mask=None):
        """Embed + inject + stack over rows [pos0, pos0+S) of the prompt (default: all)."""
        S = self.cfg.seq if S is None else S
        if pos0 == 0:
            self.embed_inject()
        x = self.x[pos0:pos0 + S]
        self.model.prefill(x, pos0, self.cos, self.sin, mask or causal_mask(), self.kv, self.ws)
        return x

    def first_token(self, logits=None, check=True):
        """lm_head + argmax of the last prompt row (writes self.tok). check: synchronize and raise
        VlmError (VLM_ERR_NONFINITE) on a non-finite row; check=False keeps the call asynchronous."""
        self.model.lmhead_argmax(self.x[self.cfg.seq - 1], self.tok, self.ws, logits)
        if check:
            token_status(self.tok)
        return self.tok

    def decode(self, n, loop=True):
        """n greedy steps from self.tok; returns the produced ids (host)."""
        if n == 0:
            return np.zeros(0, np.int64)
        t0 = self.kv.len()
        if loop:
            self.model.decode_loop(self.kv, self.cos, self.sin, self.ws, self.tok, n, hist=self.hist)
        else:
            for _ in range(n):
                self.model.decode_step(self.kv, self.cos, self.sin, self.ws, token_in=self.tok, token_out=self.tok,
                                       hist=self.hist)
        self.kv.status()   # synchronizes; raises on a non-finite step
        return self.hist[t0 + 1:t0 + 1 + n].cpu().numpy().astype(np.int64)

    def generate_sampled(self, n, temperature, top_k, top_p, penalty, u):
        """Sampled generation after prefill(): the first token from the last prompt row, then n
        decode steps, each token drawn by vlm_sample_logits from the lm_head logits with the prompt
        and the tokens so far as the penalty context; u: host float32 [n + 1] uniform draws (inputs).
        Everything stays on the device (the sampled id is written straight into the context
        buffer that the next step reads). Returns the n + 1 ids (host)."""
        from .runtime import sample_logits
        cfg = self.cfg
        S, V = cfg.seq, cfg.vocab
        ctx = torch.empty(S + n + 1, dtype=torch.int32, device="cuda")
        ctx[:S].copy_(self.ids_dev)
        ud = torch.from_numpy(np.ascontiguousarray(u, np.float32)).to("cuda")
        logits = torch.empty(V, dtype=torch.float32, device="cuda")
        scratch = torch.empty(1, dtype=torch.int32, device="cuda")
        self.model.lmhead_argmax(self.x[S - 1], scratch, self.ws, logits)
        sample_logits(logits, temperature, top_k, top_p, penalty, ctx[:S], ud[0:1], ctx[S:S + 1])
        for i in range(n):
            self.model.decode_step(self.kv, self.cos, self.sin, self.ws, x_out=self.x_row, with_head=False,
                                   token_in=ctx[S + i:S + i + 1])
            self.model.lmhead_argmax(self.x_row, scratch, self.ws, logits)
            sample_logits(logits, temperature, top_k, top_p, penalty, ctx[:S + i + 1], ud[i + 1:i + 2],
                          ctx[S + i + 1:S + i + 2])
        torch.cuda.current_stream().synchronize()
        return ctx[S:].cpu().numpy().astype(np.int64)

    def generate_sampled_loop(self, n, temperature, top_k, top_p, penalty, u):
        """generate_sampled with every decode step (layers, lm_head, sampler) replayed from HIP graphs
        (vlm_decode_loop_sampled): the first token is sampled from the last prompt row, the history
        holds the prompt ids and the tokens so far, draw i is u[i]. Returns the n + 1 ids (host)."""
        from .runtime import decode_loop_sampled, sample_logits
        cfg = self.cfg
        S, V = cfg.seq, cfg.vocab
        hist = torch.full((cfg.capacity + 1,), -2, dtype=torch.int32, device="cuda")
        hist[:S].copy_(self.ids_dev)
        ud = torch.zeros(cfg.capacity + 1, dtype=torch.float32, device="cuda")
        ud[S:S + n + 1].copy_(torch.from_numpy(np.ascontiguousarray(u, np.float32)))
        logits = torch.empty(V, dtype=torch.float32, device="cuda")
        scratch = torch.empty(1, dtype=torch.int32, device="cuda")
        self.model.lmhead_argmax(self.x[S - 1], scratch, self.ws, logits)
        sample_logits(logits, temperature, top_k, top_p, penalty, hist[:S], ud[S:S + 1], hist[S:S + 1])
        self.tok.copy_(hist[S:S + 1])
        decode_loop_sampled(self.model, self.kv, self.cos, self.sin, self.ws, self.tok, n, hist,
                            N.Sampling(temperature, top_k, top_p, penalty), ud)
        self.kv.status()
        return hist[S:S + n + 1].cpu().numpy().astype(np.int64)

    def decode_forced(self, ids):
        """Teacher-forced greedy steps: step i feeds ids[i] (host ints) and records
        the token the GPU picks next; returns those picks (host)."""
        n = len(ids)
        fin = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to("cuda")
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        for i in range(n):
            self.model.decode_step(self.kv, self.cos, self.sin, self.ws, token_in=fin[i:i + 1],
                                   token_out=out[i:i + 1])
        self.kv.status()
        return out.cpu().numpy().astype(np.int64)

    def verify_block(self, draft, logits=None):
        """Multi-token verify of a drafted block: draft[0] is the last committed token (not yet in the
        cache), draft[1:] the drafted ones. Embeds the block, prefills it as a causal chunk at the cache
        length, takes every row's argmax in one lm_head pass and commits the accepted prefix.
        Returns (accepted drafted tokens + the correction, the next token to feed)."""
        k = len(draft)
        pos0 = self.kv.len()
        ids = torch.from_numpy(np.ascontiguousarray(draft, np.int32)).to("cuda")
        xb = torch.empty((k, self.cfg.hidden), dtype=torch.float32, device="cuda")
        self.model.embed_ids(ids, xb)
        self.model.prefill(xb, pos0, self.cos, self.sin, causal_mask(), self.kv, self.ws)
        pred = torch.empty(k, dtype=torch.int32, device="cuda")
        self.model.lmhead_argmax_rows(xb, pred, self.ws, logits)
        a, nxt = self.kv.verify_commit(pos0, draft, pred)
        return [int(t) for t in draft[1:a + 1]] + [nxt], nxt

    def decode_hidden(self, rows: torch.Tensor):
        """Hidden-state decode (no vocabulary): one step per input row; returns [n][H]."""
        out = torch.empty_like(rows)
        for i in range(rows.shape[0]):
            self.model.decode_step(self.kv, self.cos, self.sin, self.ws, x_in=rows[i], x_out=out[i], with_head=False)
        return out


class VitRun:
    """Vision tower + merger: permute rows into windows, run the layers with the
    window (segment) or full mask, then post-LN, 2x2 merge MLP and un-permute."""

    def __init__(self, cfg, layer_weights, glob):
        self.cfg = cfg
        m = Model(n_layers=cfg.n_layers, hidden=cfg.hidden, n_q_heads=cfg.n_heads, n_kv_heads=cfg.n_heads,
                  head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=0, dtype=cfg.dtype, qk_norm=False, rope_segments=2,
                  eps=cfg.eps, block_kind=N.VLM_BLOCK_VIT)
        for l in range(cfg.n_layers):
            m.set_vit_layer(l, layer_weights(l))
        self.model = m
        n, m2 = cfg.n_patches, cfg.merge * cfg.merge
        self.unit_perm, self.row_perm, self.row_seg, self.pos = window_index(cfg.grid_h, cfg.grid_w, cfg.merge,
                                                                             cfg.window)
        half = cfg.head_dim // 2
        axes = np.r_[np.zeros(half // 2, np.int32), np.ones(half // 2, np.int32)]
        self.cos, self.sin = rope_table(self.pos, axes, 2, cfg.head_dim, cfg.theta)
        self.d_row_perm = torch.from_numpy(self.row_perm).to("cuda")
        self.d_unit_perm = torch.from_numpy(self.unit_perm).to("cuda")
        self.d_seg = torch.from_numpy(self.row_seg).to("cuda")
        self.x_in = torch.from_numpy(np.ascontiguousarray(glob["x"], np.float32)).to("cuda")
        self.x = torch.empty_like(self.x_in)
        self.ws = m.workspace(n)
        self.masks = [none_mask() if l in cfg.full_layers else segment_mask(self.d_seg) for l in range(cfg.n_layers)]
        self.merger = N.Merger(cfg.hidden, cfg.merge, cfg.merger_hidden, cfg.out_dim, m.dtype, cfg.eps)
        self._mk = {k: to_device(glob[k], m.dtype) for k in ("post_ln", "post_ln_b", "m1", "m1b", "m2", "m2b")}
        for f, k in (("post_ln", "post_ln"), ("post_ln_b", "post_ln_b"), ("w1", "m1"), ("b1", "m1b"), ("w2", "m2"),
                     ("b2", "m2b")):
            setattr(self.merger, f, self._mk[k].data_ptr())
        import ctypes as C
        nb = C.c_size_t()
        N.call("vlm_vit_merger_workspace_bytes", C.byref(self.merger), n, C.byref(nb))
        self.mws = torch.empty(nb.value, dtype=torch.uint8, device="cuda")
        self.out = torch.empty((n // m2, cfg.out_dim), dtype=torch.float32, device="cuda")

    def run(self):
        cfg = self.cfg
        n = cfg.n_patches
        N.call("vlm_gather_rows", ptr(self.x_in), n, ptr(self.d_row_perm), n, cfg.hidden, ptr(self.x), stream())
        self.model.prefill(self.x, 0, self.cos, self.sin, self.masks, None, self.ws)
        N.call("vlm_vit_merger", __import__("ctypes").byref(self.merger), ptr(self.x), n, ptr(self.d_unit_perm),
               ptr(self.out), ptr(self.mws), self.mws.numel(), stream())
        return self.out


def window_index(grid_h, grid_w, merge, window):
    """Host-side window permutation from the library (integer bookkeeping)."""
    import ctypes as C
    n = grid_h * grid_w
    units = n // (merge * merge)
    up = np.zeros(units, np.int32)
    rp = np.zeros(n, np.int32)
    sg = np.zeros(n, np.int32)
    pos = np.zeros((2, n), np.int32)
    P = C.POINTER(C.c_int32)
    N.call("vlm_vit_window_index", grid_h, grid_w, merge, window, up.ctypes.data_as(P), rp.ctypes.data_as(P),
           sg.ctypes.data_as(P), pos.ctypes.data_as(P))
    return up, rp, sg, pos
