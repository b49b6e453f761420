"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/vlm.h declares, and rejects bad arguments before any
device work (no compute calls are made here)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from decoder_prefill_decode_amd import native as N
from oracle import vit as ov
import vlm_synth as vs

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "vlm.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vlm_[a-z0-9_]+)\s*\(", src)))


def desc(**kw):
    base = dict(block_kind=0, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=4096,
                dtype=N.VLM_F32, qk_norm=0, rope_segments=1, norm_eps=1e-6)
    base.update(kw)
    return N.ModelDesc(**base)


def test_library_exports_every_declared_symbol():
    L = N.lib()
    names = declared()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(N._SIG), "binding signatures out of sync with the header"


def test_kv_and_workspace_sizes():
    d = desc()
    n = C.c_size_t()
    N.call("vlm_kv_bytes", C.byref(d), 64, C.byref(n))
    assert n.value == N.KV_HEADER_BYTES + 2 * 2 * 2 * 64 * 64 * 4
    d = desc(dtype=N.VLM_BF16)
    N.call("vlm_kv_bytes", C.byref(d), 64, C.byref(n))
    assert n.value == N.KV_HEADER_BYTES + 2 * 2 * 2 * 64 * 64 * 2
    N.call("vlm_workspace_bytes", C.byref(d), 512, C.byref(n))
    assert n.value > 512 * 256 * 2


def test_bf16_head72_is_accepted():
    """The bf16 attention zero-pads 72-wide heads to 80, so a bf16 vision stack of 72-wide heads is valid."""
    d = desc(block_kind=N.VLM_BLOCK_VIT, dtype=N.VLM_BF16, head_dim=72, n_kv_heads=4)
    n = C.c_size_t()
    N.call("vlm_workspace_bytes", C.byref(d), 16, C.byref(n))
    assert n.value > 0


def test_mla_cache_layout_sizes():
    """K rows 192 wide and V rows 128 wide per layer (the expanded MLA cache of the Youtu-VL port)."""
    d = desc(block_kind=N.VLM_BLOCK_MLA, head_dim=192, n_kv_heads=4, q_lora_rank=384, kv_lora_rank=512,
             qk_rope_dim=64, v_head_dim=128)
    n = C.c_size_t()
    N.call("vlm_kv_bytes", C.byref(d), 64, C.byref(n))
    assert n.value == N.KV_HEADER_BYTES + 2 * 4 * 64 * (192 + 128) * 4
    N.call("vlm_workspace_bytes", C.byref(d), 48, C.byref(n))
    assert n.value > 48 * (384 + 512 + 64) * 4


@pytest.mark.parametrize("bad,status", [
    (dict(n_q_heads=5), N.VLM_ERR_SHAPE),            # nq % nkv != 0
    (dict(head_dim=96), N.VLM_ERR_UNSUPPORTED),
    (dict(dtype=7), N.VLM_ERR_DTYPE),
    (dict(ffn=770), N.VLM_ERR_SHAPE),
    (dict(ffn=776), N.VLM_ERR_SHAPE),                 # decoder ffn not a multiple of 32
    (dict(block_kind=2, head_dim=128, n_kv_heads=4, q_lora_rank=384, kv_lora_rank=512, qk_rope_dim=64,
          v_head_dim=128), N.VLM_ERR_UNSUPPORTED),   # no MLA kernel for 128-wide keys
    (dict(n_q_heads=6, n_kv_heads=2), N.VLM_ERR_UNSUPPORTED),  # group of 3
    (dict(block_kind=1, n_kv_heads=2), N.VLM_ERR_UNSUPPORTED),
    (dict(rope_segments=3), N.VLM_ERR_ARG),
    (dict(qk_norm=3), N.VLM_ERR_ARG),
    (dict(rope_interleave=2), N.VLM_ERR_ARG),
    (dict(v_head_dim=128), N.VLM_ERR_ARG),            # MLA sizes on a GQA decoder
    (dict(block_kind=2, head_dim=192, n_kv_heads=4, q_lora_rank=384, kv_lora_rank=512, qk_rope_dim=64,
          v_head_dim=96), N.VLM_ERR_UNSUPPORTED),      # no kernel for V 96
    (dict(block_kind=2, head_dim=192, q_lora_rank=384, kv_lora_rank=512, qk_rope_dim=64,
          v_head_dim=128), N.VLM_ERR_SHAPE),           # MLA needs nkv == nq
    (dict(block_kind=2, head_dim=192, n_kv_heads=4, q_lora_rank=380, kv_lora_rank=512, qk_rope_dim=64,
          v_head_dim=128), N.VLM_ERR_SHAPE),           # rank not a multiple of 8
])
def test_desc_validation(bad, status):
    d = desc(**bad)
    n = C.c_size_t()
    assert N.lib().vlm_workspace_bytes(C.byref(d), 16, C.byref(n)) == status
    assert N.last_error()


def test_inject_count_mismatch_rejected_before_launch():
    d = desc()
    ids = np.array([1, 4095, 4095, 3], np.int32)
    fake = C.c_void_p(0x1000)        # never dereferenced: the check fails first
    st = N.lib().vlm_inject_image_embeds(C.byref(d), fake, 4, ids.ctypes.data_as(C.POINTER(C.c_int32)), fake, 4095,
                                         fake, 3, N.VLM_F32, None)
    assert st == N.VLM_ERR_COUNT_MISMATCH
    assert "2 placeholder" in N.last_error()


def test_rope_table_argument_checks():
    axes = np.zeros(32, np.int32)
    P = C.POINTER(C.c_int32)
    fake = C.c_void_p(0x1000)
    L = N.lib()
    assert L.vlm_rope_table(fake, 1, 8, axes.ctypes.data_as(P), 1, 256, 1e6, fake, fake, None) == N.VLM_ERR_UNSUPPORTED
    axes[3] = 2
    assert L.vlm_rope_table(fake, 2, 8, axes.ctypes.data_as(P), 1, 64, 1e6, fake, fake, None) == N.VLM_ERR_ARG
    axes[3] = 0
    assert L.vlm_rope_table(fake, 1, 8, axes.ctypes.data_as(P), 1, 64, -1.0, fake, fake, None) == N.VLM_ERR_ARG


def test_rope_alpha_base_matches_oracle_and_checks_arguments():
    from oracle import decoder as od
    L = N.lib()
    out = C.c_double()
    for theta, alpha, d in [(1e4, 1e3, 128), (1e6, 1.0, 64), (5e5, 3.7, 80)]:
        assert L.vlm_rope_alpha_base(theta, alpha, d, C.byref(out)) == N.VLM_OK
        assert out.value == pytest.approx(od.alpha_scaled_base(theta, alpha, d), rel=1e-15)
    for theta, alpha, d in [(0.0, 2.0, 64), (1e4, -1.0, 64), (1e4, 2.0, 2)]:
        assert L.vlm_rope_alpha_base(theta, alpha, d, C.byref(out)) == N.VLM_ERR_ARG
    assert L.vlm_rope_alpha_base(1e4, 2.0, 64, None) == N.VLM_ERR_ARG


def test_sample_logits_argument_checks():
    L = N.lib()
    fake = C.c_void_p(0x1000)   # never dereferenced: every case fails its checks first
    def st(V=1000, T=1.0, k=40, p=0.9, r=1.1, n=0, ctx=None):
        prm = N.Sampling(T, k, p, r)
        return L.vlm_sample_logits(fake, V, C.byref(prm), ctx, n, fake, fake, None)
    assert st(V=0) == N.VLM_ERR_SHAPE and st(V=(1 << 19) + 1) == N.VLM_ERR_SHAPE
    assert st(T=0.0) == N.VLM_ERR_ARG and st(T=float("nan")) == N.VLM_ERR_ARG
    assert st(k=0) == N.VLM_ERR_UNSUPPORTED and st(k=1025) == N.VLM_ERR_UNSUPPORTED
    assert st(p=0.0) == N.VLM_ERR_ARG and st(p=1.5) == N.VLM_ERR_ARG
    assert st(r=0.0) == N.VLM_ERR_ARG
    assert st(n=3, ctx=None) == N.VLM_ERR_ARG


def test_window_index_matches_oracle():
    """Integer bookkeeping of the vision window permutation: bit-exact vs the oracle."""
    from decoder_prefill_decode_amd.pipeline import window_index
    for cfg in (vs.C5, vs.scaled_vit(vs.C5, grid_h=6, grid_w=10, window=2)):
        up, rp, sg, pos = window_index(cfg.grid_h, cfg.grid_w, cfg.merge, cfg.window)
        perm, seg = ov.vit_window_order(cfg)
        assert np.array_equal(up, perm)
        row_perm = (perm[:, None] * 4 + np.arange(4)).reshape(-1)
        assert np.array_equal(rp, row_perm)
        assert np.array_equal(sg, np.repeat(seg, 4))
        assert np.array_equal(pos, ov.vit_positions(cfg)[:, row_perm])


def test_window_index_rejects_bad_grid():
    assert N.lib().vlm_vit_window_index(13, 92, 2, 8, None, None, None, None) == N.VLM_ERR_SHAPE


def test_merger_validation():
    m = N.Merger(1152, 2, 4608, 2560, N.VLM_F32, 1e-6)
    n = C.c_size_t()
    assert N.lib().vlm_vit_merger_workspace_bytes(C.byref(m), 1288, C.byref(n)) == N.VLM_ERR_ARG  # NULL weights
    for f in ("post_ln", "post_ln_b", "w1", "b1", "w2", "b2"):
        setattr(m, f, 0x1000)
    assert N.lib().vlm_vit_merger_workspace_bytes(C.byref(m), 1287, C.byref(n)) == N.VLM_ERR_SHAPE
    N.call("vlm_vit_merger_workspace_bytes", C.byref(m), 1288, C.byref(n))
    assert n.value >= 1288 * 1152 * 4 + 322 * 4608 * 4


def test_noalloc_lmhead_rejects_vocab_beyond_scratch_before_device_work():
    d = desc(vocab=300000, dtype=N.VLM_BF16)
    fake = C.c_void_p(256)
    st = N.lib().vlm_lmhead_argmax_noalloc(C.byref(d), fake, fake, fake, fake, None, None)
    assert st == N.VLM_ERR_UNSUPPORTED and "scratch" in N.last_error()


def test_verify_commit_and_status_argument_checks():
    assert N.lib().vlm_verify_commit(None, 0, None, 1, None, None, None, None) == N.VLM_ERR_ARG
    assert N.lib().vlm_kv_status(None, None, None) == N.VLM_ERR_ARG
    assert N.lib().vlm_token_status(None, None, None) == N.VLM_ERR_ARG
    d = desc(vocab=0)
    fake = C.c_void_p(256)
    tok = C.c_void_p(512)
    assert N.lib().vlm_lmhead_argmax_rows(C.byref(d), fake, fake, fake, 4, tok, None, fake, 1 << 20, None) == \
        N.VLM_ERR_SHAPE


def test_verify_head_logits_scratch_is_checked_against_the_workspace_bytes():
    """With no logits buffer the verify head keeps S x V fp32 logits in the workspace, after the S
    normalised rows, then the row argmax's partial keys (32 u64 per row at this vocabulary), and
    checks that against the caller's workspace size (a vocabulary of 128256 does not fit the S-row
    layout's own split scratch)."""
    d = desc(vocab=128256)
    n = C.c_size_t()
    N.call("vlm_workspace_bytes", C.byref(d), 8, C.byref(n))
    need = 8 * 256 * 4 + 8 * 128256 * 4 + 8 * 32 * 8   # rows, logits (both already 256-aligned), keys
    assert n.value < need
    fake = C.c_void_p(256)
    tok = C.c_void_p(512)
    st = N.lib().vlm_lmhead_argmax_rows(C.byref(d), fake, fake, fake, 8, tok, None, fake, n.value, None)
    assert st == N.VLM_ERR_WORKSPACE and str(need) in N.last_error()


def test_host_split_plan_mirror_matches_library():
    """decoder_prefill_decode_amd.csrc_info.decode_plan (the bench's byte accounting) equals the
    library's planner at every band of the 36-layer stack's window and of a long tiny one."""
    from decoder_prefill_decode_amd.csrc_info import decode_plan
    ns, ch = C.c_int32(), C.c_int32()
    for cap in (64, 1024, 1152, 2048, 2100):
        for t in list(range(0, cap, 37)) + [cap - 1]:
            N.call("vlm_decode_split_plan", cap, t, C.byref(ns), C.byref(ch))
            assert (ns.value, ch.value) == decode_plan(cap, t), (cap, t)
            assert ns.value <= 32 and ns.value * ch.value >= min(cap, (t // 64 + 1) * 64) > t
