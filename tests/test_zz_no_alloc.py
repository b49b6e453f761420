"""The allocation-free lm_head argmax (vlm_lmhead_argmax_noalloc) against the
workspace entry point it mirrors (vlm_lmhead_argmax): same token, bitwise the
same logits, on two calls in a row (the second over a smaller vocabulary, so
the library's scratch array holds the first call's partials beyond the second
call's range), and the vocabulary limit rejected before any device work."""
import ctypes as C

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _model(V, H, seed):
    from decoder_prefill_decode_amd.runtime import Model
    rng = np.random.default_rng(seed)
    m = Model(n_layers=1, hidden=H, n_q_heads=8, n_kv_heads=8, head_dim=128, ffn=3072, vocab=V, dtype="bf16")
    table = (rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    import vlm_synth as vs
    m.set_table(vs.to_bf16_values(table, inplace=True), vs.to_bf16_values(1 + 0.02 * rng.standard_normal(H).astype(np.float32)))
    x = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to("cuda")
    return m, x


def test_noalloc_lmhead_equals_workspace_entry_point():
    from decoder_prefill_decode_amd import native as N
    from decoder_prefill_decode_amd.runtime import ptr, stream
    for V, seed in ((151936, 1), (8192, 2)):
        m, x = _model(V, 1024, seed)
        ws = m.workspace(1)
        tok_a = torch.full((1,), -5, dtype=torch.int32, device="cuda")
        tok_b = torch.full((1,), -5, dtype=torch.int32, device="cuda")
        lg_a = torch.empty(V, dtype=torch.float32, device="cuda")
        lg_b = torch.empty(V, dtype=torch.float32, device="cuda")
        m.lmhead_argmax(x, tok_a, ws, lg_a)
        N.call("vlm_lmhead_argmax_noalloc", C.byref(m.desc), ptr(m.final_norm), ptr(m.embed), ptr(x), ptr(tok_b),
               ptr(lg_b), stream())
        torch.cuda.synchronize()
        assert int(tok_b[0]) == int(tok_a[0]) == int(np.argmax(lg_a.cpu().numpy()))
        assert torch.equal(lg_a, lg_b)
        tok_c = torch.full((1,), -5, dtype=torch.int32, device="cuda")
        N.call("vlm_lmhead_argmax_noalloc", C.byref(m.desc), ptr(m.final_norm), ptr(m.embed), ptr(x), ptr(tok_c),
               None, stream())
        torch.cuda.synchronize()
        assert int(tok_c[0]) == int(tok_a[0])


def test_noalloc_rejects_vocab_beyond_scratch():
    from decoder_prefill_decode_amd import native as N
    d = N.ModelDesc(0, 1, 1024, 8, 8, 128, 3072, 300000, N.VLM_BF16, 0, 1, 1e-6)
    fake = C.c_void_p(256)
    st = N.lib().vlm_lmhead_argmax_noalloc(C.byref(d), fake, fake, fake, fake, None, None)
    assert st == N.VLM_ERR_UNSUPPORTED and "scratch" in N.last_error()
