"""Vision tower -> decoder chaining on one device (the VLM data flow of the
Youtu-VL-4B ncnn port, 实现流程 §1-§6, and the HunyuanOCR v1.5 report §2): the
merged vision rows [322, 2560] that the ViT stack produces are exactly the
image rows injected into the 4B-class decoder's placeholder span.

The GPU runs the ViT, keeps its output on the device and hands it to the
decoder's injection; the oracle runs oracle/vit.py and feeds its output to
oracle/decoder.py. Gates: the merged rows within 1e-4 (fp32 tower) or 2e-2 (bf16 tower), decoder
prefill rows and first-token logits within the bf16 gate 2e-2, greedy ids
free-running and teacher-forced, exempt only below the oracle's own noise
floor (tests/_parity.py).
Stacks are cut to 2 layers each (decoder vocabulary 8192) so the oracle
finishes in seconds; the shapes at the seam are the full ones.
"""
import numpy as np
import pytest
import torch

import vlm_synth as vs
from oracle import decoder as od
from oracle import vit as ov
from tests._parity import check_ids, oracle_run

pytestmark = pytest.mark.gpu


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("vit_dtype", ["f32", "bf16"])
def test_vit_output_feeds_decoder(vit_dtype):
    from decoder_prefill_decode_amd import pipeline
    vcfg = vs.scaled_vit(vs.C5, n_layers=2, full_layers=(1,), dtype=vit_dtype)
    vtol = 1e-4 if vit_dtype == "f32" else 2e-2
    dcfg = vs.scaled(vs.C4, n_layers=2, vocab=8192, decode_steps=8)
    assert dcfg.n_img == 322 and dcfg.hidden == 2560  # the merged-token count and width of the tower
    vglob = vs.vit_globals(vcfg)
    vlayers = [vs.vit_layer_weights(vcfg, l) for l in range(vcfg.n_layers)]
    dglob = vs.decoder_globals(dcfg)
    dlayers = [vs.decoder_layer_weights(dcfg, l) for l in range(dcfg.n_layers)]

    vref = ov.run_vit(vcfg, vglob, vlayers)["out"]
    assert vref.shape == (dcfg.n_img, dcfg.hidden)
    oglob = dict(dglob)
    oglob["img"] = vref
    ref = oracle_run(dcfg, oglob, dlayers)

    vrun = pipeline.VitRun(vcfg, lambda l: vlayers[l], vglob)
    img = vrun.run()  # device fp32 [322, 2560], raster order
    assert rel(img.cpu().numpy(), vref) <= vtol
    drun = pipeline.DecoderRun(dcfg, lambda l: dlayers[l], dglob)
    drun.img = img.contiguous()
    x = drun.prefill()
    logits = torch.empty(dcfg.vocab, dtype=torch.float32, device="cuda")
    tok0 = int(drun.first_token(logits)[0])
    lg = logits.cpu().numpy()
    assert rel(x.cpu().numpy(), ref["prefill_x"]) <= 2e-2
    assert rel(lg, ref["logits0"]) <= 2e-2
    free = [tok0] + list(drun.decode(dcfg.decode_steps))
    drun.kv.truncate(dcfg.seq)
    forced = [tok0] + list(drun.decode_forced(ref["ids"][:-1]))
    print(f"chain ({vit_dtype} tower): vit err {rel(img.cpu().numpy(), vref):.2e}, "
          f"first-token logit err {np.abs(lg - ref['logits0']).max():.2e}")
    check_ids(f"chain ({vit_dtype} tower)", free, forced, ref["ids"], ref["margins"], ref["floor"])
