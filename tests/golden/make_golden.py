"""Writes the stored oracle results for the full-size workloads.

Calls only oracle/ (and the shared seeded input generators). The GPU tests at
full size compare against these files, because the oracle needs minutes per
workload there.

    python tests/golden/make_golden.py c3_qwen3_28l c4_llama_4b c5_vit_27l
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import decoder as od  # noqa: E402
from oracle import vit as ov  # noqa: E402
import vlm_synth as vs  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))


def decoder_golden(cfg):
    t = time.time()
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    print(f"{cfg.name}: inputs in {time.time() - t:.0f}s", flush=True)
    t = time.time()
    r = od.run_decoder(cfg, glob, layers)
    print(f"{cfg.name}: oracle in {time.time() - t:.0f}s", flush=True)
    lg = r["logits0"]
    top = np.argsort(-lg)[:64]
    S = cfg.seq
    rows = np.unique(np.r_[np.arange(0, S, 37), S - 1])
    slots = np.unique(np.r_[np.arange(0, S + cfg.decode_steps, 53), S + cfg.decode_steps - 1])
    Ls = [0, cfg.n_layers - 1]
    np.savez_compressed(
        os.path.join(OUT, f"{cfg.name}.npz"),
        ids=r["ids"], margins=r["margins"], logits0_top_idx=top, logits0_top_val=lg[top],
        logits0_absmax=np.abs(lg).max(), prefill_rows=rows, prefill_x_rows=r["prefill_x"][rows].astype(np.float32),
        prefill_x_absmax=np.abs(r["prefill_x"]).max(), kv_layers=np.array(Ls), kv_slots=slots,
        k_samples=r["k_cache"][Ls][:, :, slots].astype(np.float32),
        v_samples=r["v_cache"][Ls][:, :, slots].astype(np.float32),
        decode_x_last=r["decode_x"][-1].astype(np.float32))
    print(f"{cfg.name}: ids {list(r['ids'][:16])} ... min margin {r['margins'].min():.3e}", flush=True)


def vit_golden(cfg):
    t = time.time()
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    r = ov.run_vit(cfg, glob, layers)
    print(f"{cfg.name}: oracle in {time.time() - t:.0f}s", flush=True)
    units = np.arange(0, cfg.n_merged, 7)
    np.savez_compressed(os.path.join(OUT, f"{cfg.name}.npz"), units=units,
                        out_rows=r["out"][units].astype(np.float32), out_absmax=np.abs(r["out"]).max(),
                        out_row_norms=np.linalg.norm(r["out"], axis=1))


if __name__ == "__main__":
    for name in sys.argv[1:]:
        cfg = vs.ALL_CONFIGS[name]
        (vit_golden if isinstance(cfg, vs.VitConfig) else decoder_golden)(cfg)
