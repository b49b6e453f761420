"""Writes the stored oracle results for the full-size workloads.

Calls only oracle/ (and the shared seeded input generators). The GPU tests at
full size compare against these files, because the oracle needs minutes per
workload there.

    python tests/golden/make_golden.py c3_qwen3_28l c4_llama_4b c5_vit_27l c5_vit_27l_bf16

Each decoder file holds the exact-sum oracle's (bf16 mode: float64 sums of
the exact bf16 products) full tensors: every prefill row, every first-token
logit, every valid K/V slot of layers 0, L/2 and L-1 (bf16 bit patterns),
the greedy ids and their top-2 margins. It also holds the oracle's own noise
floor: the same workload rerun with float32 BLAS sums (every operand and
rounding point unchanged) and teacher-forced on the exact run's ids. The
largest logit change over all steps of that rerun is the floor below which a
greedy step is a near-tie that the arithmetic does not decide; the prefill and
KV changes are recorded next to it. No value here comes from the GPU path.
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


class Lazy:
    """Layers generated on first read, so only one layer's float32 draw is alive at a time."""

    def __init__(self, fn, n):
        self.fn, self.n = fn, n

    def __len__(self):
        return self.n

    def __iter__(self):
        return (self.fn(l) for l in range(self.n))


def kv_layers(cfg):
    return sorted({0, cfg.n_layers // 2, cfg.n_layers - 1})


def rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def decoder_golden(cfg):
    t = time.time()
    glob = vs.decoder_globals(cfg)
    layers = Lazy(lambda l: vs.decoder_layer_weights(cfg, l), cfg.n_layers)
    r = od.run_decoder(cfg, glob, layers, keep_logits=True)
    print(f"{cfg.name}: exact-sum oracle in {time.time() - t:.0f}s", flush=True)
    t = time.time()
    p = od.run_decoder(cfg, glob, layers, keep_logits=True, prec=od.BF16_F32SUM, forced_ids=r["ids"][:-1])
    print(f"{cfg.name}: float32-sum rerun in {time.time() - t:.0f}s", flush=True)
    T = cfg.seq + cfg.decode_steps
    Ls = kv_layers(cfg)
    step_floor = np.array([np.abs(a - b).max() for a, b in zip([r["logits0"]] + r["step_logits"],
                                                                 [p["logits0"]] + p["step_logits"])])
    kv_floor = [max(rel(p["k_cache"][l][:, :cfg.seq], r["k_cache"][l][:, :cfg.seq]),
                    rel(p["v_cache"][l][:, :cfg.seq], r["v_cache"][l][:, :cfg.seq])) for l in Ls]
    k = np.stack([r["k_cache"][l][:, :T] for l in Ls]).astype(np.float32)
    v = np.stack([r["v_cache"][l][:, :T] for l in Ls]).astype(np.float32)
    np.savez_compressed(
        os.path.join(OUT, f"{cfg.name}.npz"),
        ids=r["ids"], margins=r["margins"], logits0=r["logits0"].astype(np.float32),
        prefill_x=r["prefill_x"].astype(np.float32), kv_layers=np.array(Ls),
        k_bits=vs.bf16_bits(k), v_bits=vs.bf16_bits(v), decode_x_last=r["decode_x"][-1].astype(np.float32),
        floor_logit_steps=step_floor, floor_logit=step_floor.max(), floor_prefill_rel=rel(p["prefill_x"], r["prefill_x"]),
        floor_kv_rel=np.array(kv_floor), floor_ids_agree=np.array([int(a == b) for a, b in zip(p["ids"], r["ids"])]))
    assert np.array_equal(vs.bf16_bits(k).astype(np.uint32) << 16, k.view(np.uint32)), "K not bf16-exact"
    n_tie = int((r["margins"] < step_floor.max()).sum())
    print(f"{cfg.name}: ids {[int(i) for i in r['ids'][:12]]} ... {len(set(r['ids']))} distinct; logit floor "
          f"{step_floor.max():.3e}; {n_tie}/{len(r['ids'])} steps below it; prefill floor "
          f"{rel(p['prefill_x'], r['prefill_x']):.3e}; KV floor {kv_floor}; float32-sum rerun picks the exact "
          f"ids at {sum(int(a == b) for a, b in zip(p['ids'], r['ids']))}/{len(r['ids'])} steps", flush=True)


def vit_golden(cfg):
    t = time.time()
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    r = ov.run_vit(cfg, glob, layers)
    print(f"{cfg.name}: oracle in {time.time() - t:.0f}s", flush=True)
    extra = {}
    if cfg.dtype == vs.BF16:
        p = ov.run_vit(cfg, glob, layers, prec=od.BF16_F32SUM)
        extra["floor_out_rel"] = rel(p["out"], r["out"])
        print(f"{cfg.name}: float32-sum rerun moves the merged rows by {extra['floor_out_rel']:.3e}", flush=True)
    np.savez_compressed(os.path.join(OUT, f"{cfg.name}.npz"), out=r["out"].astype(np.float32), **extra)


def config(name):
    if name == "c5_vit_27l_bf16":
        return vs.scaled_vit(vs.C5, dtype=vs.BF16, name=name)
    return vs.ALL_CONFIGS[name]


if __name__ == "__main__":
    for name in sys.argv[1:]:
        cfg = config(name)
        (vit_golden if isinstance(cfg, vs.VitConfig) else decoder_golden)(cfg)
