#!/usr/bin/env python3
"""Throughput of the VLM decoder hot path on one MI355X.

One step = one pass of the decoder path over one synthetic prompt: embedding
lookup, image-row injection, parallel prefill of every layer into the KV
cache, lm_head + argmax of the last prompt row, then the workload's greedy
decode steps (one HIP-graph launch per token), starting from an empty cache.
Inputs and weights are resident in HBM before the timed region.

Default workload: the 28-layer Qwen3-style bf16 stack (hidden 1024, 16/8
heads, head_dim 128, FFN 3072, tied vocabulary 151936), 560-token prompt
with a 495-row image span, 128 decode steps.

Prints one JSON line: value = (prompt + generated tokens) / step time, with
the prefill and decode rates beside it, the roofline of the dominant kernel
(timed with HIP events on the stream it runs on) and the CPU oracle timed on
a bounded sample on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
METRIC = "prefill tok/s + decode tok/s per decoder stack; % of HBM / MFMA roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "decoder_prefill_decode_amd", "csrc", "k_gemv.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c3_qwen3_28l")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-decode-steps", type=int, default=128)
    ap.add_argument("--kernel-only", default=None,
                    help="launch one decode kernel (lmhead, qkv, o, gate_up, down) --launches times and exit")
    ap.add_argument("--launches", type=int, default=200)
    return ap.parse_args()


KERNELS = ["lmhead", "qkv", "o", "gate_up", "down"]


def kernel_bytes(cfg, name):
    """Algorithmic HBM bytes of one launch: the weight matrix once plus its vector input/output."""
    E = 2 if cfg.dtype == "bf16" else 4
    H, F, qd = cfg.hidden, cfg.ffn, cfg.n_q_heads * cfg.head_dim
    if name == "lmhead":
        return cfg.vocab * H * E + H * 4
    if name == "qkv":
        return cfg.qkv_rows * H * E + H * 4 + cfg.qkv_rows * 4
    if name == "o":
        return H * qd * E + qd * E + 2 * H * 4
    if name == "gate_up":
        return 2 * F * H * E + H * 4 + F * E
    return H * F * E + F * E + 2 * H * 4


def load_traffic(name):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t.get(name)
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if ent and ent.get("source_sha256") == sha:
            return ent.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def time_kernel(run, name, launches):
    import ctypes as C

    import torch

    from decoder_prefill_decode_amd import native as N
    from decoder_prefill_decode_amd.runtime import ptr, stream
    m = run.model
    which = KERNELS.index(name)
    x = run.x[run.cfg.seq - 1]

    def go(n):
        N.call("vlm_launch_kernel", C.byref(m.desc), m.layers, ptr(m.final_norm), ptr(m.embed), which, n, ptr(x),
               ptr(run.ws), run.ws.numel(), stream())
    go(10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    go(launches)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / launches  # us per launch (includes the one-row copy, < 1 us)


def cpu_baseline(cfg, glob, layers, n_dec):
    """The oracle, untuned, on this host: prefill of the whole prompt plus n_dec
    decode steps; scaled to a full step (prompt + all decode steps)."""
    import numpy as np

    from oracle import decoder as od
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    r = od.run_decoder(cfg, glob, layers, steps=n_dec)
    t_pre = r["t_prefill_s"]
    t_dec = r["t_decode_s"] / max(n_dec, 1)
    t_step = t_pre + cfg.decode_steps * t_dec
    return {"value": (cfg.seq + cfg.decode_steps) / t_step, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name}: oracle prefill of {cfg.seq} tokens ({t_pre:.1f} s) and {n_dec} decode steps "
                      f"({t_dec:.2f} s each), scaled to {cfg.seq} + {cfg.decode_steps} tokens",
            "prefill_tok_s": cfg.seq / t_pre, "decode_tok_s": 1.0 / t_dec, "ids_head": [int(i) for i in r["ids"][:4]]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import vlm_synth as vs
    from decoder_prefill_decode_amd.pipeline import DecoderRun

    cfg = vs.ALL_CONFIGS[args.config]
    t_gen = time.perf_counter()
    glob = vs.decoder_globals(cfg)
    keep_layers = not args.no_cpu and args.kernel_only is None
    layers = [] if not keep_layers else [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    run = DecoderRun(cfg, (lambda l: layers[l]) if keep_layers else (lambda l: vs.decoder_layer_weights(cfg, l)),
                     glob)
    torch.cuda.synchronize()
    print(f"# {cfg.name}: weights generated and resident in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)

    if args.kernel_only:
        t = time_kernel(run, args.kernel_only, args.launches)
        print(f"# {args.kernel_only}: {t:.2f} us per launch over {args.launches} launches", file=sys.stderr)
        return

    S, N = cfg.seq, cfg.decode_steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        run.reset()
        if e:
            e[0].record()
        run.prefill()
        run.first_token()
        if e:
            e[1].record()
        run.model.decode_loop(run.kv, run.cos, run.sin, run.ws, run.tok, N, hist=run.hist)
        if e:
            e[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    ids = run.hist[S + 1:S + 1 + N].cpu().numpy()
    print(f"# step {ms_step:.2f} ms: prefill {pre_ms:.3f} ms, decode {dec_ms:.2f} ms ({dec_ms / N * 1e3:.1f} us/token); "
          f"first ids {[int(run.tok[0])] if N == 0 else list(map(int, ids[:6]))}", file=sys.stderr, flush=True)

    # per-kernel timing of the decode step; the dominant one carries the roofline
    per = {}
    for k in KERNELS:
        if k == "lmhead" and cfg.vocab == 0:
            continue
        us = time_kernel(run, k, 4 * cfg.n_layers if k != "lmhead" else 40)
        count = 1 if k == "lmhead" else cfg.n_layers
        per[k] = {"us": us, "per_token_us": us * count, "gbs": kernel_bytes(cfg, k) / (us * 1e-6) / 1e9}
    dom = max(per, key=lambda k: per[k]["per_token_us"])
    b = kernel_bytes(cfg, dom)
    achieved = b / (per[dom]["us"] * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(dom),
            "kernel": dom, "bytes_per_launch": b, "avg_launch_us": round(per[dom]["us"], 3)}
    flops = 2.0 * (cfg.n_layers * (cfg.qkv_rows * cfg.hidden + cfg.hidden * cfg.n_q_heads * cfg.head_dim
                                   + 3 * cfg.ffn * cfg.hidden) * S
                   + cfg.n_layers * 2 * cfg.n_q_heads * cfg.head_dim * S * (S + 1) / 2 + cfg.vocab * cfg.hidden)
    peak_mm = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": METRIC, "value": round((S + N) / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_layers}-layer decoder, hidden {cfg.hidden}, "
                               f"{cfg.n_q_heads}/{cfg.n_kv_heads} heads x {cfg.head_dim}, FFN {cfg.ffn}, vocab {cfg.vocab}, "
                               f"prefill {S} tokens ({cfg.n_img} image rows) + {N} greedy decode steps, KV window "
                               f"{cfg.capacity}", "prefill_tokens": S, "decode_steps": N, "global_batch": 1,
                   "seq_len": S, "parallelism": "single GPU"},
        "prefill_tok_s": round(S / (pre_ms * 1e-3), 1), "decode_tok_s": round(N / (dec_ms * 1e-3), 1),
        "prefill_ms": round(pre_ms, 3), "decode_ms": round(dec_ms, 3),
        "prefill_mfma_frac": round(flops / (pre_ms * 1e-3) / (peak_mm * 1e12), 4),
        "decode_kernels_us": {k: round(v["us"], 2) for k, v in per.items()},
        "decode_kernels_gbs": {k: round(v["gbs"], 1) for k, v in per.items()},
        "roofline": roof,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, glob, layers, args.cpu_decode_steps)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
