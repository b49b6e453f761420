#!/usr/bin/env python3
"""Throughput of the VLM decoder hot path on one MI355X.

One step = one pass of the decoder path over one synthetic prompt: embedding
lookup, image-row injection, parallel prefill of every layer into the KV
cache, lm_head + argmax of the last prompt row, then the workload's greedy
decode steps (one HIP-graph launch per token), starting from an empty cache.
Inputs and weights are resident in HBM before the timed region.

Default workload: the 36-layer 4B-class bf16 stack (hidden 2560, 32/8 heads
of 80, FFN 9728, tied vocabulary 128256, 2048-slot window), 512-token prompt
with a 322-row image span, 256 decode steps. --config c3_qwen3_28l runs the
28-layer Qwen3-style stack (vocabulary 151936) the same way. --config
c5_vit_27l times the 27-layer window/full-attention vision tower with its 2x2
merger instead (one step = one tower pass over the 1288 patch rows; fp32, or
bf16 storage with fp32 accumulation with --vit-dtype bf16), with the roofline of
the whole pass against the matrix-core peak of its type.

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
KERNEL_SOURCES = {k: os.path.join(ROOT, "decoder_prefill_decode_amd", "csrc", f)
                  for k, f in (("gemv", "k_gemv.hip"), ("attn", "k_attn.hip"), ("common", "common.hpp"))}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4_llama_4b")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-decode-steps", type=int, default=32)
    ap.add_argument("--kernel-only", default=None,
                    help="launch one decode kernel (lmhead, qkv, o, gate_up, down, attn) --launches times, then "
                         "one plain copy of --copy-mib MiB (reference for HBM counters), and exit")
    ap.add_argument("--launches", type=int, default=200)
    ap.add_argument("--mfma", default=None, metavar="CSV",
                    help="summarise a rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 counter CSV of a --prefill-only run "
                         "(per prefill kernel: MFMA busy %% and counted vs algorithmic FLOPs) and exit")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="N",
                    help="run N prefills (embed, inject, all layers, first-token head) and exit; the run the "
                         "MFMA counters are collected on")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--vit-dtype", default="f32", choices=("f32", "bf16"),
                    help="storage type of the vision tower (c5_vit_27l only)")
    ap.add_argument("--next-rows", action="store_true",
                    help="time the widened rows instead of the step: the verify head and a block verify against "
                         "one-token decode, the sampler and the sampled graph loop, the expanded-MLA stack, and "
                         "the vision tower feeding the decoder prefill; prints one JSON line and exits")
    ap.add_argument("--verify-blocks", type=int, default=0, metavar="N",
                    help="after the prompt's prefill and 8 greedy steps, verify that greedy block N times "
                         "(chunked prefill of 8 rows, verify head, commit; the cache trimmed back each time), "
                         "print one JSON line with the time per block and exit (the run the verify kernel "
                         "traces are taken on)")
    ap.add_argument("--traffic", nargs=3, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV"), default=None,
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a --kernel-only run "
                         "into profiles/traffic.json and exit")
    return ap.parse_args()


KERNELS = ["lmhead", "qkv", "o", "gate_up", "down", "attn"]
# name fragments of each kernel in a --kernel-only run (the copy kernels are told apart by name too)
KERNEL_NAME = {"lmhead": "Epi)5", "qkv": "Epi)0", "o": "Epi)1", "gate_up": "Epi)2", "down": "Epi)1",
               "attn": "attn_decode_"}  # the vector-ALU (fused), matrix-core (mfma) or MLA decode attention


def kernel_bytes(cfg, name, t=None):
    """Algorithmic HBM bytes of one launch: the weight matrix once plus its vector input/output;
    attention: the K/V slots 0..t-1 it reads, the slot t it writes, q/k/v in and the split partials out."""
    E = 2 if cfg.dtype == "bf16" else 4
    H, F, qd = cfg.hidden, cfg.ffn, cfg.n_q_heads * cfg.head_dim
    if name == "attn":
        from decoder_prefill_decode_amd.csrc_info import decode_plan, partial_stride
        kvd = cfg.n_kv_heads * cfg.head_dim
        nsplit = decode_plan(cfg.capacity, t)[0]
        return 2 * kvd * t * E + 2 * kvd * E + cfg.qkv_rows * 4 + \
            cfg.n_q_heads * nsplit * partial_stride(cfg.head_dim) * 4
    if name == "lmhead":
        return cfg.vocab * H * E + H * 4
    if name == "qkv":
        return cfg.qkv_rows * H * E + H * 4 + cfg.qkv_rows * 4
    if name == "o":
        return H * qd * E + qd * E + 2 * H * 4
    if name == "gate_up":
        return 2 * F * H * E + H * 4 + F * E
    return H * F * E + F * E + 2 * H * 4


def source_sha(name):
    """Hash of the sources the kernel is built from (its own file and the shared device helpers)."""
    h = hashlib.sha256()
    for path in (KERNEL_SOURCES["attn" if name == "attn" else "gemv"], KERNEL_SOURCES["common"]):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(cfg_name, name):
    """Counter-measured HBM bytes per launch of kernel `name` on workload `cfg_name`, if taken on the
    current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            ent = json.load(f).get(f"{cfg_name}:{name}")
        if ent and ent.get("source_sha256") == source_sha(name):
            return ent.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def traffic_from_csv(cfg_name, kernel, fetch_csv, write_csv, copy_mib):
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for the plain copy of copy_mib MiB in the same run."""
    import csv

    def rows(path, counter):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rs = rows(path, counter)
        copies = [v for n, v in rs if "gather_rows_kernel" in n]
        mine = [v for n, v in rs if KERNEL_NAME[kernel] in n and "vlm::" in n]
        if not copies or not mine:
            raise SystemExit(f"{path}: no {counter} rows for the copy or for {kernel}")
        scale = copy_mib * 1024.0 / max(copies)          # KiB the copy moves / KiB the counter reports
        res[counter] = {"kib_per_launch": sum(mine) / len(mine), "copy_kib": max(copies), "scale": scale,
                        "launches": len(mine)}
    b = (res["FETCH_SIZE"]["kib_per_launch"] * res["FETCH_SIZE"]["scale"]
         + res["WRITE_SIZE"]["kib_per_launch"] * res["WRITE_SIZE"]["scale"]) * 1024.0
    try:
        with open(TRAFFIC_FILE) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    key = f"{cfg_name}:{kernel}"
    allt[key] = {"bytes_per_launch": round(b), "source_sha256": source_sha(kernel), "counters": res,
                 "copy_reference_mib": copy_mib}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allt, f, indent=1)
    print(json.dumps(allt[key]))


def time_kernel(run, name, launches):
    """Average launch duration (us) of one decode kernel, from HIP events on the stream it runs on,
    around `launches` back-to-back launches (attention at the mid-run cache length)."""
    import ctypes as C

    import torch

    from decoder_prefill_decode_amd import native as N
    from decoder_prefill_decode_amd.runtime import ptr, stream
    m = run.model
    which = KERNELS.index(name)
    x = run.x[run.cfg.seq - 1]
    if name == "attn":
        run.kv.truncate(run.cfg.seq + run.cfg.decode_steps // 2)

    def go(n):
        N.call("vlm_launch_kernel", C.byref(m.desc), m.layers, ptr(m.final_norm), ptr(m.embed), run.kv.handle,
               ptr(run.cos), ptr(run.sin), run.cos.shape[0], which, n, ptr(x), ptr(run.ws), run.ws.numel(), stream())
    go(10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    go(launches)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / launches  # us per launch (includes the one-row copy, < 1 us)


def mfma_summary(cfg_name, csv_path):
    """Markdown table of the prefill kernels' MFMA counters: MfmaUtil (busy cycles of the matrix cores over
    all SIMDs and the kernel's active cycles) and MfmaFlopsBF16 (512 x bf16 MFMA MOPs) per dispatch, next
    to the algorithmic FLOPs of the launch for the gate/up, down, O, QKV GEMMs and the causal attention."""
    import csv
    from collections import defaultdict

    import vlm_synth as vs
    cfg = vs.ALL_CONFIGS[cfg_name]
    S, H, F = cfg.seq, cfg.hidden, cfg.ffn
    qd = cfg.n_q_heads * cfg.head_dim
    algo = {"Epi)2": 2.0 * S * 2 * F * H, "Epi)0": 2.0 * S * cfg.qkv_rows * H,
            "attn_prefill": 4.0 * cfg.n_q_heads * cfg.head_dim * S * (S + 1) / 2}
    util, flops = defaultdict(list), defaultdict(list)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "gemm_lds_kernel" not in name and "attn_prefill" not in name:
                continue
            key = name.split("(vlm::GemmArgs)")[0].split("(vlm::AttnArgs)")[0].replace("vlm::", "").replace("void ", "")
            (util if r["Counter_Name"] == "MfmaUtil" else flops)[key].append(float(r["Counter_Value"]))
    print("| kernel | dispatches | MFMA busy % (mean) | counted GFLOP / launch | algorithmic GFLOP / launch |")
    print("|---|---:|---:|---:|---:|")
    for key in sorted(util, key=lambda k: -sum(util[k])):
        a = next((v for frag, v in algo.items() if frag in key), None)
        if a is None and "Epi)1" in key:   # O (K = nq*d) or down (K = F): told apart by the counted work
            c = sum(flops[key]) / max(len(flops[key]), 1)
            a = min((2.0 * S * H * qd, 2.0 * S * H * F), key=lambda v: abs(v - c))
        cf = sum(flops[key]) / max(len(flops[key]), 1) / 1e9
        print(f"| `{key}` | {len(util[key])} | {sum(util[key]) / len(util[key]):.1f} | {cf:.2f} | "
              f"{'' if a is None else f'{a / 1e9:.2f}'} |")


def measured_peaks():
    """Peaks measured on this device: HBM from a stream copy of 1 GiB (torch's vectorised copy kernel;
    read + write bytes / time, best of 6), bf16 MFMA from rocminfo's compute units x max clock x 1024 FLOP
    per clock per SIMD x 4 SIMDs per CU (the dense 32x32x16 bf16 rate)."""
    import subprocess

    import torch

    n = 1 << 28                                         # 2^28 floats = 1 GiB read, 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = 1e30
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    hbm = 2.0 * n * 4 / (best * 1e-3) / 1e9
    cus = clk = None
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        for blk in txt.split("Agent ")[1:]:
            if "gfx9" in blk and "Compute Unit" in blk:
                for line in blk.splitlines():
                    if "Max Clock Freq" in line:
                        clk = float(line.split(":")[1].split("(")[0])
                    if "Compute Unit" in line:
                        cus = int(line.split(":")[1])
                break
    except Exception:
        pass
    mfma = cus * clk * 1e6 * 4 * 1024 / 1e12 if cus and clk else None
    return {"hbm_copy_gbs": round(hbm, 1), "bf16_mfma_tflops": round(mfma, 1) if mfma else None,
            "compute_units": cus, "max_clock_mhz": clk}


def cpu_baseline(cfg, glob, layers, n_dec):
    """The oracle, untuned, on this host: prefill of the whole prompt plus n_dec
    decode steps; scaled to a full step (prompt + all decode steps)."""
    import numpy as np

    from oracle import decoder as od
    blas = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max(i.get("num_threads", 1) for i in info) or 1
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} x{i.get('num_threads')}" for i in info)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    r = od.run_decoder(cfg, glob, layers, steps=n_dec)
    t_pre = r["t_prefill_s"]
    t_dec = r["t_decode_s"] / max(n_dec, 1)
    t_step = t_pre + cfg.decode_steps * t_dec
    return {"value": (cfg.seq + cfg.decode_steps) / t_step, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name}: oracle prefill of {cfg.seq} tokens ({t_pre:.1f} s) and {n_dec} decode steps "
                      f"({t_dec:.2f} s each), scaled to {cfg.seq} + {cfg.decode_steps} tokens",
            "prefill_tok_s": cfg.seq / t_pre, "decode_tok_s": 1.0 / t_dec, "ids_head": [int(i) for i in r["ids"][:4]],
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu, "blas": blas}


def vit_flops(cfg, row_seg):
    """Algorithmic FLOPs of one tower pass: linear layers, attention over the visible pairs of each
    layer's mask (windows or full), the merger MLP."""
    import numpy as np
    N, H, F, hd = cfg.n_patches, cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim
    lin = 2.0 * N * (3 * H * hd + hd * H + 2 * F * H)
    _, counts = np.unique(row_seg, return_counts=True)
    pairs_win = float(np.sum(counts.astype(np.float64) ** 2))
    attn = [4.0 * hd * (N * N if l in cfg.full_layers else pairs_win) for l in range(cfg.n_layers)]
    m2 = cfg.merge * cfg.merge
    merger = 2.0 * (N // m2) * (m2 * H * cfg.merger_hidden + cfg.merger_hidden * cfg.out_dim)
    return cfg.n_layers * lin + sum(attn) + merger


def vit_main(args, cfg):
    """One tower pass per step; the oracle tower on this host beside it."""
    import numpy as np
    import torch

    import vlm_synth as vs
    from decoder_prefill_decode_amd.pipeline import VitRun
    if args.vit_dtype != cfg.dtype:
        cfg = vs.scaled_vit(cfg, dtype=args.vit_dtype)
    t_gen = time.perf_counter()
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    run = VitRun(cfg, lambda l: layers[l], glob)
    torch.cuda.synchronize()
    print(f"# {cfg.name} ({cfg.dtype}): weights generated and resident in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        run.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        run.run()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    pass_ms = [e[0].elapsed_time(e[1]) for e in ev]
    t_ms = float(np.median(pass_ms))
    flops = vit_flops(cfg, run.row_seg)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flops / (t_ms * 1e-3) / 1e12
    N = cfg.n_patches
    print(f"# tower pass {t_ms:.3f} ms ({flops / 1e9:.1f} GFLOP, {achieved:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": round(N / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_layers}-layer vision tower, hidden {cfg.hidden}, "
                               f"{cfg.n_heads} heads x {cfg.head_dim}, FFN {cfg.ffn}, {N} patches on a "
                               f"{cfg.grid_h}x{cfg.grid_w} grid, window {cfg.window}x{cfg.window} merged cells, "
                               f"full attention on layers {list(cfg.full_layers)}, 2x2 merge -> {cfg.out_dim}",
                   "prefill_tokens": N, "global_batch": 1, "seq_len": N, "parallelism": "single GPU"},
        "prefill_tok_s": round(N / (t_ms * 1e-3), 1), "prefill_ms": round(t_ms, 3),
        "prefill_mfma_frac": round(achieved / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None, "kernel": "whole tower pass",
                     "flops_per_pass": flops, "avg_pass_ms": round(t_ms, 3)},
        "step_ms_median": round(t_ms, 3), "step_ms_min": round(float(np.min(pass_ms)), 3),
    }
    if not args.no_cpu:
        from oracle import vit as ov
        t0 = time.perf_counter()
        ov.run_vit(cfg, glob, layers)
        t_cpu = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": N / t_cpu, "unit": "tok/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle", "sample": f"{cfg.name}: one whole oracle tower pass ({t_cpu:.1f} s)"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


def verify_blocks_main(args):
    """N verify passes of one 8-token greedy block on the configured stack (HIP events on torch's
    current stream, the stream every call runs on)."""
    import torch

    import vlm_synth as vs
    from decoder_prefill_decode_amd.pipeline import DecoderRun

    cfg = vs.ALL_CONFIGS[args.config]
    run = DecoderRun(cfg, lambda l: vs.decoder_layer_weights(cfg, l), vs.decoder_globals(cfg))
    run.prefill()
    run.first_token(check=False)
    ids = [int(run.tok[0])] + [int(t) for t in run.decode(8)]

    def verify():
        run.kv.truncate(cfg.seq)
        return run.verify_block(ids[:8])
    verify()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.verify_blocks):
        toks, _ = verify()
    e1.record()
    e1.synchronize()
    print(json.dumps({"mode": "verify_blocks", "config": cfg.name, "block": 8, "blocks": args.verify_blocks,
                      "us_per_block": round(e0.elapsed_time(e1) * 1e3 / args.verify_blocks, 1),
                      "accepted": len(toks) - 1}))


def next_rows_main(args):
    """Measurement of the widened rows on the 36-layer stack (HIP events on torch's current stream, the
    stream every call runs on): verify head (one pass over the lm_head table for a block of rows),
    block verify (chunked prefill of the block + verify head + commit) against the same number of
    one-token decode steps, the sampler on one logits row and the sampled graph loop against the
    greedy loop, the expanded-MLA stack (prefill and decode step), and the vision tower whose merged
    rows feed the decoder prefill."""
    import numpy as np
    import torch

    import vlm_synth as vs
    from decoder_prefill_decode_amd import native as N
    from decoder_prefill_decode_amd.pipeline import DecoderRun, VitRun
    from decoder_prefill_decode_amd.runtime import decode_loop_sampled, sample_logits

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us per call

    out = {"mode": "next_rows", "n_gpus": 1, "data": "synthetic"}
    cfg = vs.ALL_CONFIGS["c4_llama_4b"]
    glob = vs.decoder_globals(cfg)
    run = DecoderRun(cfg, lambda l: vs.decoder_layer_weights(cfg, l), glob)
    E, V, H, K = 2, cfg.vocab, cfg.hidden, 8
    run.prefill()
    run.first_token(check=False)
    ids = [int(run.tok[0])] + [int(t) for t in run.decode(K)]      # a greedy block to draft from
    # verify head alone: K rows, one pass over the table
    rows = run.x[:K].clone()
    pred = torch.empty(K, dtype=torch.int32, device="cuda")
    logits = torch.empty((K, V), dtype=torch.float32, device="cuda")
    us = timed(lambda: run.model.lmhead_argmax_rows(rows, pred, run.ws, logits), 20)
    b = V * H * E + K * V * 4 + K * H * 4
    out["verify_head"] = {"rows": K, "us": round(us, 2), "bytes": b, "gbs": round(b / us * 1e-3, 1),
                          "hbm_frac": round(b / us * 1e-3 / PEAK_HBM_GBS, 4)}
    # block verify of K drafted tokens (all accepted) against K one-token decode steps from the same length
    L0 = cfg.seq
    def verify():
        run.kv.truncate(L0)
        run.verify_block(ids[:K])
    def one_token():
        run.kv.truncate(L0)
        run.tok.fill_(ids[0])
        run.decode(K)
    vu, du = timed(verify, 5), timed(one_token, 5)
    out["block_verify"] = {"block": K, "verify_us": round(vu, 1), "decode_steps_us": round(du, 1),
                           "speedup": round(du / vu, 2)}
    # sampler on one logits row, context = the prompt ids
    lg = logits[0].contiguous()
    ctx = run.ids_dev
    u = torch.full((1,), 0.37, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    su = timed(lambda: sample_logits(lg, 0.8, 50, 0.9, 1.1, ctx, u, tok), 50)
    out["sampler"] = {"vocab": V, "top_k": 50, "top_p": 0.9, "context": int(ctx.numel()), "us": round(su, 2)}
    n = 64
    hist = torch.full((cfg.capacity + 1,), -2, dtype=torch.int32, device="cuda")
    hist[:L0].copy_(ctx)
    ud = torch.from_numpy(np.random.default_rng(7).random(cfg.capacity + 1).astype(np.float32)).to("cuda")
    prm = N.Sampling(0.8, 50, 0.9, 1.1)
    def greedy():
        run.kv.truncate(L0)
        run.tok.fill_(ids[0])
        run.decode(n)
    def sampled():  # fixed buffers: the captured graphs are reused from call to call
        run.kv.truncate(L0)
        run.tok.fill_(ids[0])
        hist[L0:L0 + 1].fill_(ids[0])
        decode_loop_sampled(run.model, run.kv, run.cos, run.sin, run.ws, run.tok, n, hist, prm, ud)
        run.kv.status()
    gu, smu = timed(greedy, 3), timed(sampled, 3)
    out["sampled_loop"] = {"steps": n, "greedy_tok_s": round(n / (gu * 1e-6), 1),
                           "sampled_tok_s": round(n / (smu * 1e-6), 1), "sampled_us_per_token_extra":
                           round((smu - gu) / n, 2)}
    del run, logits, rows
    torch.cuda.empty_cache()
    # expanded MLA stack (the layer shape the parity tests cover), bf16
    mcfg = vs.scaled(vs.C_MLA, dtype=vs.BF16, name="c_mla_small_bf16")
    mglob = vs.decoder_globals(mcfg)
    mrun = DecoderRun(mcfg, lambda l: vs.decoder_layer_weights(mcfg, l), mglob)
    def mla_prefill():
        mrun.reset()
        mrun.prefill()
    pu = timed(mla_prefill, 10)
    mrun.reset()
    mrun.prefill()
    mrun.first_token(check=False)
    def mla_decode():
        mrun.kv.truncate(mcfg.seq)
        mrun.tok.fill_(1)
        mrun.decode(mcfg.decode_steps)
    mu = timed(mla_decode, 5)
    out["mla_stack"] = {"config": f"{mcfg.n_layers} layers, hidden {mcfg.hidden}, {mcfg.n_q_heads} heads, "
                                  f"K {mcfg.head_dim} / V {mcfg.v_head_dim}, latent {mcfg.kv_lora_rank}, bf16",
                        "prefill_rows": mcfg.seq, "prefill_us": round(pu, 1),
                        "decode_us_per_token": round(mu / mcfg.decode_steps, 1)}
    del mrun
    torch.cuda.empty_cache()
    # vision tower (bf16 storage) -> 36-layer decoder prefill with its merged rows injected
    vcfg = vs.scaled_vit(vs.C5, dtype=vs.BF16, name="c5_vit_27l_bf16")
    vglob = vs.vit_globals(vcfg)
    vrun = VitRun(vcfg, lambda l: vs.vit_layer_weights(vcfg, l), vglob)
    drun = DecoderRun(cfg, lambda l: vs.decoder_layer_weights(cfg, l), glob)
    def chain():
        drun.img = vrun.run()
        drun.reset()
        drun.prefill()
        drun.first_token(check=False)
    tower = timed(lambda: vrun.run(), 5)
    cu = timed(chain, 5)
    out["vision_to_decoder"] = {"tower_ms": round(tower * 1e-3, 3), "tower_plus_prefill_ms": round(cu * 1e-3, 3),
                                "image_rows": cfg.n_img, "prompt_rows": cfg.seq}
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic:
        traffic_from_csv(args.config, args.traffic[0], args.traffic[1], args.traffic[2], args.copy_mib)
        return
    if args.mfma:
        mfma_summary(args.config, args.mfma)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import vlm_synth as vs
    from decoder_prefill_decode_amd.pipeline import DecoderRun
    from decoder_prefill_decode_amd.runtime import causal_mask as pipeline_causal

    if args.next_rows:
        next_rows_main(args)
        return
    if args.verify_blocks:
        verify_blocks_main(args)
        return
    cfg = vs.ALL_CONFIGS[args.config]
    if isinstance(cfg, vs.VitConfig):
        vit_main(args, cfg)
        return
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
        if args.kernel_only == "attn":
            # A cache filled to the mid-run length for the attention kernel to read: the prompt's prefill,
            # then one chunked prefill of the next decode_steps/2 rows (copies of prompt rows). Two prefills
            # are a few hundred dispatches; filling it with eager decode steps instead issued ~55k
            # dispatches before the measured launches, and a counter-collection run over that many
            # dispatches ended in a host-side fault inside the profiled launch path.
            run.prefill()
            extra = cfg.decode_steps // 2
            xr = run.x[:extra].clone()
            run.model.prefill(xr, cfg.seq, run.cos, run.sin, pipeline_causal(), run.kv, run.ws)
        t = time_kernel(run, args.kernel_only, args.launches)
        # the counters' reference: a plain row copy (the library's gather kernel with the identity
        # index) reading and writing exactly copy_mib MiB
        import ctypes as C
        from decoder_prefill_decode_amd import native as N
        from decoder_prefill_decode_amd.runtime import ptr, stream
        rows = args.copy_mib * 256
        src = torch.ones((rows, 1024), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        idx = torch.arange(rows, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        N.call("vlm_gather_rows", ptr(src), rows, ptr(idx), rows, 1024, ptr(dst), stream())
        torch.cuda.synchronize()
        print(f"# {args.kernel_only}: {t:.2f} us per launch over {args.launches} launches", file=sys.stderr)
        return

    if args.prefill_only:
        for _ in range(args.prefill_only):
            run.reset()
            run.prefill()
            run.first_token(check=False)
        torch.cuda.synchronize()
        print(f"# {args.prefill_only} prefills of {cfg.seq} rows done", file=sys.stderr)
        return

    S, N = cfg.seq, cfg.decode_steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        run.reset()
        if e:
            e[0].record()
        run.prefill()
        run.first_token(check=False)
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
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    ids = run.hist[S + 1:S + 1 + N].cpu().numpy()
    print(f"# step {ms_step:.2f} ms: prefill {pre_ms:.3f} ms, decode {dec_ms:.2f} ms ({dec_ms / N * 1e3:.1f} us/token); "
          f"first ids {[int(run.tok[0])] if N == 0 else list(map(int, ids[:6]))}", file=sys.stderr, flush=True)

    # per-kernel timing of the decode step; the dominant one carries the roofline
    per = {}
    t_mid = S + N // 2
    for k in KERNELS:
        if k == "lmhead" and cfg.vocab == 0:
            continue
        us = time_kernel(run, k, 4 * cfg.n_layers if k != "lmhead" else 40)
        count = 1 if k == "lmhead" else cfg.n_layers
        per[k] = {"us": us, "per_token_us": us * count, "gbs": kernel_bytes(cfg, k, t_mid) / (us * 1e-6) / 1e9}
    dom = max(per, key=lambda k: per[k]["per_token_us"])
    b = kernel_bytes(cfg, dom, t_mid)
    achieved = b / (per[dom]["us"] * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(cfg.name, dom),
            "kernel": dom, "bytes_per_launch": b, "avg_launch_us": round(per[dom]["us"], 3)}
    flops = 2.0 * (cfg.n_layers * (cfg.qkv_rows * cfg.hidden + cfg.hidden * cfg.n_q_heads * cfg.head_dim
                                   + 3 * cfg.ffn * cfg.hidden) * S
                   + cfg.n_layers * 2 * cfg.n_q_heads * cfg.head_dim * S * (S + 1) / 2 + cfg.vocab * cfg.hidden)
    peak_mm = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    # whole decode step: every weight once, the lm_head table, the valid K/V slots at the mid-run length
    E = 2 if cfg.dtype == "bf16" else 4
    tok_bytes = E * (cfg.n_layers * (cfg.qkv_rows * cfg.hidden + cfg.hidden * cfg.n_q_heads * cfg.head_dim
                                     + 3 * cfg.ffn * cfg.hidden + 2 * cfg.n_kv_heads * cfg.head_dim * t_mid)
                     + cfg.vocab * cfg.hidden)
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
        "decode_bytes_per_token": tok_bytes,
        "decode_hbm_frac": round(tok_bytes / (dec_ms * 1e-3 / max(N, 1)) / (PEAK_HBM_GBS * 1e9), 4),
        "decode_kernels_us": {k: round(v["us"], 2) for k, v in per.items()},
        "decode_kernels_gbs": {k: round(v["gbs"], 1) for k, v in per.items()},
        "roofline": roof,
        "step_ms_median": round(float(np.median(step_ms)), 3), "step_ms_min": round(float(np.min(step_ms)), 3),
    }
    mp = measured_peaks()
    out["measured_peaks"] = mp
    out["decode_hbm_frac_of_measured"] = round(tok_bytes / (dec_ms * 1e-3 / max(N, 1)) / (mp["hbm_copy_gbs"] * 1e9), 4)
    out["prefill_mfma_frac_of_rocminfo"] = (round(flops / (pre_ms * 1e-3) / (mp["bf16_mfma_tflops"] * 1e12), 4)
                                            if mp["bf16_mfma_tflops"] and cfg.dtype == "bf16" else None)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, glob, layers, args.cpu_decode_steps)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
