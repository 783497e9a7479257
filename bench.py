#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, with the
inputs already resident in HBM:
  1. tq_append_key     compress every key   (rotation, bucketing, QJL signs, pack)
  2. tq_append_value   compress every value (rotation, bucketing, pack)
  3. tq_attention_scores  asymmetric scores of every query head over every key
  4. tq_attend         fused softmax . V over the packed cache (+ combine, R^T)

Workload: long context, one layer, 8 sequences x 8 KV heads (64 slots),
131072 tokens each, head_dim 128, 4 query heads per KV head (32 in all),
fp16 KV-like inputs (Gaussian, 4% outlier channels x8, LogNormal(0, 0.3)
token norms), 3-bit keys (proj_dim 64) and 3-bit values.  The packed cache
(973 MB) and the inputs (2 x 2.15 GB) are larger than the 256 MB Infinity
Cache, so every stage streams from HBM.

Prints one JSON line.  value = keys per second through the whole step
(each key is compressed, its value compressed, scored and attended).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "keys compressed/s + decode score/attend HBM GB/s (fraction of peak), 3-bit d=128"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0
WORKLOAD = dict(name="long_context_8x8x131072", n_seq=64, n_tok=131072, d=128, m=64, key_bits=3,
                value_bits=3, G=4, heads_per_slot_cycle=8)


def gen_inputs(n_seq, n_tok, d, G, heads_cycle, threads=16):
    from kv_cache_vector_compress_amd import synth
    with ThreadPoolExecutor(threads) as ex:
        K = np.stack(list(ex.map(lambda s: synth.kv_slot(synth.SEED_K, s, s % heads_cycle, n_tok, d), range(n_seq))))
        V = np.stack(list(ex.map(lambda s: synth.kv_slot(synth.SEED_V, s, s % heads_cycle, n_tok, d), range(n_seq))))
        Q = np.stack(list(ex.map(lambda s: synth.kv_slot(synth.SEED_Q, s, s % heads_cycle, G, d), range(n_seq))))
    return K, V, Q


def algorithmic_bytes(w):
    """Bytes each stage must move at minimum: inputs read once, outputs written once."""
    from kv_cache_vector_compress_amd import tq
    cfg = tq.Config(w["d"], w["m"], w["key_bits"], w["value_bits"])
    rec = tq.key_record_bytes(cfg)                      # 64
    vtok = tq.value_block_bytes(cfg) / 128               # 52
    units = w["n_seq"] * w["n_tok"]
    return {
        "compress_keys": units * (2 * w["d"] + rec),      # fp16 key in, record out
        "compress_values": units * (2 * w["d"] + vtok),   # fp16 value in, block share out
        "scores": units * (rec + 4 * w["G"]),             # record in, fp32 scores out
        "attend": units * (rec + vtok),                   # records + blocks in
    }, units


def kernel_source_hash() -> str:
    """sha256 over the HIP sources (kernels and headers), sorted by name."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_vector_compress_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def counter_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (FETCH_SIZE + WRITE_SIZE, calibrated on a plain device copy), or
    None if the record is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_long_context.txt")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash() or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return int(k["fetch_bytes"] + k["write_bytes"])


def cpu_baseline(w, slots=16):
    """The fp64 oracle, untuned, on a bounded sample of the same workload."""
    from oracle import turboquant as O
    from kv_cache_vector_compress_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    d, m, T, G = w["d"], w["m"], w["n_tok"], w["G"]
    R = synth.haar_rotation(d, synth.SEED_R)
    S = synth.gaussian_projection(m, d, synth.SEED_S)
    K, V, Q = gen_inputs(slots, T, d, G, w["heads_per_slot_cycle"], threads=8)
    kbeta, kc = O.lloyd_max_codebook(d, w["key_bits"])
    vbeta, vc = O.lloyd_max_codebook(d, w["value_bits"])
    t0 = time.perf_counter()
    keys = O.compress_keys(K, R, S, kbeta, kc)
    vals = O.compress_values(V, R, vbeta, vc)
    O.key_scores(Q, R, S, kc, keys)
    O.attend(Q, R, S, kc, keys, vals, value_centroids=vc)
    dt = time.perf_counter() - t0
    return {"value": slots * T / dt, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"slots 0-{slots - 1} of {w['n_seq']} ({slots}x{T} tokens, G={G}): compress K and V, "
                      f"scores and attend, numpy fp64; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path is single-GPU); --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cache_vector_compress_amd import synth, tq

    w = WORKLOAD
    n_seq, T, d, m, G = w["n_seq"], w["n_tok"], w["d"], w["m"], w["G"]
    print(f"[bench] generating inputs {n_seq}x{T}x{d} fp16", file=sys.stderr, flush=True)
    K, V, Q = gen_inputs(n_seq, T, d, G, w["heads_per_slot_cycle"])
    dev = torch.device("cuda:0")
    Kd = torch.from_numpy(K).to(dev)
    Vd = torch.from_numpy(V).to(dev)
    Qd = torch.from_numpy(Q).to(dev)
    del K, V
    R = synth.haar_rotation(d, synth.SEED_R)
    S = synth.gaussian_projection(m, d, synth.SEED_S)
    ctx = tq.Context(d, m, w["key_bits"], w["value_bits"], R, S)
    cache = tq.KVCache(ctx, n_seq, T)
    scores = torch.empty((n_seq, G, T), dtype=torch.float32, device=dev)
    out = torch.empty((n_seq, G, d), dtype=torch.float32, device=dev)
    cache.workspace(G, T)

    stages = ["compress_keys", "compress_values", "scores", "attend"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cache.append_key(Kd, 0)
        if ev is not None:
            ev[1].record()
        cache.append_value(Vd, 0)
        if ev is not None:
            ev[2].record()
        cache.attention_scores(Qd, T, out=scores)
        if ev is not None:
            ev[3].record()
        cache.attend(Qd, T, out=out)
        if ev is not None:
            ev[4].record()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    stage_ms = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, s in enumerate(stages)}

    alg, units = algorithmic_bytes(w)
    stage_info = {}
    for s in stages:
        gbps = alg[s] / (stage_ms[s] * 1e-3) / 1e9
        stage_info[s] = {"ms": round(stage_ms[s], 4), "alg_bytes": int(alg[s]), "GBps": round(gbps, 1),
                         "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    stage_info["compress_keys"]["keys_per_s"] = units / (stage_ms["compress_keys"] * 1e-3)
    stage_info["compress_values"]["values_per_s"] = units / (stage_ms["compress_values"] * 1e-3)
    # matrix-core work of compress (algorithmic: 2(d^2 + m d) flops per key, 2 d^2 per value)
    stage_info["compress_keys"]["alg_TFLOPs"] = round(units * 2 * (d * d + m * d) / (stage_ms["compress_keys"] * 1e-3) / 1e12, 1)
    dom = max(stages, key=lambda s: stage_ms[s])
    roof = {"bound": "hbm", "kernel": dom, "achieved": stage_info[dom]["GBps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": stage_info[dom]["frac_hbm_peak"], "traffic": counter_traffic(dom),
            "alg_bytes": int(alg[dom])}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

    line = {
        "metric": METRIC, "value": round(units / (ms_per_step * 1e-3), 1), "unit": "keys/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w["name"], "n_seq": n_seq, "tokens_per_slot": T, "head_dim": d, "proj_dim": m,
                   "key_bits": w["key_bits"], "value_bits": w["value_bits"], "query_heads_per_kv": G,
                   "input_dtype": "f16"},
        "roofline": roof,
        "stages": stage_info,
        "cpu_baseline": cpu,
        "wall_s_timed": round(t_wall, 3),
    }
    print(json.dumps(line))
    ctx.close()


if __name__ == "__main__":
    main()
