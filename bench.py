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
# Issue roofline of compress: SIMD cycles per token of the kernels'
# instruction streams (a wave64 VALU instruction holds its SIMD 4 cycles, a
# 32x32x16 f16 MFMA 32 and a 16x16x32 one 16), from the instruction-mix
# counters of the long-context step (SQ_INSTS_VALU, SQ_INSTS_MFMA per
# 16-token tile: keys 551 VALU + 56 MFMA 32x32x16, values 412 VALU + 64 MFMA
# 16x16x32), against 256 CUs x 4 SIMDs at the 2.4 GHz peak clock.
SIMDS, PEAK_CLOCK_HZ = 1024, 2.4e9
COMPRESS_ISSUE_CYCLES = {"compress_keys": (551 * 4 / 16, 56 * 32 / 16),
                         "compress_values": (412 * 4 / 16, 64 * 16 / 16)}
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


# Sources the long-context step's kernels are built from (the counter record
# in profiles/ is valid only for these exact files).
STEP_SOURCES = ("tq_attend.h", "tq_attention.hip", "tq_compress.hip", "tq_device.h", "tq_internal.h")


def kernel_source_hash() -> str:
    """sha256 over the sources of the long-context step's kernels, in name order."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_vector_compress_amd", "csrc")
    for name in STEP_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
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


def host_threads():
    """Host cores this process may run on, and the BLAS numpy calls (the
    oracle's matrix products run there; its element-wise steps run on one
    thread)."""
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "blas_vendor": None, "blas_threads": None}
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas_vendor"] = "/".join(sorted({str(i.get("internal_api")) for i in blas}))
            info["blas_threads"] = max(int(i.get("num_threads", 1)) for i in blas)
    except Exception:
        pass
    return info


def _cpu_line(value, unit, sample, dt):
    h = host_threads()
    return {"value": value, "unit": unit, "cores": int(h["blas_threads"] or 1), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), "affinity_cores": h["affinity_cores"],
            "blas": {"vendor": h["blas_vendor"], "threads": h["blas_threads"]}}


def cpu_baseline(w, slots=16):
    """The fp64 oracle, untuned, on a bounded sample of the same workload."""
    from oracle import turboquant as O
    from kv_cache_vector_compress_amd import synth
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
    return _cpu_line(slots * T / dt, "keys/s",
                     f"slots 0-{slots - 1} of {w['n_seq']} ({slots}x{T} tokens, G={G}): compress K and V, "
                     f"scores and attend, numpy fp64; {dt:.1f} s", dt)


def cpu_baseline_qwen(K, V, Q, R, S, bits=3):
    """The oracle over a whole decode-shaped cache (all slots and tokens):
    compress K and V, scores and attend of every query head; per-token rate."""
    from oracle import turboquant as O
    d = K.shape[-1]
    beta, c = O.lloyd_max_codebook(d, bits)
    t0 = time.perf_counter()
    keys = O.compress_keys(K, R, S, beta, c)
    vals = O.compress_values(V, R, beta, c)
    O.key_scores(Q, R, S, c, keys)
    O.attend(Q, R, S, c, keys, vals, value_centroids=c)
    dt = time.perf_counter() - t0
    n = K.shape[0] * K.shape[1]
    return _cpu_line(n / dt, "tokens/s", f"the whole cache ({K.shape[0]}x{K.shape[1]} tokens, "
                     f"G={Q.shape[1]}): compress K and V, scores and attend, numpy fp64; {dt:.1f} s", dt)


def _timed(torch, fn, reps):
    """Average ms of fn() over reps calls, HIP events on the current stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _kv_device(torch, n_seq, T, d, seed, heads_cycle, dev):
    """KV-like fp16 slots generated on the host (synth.kv_slot) and moved to the device."""
    from kv_cache_vector_compress_amd import synth
    with ThreadPoolExecutor(16) as ex:
        X = np.stack(list(ex.map(lambda s: synth.kv_slot(seed, s, s % heads_cycle, T, d), range(n_seq))))
    return torch.from_numpy(X).to(dev)


def bench_qwen_decode(args):
    """Qwen2.5-3B-shaped decode (36 layers x 2 KV heads x 8192 tokens, 16
    query heads = GQA 8:1, 3-bit keys m=64 and values): (i) per-layer latency
    of appending one token's K and V and attending over 8192 tokens; (ii) all
    36 layers' scores and attend in one call each, cache-resident (warm) and
    rotating over 8 cache copies (cold)."""
    import torch
    from kv_cache_vector_compress_amd import synth, tq
    w = synth.QWEN_DECODE
    d, m, T, G, n_seq = w.d, w.m, w.n_tok, w.G, w.n_seq
    dev = torch.device("cuda:0")
    R, S = synth.haar_rotation(d), synth.gaussian_projection(m, d)
    ctx = tq.Context(d, m, 3, 3, R, S)
    Kh, Vh, Qh = gen_inputs(n_seq, T, d, G, n_seq)
    Qh = synth.workload_queries(w)
    K, V, Q = torch.from_numpy(Kh).to(dev), torch.from_numpy(Vh).to(dev), torch.from_numpy(Qh).to(dev)
    copies = 8
    caches = [tq.KVCache(ctx, n_seq, T) for _ in range(copies)]
    for c in caches:
        c.append_key(K, 0)
        c.append_value(V, 0)
    sc = torch.empty((n_seq, G, T), dtype=torch.float32, device=dev)
    out = torch.empty((n_seq, G, d), dtype=torch.float32, device=dev)
    caches[0].workspace(G, T)
    reps = max(args.steps, 20)
    for _ in range(max(args.warmup, 1)):  # first launches (code loading) stay out of the timed loops
        caches[0].attention_scores(Q, T, out=sc)
        caches[0].attend(Q, T, out=out)
    torch.cuda.synchronize()
    warm_s = _timed(torch, lambda: caches[0].attention_scores(Q, T, out=sc), reps)
    warm_a = _timed(torch, lambda: caches[0].attend(Q, T, out=out), reps)
    it = iter(range(10 ** 9))
    cold_s = _timed(torch, lambda: caches[next(it) % copies].attention_scores(Q, T, out=sc), reps)
    cold_a = _timed(torch, lambda: caches[next(it) % copies].attend(Q, T, out=out), reps)
    # one layer: 2 KV slots, 8191 cached tokens, append token 8191 and attend over 8192
    layer = tq.KVCache(ctx, 2, T)
    layer.append_key(K[:2, :T - 1].contiguous(), 0)
    layer.append_value(V[:2, :T - 1].contiguous(), 0)
    k1, v1, q1 = K[:2, T - 1:].contiguous(), V[:2, T - 1:].contiguous(), Q[:2].contiguous()
    o1 = torch.empty((2, G, d), dtype=torch.float32, device=dev)
    layer.workspace(G, T)

    def one_layer():
        layer.append_key(k1, T - 1)
        layer.append_value(v1, T - 1)
        layer.attend(q1, T, out=o1)
    for _ in range(max(args.warmup, 1)):
        one_layer()
    torch.cuda.synchronize()
    lat = _timed(torch, one_layer, reps)
    # the same three calls captured once in a HIP graph and replayed: the
    # device-side latency without per-call Python and launch overhead; every
    # replay is checked against the eager result
    one_layer()
    torch.cuda.synchronize()
    ref_o = o1.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        one_layer()  # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            one_layer()
    torch.cuda.synchronize()
    graph_ok = True
    for _ in range(3):
        o1.zero_()
        graph.replay()
        torch.cuda.synchronize()
        graph_ok &= bool(torch.equal(o1, ref_o))
        one_layer()
        torch.cuda.synchronize()
    lat_graph = _timed(torch, graph.replay, reps)
    # the same step through tq_decode_step: the appends and the query
    # preparation in one launch, then the attention's two
    def one_layer_fused():
        layer.decode_step(k1, v1, q1, T - 1, out=o1)
    for _ in range(max(args.warmup, 1)):
        one_layer_fused()
    torch.cuda.synchronize()
    lat_fused = _timed(torch, one_layer_fused, reps)
    fused_o = o1.clone()
    graph_f = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        one_layer_fused()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph_f, stream=side):
            one_layer_fused()
    torch.cuda.synchronize()
    for _ in range(3):
        o1.zero_()
        graph_f.replay()
        torch.cuda.synchronize()
        graph_ok &= bool(torch.equal(o1, fused_o))
    lat_fused_graph = _timed(torch, graph_f.replay, reps)
    fused_vs_calls = float((fused_o - ref_o).norm() / ref_o.norm())
    b_sc = n_seq * T * (tq.key_record_bytes(ctx.cfg) + 4 * G)
    b_at = n_seq * T * (tq.key_record_bytes(ctx.cfg) + tq.value_block_bytes(ctx.cfg) / 128)
    gb = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 1)
    line = {"metric": "per-layer decode latency (append 1 token K+V, attend 8192) and 36-layer score/attend HBM GB/s",
            "value": round(lat * 1e3, 2), "unit": "us/layer", "higher_is_better": False, "n_gpus": 1,
            "graph_replay_us_per_layer": round(lat_graph * 1e3, 2), "graph_replays_match_eager": graph_ok,
            "decode_step_us_per_layer": round(lat_fused * 1e3, 2),
            "decode_step_graph_us_per_layer": round(lat_fused_graph * 1e3, 2),
            "decode_step_vs_three_calls_rel": fused_vs_calls,
            "data": "synthetic", "dtype": "f16",
            "config": {"workload": w.name, "n_seq": n_seq, "tokens_per_slot": T, "head_dim": d, "proj_dim": m,
                       "key_bits": 3, "value_bits": 3, "query_heads_per_kv": G},
            "all_layers": {"scores_warm": {"ms": round(warm_s, 4), "GBps": gb(b_sc, warm_s)},
                           "attend_warm": {"ms": round(warm_a, 4), "GBps": gb(b_at, warm_a)},
                           "scores_cold": {"ms": round(cold_s, 4), "GBps": gb(b_sc, cold_s)},
                           "attend_cold": {"ms": round(cold_a, 4), "GBps": gb(b_at, cold_a)},
                           "alg_bytes": {"scores": int(b_sc), "attend": int(b_at)},
                           "cold_copies": copies, "hbm_peak_GBps": HBM_PEAK_GBPS}}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_qwen(Kh, Vh, Qh, R, S)
    print(json.dumps(line))
    ctx.close()


def bench_bit_sweep(args):
    """Bit-width sweep on the Qwen decode shape (72 slots x 8192 tokens): for
    2-, 3- and 4-bit keys (m=64) and values, and for the bit budget variant
    with (b - 1)-bit key codes at b = 1..4 (0-bit keys are QJL signs only),
    bulk compression rate, score GB/s, and fidelity of the attention weights
    against exact fp16 attention
    (cosine of the softmax rows and top-1 match, evaluated with torch on the
    GPU), with the plain queries and with queries rescaled to a logit
    standard deviation of 2 (a diagnostic: plain queries give nearly uniform
    attention)."""
    import torch
    from kv_cache_vector_compress_amd import synth, tq
    w = synth.QWEN_DECODE
    d, m, T, G, n_seq = w.d, w.m, w.n_tok, w.G, w.n_seq
    dev = torch.device("cuda:0")
    R, S = synth.haar_rotation(d), synth.gaussian_projection(m, d)
    Kh, Vh, _ = gen_inputs(n_seq, T, d, G, n_seq)
    Qh = synth.workload_queries(w)
    K, V, Q = torch.from_numpy(Kh).to(dev), torch.from_numpy(Vh).to(dev), torch.from_numpy(Qh).to(dev)
    exact = torch.matmul(Q.float(), K.float().transpose(1, 2).contiguous())   # (n_seq, G, T)
    scale = 1.0 / d ** 0.5
    rescale = 2.0 / float((exact * scale).std())
    reps = max(args.steps, 10)
    res = {}
    # b-bit keys (b-bit codes plus m QJL signs) at 2-4 bits, then the bit
    # budget variant: (b - 1)-bit codes plus the signs at b = 1..4 (key_bits
    # 0 at b = 1 is pure QJL), values at b bits
    for b, kb in ((2, 2), (3, 3), (4, 4), (1, 0), (2, 1), (3, 2), (4, 3)):
        ctx = tq.Context(d, m, kb, b, R, S)
        cache = tq.KVCache(ctx, n_seq, T)
        sc = torch.empty((n_seq, G, T), dtype=torch.float32, device=dev)
        cache.workspace(G, T)
        cache.append_key(K, 0)  # first launches stay out of the timed loops
        cache.append_value(V, 0)
        cache.attention_scores(Q, T, out=sc)
        torch.cuda.synchronize()
        ck = _timed(torch, lambda: cache.append_key(K, 0), reps)
        cv = _timed(torch, lambda: cache.append_value(V, 0), reps)
        ts = _timed(torch, lambda: cache.attention_scores(Q, T, out=sc), reps)
        fid = {}
        for tag, f in (("plain", 1.0), ("logit_std_2", rescale)):
            pe = torch.softmax(exact * (scale * f), dim=-1)
            pq = torch.softmax(sc * (scale * f), dim=-1)
            cos = torch.nn.functional.cosine_similarity(pe, pq, dim=-1)
            top1 = (pe.argmax(-1) == pq.argmax(-1)).float().mean()
            fid[tag] = {"cosine_mean": round(float(cos.mean()), 5), "cosine_min": round(float(cos.min()), 5),
                        "top1": round(float(top1), 4)}
        b_sc = n_seq * T * (tq.key_record_bytes(ctx.cfg) + 4 * G)
        res[f"{b}bit" if kb == b else f"budget_{b}bit_keys{kb}"] = {
                          "key_record_bytes": tq.key_record_bytes(ctx.cfg),
                          "compress_keys_per_s": round(n_seq * T / (ck * 1e-3), 1),
                          "compress_values_per_s": round(n_seq * T / (cv * 1e-3), 1),
                          "scores_ms": round(ts, 4), "scores_GBps": round(b_sc / (ts * 1e-3) / 1e9, 1),
                          "fidelity": fid}
        ctx.close()
        if not args.no_cpu_baseline and kb == b:
            print(f"[bench] cpu baseline (oracle) {b} bits", file=sys.stderr, flush=True)
            res[f"{b}bit"]["cpu_baseline"] = cpu_baseline_qwen(Kh, Vh, Qh, R, S, bits=b)
    line = {"metric": "bit-width sweep: compress keys/s, score GB/s, attention cosine and top-1 vs fp16",
            "value": res["3bit"]["compress_keys_per_s"], "unit": "keys/s (3-bit)", "higher_is_better": True,
            "n_gpus": 1, "data": "synthetic", "dtype": "f16",
            "config": {"workload": "bit_sweep_" + w.name, "n_seq": n_seq, "tokens_per_slot": T, "head_dim": d,
                       "proj_dim": m, "query_heads_per_kv": G, "logit_rescale": round(rescale, 3)},
            "sweep": res}
    print(json.dumps(line))


def bench_vector_search(args):
    """Vector search: 2,000,000 unit-norm fp32 vectors at d = 1024 (half
    isotropic Gaussian, half a 64-cluster mixture normalise(mu_c + 0.3 g /
    sqrt(d)), generated on the device with a seeded torch generator), 4-bit
    keys with proj_dim 512, 512 unit-norm queries: compress rate, the fused
    top-10 search (tq_topk_scores: no score matrix) and, beside it, the
    materialised scores for all 512 queries; recall@10 of the fused top-10
    against brute-force fp32 inner products (torch, evaluation only)."""
    import torch
    from kv_cache_vector_compress_amd import synth, tq
    d, m, b, N, G = 1024, 512, 4, 2_000_000, 512
    dev = torch.device("cuda:0")
    R, S = synth.haar_rotation(d), synth.gaussian_projection(m, d)
    ctx = tq.Context(d, m, b, b, R, S)
    X, Q = synth.vector_search_device(torch, N, d, G, dev)
    cache = tq.KVCache(ctx, 1, -(-N // 128) * 128)
    sc = torch.empty((1, G, N), dtype=torch.float32, device=dev)
    cache.workspace(G, N)
    reps = 3
    cache.append_key(X, 0)
    cache.attention_scores(Q, N, out=sc)
    top_s, top_i = cache.topk(Q, N, 10)
    tc = _timed(torch, lambda: cache.append_key(X, 0), reps)
    ts = _timed(torch, lambda: cache.attention_scores(Q, N, out=sc), reps)
    tk = _timed(torch, lambda: cache.topk(Q, N, 10), reps)
    top_s, top_i = cache.topk(Q, N, 10)
    torch.cuda.synchronize()
    rec = []
    for q0 in range(0, G, 64):
        ex = torch.matmul(Q[0, q0:q0 + 64], X[0].T)
        t_true = ex.topk(10, dim=1).indices
        t_est = top_i[0, q0:q0 + 64].long()
        rec.append(float((t_true[:, :, None] == t_est[:, None, :]).any(-1).float().mean()))
    executed = N * (2 * d * d * 3 + 2 * m * d * 3)   # split-fp16 MFMA flops actually issued (fp32 inputs)
    line = {"metric": "vector search: vectors compressed/s, score rate for 512 queries, recall@10 vs fp32",
            "value": round(N / (tc * 1e-3), 1), "unit": "vectors/s", "higher_is_better": True, "n_gpus": 1,
            "data": "synthetic", "dtype": "f32",
            "config": {"workload": "vector_search_2M_d1024", "n_vectors": N, "head_dim": d, "proj_dim": m,
                       "key_bits": b, "queries": G},
            "compress_ms": round(tc, 3), "topk10_ms": round(tk, 3), "scores_ms": round(ts, 3),
            "topk10_read_GBps": round(N * tq.key_record_bytes(ctx.cfg) / (tk * 1e-3) / 1e9, 1),
            "compress_mfma": {"achieved_TFLOPs": round(executed / (tc * 1e-3) / 1e12, 1), "peak_TFLOPs": FP16_MFMA_PEAK_TFLOPS,
                              "frac": round(executed / (tc * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)},
            "scores_alg_TFLOPs": round(N * G * 2 * (d + m) / (ts * 1e-3) / 1e12, 1),
            "topk10_alg_TFLOPs": round(N * G * 2 * (d + m) / (tk * 1e-3) / 1e12, 1),
            "recall_at_10": round(float(np.mean(rec)), 4)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        from oracle import turboquant as O
        n_cpu = 131072
        Xs = X[0, :n_cpu].cpu().numpy()[None]
        Qs = Q.cpu().numpy()
        beta, c = O.lloyd_max_codebook(d, b)
        t0 = time.perf_counter()
        keys = O.compress_keys(Xs, R, S, beta, c)
        O.key_scores(Qs, R, S, c, keys)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = _cpu_line(n_cpu / dt, "vectors/s", f"slice: the first {n_cpu} of {N} vectors, all "
                                         f"{G} queries: compress and scores, numpy fp64; {dt:.1f} s", dt)
    print(json.dumps(line))
    ctx.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--workload", default="long_context",
                    choices=["long_context", "qwen_decode", "bit_sweep", "vector_search"],
                    help="long_context (default): the full hot-path step; the others print one extra "
                         "JSON line for the decode, bit-width sweep and vector-search configurations")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path is single-GPU); --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)
    if args.workload != "long_context":
        {"qwen_decode": bench_qwen_decode, "bit_sweep": bench_bit_sweep,
         "vector_search": bench_vector_search}[args.workload](args)
        return

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
    # Matrix-core work of compress against the fp16 MFMA peak: algorithmic
    # flops (2(d^2 + m d) per key, 2 d^2 per value) and the flops the split-
    # fp16 arithmetic executes (rotation R_hi k + R_lo k: 2 x 2 d^2; projection
    # S_hi r_hi + S_lo r_hi + S_hi r_lo: 3 x 2 m d; values 2 x 2 d^2).
    for s_, alg_f, exe_f in (("compress_keys", 2 * (d * d + m * d), 2 * 2 * d * d + 3 * 2 * m * d),
                             ("compress_values", 2 * d * d, 2 * 2 * d * d)):
        sec = stage_ms[s_] * 1e-3
        stage_info[s_]["mfma"] = {
            "alg_TFLOPs": round(units * alg_f / sec / 1e12, 1),
            "executed_TFLOPs": round(units * exe_f / sec / 1e12, 1),
            "peak_TFLOPs": FP16_MFMA_PEAK_TFLOPS,
            "alg_frac": round(units * alg_f / sec / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
            "executed_frac": round(units * exe_f / sec / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)}
        # issue roofline: the VALU and MFMA cycles of the instruction stream
        # spread over every SIMD at the peak clock, overlapped (the larger of
        # the two) or back to back (their sum)
        valu_c, mfma_c = COMPRESS_ISSUE_CYCLES[s_]
        t_valu = units * valu_c / SIMDS / PEAK_CLOCK_HZ * 1e3
        t_mfma = units * mfma_c / SIMDS / PEAK_CLOCK_HZ * 1e3
        stage_info[s_]["issue_roofline"] = {
            "valu_ms": round(t_valu, 4), "mfma_ms": round(t_mfma, 4),
            "overlapped_ms": round(max(t_valu, t_mfma), 4), "additive_ms": round(t_valu + t_mfma, 4),
            "frac_overlapped": round(max(t_valu, t_mfma) / stage_ms[s_], 4),
            "frac_additive": round((t_valu + t_mfma) / stage_ms[s_], 4)}
    dom = max(stages, key=lambda s: stage_ms[s])
    roof = {"bound": "hbm", "kernel": dom, "achieved": stage_info[dom]["GBps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": stage_info[dom]["frac_hbm_peak"], "traffic": counter_traffic(dom),
            "alg_bytes": int(alg[dom])}
    if "issue_roofline" in stage_info[dom]:
        # the bound that binds compress on this chip: SIMD issue, beside HBM
        roof["issue_roofline"] = stage_info[dom]["issue_roofline"]

    # Practical HBM ceiling beside the theoretical peak: a plain read stream
    # over the 2 GiB key input, and the same with writes interleaved 4:1 (the
    # read/write mix of the score kernel and of compress), each the best over
    # grids of 8 to 64 waves per compute unit and over 4, 8 or 16 loads in
    # flight per lane, plain or nontemporal.  Each stage is also reported
    # against the stream with its own mix.  A torch sum over the same bytes
    # is an independent check of the read figure.
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    dst = torch.empty(Kd.numel() * Kd.element_size() // 16, dtype=torch.float32, device=dev)
    stream_ms, stream_cfg, sweep = {}, {}, []
    nbytes_k = Kd.numel() * Kd.element_size()
    for name, d_ in (("read", None), ("read4_write1", dst)):
        for nl, nt in ((4, False), (8, True), (16, True)):
            for wpc in (8, 16, 32, 64):
                for _ in range(2):
                    tq.hbm_stream(Kd, d_, sink, wpc, loads_in_flight=nl, nontemporal=nt)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    tq.hbm_stream(Kd, d_, sink, wpc, loads_in_flight=nl, nontemporal=nt)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 10
                sweep.append({"mix": name, "loads_in_flight": nl, "nontemporal": nt, "waves_per_cu": wpc,
                              "GBps": round((nbytes_k * (1.25 if d_ is not None else 1.0)) / (ms * 1e-3) / 1e9, 1)})
                if name not in stream_ms or ms < stream_ms[name]:
                    stream_ms[name] = ms
                    stream_cfg[name] = {"waves_per_cu": wpc, "loads_in_flight": nl, "nontemporal": nt}
    del dst
    nbytes = Kd.numel() * Kd.element_size()
    flat = Kd.view(-1).view(torch.float32)  # (the words' values do not matter to the timing)
    torch_ms = min(_timed(torch, lambda: flat.sum(), 5) for _ in range(2))
    hbm_stream = {"read_GBps": round(nbytes / (stream_ms["read"] * 1e-3) / 1e9, 1),
                  "read4_write1_GBps": round(nbytes * 1.25 / (stream_ms["read4_write1"] * 1e-3) / 1e9, 1),
                  "torch_sum_read_GBps": round(nbytes / (torch_ms * 1e-3) / 1e9, 1),
                  "bytes_read": nbytes, "best": stream_cfg, "sweep": sweep}
    mix = {"compress_keys": "read4_write1_GBps", "compress_values": "read4_write1_GBps",
           "scores": "read4_write1_GBps", "attend": "read_GBps"}
    for s_ in stages:
        stage_info[s_]["frac_of_stream"] = round(stage_info[s_]["GBps"] / hbm_stream[mix[s_]], 4)

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
        "hbm_stream": hbm_stream,
        "stages": stage_info,
        "cpu_baseline": cpu,
        "wall_s_timed": round(t_wall, 3),
    }
    print(json.dumps(line))
    ctx.close()


if __name__ == "__main__":
    main()
