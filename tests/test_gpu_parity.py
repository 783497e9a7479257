"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case uses seeded synthetic inputs from kv_cache_vector_compress_amd.synth;
the oracle gets the same arrays.  Acceptance rules: tests/parity_util.py.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import turboquant as O
from kv_cache_vector_compress_amd import synth, tq
from tests import parity_util as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[parity]", *a, flush=True)


def make_ctx(d=128, m=64, kb=3, vb=3):
    R = synth.haar_rotation(d, synth.SEED_R)
    S = synth.gaussian_projection(m, d, synth.SEED_S)
    return tq.Context(d, m, kb, vb, R, S), R, S


def run_case(K, V, Q, kb=3, vb=3, m=64, capacity=None, chunks=None, n_tokens=None, scale=0.0,
             check_attend=True):
    """Append K/V (np arrays (n_seq, T, d)) in the given chunks, then score and
    attend with Q (n_seq, G, d); compare every output with the oracle."""
    n_seq, T, d = K.shape
    G = Q.shape[1]
    cap = capacity or -(-T // 128) * 128
    ctx, R, S = make_ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, cap)
    chunks = chunks or [T]
    pos = 0
    for n in chunks:
        kt = torch.from_numpy(np.ascontiguousarray(K[:, pos:pos + n])).cuda()
        vt = torch.from_numpy(np.ascontiguousarray(V[:, pos:pos + n])).cuda()
        cache.append_key(kt, pos)
        cache.append_value(vt, pos)
        pos += n
    assert pos == T
    torch.cuda.synchronize()
    nt = n_tokens or T

    kbeta, kc = O.lloyd_max_codebook(d, kb)
    vbeta, vc = O.lloyd_max_codebook(d, vb)
    ref_k = O.compress_keys(K, R, S, kbeta, kc)
    ref_v = O.compress_values(V, R, vbeta, vc)
    gk = P.unpack_gpu_keys(cache, d, m, kb, T)
    gv = P.unpack_gpu_values(cache, d, vb, T)
    st = P.check_keys(gk, ref_k, kbeta, S, kc)
    flip_tok = st.pop("flip_tokens")
    vst = P.check_values(gv, ref_v, vbeta)
    vflip = vst.pop("flip_tokens")
    st.update({"v_" + k: v for k, v in vst.items()})

    qt = torch.from_numpy(np.ascontiguousarray(Q)).cuda()
    sc = cache.attention_scores(qt, nt).cpu().numpy()
    qn = np.linalg.norm(Q.astype(np.float64), axis=-1)
    kn = np.linalg.norm(K.astype(np.float64), axis=-1)[:, :nt]
    # (a) score kernel against the oracle evaluated on the GPU's own codes
    gk_nt = {k: v[:, :nt] for k, v in gk.items()}
    ref_on_gpu_codes = O.key_scores(Q, R, S, kc, gk_nt)
    st["score_vs_gpu_codes"] = P.check_scores(sc, ref_on_gpu_codes, qn, kn)
    # (b) end to end against the oracle's own codes
    ref_k_nt = {k: v[:, :nt] for k, v in ref_k.items()}
    ref_scores = O.key_scores(Q, R, S, kc, ref_k_nt)
    st["score_end_to_end"] = P.check_scores(sc, ref_scores, qn, kn, skip_tokens=flip_tok[:, :nt])
    if check_attend:
        out = cache.attend(qt, nt, scale=scale).cpu().numpy()
        sc_ = None if scale <= 0 else scale
        ref_v_nt = {k: v[:, :nt] for k, v in ref_v.items()}
        gv_nt = {k: v[:, :nt] for k, v in gv.items()}
        on_gpu = O.attend(Q, R, S, kc, gk_nt, gv_nt, scale=sc_, value_centroids=vc)
        e2e = O.attend(Q, R, S, kc, ref_k_nt, ref_v_nt, scale=sc_, value_centroids=vc)
        st["attend_rel"], st["attend_e2e"], st["attend_flip_slots"] = P.check_attend_two_level(
            out, on_gpu, e2e, (flip_tok | vflip)[:, :nt])
    ctx.close()
    return st


def test_tiny_unit_gaussian_fp32():
    """Tiny case: 1 slot, d=128, 3-bit, m=64, 1024 unit fp32 keys/values, 4 queries."""
    w = synth.TINY
    K, V, Q = synth.workload_keys(w), synth.workload_values(w), synth.workload_queries(w)
    _say("tiny", K.shape, Q.shape)
    st = run_case(K, V, Q)
    _say(st)


@pytest.mark.parametrize("kb,vb,m", [(1, 1, 64), (2, 2, 64), (3, 3, 64), (4, 4, 64), (3, 2, 128), (2, 4, 128)])
def test_bits_and_proj_dim_fp16_ragged(kb, vb, m):
    """fp16 KV-like inputs, ragged token count (several tiles and a tail)."""
    d, T, n_seq, G = 128, 1000, 3, 8
    K = np.stack([synth.kv_slot(synth.SEED_K, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(synth.SEED_V, s, s, T, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(synth.SEED_Q, s, s, G, d) for s in range(n_seq)])
    _say("bits", kb, vb, m)
    _say(run_case(K, V, Q, kb=kb, vb=vb, m=m))


@pytest.mark.parametrize("G", [1, 2, 4, 5, 7, 8, 9, 12, 15, 16])
def test_query_group_sizes(G):
    d, T, n_seq = 128, 515, 2
    K = np.stack([synth.kv_slot(10, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(11, s, s, T, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(12, s, s, G, d) for s in range(n_seq)]) * np.float16(3.0)
    _say("G", G)
    _say(run_case(K, V, Q))


def test_streaming_appends_unaligned():
    """Prefill 300 tokens, then single-token decode appends, then a ragged
    chunk: blocks shared by several appends must keep earlier codes."""
    d, n_seq, G = 128, 2, 4
    chunks = [300, 1, 1, 1, 1, 1, 77, 130, 1]
    T = sum(chunks)
    K = np.stack([synth.kv_slot(20, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(21, s, s, T, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(22, s, s, G, d) for s in range(n_seq)])
    _say("streaming", chunks)
    _say(run_case(K, V, Q, chunks=chunks, capacity=1024))


def test_partial_token_window_and_scale():
    """Attention over the first n_tokens only (not a multiple of 16), custom scale."""
    d, T, n_seq, G = 128, 700, 2, 8
    K = np.stack([synth.kv_slot(30, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(31, s, s, T, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(32, s, s, G, d) for s in range(n_seq)])
    _say("window")
    _say(run_case(K, V, Q, n_tokens=509, scale=0.3))


@pytest.mark.parametrize("kb,vb,dtype", [(3, 3, np.float16), (4, 4, np.float16), (2, 1, np.float32),
                                         (1, 2, np.float32)])
def test_zero_and_single_token(kb, vb, dtype):
    """Zero key/value rows are encoded as direction 0 (every cell L/2 - 1)
    and score 0, in bulk appends of each code width and input type; a cache
    of one token attends to exactly that token's dequantised value."""
    d, T, n_seq, G = 128, 40, 1, 4
    K = synth.kv_slot(40, 0, 0, T, d, dtype=dtype)[None].copy()
    V = synth.kv_slot(41, 0, 0, T, d, dtype=dtype)[None].copy()
    K[0, 5] = 0
    V[0, 7] = 0
    V[0, 33] = 0
    Q = synth.kv_slot(42, 0, 0, G, d, dtype=dtype)[None]
    _say("zeros", kb, vb, np.dtype(dtype).name)
    _say(run_case(K, V, Q, kb=kb, vb=vb))
    _say(run_case(K[:, :1], V[:, :1], Q, kb=kb, vb=vb))


def test_fp32_inputs_kv_like():
    d, T, n_seq, G = 128, 333, 2, 4
    K = np.stack([synth.kv_slot(50, s, s, T, d, dtype=np.float32) for s in range(n_seq)]) * 7.5
    V = np.stack([synth.kv_slot(51, s, s, T, d, dtype=np.float32) for s in range(n_seq)]) * 0.01
    Q = np.stack([synth.kv_slot(52, s, s, G, d, dtype=np.float32) for s in range(n_seq)])
    _say("fp32 kv-like")
    _say(run_case(K.astype(np.float32), V.astype(np.float32), Q.astype(np.float32)))


def test_qwen_decode_shape_full():
    """Qwen2.5-3B-shaped decode step at full size: 36 layers x 2 KV heads
    (72 slots) x 8192 fp16 tokens, 16 query heads (GQA 8:1), 3-bit keys
    (m=64) and values, every output compared with the oracle."""
    w = synth.QWEN_DECODE
    K, V, Q = synth.workload_keys(w), synth.workload_values(w), synth.workload_queries(w)
    _say("qwen full", K.shape, Q.shape)
    _say(run_case(K, V, Q))


def test_long_context_full_size_sampled():
    """The benchmark workload at full size, in the launch configuration
    bench.py times: 8 sequences x 8 KV heads (64 slots) x 131072 fp16 tokens,
    3-bit keys (m=64) and values, 4 query heads per KV head, one
    tq_append_key / tq_append_value / tq_attention_scores / tq_attend call
    each over the whole cache.  The oracle recomputes sampled tokens of four
    slots one by one (codes, signs, norms, gamma, scores) and the full
    attention of one slot."""
    from concurrent.futures import ThreadPoolExecutor
    w = synth.LONG_CONTEXT
    n_seq, T, d, m, G = w.n_seq, w.n_tok, w.d, w.m, w.G
    _say("long context: generating", (n_seq, T, d))
    with ThreadPoolExecutor(8) as ex:
        K = np.stack(list(ex.map(lambda s: synth.kv_slot(synth.SEED_K, s, w.head_of_slot(s), T, d), range(n_seq))))
        V = np.stack(list(ex.map(lambda s: synth.kv_slot(synth.SEED_V, s, w.head_of_slot(s), T, d), range(n_seq))))
    Q = synth.workload_queries(w)
    ctx, R, S = make_ctx(d, m, 3, 3)
    cache = tq.KVCache(ctx, n_seq, T)
    kd, vd, qd = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), torch.from_numpy(Q).cuda()
    cache.append_key(kd, 0)
    cache.append_value(vd, 0)
    sc = cache.attention_scores(qd, T).cpu().numpy()
    out = cache.attend(qd, T).cpu().numpy()
    torch.cuda.synchronize()
    del kd, vd
    kw_all, vw_all = cache.key_words(), cache.value_words()
    _say("long context: GPU pass done")
    beta, c = O.lloyd_max_codebook(d, 3)
    rng = np.random.default_rng(2024)
    for slot in (0, 21, 42, 63):
        toks = np.unique(np.concatenate([rng.choice(T, 1024, replace=False), np.arange(T - 16, T)]))
        ks, vs = K[slot:slot + 1, toks], V[slot:slot + 1, toks]
        ref_k = O.compress_keys(ks, R, S, beta, c)
        ref_v = O.compress_values(vs, R, beta, c)
        gk = O.unpack_keys(kw_all[slot:slot + 1, toks], d, m, 3)
        gv_all = O.unpack_values(vw_all[slot:slot + 1], d, 3, n_tokens=T)
        gv = {k: v[:, toks] for k, v in gv_all.items()}
        st = P.check_keys(gk, ref_k, beta, S, c)
        flips = st.pop("flip_tokens")
        vst = P.check_values(gv, ref_v, beta)
        vst.pop("flip_tokens")
        st.update({"v_" + k: v for k, v in vst.items()})
        qn = np.linalg.norm(Q[slot:slot + 1].astype(np.float64), axis=-1)
        kn = np.linalg.norm(ks.astype(np.float64), axis=-1)
        g_sc = sc[slot:slot + 1][:, :, toks]
        st["score"] = P.check_scores(g_sc, O.key_scores(Q[slot:slot + 1], R, S, c, ref_k), qn, kn,
                                     skip_tokens=flips)
        _say("long context slot", slot, st)
    slot = 42
    ref_k = O.compress_keys(K[slot:slot + 1], R, S, beta, c)
    ref_v = O.compress_values(V[slot:slot + 1], R, beta, c)
    gk = O.unpack_keys(kw_all[slot:slot + 1], d, m, 3)
    gv = O.unpack_values(vw_all[slot:slot + 1], d, 3, n_tokens=T)
    kst = P.check_keys(gk, ref_k, beta, S, c)
    vst = P.check_values(gv, ref_v, beta)
    flips = kst.pop("flip_tokens") | vst.pop("flip_tokens")
    on_gpu = O.attend(Q[slot:slot + 1], R, S, c, gk, gv, value_centroids=c)
    e2e = O.attend(Q[slot:slot + 1], R, S, c, ref_k, ref_v, value_centroids=c)
    _say("long context attend slot", slot, kst, vst,
         P.check_attend_two_level(out[slot:slot + 1], on_gpu, e2e, flips))
    ctx.close()


# ---------------------------------------------------------------------------
# general shapes: head_dim a multiple of 64 up to 1024, proj_dim a multiple
# of 32 up to 512 (tiled rotation / projection kernels; a head_dim of
# 128 n + 64 ends in a half code chunk, a proj_dim of 64 n + 32 in a half
# sign block)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,m,kb,vb,dtype,G", [
    (256, 128, 3, 3, np.float16, 4),
    (128, 256, 2, 4, np.float16, 8),
    (512, 192, 1, 2, np.float32, 3),
    (384, 64, 4, 3, np.float16, 40),
    (1024, 512, 4, 4, np.float32, 16),
    # head_dim 64 with its proj_dim 32 (d / 2), 2- to 4-bit codes, fp16 and fp32
    (64, 32, 2, 2, np.float16, 4),
    (64, 32, 2, 3, np.float32, 8),
    (64, 32, 3, 3, np.float16, 8),
    (64, 32, 3, 4, np.float32, 4),
    (64, 32, 4, 4, np.float16, 16),
    (64, 32, 4, 2, np.float32, 20),    # scores only (G > 16)
    (64, 64, 1, 1, np.float16, 2),
    (192, 96, 3, 3, np.float16, 5),    # a full and a half chunk, a full and a half sign block
    (320, 160, 2, 4, np.float32, 12),
    (128, 32, 3, 3, np.float16, 8),    # head_dim 128 with a single half sign block
    (960, 480, 4, 1, np.float32, 3),
    # many head groups (the blocked score kernel: head groups 4 at a time)
    (192, 96, 3, 3, np.float16, 130),  # 9 live groups of a 16-group bucket, half chunk, half sign block
    (128, 64, 2, 2, np.float32, 100),  # head_dim 128 beyond 16 query heads
])
def test_general_shapes_ragged_chunks(d, m, kb, vb, dtype, G):
    """Codes, signs, norms, gamma of keys and values, scores and (G <= 16)
    attention on the general path; appended in unaligned chunks (partial
    value blocks)."""
    n_seq, T = 2, 700
    K = np.stack([synth.kv_slot(60 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(61 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(62 + d, s, s, G, d, dtype=dtype) for s in range(n_seq)])
    _say("general", (d, m, kb, vb, dtype.__name__, G))
    _say(run_case(K, V, Q, kb=kb, vb=vb, m=m, chunks=[130, 1, 300, 269], check_attend=G <= 16))


@pytest.mark.parametrize("T,G", [(333, 136), (18, 129)])
def test_many_head_scores_ragged_tokens(T, G):
    """The blocked score kernel with a token count that is not a multiple of
    4 (per-score stores) and a last wave holding fewer than 4 tiles; scores
    against the oracle."""
    d, m, kb, n_seq = 256, 128, 4, 2
    K = np.stack([synth.kv_slot(140, s, s, T, d, dtype=np.float16) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(141, s, s, T, d, dtype=np.float16) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(142, s, s, G, d, dtype=np.float16) for s in range(n_seq)])
    _say("many heads, ragged tokens", (T, G))
    _say(run_case(K, V, Q, kb=kb, vb=2, m=m, chunks=[T], check_attend=False))


def test_vector_search_shape():
    """The vector-search configuration's shape at a reduced count: unit-norm
    fp32 database rows (Gaussian plus cluster mixture) at d = 1024, 4-bit keys
    with proj_dim 512, scored against 64 and against 512 queries."""
    d, m, b = 1024, 512, 4
    N = 3000
    X = synth.vector_database(N, d, seed=5)[None]
    Qd = synth.vector_database(512, d, seed=6)[None]
    ctx, R, S = make_ctx(d, m, b, b)
    cache = tq.KVCache(ctx, 1, -(-N // 128) * 128)
    cache.append_key(torch.from_numpy(X).cuda(), 0)
    beta, c = O.lloyd_max_codebook(d, b)
    ref = O.compress_keys(X, R, S, beta, c)
    gk = P.unpack_gpu_keys(cache, d, m, b, N)
    st = P.check_keys(gk, ref, beta, S, c)
    flips = st.pop("flip_tokens")
    kn = np.linalg.norm(X.astype(np.float64), axis=-1)
    for G in (64, 512):
        Q = Qd[:, :G]
        sc = cache.attention_scores(torch.from_numpy(np.ascontiguousarray(Q)).cuda(), N).cpu().numpy()
        qn = np.linalg.norm(Q.astype(np.float64), axis=-1)
        st[f"score_G{G}"] = P.check_scores(sc, O.key_scores(Q, R, S, c, ref), qn, kn, skip_tokens=flips)
    _say("vector search shape", st)
    ctx.close()


def test_general_attend_long_range_scale():
    """General-shape attention over several 128-token ranges per slot (the
    split-and-merge path) with a non-default scale, d = 256, m = 128."""
    d, m, T, n_seq, G = 256, 128, 3000, 2, 8
    K = np.stack([synth.kv_slot(70, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(71, s, s, T, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(72, s, s, G, d) for s in range(n_seq)])
    _say("general attend", (d, m, T))
    _say(run_case(K, V, Q, m=m, n_tokens=2900, scale=0.11))


# ---------------------------------------------------------------------------
# argument errors: documented code, nothing written
# ---------------------------------------------------------------------------

def test_error_paths_leave_buffers_untouched():
    ctx, R, S = make_ctx()
    cache = tq.KVCache(ctx, 2, 256)
    canary = 0x5A5A5A5A
    cache.key_records.fill_(canary)
    cache.value_blocks.fill_(canary)
    k = torch.zeros((2, 10, 128), dtype=torch.float16, device="cuda")
    q = torch.zeros((2, 4, 128), dtype=torch.float16, device="cuda")

    def expect(code, fn):
        with pytest.raises(tq.TQError) as e:
            fn()
        assert e.value.code == code, str(e.value)

    expect(-2, lambda: cache.append_key(k, 250))                    # capacity
    expect(-2, lambda: cache.append_value(k, -1))                   # negative position
    expect(-1, lambda: tq._check(tq.lib().tq_append_key(ctx.handle, tq.ctypes.byref(cache.view),
                                                       tq.ctypes.c_void_p(k.data_ptr()), 7, 0, 10, None)))  # dtype
    expect(-1, lambda: cache.attention_scores(q, 0))                # n_tokens
    expect(-1, lambda: cache.attention_scores(q, 257))              # n_tokens > capacity
    q17 = torch.zeros((2, 17, 128), dtype=torch.float16, device="cuda")
    expect(-1, lambda: cache.attend(q17, 10))                       # G above 16 (attend)
    q513 = torch.zeros((2, 513, 128), dtype=torch.float16, device="cuda")
    expect(-1, lambda: cache.attention_scores(q513, 10))            # G above 512 (scores)
    ws = cache.workspace(4, 10)
    out = torch.empty((2, 4, 10), dtype=torch.float32, device="cuda")
    expect(-7, lambda: tq._check(tq.lib().tq_attention_scores(
        ctx.handle, tq.ctypes.byref(cache.view), tq.ctypes.c_void_p(q.data_ptr()), 1, 4, 10,
        tq.ctypes.c_void_p(out.data_ptr()), tq.ctypes.c_void_p(ws.data_ptr()), 16, None)))
    kmis = torch.zeros(2 * 10 * 128 + 4, dtype=torch.float16, device="cuda")[4:]
    expect(-1, lambda: tq._check(tq.lib().tq_append_key(ctx.handle, tq.ctypes.byref(cache.view),
                                                       tq.ctypes.c_void_p(kmis.data_ptr()), 1, 0, 10, None)))
    # a codebook that is not symmetric about 0 is rejected
    D = tq.ctypes.POINTER(tq.ctypes.c_double)
    c_bad = np.array([-0.2, -0.05, 0.06, 0.2])
    b_bad = np.array([-0.1, 0.0, 0.1])
    expect(-1, lambda: tq._check(tq.lib().tq_codebook_load(ctx.handle, 2, c_bad.ctypes.data_as(D),
                                                          b_bad.ctypes.data_as(D))))
    # 0 bits: the single centroid must be 0 (boundaries may be NULL); bits outside 0..4
    c_one = np.array([0.01])
    expect(-1, lambda: tq._check(tq.lib().tq_codebook_load(ctx.handle, 0, c_one.ctypes.data_as(D), None)))
    c_zero = np.array([0.0])
    tq._check(tq.lib().tq_codebook_load(ctx.handle, 0, c_zero.ctypes.data_as(D), None))
    expect(-1, lambda: tq._check(tq.lib().tq_codebook_load(ctx.handle, 5, c_bad.ctypes.data_as(D),
                                                          b_bad.ctypes.data_as(D))))
    # no codebook for the requested bits
    ctx2 = tq.Context(128, 64, 2, 2, R, S, load_codebooks=False)
    cache2 = tq.KVCache(ctx2, 2, 256)
    expect(-3, lambda: cache2.append_key(k, 0))
    expect(-3, lambda: cache2.attend(q, 5))
    ctx3 = tq.Context(128, 64, 0, 2, R, S, load_codebooks=False)   # 0-bit keys need their codebook too
    cache3 = tq.KVCache(ctx3, 2, 256)
    expect(-3, lambda: cache3.append_key(k, 0))
    expect(-3, lambda: cache3.attention_scores(q, 5))
    torch.cuda.synchronize()
    assert bool((cache.key_records == canary).all()) and bool((cache.value_blocks == canary).all())
    assert bool((cache2.key_records == 0).all())
    # n_new == 0 is a no-op
    cache.append_key(k[:, :0].contiguous(), 0)
    torch.cuda.synchronize()
    assert bool((cache.key_records == canary).all())
    ctx.close()
    ctx2.close()
    ctx3.close()


@pytest.mark.parametrize("d,m,kb,vb,T,chunks,rng", [
    (128, 64, 3, 3, 300, [37, 263], (0, 300)),
    (128, 64, 3, 3, 300, [300], (37, 200)),
    (128, 64, 1, 2, 200, [129, 71], (5, 190)),
    (128, 128, 4, 4, 160, [160], (0, 160)),
    (256, 128, 2, 3, 200, [200], (11, 170)),
    (1024, 512, 4, 4, 40, [40], (0, 40)),
    (64, 32, 3, 2, 200, [129, 71], (3, 190)),
    (192, 96, 4, 3, 160, [160], (0, 160)),
])
def test_reconstruction_matches_oracle(d, m, kb, vb, T, chunks, rng):
    """tq_get_keys / tq_get_values (TurboQuantMSE.dequantize,
    TurboQuantKVCache.get_values): ||x|| R^T c[idx] for a token range,
    against the oracle's dequantize_values on the GPU's own codes and, for
    tokens without an index flip, on the oracle's codes."""
    n_seq = 2
    K = np.stack([synth.kv_slot(70, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(71, s, s, T, d) for s in range(n_seq)])
    K[1, 3] = 0  # a zero row reconstructs to 0
    _say("reconstruction", (d, m, kb, vb, T, rng))
    ctx, R, S = make_ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, -(-T // 128) * 128)
    pos = 0
    for n in chunks:
        cache.append_key(torch.from_numpy(np.ascontiguousarray(K[:, pos:pos + n])).cuda(), pos)
        cache.append_value(torch.from_numpy(np.ascontiguousarray(V[:, pos:pos + n])).cuda(), pos)
        pos += n
    p0, nt = rng
    gk_out = cache.get_keys(p0, nt).cpu().numpy()
    gv_out = cache.get_values(p0, nt).cpu().numpy()
    torch.cuda.synchronize()
    kbeta, kc = O.lloyd_max_codebook(d, kb)
    vbeta, vc = O.lloyd_max_codebook(d, vb)
    sl = lambda dct: {k: v[:, p0:p0 + nt] for k, v in dct.items()}
    gk = sl(P.unpack_gpu_keys(cache, d, m, kb, T))
    gv = sl(P.unpack_gpu_values(cache, d, vb, T))
    st = {"keys_gpu_codes": P.check_dequant(gk_out, O.dequantize_values(R, kc, gk), gk["norm"]),
          "values_gpu_codes": P.check_dequant(gv_out, O.dequantize_values(R, vc, gv), gv["norm"])}
    ref_k = sl(O.compress_keys(K, R, S, kbeta, kc))
    ref_v = sl(O.compress_values(V, R, vbeta, vc))
    st["keys_end_to_end"] = P.check_dequant(gk_out, O.dequantize_values(R, kc, ref_k), ref_k["norm"],
                                            skip_tokens=(gk["idx"] != ref_k["idx"]).any(-1))
    st["values_end_to_end"] = P.check_dequant(gv_out, O.dequantize_values(R, vc, ref_v), ref_v["norm"],
                                              skip_tokens=(gv["idx"] != ref_v["idx"]).any(-1))
    # an empty range is a no-op; a range past the capacity is rejected
    cache.get_values(0, 0)
    with pytest.raises(tq.TQError) as e:
        cache.get_keys(cache.capacity - 3, 4)
    assert e.value.code == -2
    _say(st)
    ctx.close()


def _topk_reference(scores, k):
    """Indices of the k best scores per row by (score desc, index asc)."""
    n = scores.shape[-1]
    order = np.lexsort((np.broadcast_to(np.arange(n), scores.shape), -scores), axis=-1)
    return order[..., :k]


@pytest.mark.parametrize("d,m,b,n_seq,N,G,k", [
    (128, 64, 3, 2, 3000, 40, 10),
    (128, 64, 2, 1, 700, 16, 16),
    (256, 128, 3, 2, 1000, 20, 1),
    (1024, 512, 4, 1, 2500, 64, 10),
    (128, 64, 3, 1, 5, 4, 10),
    (128, 64, 0, 2, 3000, 40, 10),     # 0-bit keys: QJL signs only
    (1024, 512, 0, 1, 2500, 64, 10),
    (64, 32, 3, 1, 1500, 20, 10),      # half chunk and half sign block
    (64, 32, 2, 1, 700, 33, 4),
    (192, 96, 4, 2, 900, 8, 5),
    (64, 32, 0, 1, 900, 4, 3),
])
def test_topk_matches_scores(d, m, b, n_seq, N, G, k):
    """tq_topk_scores: the k best tokens of each query (vector search over the
    packed keys) equal the top-k of tq_attention_scores' own output (same
    estimate, same order: score desc, position asc), and form a valid top-k
    of the oracle's estimates within the score tolerance."""
    _say("topk", (d, m, b, n_seq, N, G, k))
    X = np.stack([synth.vector_database(N, d, seed=80 + s) for s in range(n_seq)])
    Q = np.stack([synth.unit_gaussian(G, d, seed=90 + s) for s in range(n_seq)])
    ctx, R, S = make_ctx(d, m, b, max(b, 1))
    cache = tq.KVCache(ctx, n_seq, -(-N // 128) * 128)
    cache.append_key(torch.from_numpy(X).cuda(), 0)
    qt = torch.from_numpy(Q).cuda()
    ts, ti = cache.topk(qt, N, k)
    sc = cache.attention_scores(qt, N)
    ts, ti, sc = ts.cpu().numpy(), ti.cpu().numpy(), sc.cpu().numpy()
    kk = min(k, N)
    ref_i = _topk_reference(sc, kk)
    assert np.array_equal(ti[..., :kk], ref_i), "top-k indices differ from the materialised scores' top-k"
    assert np.array_equal(ts[..., :kk], np.take_along_axis(sc, ref_i, -1)), "top-k scores differ"
    if kk < k:
        assert np.all(ti[..., kk:] == -1) and np.all(np.isneginf(ts[..., kk:]))
    # validity against the oracle's estimates on the GPU's codes
    beta, c = O.lloyd_max_codebook(d, b)
    gk = P.unpack_gpu_keys(cache, d, m, b, N)
    ref = O.key_scores(Q.astype(np.float64), R, S, c, gk)
    qn = np.linalg.norm(Q.astype(np.float64), axis=-1)[..., None]
    kn = np.linalg.norm(X.astype(np.float64), axis=-1)[:, None, :]
    tol = P.SCORE_TOL * qn * kn
    picked = np.zeros(ref.shape, dtype=bool)
    np.put_along_axis(picked, ti[..., :kk].astype(np.int64), True, axis=-1)
    lo = np.min(np.where(picked, ref + tol, np.inf), axis=-1)
    hi = np.max(np.where(picked, -np.inf, ref - tol), axis=-1)
    assert np.all(hi <= lo), "a token left out beats a returned one by more than the score tolerance"
    _say({"worst_margin": float(np.max(hi - lo)) if kk < N else None})
    ctx.close()


@pytest.mark.parametrize("d,m,kb,vb,dtype", [
    (128, 64, 3, 3, np.float16),
    (128, 128, 4, 2, np.float32),
    (256, 128, 2, 3, np.float16),
    (1024, 512, 1, 4, np.float32),
    (64, 32, 3, 3, np.float16),
    (192, 96, 4, 2, np.float32),
])
def test_small_appends_decode_like(d, m, kb, vb, dtype):
    """Appends of 1..16 tokens (the decode-step path: fp32 vector arithmetic,
    no matrix-core tiles) between bulk appends, crossing 128-token block
    boundaries, with zero key/value rows inside the small chunks; every code,
    sign, norm, score and the attention output against the oracle."""
    T, n_seq, G = 300, 2, 4
    K = np.stack([synth.kv_slot(100, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(101, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(102, s, s, G, d, dtype=dtype) for s in range(n_seq)])
    K[0, 131] = 0  # inside the 16-token chunk at 131
    V[1, 128] = 0  # the one-token chunk at 128
    chunks = [120, 8, 1, 1, 1, 16, 3, 5, 1, 144]
    _say("small appends", (d, m, kb, vb, np.dtype(dtype).name), chunks)
    _say(run_case(K, V, Q, kb=kb, vb=vb, m=m, chunks=chunks))


@pytest.mark.parametrize("d,m,kb,vb,dtype,G", [
    (128, 64, 3, 3, np.float16, 4),
    (128, 128, 4, 2, np.float32, 8),
    (128, 64, 2, 1, np.float16, 16),
    (128, 64, 3, 4, np.float16, 11),   # 9 <= G <= 15: the attend instance with unused head columns
    (256, 128, 3, 3, np.float16, 4),   # not a single-kernel shape: the three calls in order
    (128, 64, 0, 3, np.float16, 8),    # 0-bit keys: fused appends and query preparation, like 1-4 bits
    (64, 32, 3, 3, np.float16, 4),     # head_dim 64 / proj_dim 32: the three calls
])
def test_decode_steps_match_oracle(d, m, kb, vb, dtype, G):
    """tq_decode_step after a prefill: each step appends 1..16 tokens (crossing
    128-token blocks, one step of 17 taking the unfused form) and attends over
    the whole cache so far; every step's output against the oracle's attention
    over the oracle's codes of that prefix, and at the end every code, sign and
    norm of the cache against the oracle."""
    n_seq, prefill = 2, 120
    steps = [1, 1, 5, 1, 16, 1, 17, 2]
    T = prefill + sum(steps)
    K = np.stack([synth.kv_slot(110, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(111, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    K[1, prefill + 2] = 0  # a zero key inside a decode step
    Qs = [np.stack([synth.kv_slot(112 + i, s, s, G, d, dtype=dtype) for s in range(n_seq)]) for i in range(len(steps))]
    _say("decode steps", (d, m, kb, vb, np.dtype(dtype).name, G), steps)
    ctx, R, S = make_ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, 512)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cache.append_key(dev(K[:, :prefill]), 0)
    cache.append_value(dev(V[:, :prefill]), 0)
    kbeta, kc = O.lloyd_max_codebook(d, kb)
    vbeta, vc = O.lloyd_max_codebook(d, vb)
    ref_k = O.compress_keys(K, R, S, kbeta, kc)
    ref_v = O.compress_values(V, R, vbeta, vc)
    pos, outs = prefill, []
    for n, Q in zip(steps, Qs):
        outs.append(cache.decode_step(dev(K[:, pos:pos + n]), dev(V[:, pos:pos + n]), dev(Q), pos).cpu().numpy())
        pos += n
    # codes first (the attention below is judged on the GPU's own codes)
    gk = P.unpack_gpu_keys(cache, d, m, kb, T)
    gv = P.unpack_gpu_values(cache, d, vb, T)
    st = P.check_keys(gk, ref_k, kbeta, S, kc)
    vst = P.check_values(gv, ref_v, vbeta)
    flips = st.pop("flip_tokens") | vst.pop("flip_tokens")
    st.update({"v_" + k: v for k, v in vst.items()})
    _say(st)
    # each step's output at two levels (P.check_attend_two_level): against
    # the oracle's attention on the GPU's codes of that prefix, and end to end
    # for every slot whose prefix holds no flipped token
    pos, errs = prefill, []
    for n, Q, out in zip(steps, Qs, outs):
        pos += n
        on_gpu = O.attend(Q, R, S, kc, {k: a[:, :pos] for k, a in gk.items()},
                          {k: a[:, :pos] for k, a in gv.items()}, value_centroids=vc)
        e2e = O.attend(Q, R, S, kc, {k: a[:, :pos] for k, a in ref_k.items()},
                       {k: a[:, :pos] for k, a in ref_v.items()}, value_centroids=vc)
        errs.append((pos, *P.check_attend_two_level(out, on_gpu, e2e, flips[:, :pos])))
    _say("per step (n_tokens, vs oracle on GPU codes, end to end on clean slots, slots with a flip)", errs)
    ctx.close()


# ---------------------------------------------------------------------------
# 0-bit keys: the (b - 1)-bit + QJL budget at b = 1, signs and norms only
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,m,vb,dtype,G", [
    (128, 64, 3, np.float16, 8),
    (128, 128, 2, np.float32, 4),
    (256, 128, 4, np.float16, 20),   # scores only (G > 16)
    (1024, 512, 4, np.float32, 16),
    (64, 32, 2, np.float16, 8),
    (128, 32, 3, np.float32, 4),
])
def test_zero_bit_keys(d, m, vb, dtype, G):
    """key_bits = 0: records of m sign bits of S R k/||k|| and the two norms
    (gamma = 1), appended in unaligned chunks (one-token and bulk appends)
    with a zero key inside; signs, norms, scores (the plain QJL estimate) and
    attention against the oracle.  The key reconstruction is all zeros, and
    top-k returns the best of the materialised scores."""
    n_seq, T = 2, 700
    K = np.stack([synth.kv_slot(130 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(131 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(132 + d, s, s, G, d, dtype=dtype) for s in range(n_seq)])
    K[1, 130] = 0  # the one-token chunk at 130
    K[0, 400] = 0
    _say("zero-bit keys", (d, m, vb, np.dtype(dtype).name, G))
    assert tq.key_record_bytes(tq.Config(d, m, 0, vb)) == 4 * (m // 32 + 2)
    _say(run_case(K, V, Q, kb=0, vb=vb, m=m, chunks=[130, 1, 300, 269], check_attend=G <= 16))
    ctx, R, S = make_ctx(d, m, 0, vb)
    cache = tq.KVCache(ctx, n_seq, 768)
    cache.append_key(torch.from_numpy(np.ascontiguousarray(K[:, :50])).cuda(), 0)
    rec = P.unpack_gpu_keys(cache, d, m, 0, 50)
    assert np.all(np.abs(rec["gamma"][K[:, :50].any(-1)] - 1.0) < 1e-6)
    assert not cache.get_keys(0, 50).cpu().numpy().any()
    qt = torch.from_numpy(np.ascontiguousarray(Q[:, :4])).cuda()
    ts, ti = cache.topk(qt, 50, 4)
    sc = cache.attention_scores(qt, 50)
    assert torch.equal(ts, torch.topk(sc, 4, dim=-1).values)
    assert torch.equal(torch.gather(sc, -1, ti.long()), ts)
    ctx.close()


def test_topk_at_maximum_capacity():
    """Top-k over a slot of the maximum capacity (2^24 tokens) of 584-byte
    records (d = 1024, m = 512, 4-bit): 9.8 GB of records, so the tokens at
    the end of the slot sit past 2^32 bytes from its start.  3000 keys are
    appended at the end (the rest are zero records, which score 0); the top-k
    over all 2^24 tokens equals the top-k of tq_attention_scores' estimates
    of the appended tokens, and is a valid top-k of the oracle's estimates."""
    d, m, b, G, k, N = 1024, 512, 4, 64, 10, 3000
    cap = 1 << 24
    pos = cap - N - 5
    _say("topk at maximum capacity", (d, m, b, cap, pos, G, k))
    X = synth.vector_database(N, d, seed=140)[None]
    Q = synth.unit_gaussian(G, d, seed=141)[None]
    ctx, R, S = make_ctx(d, m, b, b)
    cache = tq.KVCache(ctx, 1, cap)
    cache.append_key(torch.from_numpy(X).cuda(), pos)
    qt = torch.from_numpy(Q).cuda()
    ts, ti = cache.topk(qt, cap, k)
    sc = cache.attention_scores(qt, cap)[..., pos:pos + N].cpu().numpy()
    ts, ti = ts.cpu().numpy(), ti.cpu().numpy()
    assert np.all((sc > 0).sum(-1) >= k)  # the zero records (score 0) cannot enter
    ref_i = _topk_reference(sc, k)
    assert np.array_equal(ti, ref_i + pos), "top-k indices differ from the materialised scores' top-k"
    assert np.array_equal(ts, np.take_along_axis(sc, ref_i, -1)), "top-k scores differ"
    rw = tq.key_record_bytes(ctx.cfg) // 4
    recs = cache.key_records.view(1, cap, rw)[:, pos:pos + N].cpu().numpy().view(np.uint32)
    beta, c = O.lloyd_max_codebook(d, b)
    gk = O.unpack_keys(recs, d, m, b)
    ref = O.key_scores(Q.astype(np.float64), R, S, c, gk)
    tol = P.SCORE_TOL * np.linalg.norm(Q, axis=-1)[..., None] * np.linalg.norm(X, axis=-1)[:, None, :]
    picked = np.zeros(ref.shape, dtype=bool)
    np.put_along_axis(picked, (ti - pos).astype(np.int64), True, axis=-1)
    lo = np.min(np.where(picked, ref + tol, np.inf), axis=-1)
    hi = np.max(np.where(picked, -np.inf, ref - tol), axis=-1)
    assert np.all(hi <= lo), "a token left out beats a returned one by more than the score tolerance"
    del cache
    ctx.close()


def test_general_scores_beyond_one_launch():
    """The general score kernel runs one wave per (slot, 16-token tile) and is
    launched in pieces of 2^24 waves: 17 slots of 2^24 tokens (0-bit keys,
    4.6 GB of records) need two.  Keys appended at the end of every slot
    (the last slot's in the second piece) score as the oracle says on the
    GPU's records; the zero records score 0."""
    d, m, kb, vb, G, N = 128, 64, 0, 1, 4, 500
    n_seq, cap = 17, 1 << 24
    pos = cap - N
    _say("general scores in pieces", (n_seq, cap, kb, G))
    K = np.stack([synth.kv_slot(150, s, s, N, d) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(151, s, s, G, d) for s in range(n_seq)])
    ctx, R, S = make_ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, cap)
    cache.append_key(torch.from_numpy(K).cuda(), pos)
    sc_all = cache.attention_scores(torch.from_numpy(Q).cuda(), cap)
    sc = sc_all[..., pos:].cpu().numpy()
    assert float(sc_all[..., :pos].abs().max()) == 0.0
    del sc_all
    rw = tq.key_record_bytes(ctx.cfg) // 4
    recs = cache.key_records.view(n_seq, cap, rw)[:, pos:].cpu().numpy().view(np.uint32)
    _, c = O.lloyd_max_codebook(d, kb)
    ref = O.key_scores(Q.astype(np.float64), R, S, c, O.unpack_keys(recs, d, m, kb))
    qn = np.linalg.norm(Q.astype(np.float64), axis=-1)
    kn = np.linalg.norm(K.astype(np.float64), axis=-1)
    _say({"score_vs_gpu_codes": P.check_scores(sc, ref, qn, kn)})
    del cache
    ctx.close()


def test_vector_search_full_size_sampled():
    """The vector-search workload at full size, in the launch configuration
    bench.py times: 2,000,000 unit-norm fp32 vectors (d = 1024) compressed in
    one tq_append_key call (4-bit keys, proj_dim 512), scored against 512
    queries (tq_attention_scores) and searched for the top 10 (tq_topk_scores).
    The oracle recomputes the records and scores of sampled rows; the top-10
    of every query equals the 10 best of the materialised scores."""
    d, m, b, N, G, k = 1024, 512, 4, 2_000_000, 512, 10
    _say("vector search full size", (N, d, m, b, G))
    dev = torch.device("cuda:0")
    X, Q = synth.vector_search_device(torch, N, d, G, dev)
    ctx, R, S = make_ctx(d, m, b, b)
    cache = tq.KVCache(ctx, 1, -(-N // 128) * 128)
    cache.append_key(X, 0)
    sc = cache.attention_scores(Q, N)
    ts, ti = cache.topk(Q, N, k)
    # top-k against the materialised scores, on the device: the same values
    # in descending order, at the returned positions, no position twice
    ref_s = torch.topk(sc, k, dim=-1).values
    assert torch.equal(ts, ref_s), "top-k scores differ from the 10 best materialised scores"
    assert torch.equal(torch.gather(sc, -1, ti.long()), ts), "top-k positions do not hold their scores"
    assert bool((ti.sort(dim=-1).values.diff(dim=-1) > 0).all()), "a position returned twice"
    # sampled rows against the oracle: records, then scores
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([rng.choice(N, 1500, replace=False), np.arange(N - 16, N)]))
    tt = torch.from_numpy(toks).to(dev)
    xs = X[0, tt].cpu().numpy()[None]
    rw = tq.key_record_bytes(ctx.cfg) // 4
    recs = cache.key_records.view(1, cache.capacity, rw)[0, tt].cpu().numpy().view(np.uint32)[None]
    beta, c = O.lloyd_max_codebook(d, b)
    ref = O.compress_keys(xs, R, S, beta, c)
    st = P.check_keys(O.unpack_keys(recs, d, m, b), ref, beta, S, c)
    flips = st.pop("flip_tokens")
    q = Q.cpu().numpy()
    st["score"] = P.check_scores(sc[:, :, tt].cpu().numpy(), O.key_scores(q, R, S, c, ref),
                                 np.linalg.norm(q.astype(np.float64), axis=-1),
                                 np.linalg.norm(xs.astype(np.float64), axis=-1), skip_tokens=flips)
    _say("vector search full size", st)
    del cache, sc, X
    ctx.close()


def _pow2_rows(X, exps):
    """Rows of X (n_seq, T, d) scaled by powers of two cycling through exps,
    as fp32 (exact scalings; 2^-135 gives subnormal coordinates)."""
    e = np.asarray(exps, dtype=np.float64)[np.arange(X.shape[1]) % len(exps)]
    return (X.astype(np.float64) * np.exp2(e)[None, :, None]).astype(np.float32)


@pytest.mark.parametrize("d,m,chunks", [(128, 64, [256, 3, 41]), (256, 128, [200, 100])])
def test_extreme_fp32_magnitudes(d, m, chunks):
    """fp32 inputs across the fp32 range: keys and values with per-token
    scales 2^-135 (subnormal coordinates) .. 2^100 and queries 2^-10 .. 2^10,
    appended in bulk and in small chunks (single-kernel, small-append and
    general paths).  Norms are taken over rows pre-shifted by their largest
    magnitude, so codes, signs, norms and scores match the oracle at every
    scale (products |q| ||k|| stay inside the fp32 range).  Attention with
    values at 2^-120 .. 2^120 and moderate keys matches as well."""
    n_seq, T, G = 2, 300, 4
    exps = [-135, -126, -100, -60, -20, 0, 20, 60, 100]
    K0 = np.stack([synth.kv_slot(170 + d, s, s, T, d, dtype=np.float32) for s in range(n_seq)])
    V0 = np.stack([synth.kv_slot(171 + d, s, s, T, d, dtype=np.float32) for s in range(n_seq)])
    Q0 = np.stack([synth.kv_slot(172 + d, s, s, G, d, dtype=np.float32) for s in range(n_seq)])
    K, V = _pow2_rows(K0, exps), _pow2_rows(V0, exps[::-1])
    Q = (Q0.astype(np.float64) * np.exp2([-10.0, 0.0, 10.0, 3.0])[None, :, None]).astype(np.float32)
    _say("extreme magnitudes", (d, m, chunks))
    _say(run_case(K, V, Q, kb=3, vb=3, m=m, chunks=chunks, check_attend=False))
    V2 = _pow2_rows(V0, [-120, -60, 0, 60, 120, 7, -7])
    _say(run_case(K0, V2, Q0, kb=3, vb=3, m=m, chunks=chunks, check_attend=True))


def test_extreme_fp32_magnitudes_decode_step():
    """The fused decode step (small appends and query preparation in one
    launch) on fp32 rows at 2^-130 .. 2^100 and queries at 2^-100 and 2^-96:
    codes and norms against the oracle, attention against the oracle on the
    GPU's codes."""
    d, m, G, n_seq, prefill = 128, 64, 4, 2, 130
    steps = [1, 3, 1]
    T = prefill + sum(steps)
    K = _pow2_rows(np.stack([synth.kv_slot(180, s, s, T, d, dtype=np.float32) for s in range(n_seq)]),
                   [-130, 0, 100, -60, 30])
    V = _pow2_rows(np.stack([synth.kv_slot(181, s, s, T, d, dtype=np.float32) for s in range(n_seq)]),
                   [100, -130, 0, 50])
    Q0 = np.stack([synth.kv_slot(182, s, s, G, d, dtype=np.float32) for s in range(n_seq)])
    _say("extreme magnitudes, decode steps")
    ctx, R, S = make_ctx(d, m, 3, 3)
    cache = tq.KVCache(ctx, n_seq, 256)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cache.append_key(dev(K[:, :prefill]), 0)
    cache.append_value(dev(V[:, :prefill]), 0)
    pos, outs, qs = prefill, [], []
    for i, n in enumerate(steps):
        # tiny queries against the 2^100 keys keep the logits moderate (no
        # hard argmax between nearly equal estimates)
        Q = (Q0.astype(np.float64) * 2.0 ** (-100 if i % 2 == 0 else -96)).astype(np.float32)
        qs.append(Q)
        outs.append(cache.decode_step(dev(K[:, pos:pos + n]), dev(V[:, pos:pos + n]), dev(Q), pos).cpu().numpy())
        pos += n
    beta, c = O.lloyd_max_codebook(d, 3)
    gk = P.unpack_gpu_keys(cache, d, m, 3, T)
    gv = P.unpack_gpu_values(cache, d, 3, T)
    st = P.check_keys(gk, O.compress_keys(K, R, S, beta, c), beta, S, c)
    st.pop("flip_tokens")
    vst = P.check_values(gv, O.compress_values(V, R, beta, c), beta)
    vst.pop("flip_tokens")
    st.update({"v_" + k: v for k, v in vst.items()})
    pos, errs = prefill, []
    for n, Q, out in zip(steps, qs, outs):
        pos += n
        ref = O.attend(Q, R, S, c, {k: a[:, :pos] for k, a in gk.items()}, {k: a[:, :pos] for k, a in gv.items()})
        errs.append(P.check_attend(out, ref))
    _say(st, errs)
    ctx.close()


@pytest.mark.parametrize("d,m,dtype", [(128, 64, np.float16), (256, 128, np.float32)])
def test_zero_query_heads(d, m, dtype):
    """A query head of all zeros scores exactly 0 against every key, and its
    attention is the plain average of the dequantised values (softmax of
    equal logits), as the oracle has it; the other heads are unaffected."""
    n_seq, T, G = 2, 200, 4
    K = np.stack([synth.kv_slot(190 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(191 + d, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    Q = np.stack([synth.kv_slot(192 + d, s, s, G, d, dtype=dtype) for s in range(n_seq)])
    Q[0, 1] = 0
    Q[1, 3] = 0
    _say("zero query heads", (d, m, np.dtype(dtype).name))
    ctx, R, S = make_ctx(d, m, 3, 3)
    cache = tq.KVCache(ctx, n_seq, 256)
    cache.append_key(torch.from_numpy(K).cuda(), 0)
    cache.append_value(torch.from_numpy(V).cuda(), 0)
    qt = torch.from_numpy(Q).cuda()
    sc = cache.attention_scores(qt, T).cpu().numpy()
    out = cache.attend(qt, T).cpu().numpy()
    assert not sc[0, 1].any() and not sc[1, 3].any()
    gk = P.unpack_gpu_keys(cache, d, m, 3, T)
    gv = P.unpack_gpu_values(cache, d, 3, T)
    _, c = O.lloyd_max_codebook(d, 3)
    ref = O.attend(Q, R, S, c, gk, gv)
    np.testing.assert_allclose(ref[0, 1], O.dequantize_values(R, c, gv)[0].mean(0), rtol=1e-12, atol=1e-12)
    _say({"attend_rel": P.check_attend(out, ref)})
    ctx.close()


def test_scores_and_attend_at_maximum_capacity():
    """The single-kernel score and attend kernels over a slot of the maximum
    capacity (2^24 tokens; ~1 GB of key records and ~0.9 GB of value blocks
    addressed through per-slot buffer descriptors).  300 tokens are appended
    at the very end; the zero records before them score exactly 0, and in the
    softmax they add N_zero exp(0 - M) to the denominator and nothing to the
    numerator (zero values), so the oracle's attention over all 2^24 tokens is
    formed from the 300 real tokens in closed form."""
    d, m, b, G, N = 128, 64, 3, 4, 300
    cap = 1 << 24
    pos = cap - N
    _say("scores and attend at maximum capacity", (cap, pos, G))
    K = synth.kv_slot(200, 0, 0, N, d)[None]
    V = synth.kv_slot(201, 0, 0, N, d)[None]
    Q = synth.kv_slot(202, 0, 0, G, d)[None] * 4
    ctx, R, S = make_ctx(d, m, b, b)
    cache = tq.KVCache(ctx, 1, cap)
    cache.append_key(torch.from_numpy(K).cuda(), pos)
    cache.append_value(torch.from_numpy(V).cuda(), pos)
    qt = torch.from_numpy(np.ascontiguousarray(Q)).cuda()
    sc_all = cache.attention_scores(qt, cap)
    out = cache.attend(qt, cap).cpu().numpy()
    assert float(sc_all[..., :pos].abs().max()) == 0.0
    sc = sc_all[..., pos:].cpu().numpy()
    del sc_all
    rw = tq.key_record_bytes(ctx.cfg) // 4
    recs = cache.key_records.view(1, cap, rw)[:, pos:].cpu().numpy().view(np.uint32)
    bw = tq.value_block_bytes(ctx.cfg) // 4
    blocks = cache.value_blocks.view(1, cap // 128, bw)[:, (pos // 128):].cpu().numpy().view(np.uint32)
    _, c = O.lloyd_max_codebook(d, b)
    gk = O.unpack_keys(recs, d, m, b)
    gv_blk = O.unpack_values(blocks, d, b)
    off = pos - (pos // 128) * 128
    gv = {k: v[:, off:off + N] for k, v in gv_blk.items()}
    est = O.key_scores(Q.astype(np.float64), R, S, c, gk)
    qn = np.linalg.norm(Q.astype(np.float64), axis=-1)
    kn = np.linalg.norm(K.astype(np.float64), axis=-1)
    st = {"score": P.check_scores(sc, est, qn, kn)}
    lg = est / np.sqrt(d)                                          # (1, G, N) logits of the real tokens
    M = np.maximum(lg.max(-1, keepdims=True), 0.0)                 # the zero records' logit is 0
    w = np.exp(lg - M)
    den = w.sum(-1) + (cap - N) * np.exp(-M[..., 0])
    ref = np.einsum("sgt,std->sgd", w, O.dequantize_values(R, c, gv)) / den[..., None]
    st["attend_rel"] = P.check_attend(out, ref)
    _say(st)
    del cache
    ctx.close()


@pytest.mark.parametrize("d,m,kb,vb", [(128, 64, 3, 3), (128, 128, 0, 2), (1024, 512, 4, 4), (256, 128, 2, 1),
                                        (64, 32, 3, 2), (192, 96, 0, 4)])
def test_context_size_queries(d, m, kb, vb):
    """tq_key_record_bytes / tq_value_record_bytes / tq_attend_workspace_bytes
    of a live context agree with the configuration's layout sizes."""
    ctx, _, _ = make_ctx(d, m, kb, vb)
    assert ctx.key_record_bytes() == tq.key_record_bytes(ctx.cfg) == 4 * O.key_record_words(d, m, kb)
    assert ctx.value_record_bytes() * 128 == tq.value_block_bytes(ctx.cfg)
    for n_seq, G, T in [(4, 4, 1000), (64, 4, 131072), (1, 512, 2_000_000), (2, 16, 7)]:
        assert ctx.attend_workspace_bytes(n_seq, G, T) == tq.workspace_bytes(ctx.cfg, n_seq, G, T) > 0
    assert ctx.attend_workspace_bytes(4, 513, 1000) == 0
    ctx.close()


def test_binding_rejects_mismatched_tensor_shapes():
    """The binding checks every tensor against the cache's shape before the
    call (the C ABI sees raw pointers only); nothing is launched."""
    ctx, _, _ = make_ctx()
    cache = tq.KVCache(ctx, 2, 256)
    dev = torch.device("cuda")
    k_bad = torch.zeros((2, 10, 64), dtype=torch.float16, device=dev)
    k_seq = torch.zeros((3, 10, 128), dtype=torch.float16, device=dev)
    q = torch.zeros((2, 4, 128), dtype=torch.float16, device=dev)
    for bad in (k_bad, k_seq):
        with pytest.raises(ValueError):
            cache.append_key(bad, 0)
        with pytest.raises(ValueError):
            cache.append_value(bad, 0)
        with pytest.raises(ValueError):
            cache.attend(bad, 10)
    with pytest.raises(ValueError):
        cache.attention_scores(q, 10, out=torch.empty((2, 4, 9), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        cache.attend(q, 10, out=torch.empty((2, 4, 128), dtype=torch.float16, device=dev))
    k = torch.zeros((2, 1, 128), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError):
        cache.decode_step(k, torch.zeros((2, 2, 128), dtype=torch.float16, device=dev), q, 0)
    ctx.close()


def test_decode_step_single_launch_workgroups_and_graph_replay():
    """The single-launch decode step with two attention workgroups and the
    append workgroup per slot (6 blocks per slot at 700 tokens, 5 slots),
    step by step against the oracle on the GPU's codes; then the same step
    captured in a HIP graph and replayed several times (each replay finds
    the slots' arrival counts back at their start), every replay equal to
    the eager output, with eager work and synchronisations between
    replays."""
    d, m, G, n_seq, prefill = 128, 64, 8, 5, 690
    steps = [1, 3, 1, 5]
    T = prefill + sum(steps)
    K = np.stack([synth.kv_slot(230, s, s, T, d) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(231, s, s, T, d) for s in range(n_seq)])
    Qs = [np.stack([synth.kv_slot(232 + i, s, s, G, d) for s in range(n_seq)]) for i in range(len(steps))]
    _say("decode step, several workgroups per slot", (n_seq, T, G))
    ctx, R, S = make_ctx(d, m, 3, 3)
    cache = tq.KVCache(ctx, n_seq, 768)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cache.append_key(dev(K[:, :prefill]), 0)
    cache.append_value(dev(V[:, :prefill]), 0)
    pos, outs = prefill, []
    for n, Q in zip(steps, Qs):
        outs.append(cache.decode_step(dev(K[:, pos:pos + n]), dev(V[:, pos:pos + n]), dev(Q), pos).cpu().numpy())
        pos += n
    kbeta, kc = O.lloyd_max_codebook(d, 3)
    gk = P.unpack_gpu_keys(cache, d, m, 3, T)
    gv = P.unpack_gpu_values(cache, d, 3, T)
    st = P.check_keys(gk, O.compress_keys(K, R, S, kbeta, kc), kbeta, S, kc)
    st.pop("flip_tokens")
    pos, errs = prefill, []
    for n, Q, out in zip(steps, Qs, outs):
        pos += n
        ref = O.attend(Q, R, S, kc, {k: a[:, :pos] for k, a in gk.items()}, {k: a[:, :pos] for k, a in gv.items()})
        errs.append(P.check_attend(out, ref))
    _say(st, errs)
    # graph capture and replay of one more step (re-appending the last token)
    k1, v1, q1 = dev(K[:, T - 1:T]), dev(V[:, T - 1:T]), dev(Qs[-1])
    o = torch.empty((n_seq, G, d), dtype=torch.float32, device="cuda")
    cache.decode_step(k1, v1, q1, T - 1, out=o)
    torch.cuda.synchronize()
    eager = o.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        cache.decode_step(k1, v1, q1, T - 1, out=o, stream=side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            cache.decode_step(k1, v1, q1, T - 1, out=o, stream=side)
    torch.cuda.synchronize()
    for r in range(4):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager), f"graph replay {r} differs from the eager step"
        cache.decode_step(k1, v1, q1, T - 1)  # eager work between replays
        torch.cuda.synchronize()
    del g
    ctx.close()


@pytest.mark.parametrize("d,m", [(128, 64), (256, 128)])
def test_attend_values_near_fp32_max_over_many_partials(d, m):
    """Value norms of 2^120 with uniform attention (zero queries) over 8000
    tokens: each attend partial's share of the output is near 2^124 and the
    merge adds tens of them, which overflowed fp32 while partials were stored
    scaled back to the norms' magnitude.  With the exponent stored beside the
    accumulator the output (a mean of 2^120-sized vectors) is finite and
    matches the oracle on the GPU's codes; on both the single-kernel and the
    general attend."""
    n_seq, T, G = 1, 8000, 4
    K = np.stack([synth.kv_slot(240, s, s, T, d, dtype=np.float32) for s in range(n_seq)])
    V = (np.stack([synth.kv_slot(241, s, s, T, d, dtype=np.float32) for s in range(n_seq)]).astype(np.float64)
         / np.linalg.norm(np.stack([synth.kv_slot(241, s, s, T, d, dtype=np.float32) for s in range(n_seq)])
                          .astype(np.float64), axis=-1, keepdims=True) * 2.0 ** 120).astype(np.float32)
    Q = np.zeros((n_seq, G, d), dtype=np.float32)
    Q[0, 1] = synth.kv_slot(242, 0, 0, 1, d, dtype=np.float32)[0] * 1e-3  # nearly uniform
    _say("values near fp32 max", (d, m, T))
    ctx, R, S = make_ctx(d, m, 3, 3)
    cache = tq.KVCache(ctx, n_seq, 8064)
    cache.append_key(torch.from_numpy(K).cuda(), 0)
    cache.append_value(torch.from_numpy(V).cuda(), 0)
    out = cache.attend(torch.from_numpy(Q).cuda(), T).cpu().numpy()
    assert np.isfinite(out).all(), "attention output overflowed"
    _, c = O.lloyd_max_codebook(d, 3)
    gk = P.unpack_gpu_keys(cache, d, m, 3, T)
    gv = P.unpack_gpu_values(cache, d, 3, T)
    ref = O.attend(Q, R, S, c, gk, gv)
    _say({"attend_rel": P.check_attend(out, ref), "max_abs": float(np.abs(out).max())})
    ctx.close()
