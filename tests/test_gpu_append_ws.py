"""Appends with a caller-owned workspace (tq_append_key_ws /
tq_append_value_ws): bit-identical to the appends on the context's scratch,
safe on several streams at once, and not limited by the context's scratch
to 256 slots.  Codes are judged against the oracle with the rules of
tests/parity_util.py."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import turboquant as O
from kv_cache_vector_compress_amd import synth, tq
from tests import parity_util as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[append-ws]", *a, flush=True)


def _ctx(d, m, kb, vb):
    R = synth.haar_rotation(d, synth.SEED_R)
    S = synth.gaussian_projection(m, d, synth.SEED_S)
    return tq.Context(d, m, kb, vb, R, S), R, S


def _kv(seed, n_seq, T, d, dtype):
    K = np.stack([synth.kv_slot(seed, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    V = np.stack([synth.kv_slot(seed + 1, s, s, T, d, dtype=dtype) for s in range(n_seq)])
    return K, V


@pytest.mark.parametrize("d,m,kb,vb,dtype", [
    (256, 128, 3, 3, np.float16),
    (64, 32, 4, 2, np.float32),
    (128, 32, 2, 4, np.float16),   # general keys (proj_dim 32), single-kernel values
])
def test_workspace_appends_equal_context_scratch_appends(d, m, kb, vb, dtype):
    """The same chunks appended both ways give identical records and blocks;
    the workspace size query is 0 exactly for the appends that use none."""
    n_seq, chunks = 3, [300, 5, 200, 1]
    T = sum(chunks)
    K, V = _kv(150, n_seq, T, d, dtype)
    ctx, _, _ = _ctx(d, m, kb, vb)
    a, b = tq.KVCache(ctx, n_seq, 512), tq.KVCache(ctx, n_seq, 512)
    assert ctx.append_workspace_bytes(n_seq, 16) == 0
    assert ctx.append_workspace_bytes(n_seq, 300) > 0
    pos = 0
    for n in chunks:
        kt = torch.from_numpy(np.ascontiguousarray(K[:, pos:pos + n])).cuda()
        vt = torch.from_numpy(np.ascontiguousarray(V[:, pos:pos + n])).cuda()
        a.append_key(kt, pos)
        a.append_value(vt, pos)
        b.append_key_ctx_scratch(kt, pos)
        b.append_value_ctx_scratch(vt, pos)
        pos += n
    torch.cuda.synchronize()
    assert torch.equal(a.key_records, b.key_records)
    assert torch.equal(a.value_blocks, b.value_blocks)
    _say("identical", (d, m, kb, vb, np.dtype(dtype).name))
    ctx.close()


def test_workspace_appends_on_two_streams_at_once():
    """Two caches of one context filled by bulk general-path appends on two
    streams concurrently (each with its own workspace) hold the same records
    as when filled one after the other."""
    d, m, kb, vb, n_seq, T = 192, 96, 3, 3, 4, 2048
    K, V = _kv(160, n_seq, T, d, np.float16)
    ctx, _, _ = _ctx(d, m, kb, vb)
    caches = [tq.KVCache(ctx, n_seq, T) for _ in range(2)]
    ref = [tq.KVCache(ctx, n_seq, T) for _ in range(2)]
    inputs = [(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()),
              (torch.from_numpy(np.ascontiguousarray(K[::-1])).cuda(),
               torch.from_numpy(np.ascontiguousarray(V[::-1])).cuda())]
    for c, (kt, vt) in zip(ref, inputs):
        c.append_key(kt, 0)
        c.append_value(vt, 0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for c in caches:
            c.key_records.zero_()
            c.value_blocks.zero_()
        torch.cuda.synchronize()
        for c, st, (kt, vt) in zip(caches, streams, inputs):
            with torch.cuda.stream(st):
                for off in range(0, T, 512):  # several launches in flight on each stream
                    c.append_key(kt[:, off:off + 512].contiguous(), off, stream=st)
                    c.append_value(vt[:, off:off + 512].contiguous(), off, stream=st)
        torch.cuda.synchronize()
        for c, r in zip(caches, ref):
            assert torch.equal(c.key_records, r.key_records), f"replay {rep}: key records differ"
            assert torch.equal(c.value_blocks, r.value_blocks), f"replay {rep}: value blocks differ"
    _say("two streams: identical over 3 rounds")
    ctx.close()


def test_workspace_appends_beyond_256_slots():
    """A bulk general-path append into 300 slots: the context's scratch
    rejects it (TQ_EUNSUPPORTED, nothing written), the workspace form
    appends it, codes and norms against the oracle."""
    d, m, kb, vb, n_seq, T = 64, 32, 3, 2, 300, 130
    K, V = _kv(170, n_seq, T, d, np.float16)
    ctx, R, S = _ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, 256)
    kt, vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    with pytest.raises(tq.TQError) as e:
        cache.append_key_ctx_scratch(kt, 0)
    assert e.value.code == -6
    with pytest.raises(tq.TQError) as e:
        cache.append_value_ctx_scratch(vt, 0)
    assert e.value.code == -6
    torch.cuda.synchronize()
    assert not cache.key_records.any() and not cache.value_blocks.any()
    cache.append_key(kt, 0)
    cache.append_value(vt, 0)
    torch.cuda.synchronize()
    kbeta, kc = O.lloyd_max_codebook(d, kb)
    vbeta, vc = O.lloyd_max_codebook(d, vb)
    st = P.check_keys(P.unpack_gpu_keys(cache, d, m, kb, T), O.compress_keys(K, R, S, kbeta, kc), kbeta, S, kc)
    st.pop("flip_tokens")
    vst = P.check_values(P.unpack_gpu_values(cache, d, vb, T), O.compress_values(V, R, vbeta, vc), vbeta)
    vst.pop("flip_tokens")
    _say("300 slots", st, vst)
    ctx.close()


def test_workspace_too_small_is_rejected_before_any_write():
    d, m, kb, vb, n_seq, T = 256, 128, 3, 3, 2, 300
    K, V = _kv(180, n_seq, T, d, np.float16)
    ctx, _, _ = _ctx(d, m, kb, vb)
    cache = tq.KVCache(ctx, n_seq, 512)
    cache.key_records.fill_(0x5A5A5A5A)
    cache.value_blocks.fill_(0x5A5A5A5A)
    need = ctx.append_workspace_bytes(n_seq, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    kt, vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    lib = tq.lib()
    for fn, x in ((lib.tq_append_key_ws, kt), (lib.tq_append_value_ws, vt)):
        rc = fn(ctx.handle, ctypes.byref(cache.view), ctypes.c_void_p(x.data_ptr()), 1, 0, T,
                ctypes.c_void_p(ws.data_ptr()), need - 1, None)
        assert rc == -7, tq.last_error()
        rc = fn(ctx.handle, ctypes.byref(cache.view), ctypes.c_void_p(x.data_ptr()), 1, 0, T, None, need, None)
        assert rc == -1, tq.last_error()
    torch.cuda.synchronize()
    assert bool((cache.key_records == 0x5A5A5A5A).all()) and bool((cache.value_blocks == 0x5A5A5A5A).all())
    ctx.close()
