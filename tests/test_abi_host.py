"""Host-side checks of libtq.so that need no GPU: it loads, exports every
function include/tq.h declares, its host Lloyd-Max builder agrees with the
oracle's numerically integrated codebook, size queries follow the record
layout, and argument errors are reported before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import turboquant as O
from kv_cache_vector_compress_amd import tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = tq.lib()
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tq.h but not exported"
    out = os.popen(f"nm -D --defined-only {tq.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not a defined text symbol"


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 1024])
def test_host_codebook_matches_oracle(bits, d):
    c, b = tq.lloyd_max_codebook(d, bits)
    ob, oc = O.lloyd_max_codebook(d, bits)
    np.testing.assert_allclose(c, oc, rtol=0, atol=1e-13 / np.sqrt(d))
    np.testing.assert_allclose(b, ob, rtol=0, atol=1e-13 / np.sqrt(d))


def test_codebook_builder_rejects_bad_arguments():
    c = np.zeros(16)
    b = np.zeros(16)
    P = c.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    Q = b.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    lib = tq.lib()
    assert lib.tq_lloyd_max_codebook(128, -1, P, Q) == -1
    assert lib.tq_lloyd_max_codebook(128, 5, P, Q) == -1
    assert lib.tq_lloyd_max_codebook(0, 3, P, Q) == -1
    assert lib.tq_lloyd_max_codebook(128, 3, None, Q) == -1
    assert "bits" in tq.last_error()


def test_zero_bit_codebook():
    """0 bits: the one centroid 0 and no boundary, as the oracle has it."""
    c, b = tq.lloyd_max_codebook(128, 0)
    ob, oc = O.lloyd_max_codebook(128, 0)
    assert c.tolist() == oc.tolist() == [0.0] and b.size == ob.size == 0
    cc = np.zeros(1)
    assert tq.lib().tq_lloyd_max_codebook(128, 0, cc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), None) == 0


@pytest.mark.parametrize("kb,vb,m", [(3, 3, 64), (2, 4, 128), (1, 1, 64), (4, 2, 512), (0, 3, 64), (0, 1, 512)])
def test_sizes_follow_record_layout(kb, vb, m):
    cfg = tq.Config(128, m, kb, vb)
    assert tq.key_record_bytes(cfg) == 4 * (kb * 128 // 32 + m // 32 + 2) == 4 * O.key_record_words(128, m, kb)
    assert tq.value_block_bytes(cfg) == 4 * O.value_block_words(128, vb)
    assert tq.cache_key_bytes(cfg, 3, 256) == 3 * 256 * tq.key_record_bytes(cfg)
    assert tq.cache_value_bytes(cfg, 3, 256) == 3 * 2 * tq.value_block_bytes(cfg)
    assert tq.cache_key_bytes(cfg, 3, 100) == 0       # capacity not a multiple of 128
    assert tq.workspace_bytes(cfg, 4, 4, 1000) > 0
    assert tq.workspace_bytes(cfg, 4, 17, 1000) > 0   # scores only (general kernel)
    assert tq.workspace_bytes(cfg, 4, 513, 1000) == 0  # G out of range
    assert tq.workspace_bytes(cfg, 4, 4, 0) == 0


@pytest.mark.parametrize("d,m,kb,vb", [(256, 128, 3, 3), (1024, 512, 4, 4), (128, 256, 2, 2), (512, 64, 1, 4),
                                        (64, 32, 3, 3), (192, 96, 2, 4), (128, 32, 4, 1), (960, 480, 1, 2),
                                        (64, 32, 0, 2)])
def test_general_shape_sizes_follow_record_layout(d, m, kb, vb):
    """head_dim a multiple of 64 up to 1024, proj_dim a multiple of 32 up to
    512: the same record layout, sized from the oracle's word counts."""
    cfg = tq.Config(d, m, kb, vb)
    assert tq.key_record_bytes(cfg) == 4 * O.key_record_words(d, m, kb)
    assert tq.value_block_bytes(cfg) == 4 * O.value_block_words(d, vb)
    assert tq.workspace_bytes(cfg, 2, 512, 4096) > 0
    assert tq.workspace_bytes(cfg, 2, 513, 4096) == 0


def test_vector_search_record_is_584_bytes():
    # 4-bit codes of 1024 coordinates (512 B), 512 sign bits (64 B), two fp32 norms
    assert tq.key_record_bytes(tq.Config(1024, 512, 4, 4)) == 584


def test_3bit_record_is_64_bytes_and_block_is_52_bytes_per_token():
    cfg = tq.Config(128, 64, 3, 3)
    assert tq.key_record_bytes(cfg) == 64
    assert tq.value_block_bytes(cfg) == 52 * 128


@pytest.mark.parametrize("cfg,code", [
    ((100, 64, 3, 3), -1), ((128, 48, 3, 3), -1), ((128, 64, -1, 3), -1), ((128, 64, 3, 5), -1),
    ((128, 64, 3, 0), -1), ((128, 64, 5, 3), -1),
    ((2048, 64, 3, 3), -1), ((1152, 64, 3, 3), -1), ((96, 64, 3, 3), -1), ((128, 576, 3, 3), -1),
    ((128, 80, 3, 3), -1), ((32, 32, 3, 3), -1), ((128, 16, 3, 3), -1), ((1088, 64, 3, 3), -1)])
def test_create_rejects_configs_before_any_device_call(cfg, code):
    R = np.eye(cfg[0])
    S = np.ones((max(cfg[1], 1), cfg[0]))
    h = ctypes.c_void_p()
    c = tq.Config(*cfg)
    D = ctypes.POINTER(ctypes.c_double)
    rc = tq.lib().tq_create(ctypes.byref(c), R.ctypes.data_as(D), S.ctypes.data_as(D), ctypes.byref(h))
    assert rc == code, tq.last_error()
    assert not h.value


def test_create_rejects_null_and_nonfinite_matrices():
    c = tq.Config(128, 64, 3, 3)
    h = ctypes.c_void_p()
    D = ctypes.POINTER(ctypes.c_double)
    R = np.eye(128)
    S = np.ones((64, 128))
    assert tq.lib().tq_create(ctypes.byref(c), None, S.ctypes.data_as(D), ctypes.byref(h)) == -1
    R[3, 4] = np.nan
    assert tq.lib().tq_create(ctypes.byref(c), R.ctypes.data_as(D), S.ctypes.data_as(D), ctypes.byref(h)) == -1
    assert "non-finite" in tq.last_error()


def test_hot_path_entry_points_reject_null_context():
    lib = tq.lib()
    view = tq.CacheView(16, 16, 128, 1)
    assert lib.tq_append_key(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 0, 1, None) == -1
    assert lib.tq_append_value(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 0, 1, None) == -1
    assert lib.tq_append_key_ws(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 0, 1, ctypes.c_void_p(16),
                                1 << 20, None) == -1
    assert lib.tq_append_value_ws(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 0, 1, ctypes.c_void_p(16),
                                  1 << 20, None) == -1
    assert lib.tq_append_workspace_bytes(None, 4, 1000) == 0
    assert lib.tq_attention_scores(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 4, 1,
                                   ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 20, None) == -1
    assert lib.tq_attend(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 4, 1, 0.0,
                         ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 20, None) == -1
    assert lib.tq_topk_scores(None, ctypes.byref(view), ctypes.c_void_p(16), 1, 4, 1, 10, ctypes.c_void_p(16),
                              ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 20, None) == -1
    assert lib.tq_get_values(None, ctypes.byref(view), 0, 1, ctypes.c_void_p(16), None) == -1
    assert lib.tq_get_keys(None, ctypes.byref(view), 0, 1, ctypes.c_void_p(16), None) == -1
    assert lib.tq_decode_step(None, ctypes.byref(view), ctypes.c_void_p(16), ctypes.c_void_p(16), 1, 0, 1,
                              ctypes.c_void_p(16), 4, 0.0, ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 20,
                              None) == -1
    assert lib.tq_codebook_load(None, 3, None, None) == -1
    assert lib.tq_destroy(None) == 0



def test_topk_workspace_rejects_bad_arguments():
    cfg = tq.Config(128, 64, 3, 3)
    ws = lambda *a: tq.lib().tq_topk_workspace_bytes(ctypes.byref(cfg), *a)
    assert ws(1, 512, 2_000_000, 10) > 0
    assert ws(1, 4, 100, 16) > 0
    for bad in [(0, 4, 100, 10), (1, 0, 100, 10), (1, 513, 100, 10), (1, 4, 0, 10), (1, 4, 100, 0), (1, 4, 100, 17)]:
        assert ws(*bad) == 0, bad


def _hip_device_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0   # counts devices without initialising one
    except Exception:
        return False


@pytest.mark.skipif(_hip_device_visible(), reason="made-up device addresses: run only where no GPU is visible")
def test_hbm_stream_rejects_bad_arguments_before_any_device_call():
    """tq_hbm_stream checks pointers, alignment and sizes on the host (fake
    addresses: an accepted call would fault, so only rejected ones are made,
    and only on a host without a GPU)."""
    lib = tq.lib()
    A = ctypes.c_void_p(1 << 40)       # aligned, never dereferenced
    U = ctypes.c_void_p((1 << 40) + 4)  # misaligned
    assert lib.tq_hbm_stream(None, 4096, None, 0, A, 0, 0, None) == -1
    assert lib.tq_hbm_stream(U, 4096, None, 0, A, 0, 0, None) == -1
    assert lib.tq_hbm_stream(A, 0, None, 0, A, 0, 0, None) == -1
    assert lib.tq_hbm_stream(A, 4096 + 16, None, 0, A, 0, 0, None) == -1
    assert lib.tq_hbm_stream(A, 8192, None, 2048, A, 0, 0, None) == -1      # writes without dst
    assert lib.tq_hbm_stream(A, 8192, A, 3000, A, 0, 0, None) == -1         # ratio not 1, 2 or 4
    assert lib.tq_hbm_stream(A, 8192, A, 8192 // 8, A, 0, 0, None) == -1    # ratio 8
    assert lib.tq_hbm_stream(A, 8192, A, 2048, None, 0, 0, None) == -1   # no sink
    assert lib.tq_hbm_stream(A, 8192, A, 2048, ctypes.c_void_p((1 << 40) + 2), 0, 0, None) == -1
    assert lib.tq_hbm_stream(A, 8192, A, 2048, A, 6, 0, None) == -1      # waves per CU not a multiple of 4
    assert lib.tq_hbm_stream(A, 8192, A, 2048, A, 68, 0, None) == -1     # above 64
    assert lib.tq_hbm_stream(A, 8192, A, 2048, A, -4, 0, None) == -1
    assert lib.tq_hbm_stream(A, 8192, A, 2048, A, 0, 3, None) == -1              # unknown flag bit
    assert lib.tq_hbm_stream(A, 8192, A, 2048, A, 0, 12 << 8, None) == -1        # 12 loads in flight
    assert lib.tq_hbm_stream(A, 8192, None, 0, A, 0, 16 << 8, None) == -1        # not a multiple of 16 KiB
    assert "tq_hbm_stream" in tq.last_error()


def test_zero_bit_keys_take_the_single_kernel_workspace():
    """0-bit keys at head_dim 128 attend on the single-kernel path: the same
    workspace plan as any other key width (it depends on m, n_seq, G and the
    token count only); at other head_dims they take the general plan."""
    for m in (64, 128):
        for G in (1, 4, 8, 16):
            a = tq.workspace_bytes(tq.Config(128, m, 0, 3), 4, G, 5000)
            b = tq.workspace_bytes(tq.Config(128, m, 3, 3), 4, G, 5000)
            assert a == b > 0
    assert tq.workspace_bytes(tq.Config(256, 128, 0, 3), 4, 8, 5000) == \
        tq.workspace_bytes(tq.Config(256, 128, 2, 3), 4, 8, 5000) > 0


def test_context_size_queries_reject_null_context():
    """The size queries of a context (tq_key_record_bytes,
    tq_value_record_bytes, tq_attend_workspace_bytes) return 0 for NULL;
    their values for a live context are checked on the GPU."""
    lib = tq.lib()
    assert lib.tq_key_record_bytes(None) == 0
    assert lib.tq_value_record_bytes(None) == 0
    assert lib.tq_attend_workspace_bytes(None, 4, 4, 1000) == 0


@pytest.mark.parametrize("d,m,kb,vb", [(128, 64, 3, 3), (128, 128, 0, 2), (1024, 512, 4, 4), (256, 128, 2, 1)])
def test_value_record_is_the_per_token_share_of_a_block(d, m, kb, vb):
    """4 (b d/32 + 1) bytes per token: the block of 128 tokens holds b d/32
    code words and one fp32 norm per token."""
    cfg = tq.Config(d, m, kb, vb)
    assert tq.value_block_bytes(cfg) == 128 * 4 * (vb * d // 32 + 1)


def test_layout_version_is_2():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    assert re.search(r"#define\s+TQ_LAYOUT_VERSION\s+2\b", src)
