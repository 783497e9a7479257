"""GPU check of the HBM stream used as the bandwidth baseline (tq_hbm_stream):
it reads every word of the source (the XOR it folds matches numpy's) and,
with writes, fills the whole destination, at each allowed read/write ratio."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from kv_cache_vector_compress_amd import tq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("read_bytes,ratio,wpc,nl,nt", [
    (4096, 0, 0, 4, False), (1 << 20, 0, 16, 8, True), (3 << 20, 4, 0, 4, False), (1 << 22, 2, 64, 16, True),
    (1 << 21, 1, 4, 8, False), (64 << 20, 4, 32, 16, True), (64 << 20, 0, 64, 4, True), (48 << 10, 4, 8, 16, False)])
def test_stream_reads_everything_and_writes_everything(read_bytes, ratio, wpc, nl, nt):
    rng = np.random.default_rng(read_bytes + ratio)
    words = rng.integers(0, 2**32, size=read_bytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    dst = torch.zeros(read_bytes // 4 // ratio, dtype=torch.float32, device="cuda") if ratio else None
    sink = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    print("[stream]", read_bytes, ratio, wpc, nl, nt, flush=True)
    tq.hbm_stream(src, dst, sink, waves_per_cu=wpc, loads_in_flight=nl, nontemporal=nt)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(words) ^ np.uint32(0x5A5A5A5A)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == expect
    if dst is not None:
        assert bool((dst == 1.0).all())
