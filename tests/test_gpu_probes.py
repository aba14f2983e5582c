"""The measurement kernels beside the path, through the C ABI on cuda:0: the
streaming-read probe reads every byte exactly once (the xor of its per-
workgroup checksums is the xor of all words), and the copy probe copies."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("n_words", [4, 4096 * 64 * 4 + 12, 3 * (1 << 20) + 4])
def test_probe_read_reads_every_word_once(n_words):
    import torch
    import paged_kv_cache_227_amd as P
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 1 << 32, size=n_words, dtype=np.uint64).astype(np.uint32)
    say("case probe_read, %d words" % n_words)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    P.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_probe_copy_copies():
    import torch
    import paged_kv_cache_227_amd as P
    src = torch.randint(-(1 << 31), 1 << 31, ((1 << 20) + 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    P.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
