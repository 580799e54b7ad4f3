"""The streaming-read probe (a measurement helper of the benchmark) reads every 16-byte chunk exactly once: the
XOR of its per-workgroup checksums equals the XOR of every word of the buffer, for sizes that leave a partial
unrolled round and a tail."""
import numpy as np
import pytest
import torch

import rank_shared_kv_amd as lk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20, (64 << 20) + 2048 * 256 * 16 * 3 + 160])
def test_read_probe_reads_every_chunk_once(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    words = np.random.default_rng(nbytes % 1000).integers(0, 2 ** 31, nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(words).cuda()
    sink = torch.zeros(lk.READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    lk.lrkv_read_probe(src, nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words.view(np.uint32))
