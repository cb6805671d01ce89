"""The read-stream reference the benchmark prints beside every decode
fraction (kvq_read_stream): it must read every byte it is given, so each
16 KB chunk's XOR of 32-bit words is checked against numpy, bit for bit,
including a short last chunk and a single-load buffer."""
import numpy as np
import pytest
import torch

import mixed_precision_kv_amd as kvq

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]


@pytest.mark.parametrize("nbytes", [16, 16384, 3 * 16384 + 4096 + 48, 11776 * 257])
def test_read_stream_reads_every_byte(nbytes):
    print(f"\n[case] read stream {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    chunks = (nbytes + 16383) // 16384
    sink = torch.full((chunks + 1,), -1, dtype=torch.int32, device="cuda")   # one word past the chunks
    kvq.kvq_read_stream(src, nbytes, sink, chunks * 4)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = np.zeros(chunks * 4096, dtype=np.uint32)
    words[:nbytes // 4] = host.view("<u4")
    want = np.bitwise_xor.reduce(words.reshape(chunks, 4096), axis=1)
    assert np.array_equal(got[:chunks], want)
    assert got[chunks] == 0xFFFFFFFF   # nothing written past the chunks
