"""GPU check of the streaming-read probe used as the bandwidth reference for
decode: it must read every byte of both buffers exactly once, which the XOR of
all their 32-bit words (computed on the host) pins."""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 * (1 << 20) + 48, 64 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    print(f"[read probe] {nbytes} bytes per buffer", flush=True)
    g = torch.Generator().manual_seed(nbytes % 1000003)
    a = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    b = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    want = np.bitwise_xor.reduce(np.concatenate([a.numpy(), b.numpy()]).view(np.uint32))
    for words in (1, 7, 1024):
        sink = torch.zeros(words, dtype=torch.int32, device="cuda")
        pa.read_probe(a.cuda(), b.cuda(), sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert int(got) == int(want), words
        # a second call folds the same value in again: XOR back to zero
        pa.read_probe(a.cuda(), b.cuda(), sink)
        torch.cuda.synchronize()
        assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == 0
