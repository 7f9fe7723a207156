"""The read-rate probe (nvfp4_read_probe) reads every 16-byte chunk of its buffer
exactly once: each workgroup's XOR fold equals the XOR of the 32-bit words of its
contiguous share, including shares past the end (fold 0) when there are more
workgroups than chunks."""
import numpy as np
import pytest

from gpu_util import DEV, nv, say, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (4096, 300), ((1 << 20) + 48, 7), (1 << 22, 256),
                                       (12288 * 5120 * 9 // 16, 256), (12288 * 5120 * 9 // 16, 1024)])
def test_read_probe_folds_every_chunk_once(nbytes, wg):
    say(f"[read probe] bytes={nbytes} workgroups={wg}")
    g = torch.Generator(device="cpu").manual_seed(nbytes + wg)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(DEV)
    sink = torch.full((wg,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    nv.nvfp4_read_probe(buf, nbytes, wg, sink)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32)
    n16 = nbytes // 16
    per = -(-n16 // wg)
    want = np.zeros(wg, dtype=np.uint32)
    for b in range(wg):
        lo, hi = min(b * per, n16) * 4, min((b + 1) * per, n16) * 4
        if hi > lo:
            want[b] = np.bitwise_xor.reduce(words[lo:hi])
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
