"""kpa_stream_xor on the GPU: the streaming read the decode kernels' HBM rate
is set against.  Its defined result (per workgroup, the XOR of the 32-bit
words of one contiguous share) is checked against numpy on random bytes, for
ragged sizes, more workgroups than 16-byte words, and the decode-sized grid."""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa

pytestmark = pytest.mark.gpu


def _expected(words32, n_blocks):
    n16 = words32.size // 4
    share = -(-n16 // n_blocks)
    out = np.zeros(n_blocks, np.uint32)
    for w in range(n_blocks):
        lo, hi = w * share, min((w + 1) * share, n16)
        if lo < hi:
            out[w] = np.bitwise_xor.reduce(words32[4 * lo:4 * hi])
    return out


@pytest.mark.parametrize("nbytes,n_blocks", [(16, 1), (1048576 + 48, 7), (4096, 1000), (64 << 20, 768),
                                             ((3 << 20) + 16 * 1001, 257)])
def test_stream_xor_matches_numpy(gpu_lib, nbytes, n_blocks):
    g = torch.Generator().manual_seed(nbytes % 1000 + n_blocks)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4 + 8,), generator=g, dtype=torch.int32)
    buf = host.cuda()
    partial = torch.full((n_blocks + 1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    kpa.kpa_stream_xor(buf, partial, n_blocks=n_blocks, nbytes=nbytes)
    torch.cuda.synchronize()
    got = partial.cpu().numpy().view(np.uint32)
    want = _expected(host.numpy().view(np.uint32)[:nbytes // 4], n_blocks)
    assert np.array_equal(got[:n_blocks], want)
    assert got[n_blocks] == 0x5A5A5A5A  # nothing past n_blocks is written


def test_stream_xor_kernel_timing_hook(gpu_lib):
    buf = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    partial = torch.zeros(768, dtype=torch.int32, device="cuda")
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()  # created on the device before the hook stamps them
    torch.cuda.synchronize()
    assert kpa.load().kpa_time_next_decode_kernel(a.cuda_event, b.cuda_event) == 0
    kpa.kpa_stream_xor(buf, partial)
    torch.cuda.synchronize()
    t = a.elapsed_time(b)
    assert 0 < t < 50.0
    assert int(partial.abs().sum().item()) == 0
