"""The streaming-read reference of the measurements (kvq_stream_read): every
workgroup reads exactly its slice, checked through the XOR of the words each
one read, on slices that do not divide evenly."""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("threads", [256, 1024])
@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096, 3), (1 << 20, 7), (9479168, 256), (3 * 16 * 1024 + 48, 5),
                                         (9479168, 2048)])
def test_stream_read_covers_each_slice_once(nbytes, grid, threads):
    import torch

    import decode_attention_quantized_amd as kvq
    say("case stream read", nbytes, "bytes over", grid, "workgroups of", threads)
    rng = np.random.default_rng(nbytes + grid)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).cuda()
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    kvq.kvq_stream_read(src, grid, sink, threads=threads)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    words = host.reshape(n16, 4)
    want = np.array([np.bitwise_xor.reduce(words[n16 * g // grid:n16 * (g + 1) // grid].ravel(), initial=np.uint32(0))
                     for g in range(grid)], dtype=np.uint32)
    assert np.array_equal(got, want)
