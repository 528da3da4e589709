"""Key-block summaries of the host library (kvq_key_norms) against the
oracle's definition (oracle.kskip.cache_block_norms): bit-exact for every
format, capacities with a partial last block, unwritten (zero) rows and
extreme scales. CPU only."""
import numpy as np
import pytest

import decode_attention_quantized_amd as kvq
from oracle import formats as F
from oracle import kskip as K


@pytest.mark.parametrize("fmt,dim", [("q8_0", 128), ("q4_0", 128), ("lut3", 128), ("lut3_wht", 128),
                                     ("fp8_b128", 576), ("q8_0", 64), ("q4_0", 256)])
@pytest.mark.parametrize("cap", [1, 64, 150, 256])
def test_host_summaries_match_the_oracle(fmt, dim, cap):
    rng = np.random.default_rng(cap * 7 + dim)
    x = rng.standard_normal((2, 3, cap, dim)) * rng.uniform(0.01, 30.0, (2, 3, cap, 1))
    x[0, 1, : cap // 2] = 0.0                           # never-written rows read as zero planes
    x = x.astype(np.float32)
    codes, scales = F.pack(fmt, x)
    got = kvq.kvq_key_norms(fmt, codes, scales, dim)
    want = K.cache_block_norms(fmt, codes, scales, dim)
    assert got.shape == want.shape == (2, 3, (cap + 63) // 64)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), fmt


def test_host_summaries_reject_bad_arguments():
    codes = np.zeros((1, 1, 64, 64), np.uint8)
    scales = np.zeros((1, 1, 64, 8), np.uint8)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_key_norms("q4_0", codes, scales, 100)   # dim not a multiple of 32
