"""The kernels' fp32 -> e4m3fn conversion against the oracle encoder, over
every binary32 value with |y| < 464 (both signs), through the C-ABI."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
from gpu_util import DEV, assert_equal, say

pytestmark = pytest.mark.gpu

TOP = int(np.float32(464.0).view(np.uint32))  # first pattern not compared
CHUNK = 1 << 27


def test_encode_fixed_values():
    vals = np.array([448.0, 449.0, 463.9, 2.0 ** -10, 1.5 * 2.0 ** -10, -0.0,
                     2.0 ** -9, 2.0 ** -6, 1.0, 1.0625, 1.1875, 432.0, -448.0,
                     0.0, 1e-40, -1e-40], np.float32)
    say("codec fixed values")
    got = mxq.mxq_e4m3_encode_f32(torch.from_numpy(vals).to(DEV)).cpu().numpy()
    import oracle
    assert_equal(got, oracle.e4m3_encode(vals), "fixed values")


def test_encode_odd_lengths():
    import oracle
    rng = np.random.default_rng(0)
    for n in (1, 2, 3, 5, 7, 1023, 4097):
        v = (rng.standard_normal(n) * 50).astype(np.float32)
        say("codec length", n)
        got = mxq.mxq_e4m3_encode_f32(torch.from_numpy(v).to(DEV)).cpu().numpy()
        assert_equal(got, oracle.e4m3_encode(v), "n=%d" % n)


def test_encode_exhaustive_below_464():
    import oracle
    for w0 in range(0, TOP, CHUNK):
        n = min(CHUNK, TOP - w0)
        say("codec exhaustive chunk", hex(w0), n)
        bits = torch.arange(w0, w0 + n, dtype=torch.int32, device=DEV)
        x = bits.view(torch.float32)
        got_pos = mxq.mxq_e4m3_encode_f32(x).cpu().numpy()
        got_neg = mxq.mxq_e4m3_encode_f32(-x).cpu().numpy()
        del bits, x
        want_pos = oracle.e4m3_encode_bits_range(w0, n)
        assert_equal(got_pos, want_pos, "positive chunk %#x" % w0)
        want_neg = oracle.e4m3_encode_bits_range(w0 | 0x80000000, n)
        assert_equal(got_neg, want_neg, "negative chunk %#x" % w0)
