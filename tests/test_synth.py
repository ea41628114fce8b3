"""The seeded input generator: partial draws equal the slices of whole draws
(the CPU oracle's workers draw only the rows they need)."""

import numpy as np
import torch

from block_sparse_masked_mask_amd import synth


def test_normal_range_equals_slices_across_chunks():
    n = 2 * synth.CHUNK + 12345
    whole = synth.normal((n,), 3, synth.TID_K, scale=0.5)
    for lo, hi in ((0, 10), (5, synth.CHUNK + 7), (synth.CHUNK - 3, synth.CHUNK + 3),
                   (synth.CHUNK, 2 * synth.CHUNK), (2 * synth.CHUNK + 100, n), (7, 7)):
        np.testing.assert_array_equal(synth.normal_range(3, synth.TID_K, lo, hi, 0.5),
                                      whole[lo:hi], err_msg=f"[{lo}, {hi})")


def test_normal_rows_equal_tensor_rows():
    shape = (3, 5000, 4, 128)   # 7.7M elements: batches straddle chunk boundaries
    whole = synth.normal_tensor(shape, 1, synth.TID_Q, "bf16", 0.5)
    for b, r0, r1 in ((0, 0, 128), (1, 4000, 5000), (2, 17, 18), (1, 0, 5000)):
        got = synth.normal_rows(shape, 1, synth.TID_Q, b, r0, r1, "bf16", 0.5)
        assert got.shape == (1, r1 - r0, 4, 128)
        assert torch.equal(got, whole[b:b + 1, r0:r1])
