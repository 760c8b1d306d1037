"""The packed expert-weight layout (include/zc_moe.h, zc_moe_pack_weights) as
the GPU tests check it: the numpy permutation they compare against is pinned
here, element by element, to the index formula the header documents."""
import numpy as np

from tests import gpu_harness as H


def test_pack_reference_follows_the_documented_formula():
    rng = np.random.default_rng(0)
    n, R, C = 2, 64, 48
    w = rng.integers(0, 1 << 16, size=(n, R, C), dtype=np.uint16)
    p = H.pack_ref(w).reshape(n, -1)
    for m in range(n):
        for r in range(R):
            for c in range(C):
                idx = ((r // 32) * (C // 16) + c // 16) * 512 + (r % 32 + 32 * ((c // 8) % 2)) * 8 + c % 8
                assert p[m, idx] == w[m, r, c]


def test_pack_reference_is_a_permutation_of_whole_16_byte_chunks():
    # every 8-element chunk of a packed block is 8 consecutive reduction steps
    # of one output column: what one lane loads as an MFMA operand
    n, R, C = 1, 96, 64
    w = np.arange(n * R * C, dtype=np.int64).reshape(n, R, C)
    chunks = H.pack_ref(w).reshape(-1, 8)
    assert (np.diff(chunks, axis=1) == 1).all()
    assert sorted(chunks[:, 0]) == sorted(w.reshape(-1, 8)[:, 0])
