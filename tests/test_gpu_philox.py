"""The device Philox stream against the oracle's, bit for bit, over more than
10^7 counters.

The accept test and the draws take U(seed, row, pos, tag) = (w >> 8) * 2^-24,
w the first output word of Philox4x32-10 (Salmon et al., SC'11) at counter
(pos, row, tag, 0) under key (low, high 32 bits of the seed): the uniforms
keyed by (seed, batch row, position) that make the decisions reproducible.
The oracle's generator is pinned against rocRAND's engine in
test_oracle_philox.py; here the library's device copy (spec_philox_uniforms,
the same device function the kernels call) must equal it on every counter of
blocks that cover small and huge seeds, all tags the path uses plus others,
and rows and positions next to 0 and next to 2^32 (where they wrap).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

BLOCKS = [
    # seed, row0, nrow, pos0, npos, tag
    (0, 0, 128, 0, 8192, 0),
    (0, 0, 128, 0, 8192, 1),
    (1, 0, 64, 0, 16384, 2),
    (12345678901234567, 7, 256, 0, 4096, 0),
    (2 ** 64 - 1, 2 ** 32 - 100, 200, 0, 4096, 1),
    (0xDEADBEEF00000000, 0, 64, 2 ** 32 - 2048, 4096, 0),
    (0x00000000CAFEBABE, 1000, 128, 2 ** 31 - 1000, 8192, 3),
    (2 ** 63, 5, 64, 17, 8192, 0xFFFFFFFF),
    (987654321, 0, 512, 0, 2048, 1),
    (42, 0, 1024, 0, 3072, 0),
]


def test_blocks_cover_ten_million_counters():
    assert sum(b[2] * b[4] for b in BLOCKS) >= 10_000_000


@pytest.mark.parametrize("blk", BLOCKS, ids=[f"seed{b[0]:x}_row{b[1]}_pos{b[3]}_tag{b[5]}" for b in BLOCKS])
def test_device_philox_equals_oracle(blk):
    import lossless_draft_verification_amd as L
    seed, row0, nrow, pos0, npos, tag = blk
    got = L.philox_uniforms(seed, row0, nrow, pos0, npos, tag)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    want = oracle.default().uniform_grid(seed, row0, nrow, pos0, npos, tag)
    bad = np.nonzero(g != want)
    assert bad[0].size == 0, (blk, bad[0][:5], bad[1][:5], g[bad][:5], want[bad][:5])
    # 24-bit uniforms in [0, 1 - 2^-24]
    assert g.min() >= 0.0 and g.max() <= 1.0 - 2.0 ** -24
    assert np.all(g * 2.0 ** 24 == np.floor(g * 2.0 ** 24))
