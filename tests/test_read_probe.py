"""The read probe (GPU): every 16-byte word read once, whatever the grid size.

The sum of the per-group partials (wrapping 32-bit adds) must equal the sum of all 32-bit words
of the buffer modulo 2^32, computed here on the host. A wrong stride, a skipped tail or a word
read twice changes the sum.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

import lossless_draft_verification_sv_amd as sv  # noqa: E402
from tests.gpu_util import say  # noqa: E402


@pytest.mark.parametrize("nbytes,groups", [(16, 1), (4096, 3), (1 << 20, 256),
                                            ((1 << 24) + 48, 2048), (1000 * 16, 8192)])
def test_probe_reads_every_word_once(nbytes, groups):
    rng = np.random.default_rng(nbytes + groups)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    say(f"[gpu] read probe {nbytes} bytes, {groups} groups")
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    part = sv.sv_read_probe(dev, groups)
    torch.cuda.synchronize()
    got = int(part.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % 2**32
    want = int(host.astype(np.uint64).sum()) % 2**32
    assert got == want
