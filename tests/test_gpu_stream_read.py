"""qmvdbg_stream_read, the streaming-read ceiling that bench.py reports next to
the GEMV bandwidths: every 32-bit word of the buffer is read exactly once,
checked through the per-workgroup XORs it stores (a word read twice or
skipped changes their XOR), for ragged sizes and grids (more workgroups than
16-byte words included), with the 65 MB of one C2 matrix."""
import numpy as np
import pytest
import torch

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 65028096])
@pytest.mark.parametrize("workgroups", [1, 7, 2048])
def test_every_word_read_once(nbytes, workgroups):
    say(f"qmvdbg_stream_read bytes={nbytes} workgroups={workgroups}")
    qmv = _qmv()
    rng = np.random.default_rng(nbytes % 1000 + workgroups)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = dev(words.view(np.uint8))
    out = torch.full((workgroups + 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda:0")
    qmv.qmvdbg_stream_read(buf, nbytes, out, workgroups)
    got = out.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(got[:workgroups]) == np.bitwise_xor.reduce(words)
    assert np.all(got[workgroups:] == 0x5A5A5A5A)
