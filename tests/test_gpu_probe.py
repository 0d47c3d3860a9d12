"""GPU check of the streaming-read probe (dcp_hbm_read_probe), the measured
read ceiling bench.py sets the decode kernels against: every byte of the
buffer is read exactly once, so the XOR of the per-workgroup digests equals
the XOR of every 32-bit word of the buffer, computed on the host. Sizes cover
a buffer smaller than one load per wavefront (most wavefronts read nothing),
runs that end inside an unrolled iteration (a ragged tail), and runs of many
unrolled iterations."""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 77, 64 << 20])
def test_probe_reads_every_word_once(device, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(device)
    blocks = dcp.dcp_hbm_read_probe_blocks()
    digest = torch.zeros(blocks, dtype=torch.int32, device=device)
    dcp.dcp_hbm_read_probe(buf, digest)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(digest.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
