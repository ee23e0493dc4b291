"""The read-bandwidth probe (a measurement utility of the library, not a step
of the path) through the C ABI: it reads every byte once, and each
workgroup's word is the XOR of the 16-byte pieces it covers (workgroup b
reads pieces j with (j // 1024) % num_blocks == b), checked against the
same XOR on the host for a ragged size."""

import numpy as np
import pytest
import torch

from sparse_attention_09_amd import dsa
from tests._harness import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pieces,blocks", [(1, 1), (5000, 3), (70001, 8)])
def test_read_probe_reads_every_piece_once(pieces, blocks):
    g = np.random.default_rng(pieces)
    host = g.integers(0, 2**32, size=(pieces, 4), dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda:0")
    say(f"[case] read probe pieces={pieces} blocks={blocks}")
    dsa.read_probe(buf, out)
    torch.cuda.synchronize()
    words = np.bitwise_xor.reduce(host, axis=1)
    owner = (np.arange(pieces) // 1024) % blocks
    want = np.array([np.bitwise_xor.reduce(words[owner == b]) if (owner == b).any() else 0
                     for b in range(blocks)], dtype=np.uint32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
