"""The plain read kernel that sets the decode rate beside the part's practical
read ceiling (tq_read_probe): it must read every 16-byte piece of the buffer
exactly once, which the XOR of the buffer's 32-bit words shows (a missed or
repeated piece changes it, up to chance)."""
import numpy as np
import pytest
import torch

from kv_cache_vector_06_amd import torch_api as T
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32))) if a.size else 0


# 16 B; under one workgroup; several workgroups with a ragged end; more than
# one full round of the grid plus a tail of single loads.
@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, (1 << 20) + 7 * 16, (64 << 20) + 48])
def test_read_probe_reads_every_word_once(nbytes):
    say(f"read probe: {nbytes} bytes")
    g = np.random.default_rng(91 + nbytes % 1000)
    host = g.integers(0, 256, size=nbytes + 16, dtype=np.uint8)
    buf = torch.from_numpy(host).to(DEV)
    view = buf[16:]                                  # a 16-byte aligned view at an offset
    xo = torch.tensor([0x12345678], dtype=torch.int32, device=DEV)
    T.read_probe(view, xo)
    got = int(xo.cpu().numpy().view(np.uint32)[0])
    assert got == 0x12345678 ^ _xor_words(host[16:])
    xo.zero_()
    T.read_probe(view, xo)
    T.read_probe(view, xo)                           # twice: XORs cancel
    torch.cuda.synchronize()
    assert int(xo.cpu()[0]) == 0
