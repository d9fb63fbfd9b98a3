"""The HBM probes bench.py takes its ceilings from: the copy reproduces the buffer, and the
read probe's sink words XOR to the XOR of every word it read (each word folded in once)."""
import numpy as np
import pytest
import torch

from speculative_decoding_decode_amd import _lib
from cases import say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (8 << 20) + 16 * 77])
def test_probes(nbytes):
    lib = _lib.load()
    say(f"[probe] {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    s = src.to(dev())
    grid = lib.spec_hbm_probe_grid()
    sink = torch.zeros(4 * grid, dtype=torch.int32, device=dev())
    dst = torch.zeros_like(s)
    stream = torch.cuda.current_stream(dev()).cuda_stream
    _lib.check("spec_hbm_probe", lib.spec_hbm_probe(0, s.data_ptr(), sink.data_ptr(), nbytes,
                                                    stream if stream else None))
    _lib.check("spec_hbm_probe", lib.spec_hbm_probe(1, s.data_ptr(), dst.data_ptr(), nbytes,
                                                    stream if stream else None))
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src)
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
