"""spec_lm_head_noalloc (the lm-head entry point that allocates nothing: its scratch is a
static device array) against spec_lm_head with a workspace: logits and p bit-identical, on two
calls in a row, the second smaller than the first (the array keeps the first call's
statistics, which the second must not read), then once more at the first size."""
import math

import numpy as np
import pytest
import torch

import speculative_decoding_decode_amd as sv
from speculative_decoding_decode_amd import _lib
from cases import say, dev

pytestmark = pytest.mark.gpu


def inputs(R, H, V, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(R, H, generator=g).to(dtype)
    W = (torch.randn(V, H, generator=g) / math.sqrt(H)).to(dtype)
    t = torch.tensor([(1.0, 0.0, 0.7, 2.0)[r % 4] for r in range(R)], dtype=torch.float32)
    return x.to(dev()), W.to(dev()), t.to(dev())


def noalloc_call(x, W, t, logits, probs):
    lib = _lib.load()
    R, H = x.shape
    V = W.shape[0]
    s = torch.cuda.current_stream(dev()).cuda_stream
    rc = lib.spec_lm_head_noalloc(x.data_ptr(), W.data_ptr(), t.data_ptr(), logits.data_ptr(),
                                  probs.data_ptr(), R, H, V,
                                  sv.SPEC_BF16 if x.dtype == torch.bfloat16 else sv.SPEC_F32,
                                  s if s else None)
    _lib.check("spec_lm_head_noalloc", rc)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_workspace_entry_point(dtype):
    shapes = [(96, 2560, 50021), (3, 1032, 4099), (96, 2560, 50021)]
    for i, (R, H, V) in enumerate(shapes):
        say(f"[noalloc] call {i}: R={R} H={H} V={V} {dtype}")
        x, W, t = inputs(R, H, V, dtype, seed=100 + i)
        ref_z, ref_p = sv.lm_head(x, W, t, want_logits=True)
        z = torch.full((R, V), float("nan"), device=dev())
        p = torch.full((R, V), float("nan"), device=dev())
        noalloc_call(x, W, t, z, p)
        torch.cuda.synchronize()
        assert torch.equal(z, ref_z)
        assert torch.equal(p, ref_p)
        np.testing.assert_allclose(p.double().sum(1).cpu().numpy(), 1.0, atol=1e-5)
