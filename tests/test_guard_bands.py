"""The guard-band allocator of the GPU tests on the CPU: buffers are views
inside sentinel margins, a write past either end is reported, and the
binding's allocator is restored afterwards."""
import pytest
import torch

import bit_microscaled_numerics_amd as nv
import parity


def test_views_sit_inside_the_margins_and_overruns_are_caught(monkeypatch):
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    g = parity.GuardBands()
    a = g.empty(3, 5, dtype=torch.float32, device="cpu")
    assert a.shape == (3, 5) and a.dtype == torch.float32 and a.is_contiguous()
    assert (a.data_ptr() - g.bufs[-1][0].data_ptr()) == parity.GUARD_BYTES
    a.fill_(1.0)
    g.check()                                   # writes inside: fine
    b = g.empty(16, dtype=torch.uint8, device="cpu")
    raw, n = g.bufs[-1]
    raw[parity.GUARD_BYTES + n] = 0             # one byte past the end
    with pytest.raises(AssertionError, match="outside an output buffer"):
        g.check()
    del b


def test_context_restores_the_allocator(monkeypatch):
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    saved = nv._empty
    with parity.guard_bands() as g:
        assert nv._empty == g.empty
        t = nv._empty(4, dtype=torch.uint8, device="cpu")
        t.fill_(7)
    assert nv._empty is saved
