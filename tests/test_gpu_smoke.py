"""The package's smoke check (two fused AdamW steps on three ragged tensors,
compared with the oracle bit for bit), run as a test so that a change to the
state layout or the binding that breaks it fails the GPU suite."""
import pytest


@pytest.mark.gpu
def test_smoke():
    import __graft_entry__
    __graft_entry__.smoke()
