"""The round-end smoke entry point (`__graft_entry__.smoke()`): one small layer through the C ABI,
checked against the oracle.  Run here so that a change to the layer's call sequence cannot leave it
checking a buffer the layer no longer writes."""
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def test_smoke_entry_point():
    print("\n[gpu] __graft_entry__.smoke()", flush=True)
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import __graft_entry__
    __graft_entry__.smoke()
