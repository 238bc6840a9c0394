"""The read-ceiling probe (a measurement helper): it reads and leaves its sink alone."""
import pytest
import torch

import ssm_decode_amd as rs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 4096 + 4, 3 << 20])
def test_probe_read_runs_and_keeps_sink(n):
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    rs.probe_read(src, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0.0
