"""ffnq_stream_read, the plain streaming read that bench.py sets beside the
weight-streaming kernels: it runs over sizes with a ragged tail (not a multiple
of its grid's threads), leaves the buffer and the sink as they were, and its
launch takes the timing events."""
import pytest
import torch

import moe_expert_dequant_amd as fq
from test_gpu_parity import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (33 << 20) + 16 * 7])
def test_stream_read(nbytes):
    say("stream read", nbytes)
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")   # every 32-bit word 0x01010101: the fold is 0
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = fq.PhaseEvents()
    with ev:
        fq.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert bool((buf == 1).all())
    assert ev.durations()[0] > 0.0
