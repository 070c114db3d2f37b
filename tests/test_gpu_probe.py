"""The read-bandwidth probe (include/iq_probe.h) on the GPU: it reads a
buffer through the C ABI, returns IQ_OK and leaves the sink untouched for
data whose fold is not the probe's fixed value."""

import pytest

from compressed_space_attention_isoquant_amd import binding as B
from tests.gpu_helpers import DEV, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 64 << 20])
def test_probe_reads_buffer(nbytes):
    t = torch()
    buf = t.zeros(nbytes, dtype=t.uint8, device=DEV)
    sink = t.full((1,), 7, dtype=t.int32, device=DEV)
    B.iq_probe_stream_read(buf, sink)
    t.cuda.synchronize()
    assert int(sink.item()) == 7
