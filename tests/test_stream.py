"""GPU check of the streaming-read reference kernel (mxgemm_stream_read):
it runs on buffers of several sizes (whole and partial sweeps of its grid)
and leaves its sink word alone for data whose XOR is not its trigger."""
import pytest

import block_scaled_precision_mxfp4_amd as mx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, 35672320, (1 << 31) - 16])
def test_stream_read_runs_and_leaves_sink(nbytes):
    mx.lib()
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 0x1234, dtype=torch.int32, device="cuda")
    mx.mxgemm_stream_read(src, nbytes, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0x1234
