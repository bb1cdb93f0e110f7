"""GPU check of qd_stream_read, the read-only stream the GEMV's bandwidth is
compared against: it reads the whole buffer and writes the sink only when
the XOR of every loaded word is 0x9E3779B9."""
import numpy as np
import pytest
import torch

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9


@pytest.mark.parametrize("nbytes", [16, 2048, 4096 + 16, 9437184])
def test_stream_reads_every_word(nbytes):
    # the marker word sits in the last 16 bytes: the sink is written only if
    # the reads reach the end of the buffer (and read nothing beyond it)
    words = np.zeros(nbytes // 4, np.uint32)
    words[-4] = MARK
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    qd.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) & 0xFFFFFFFF == MARK


def test_stream_leaves_the_sink_alone():
    buf = torch.randint(-2**31, 2**31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    qd.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
