"""GPU check of the counter-calibration stream (global -> LDS copies of a
known size): it runs on every slice of the source and each slice's sink word
holds four source bytes as they landed in LDS."""

import pytest
import torch

from segment_autoregressive_dit_amd import nomas

from _gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1024, 5 << 20, (3 << 20) + 7 * 1024])
def test_lds_stream_reads_every_slice(nbytes):
    say(f"calibrate: lds stream of {nbytes} bytes")
    src = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(nomas.lib().nomas_calibrate_lds_stream_blocks(nbytes) + 1, dtype=torch.int32, device="cuda")
    nomas.nomas_calibrate_lds_stream(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().tolist()
    assert got[:-1] == [0x5A5A5A5A] * (len(got) - 1)
    assert got[-1] == 0   # nothing written past the slices
