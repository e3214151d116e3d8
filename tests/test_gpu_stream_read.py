"""GPU: dflash_stream_read, the plain read the bench sets the attention against,
and dflash_mfma_peak, the matrix-core probe beside the projections.

The kernel folds every 16-byte word a lane reads into one value by XOR and
stores it only when it equals one constant.  A buffer of zeros holding that
constant in a single word therefore shows which words were read: the sink is
written exactly when the planted word lies inside the range, at the start,
the end, a grid-stride boundary or a ragged tail.  (Two lanes never fold the
same word, so no other lane can cancel it.)
"""
import ctypes as C

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU visible", allow_module_level=True)

from block_diffusion_draft_fc_amd import _lib as L  # noqa: E402

MAGIC = 0x9E3779B9


def _read(nbytes, planted_word):
    """Words of 16 bytes; the one at index planted_word carries the constant."""
    words = max(nbytes // 16, planted_word + 1) + 4
    buf = torch.zeros(words * 4, dtype=torch.int32, device="cuda")
    buf[4 * planted_word] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = L.LIB.dflash_stream_read(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(sink.data_ptr()), None)
    assert st == 0
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("n16", [1, 7, 1024, 1025, 4096 * 3 + 5, 8192 * 1024 + 3, 8192 * 1024 * 2 + 17])
def test_stream_read_covers_its_range(n16):
    nbytes = 16 * n16
    inside = sorted({0, 1, 255, 256, 1023, 1024, n16 // 2, n16 - 1} & set(range(n16)))
    for w in inside:
        assert _read(nbytes, w) == MAGIC, f"word {w} of {n16} not read"
    # the word just past the range is never read (nor a partial last word)
    assert _read(nbytes, n16) == 0
    assert _read(nbytes + 15, n16) == 0


def test_mfma_peak_runs_and_writes_nothing():
    """The probe's accumulators never reach the stored value: the sink keeps
    its bits, and a timed run reports a positive rate."""
    sink = torch.full((1,), -7.0, dtype=torch.float32, device="cuda")
    assert L.LIB.dflash_mfma_peak(64, 512, C.c_void_p(sink.data_ptr()), None) == 0
    torch.cuda.synchronize()
    assert sink.item() == -7.0
    L.timing_reset()
    L.timing_enable(True)
    L.dflash_mfma_peak(256, 1024)
    torch.cuda.synchronize()
    n, ms = L.timing_read()["mfma_peak"]
    L.timing_enable(False)
    assert n == 1 and ms > 0
