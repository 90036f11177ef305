"""GPU checks of the benchmark hooks: the streaming-read kernel reads every
vector of its buffer, tail included, and nothing beyond it; the device
query reports this device.

The read kernel combines each thread's words with XOR and stores the magic
word 0x9e3779b9 only when that combination equals it.  In a zero buffer with
the magic word at one position, exactly the thread that loads that vector
stores it, so the sink shows whether that position was read.
"""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAGIC = 0x9E3779B9


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def _read(rk, buf, nbytes, grid, sink):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rk.rk_debug_stream_read(buf.data_ptr(), nbytes, grid, sink.data_ptr(), st)
    torch.cuda.synchronize()


@pytest.mark.parametrize("nvec", [1, 7, 2048, 2049, 65536 + 13, 1_000_003])
@pytest.mark.parametrize("grid", [0, 1, 3, 512])
def test_stream_read_reaches_every_vector(nvec, grid):
    rk = _rk()
    words = torch.zeros(4 * nvec + 8, dtype=torch.int32, device=DEV)   # 2 vectors of guard after
    magic = torch.tensor([MAGIC], dtype=torch.int64).to(torch.int32).item()
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for pos in sorted({0, nvec // 2, nvec - 1}):
        words.zero_()
        words[4 * pos + pos % 4] = magic
        sink.zero_()
        _read(rk, words, 16 * nvec, grid, sink)
        assert sink.item() == magic, (nvec, grid, pos)
    # a magic word just past the end is never read
    words.zero_()
    words[4 * nvec] = magic
    sink.zero_()
    _read(rk, words, 16 * nvec, grid, sink)
    assert sink.item() == 0


def test_device_info():
    rk = _rk()
    info = rk.rk_debug_device_info()
    assert info["num_cus"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert info["mem_clock_khz"] > 0 and info["mem_bus_bits"] > 0
