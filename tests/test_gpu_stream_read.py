"""The streaming-read kernel (the measured read ceiling beside the linear):
it must read every word of the buffer once.  The kernel xors every 32-bit
word into the sink, so from a zeroed sink it leaves the xor of the whole
buffer, which the host computes independently."""
import numpy as np
import pytest

SIZES = [16, 4096 + 16, 16384 * 3 + 48, (9 << 20) + 1040, (64 << 20) + 16]


def _words(nbytes, seed):
    return np.random.default_rng(seed).integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", SIZES)
def test_stream_read_folds_every_word(nbytes):
    import torch
    import block_scaled_fp4_act_amd as rs
    w = _words(nbytes, nbytes)
    src = torch.from_numpy(w.view(np.uint8)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rs.stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(w))
    # a second read xors the same value in again: back to zero
    rs.stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.gpu
def test_stream_read_rejects_misaligned_source():
    import torch
    import block_scaled_fp4_act_amd as rs
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        rs.stream_read(buf[4:], torch.zeros(1, dtype=torch.int32, device="cuda"))


@pytest.mark.gpu
def test_stream_read_rejects_ragged_size():
    import torch
    import block_scaled_fp4_act_amd as rs
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        rs.stream_read(buf[:4088], torch.zeros(1, dtype=torch.int32, device="cuda"))
