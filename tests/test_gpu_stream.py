"""The streaming-read ceiling kernel (a measurement aid of the bench) reads
every byte it is given: its XOR checksum equals numpy's on ragged sizes."""
import numpy as np
import pytest
import torch

import bit_quantized_gemv_amd as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 16 * (491520 * 2 + 7), 33216000])
def test_stream_read_checksum(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    buf = host.to("cuda:0")
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    print(f"stream_read {nbytes} B", flush=True)
    assert q.stream_read_ptr(buf.data_ptr(), nbytes, out.data_ptr(), checksum=True,
                             stream=torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    assert (int(out.item()) & 0xffffffff) == want


@pytest.mark.parametrize("shape", [(1, 16, 16, 0), (2, 4, 1, 1), (8, 8, 8, 1), (16, 2, 2, 0)])
def test_stream_read_ex_checksum(shape):
    """Every launch shape of the swept ceiling reads every byte exactly once."""
    nbytes = 16 * (491520 * 3 + 5)
    g = torch.Generator().manual_seed(17)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    buf = host.to("cuda:0")
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    print(f"stream_read_ex {nbytes} B shape {shape}", flush=True)
    assert q.stream_read_ex_ptr(buf.data_ptr(), nbytes, out.data_ptr(), *shape, checksum=True,
                                stream=torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    assert (int(out.item()) & 0xffffffff) == want
