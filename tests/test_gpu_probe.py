"""The HBM rate probes (libepdc_probe.so) on the GPU: the write and copy
kernels produce exactly the documented bytes, and the read kernel reads
every block (its flag fires for the magic a block's words XOR to, and only
then)."""
import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import probe

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 * 37 + 48])
def test_write_and_copy(nbytes):
    print(f"probe write/copy {nbytes} B", flush=True)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    probe.write(dst.data_ptr(), nbytes, 0x1234ABCD, stream())
    torch.cuda.synchronize()
    words = dst[:nbytes].view(torch.int32).cpu().numpy().view(np.uint32)
    want = np.uint32(0x1234ABCD) ^ (np.arange(words.size, dtype=np.uint32) % 4)
    np.testing.assert_array_equal(words, want)
    assert int(dst[nbytes:].sum()) == 0  # nothing past the end
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
    out = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    probe.copy(src.data_ptr(), out.data_ptr(), nbytes, stream())
    torch.cuda.synchronize()
    assert torch.equal(out[:nbytes], src) and int(out[nbytes:].sum()) == 0


def test_read_flag():
    block = 32 << 10  # bytes one read block covers
    nbytes = 3 * block + 4096
    print(f"probe read {nbytes} B", flush=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    host = torch.randint(0, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = host.to(DEV)
    words = host.numpy().view(np.uint32)
    per_block = [int(np.bitwise_xor.reduce(words[i:i + block // 4]))
                 for i in range(0, words.size, block // 4)]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    magic = per_block[-1]  # the short last block
    probe.read(src.data_ptr(), nbytes, magic, flag.data_ptr(), stream())
    torch.cuda.synchronize()
    assert int(flag.item()) & 0xFFFFFFFF == magic
    absent = next(m for m in range(1, 1 << 20) if m not in per_block)
    flag.zero_()
    probe.read(src.data_ptr(), nbytes, absent, flag.data_ptr(), stream())
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
