"""GPU: the measurement probes compute what their header says. With all-ones
bf16 operands every MFMA adds K products of 1 to each accumulator element, so
the per-thread checksum is exact in float32: 32x32x16 loop, 4 accumulators of
16 elements, each gaining 4 MFMAs x 16 per iteration; 16x16x32 loop, 8
accumulators of 4 elements, each gaining 4 MFMAs x 32 per iteration: 4096 per
iteration either way. The streaming read's per-thread XOR checksums, XORed
together, equal the XOR of the whole buffer's 32-bit words."""
import numpy as np
import pytest

import global_attention_amd as ga

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [32, 16])
def test_mfma_probe_checksum(shape):
    import torch
    nb, iters = 8, 10
    ones = torch.ones((nb * 256 * 128,), device="cuda").to(torch.bfloat16).view(torch.int32)
    out = torch.full((nb * 256,), -1.0, dtype=torch.float32, device="cuda")
    probe = ga.probe_mfma_bf16 if shape == 32 else ga.probe_mfma16_bf16
    flops = probe(ones, nb, iters, 1, out)
    torch.cuda.synchronize()
    assert flops == nb * 4 * iters * 16 * 32768
    assert torch.all(out == 4096.0 * iters), out[:8]


def test_mfma_probe_arguments():
    import torch
    ops = torch.zeros((256 * 64,), dtype=torch.int32, device="cuda")
    for probe in (ga.probe_mfma_bf16, ga.probe_mfma16_bf16):
        with pytest.raises(ga.BeamError) as e:
            probe(ops, 1, 10, 9)
        assert e.value.status == 3


def test_stream_read_checksum():
    import torch
    n = 1 << 20
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int64, device="cuda").to(torch.int32)
    nb = 64
    out = torch.empty((nb * 256,), dtype=torch.int32, device="cuda")
    nbytes = ga.probe_stream_read(buf, nb, out)
    torch.cuda.synchronize()
    assert nbytes == 4 * n
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    assert got == want
