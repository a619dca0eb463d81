"""The roofline probes on the GPU: the copy kernel copies (ragged tail included), every
matrix-core format launches and completes, and the device query answers."""

import numpy as np
import pytest
import torch

from long_context_attention_07_amd import probe

pytestmark = pytest.mark.gpu


def test_device_query():
    n_cu, khz = probe.device()
    print("device", n_cu, "CUs", khz, "kHz", flush=True)
    assert n_cu >= 1 and khz > 0


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 257])
def test_copy_copies(nbytes):
    print("copy", nbytes, flush=True)
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    probe.copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].abs().sum()) == 0  # nothing past the end


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 257])
def test_read_reads_every_word(nbytes):
    print("read", nbytes, flush=True)
    n_cu, _ = probe.device()
    g = torch.Generator(device="cuda").manual_seed(nbytes + 1)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.zeros(4 * probe.STREAM_WG_PER_CU * n_cu, dtype=torch.int32, device="cuda")
    probe.read(src, nbytes, sink)
    torch.cuda.synchronize()
    # the waves' words fold to the XOR of every word read, however the grid split the data
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("fmt", list(probe.FORMATS))
def test_mfma_launches(fmt):
    print("mfma", fmt, flush=True)
    n_wg = 8
    sink = torch.full((n_wg * 4,), float("nan"), dtype=torch.float32, device="cuda")
    probe.mfma(probe.FORMATS[fmt], n_wg, 16, sink)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())  # every wave wrote its value
