"""CPU checks of the input generators the GPU tests use for tensors too large to draw on the
host: the torch MXFP4 encoder must write exactly the bytes the oracle's encoder writes
(ties to even, saturation, -0, zero and subnormal blocks), so that device-drawn MXFP4
inputs follow the same recipe as host-drawn ones."""

import numpy as np
import torch

from oracle import formats as F

from harness import device_outlier_normal, mxfp4_encode_torch


def test_mxfp4_torch_encoder_matches_oracle():
    g = np.random.default_rng(5)
    x = (g.standard_normal((4000, 128)) * np.exp(g.uniform(-20, 20, (4000, 1)))).astype(np.float32)
    # exact ties on the e2m1 grid at every step size, saturation, signed zeros
    x[0, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -0.75, 0.0, -0.0, 6.0, -6.0, 0.1, 0.2]
                         + [1.0] * 16, dtype=np.float32)
    x[1, :32] = 0.0
    x[1, 32:64] = -0.0
    x[2, :32] = np.float32(2.0 ** -130)   # subnormal float32 block
    x[3, :32] = np.float32(3.0 * 2.0 ** 100)
    p, s = mxfp4_encode_torch(torch.from_numpy(x))
    pr, sr = F.quant_mxfp4(x.astype(np.float64))
    assert np.array_equal(p.numpy(), pr)
    assert np.array_equal(s.numpy(), sr)


def test_device_outlier_normal_recipe():
    gen = torch.Generator()
    gen.manual_seed(3)
    x = device_outlier_normal(gen, (2000, 512), "cpu")
    big = (x.abs() > 12).float().mean().item()
    assert 0.0005 < big < 0.0015, big          # Bernoulli(0.001) outliers at +-20
    assert abs(x[x.abs() < 8].std().item() - 1.0) < 0.01
