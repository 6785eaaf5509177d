"""GPU nvfp4_to_w2 against the exact oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import requant
import workloads

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _gpu(e2m1, e4m3, s2):
    codes, scales = moe.nvfp4_to_w2(dev(e2m1), dev(e4m3), dev(np.asarray(s2, np.float32)))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_workload_tensors_bit_exact(gpu):
    tens = [workloads.nvfp4_tensor(i, R=64, C=6144) for i in range(3)]
    e2m1 = np.stack([t[0] for t in tens]); e4m3 = np.stack([t[1] for t in tens])
    s2 = np.array([t[2] for t in tens], np.float32)
    c, s = _gpu(e2m1, e4m3, s2)
    wc, ws = requant.nvfp4_to_w2(e2m1, e4m3, s2, window=False)
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


def test_full_range_inputs_bit_exact(gpu):
    rng = np.random.default_rng(13)
    n, R, C = 24, 16, 256
    e2m1 = rng.integers(0, 256, size=(n, R, C // 2), dtype=np.uint8)
    e4m3 = rng.integers(0, 256, size=(n, R, C // 16), dtype=np.uint8)
    e4m3[(e4m3 & 0x7F) == 0x7F] = 0x00
    s2 = (2.0 ** rng.integers(-149, 127, size=n) * rng.uniform(1, 2, size=n)).astype(np.float32)
    s2[0] = np.float32(1.4e-45)     # smallest subnormal
    s2[1] = np.float32(3.4e38)
    s2[2] = np.float32(-0.01)       # negative per-tensor scale flips every sign
    s2[3] = np.float32(0.0)
    # constructed blocks: all zero (+0 / -0), single magnitude, midpoint
    e2m1[4, 0, :16] = 0x00; e2m1[4, 0, 16:] = 0x88
    e2m1[5, 0, :16] = 0x22; e4m3[5, 0, :2] = 0x38
    c, s = _gpu(e2m1, e4m3, s2)
    wc, ws = requant.nvfp4_to_w2(e2m1, e4m3, s2, window=False)
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


def test_nan_inputs_are_reported(gpu):
    e2m1 = np.zeros((1, 1, 16), np.uint8)
    e4m3 = np.array([[[0x38, 0x7F]]], np.uint8)
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(e2m1, e4m3, np.array([1.0], np.float32))
    assert ei.value.status == -7
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(e2m1, np.array([[[0x38, 0x38]]], np.uint8), np.array([np.inf], np.float32))
    assert ei.value.status == -7
