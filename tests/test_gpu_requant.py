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


def test_half_blocks_at_opposite_scale_ends_bit_exact(gpu):
    """The two 16-element halves of each 32-block with e4m3 scales at opposite ends of the range
    (one near 448, one subnormal or zero), over scale_2 from the smallest subnormal to 2^100: the
    widest spread between the halves' exponents, where the candidates' exact scores are largest."""
    rng = np.random.default_rng(17)
    n, R, C = 8, 32, 512
    e2m1 = rng.integers(0, 256, size=(n, R, C // 2), dtype=np.uint8)
    e4m3 = np.empty((n, R, C // 16), np.uint8)
    e4m3[..., 0::2] = rng.integers(0x70, 0x7F, size=(n, R, C // 32))            # large, finite
    e4m3[..., 1::2] = rng.integers(0, 8, size=(n, R, C // 32))                  # subnormal or zero
    e4m3[:, ::2] = np.flip(e4m3[:, ::2], axis=-1)                               # either half large
    e4m3 |= (rng.integers(0, 2, size=e4m3.shape) << 7).astype(np.uint8)         # random signs
    s2 = np.array([1.4e-45, 2.0 ** -126, 3.7e-3, 1.0, -0.75, 7.0, 2.0 ** 100, -3.0e38], np.float32)
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


# ------------------------------------------------------------------------------------------------
# fp8_block128_to_w2 and mxfp4_to_w2 ("The v0.24.0 port", section "Our hooks", fp8.py bullet;
# README: the FP8 block-quant and FP4 checkpoint flavours): bit-exact against the oracle's exact
# search (itself pinned against the full-scan rational reference).
# ------------------------------------------------------------------------------------------------

def test_fp8_block128_bit_exact_full_range(gpu):
    rng = np.random.default_rng(21)
    n, R, C = 3, 256, 512
    e4m3 = np.stack([workloads.fp8_block_tensor(i, R, C)[0] for i in range(n)])
    bs = (2.0 ** rng.uniform(-140, 100, size=(n, R // 128, C // 128))).astype(np.float32)
    bs[0, 0, 0] = np.float32(1.4e-45)      # subnormal scale
    bs[0, 0, 1] = np.float32(-0.25)        # negative scale flips every sign
    bs[0, 1, 0] = np.float32(0.0)
    bs[1, 1, 1] = np.float32(3.4e38)
    e4m3[2, :4, :64] = 0x80                 # -0 blocks
    e4m3[2, 4, :32] = 0x38                  # single magnitude
    c, s = moe.fp8_block128_to_w2(dev(e4m3), dev(bs))
    torch.cuda.synchronize()
    wc, ws = requant.fp8_block128_to_w2(e4m3, bs, window=False)
    assert np.array_equal(s.cpu().numpy(), ws)
    assert np.array_equal(c.cpu().numpy(), wc)


def test_fp8_block128_workload_tensor_bit_exact(gpu):
    e4m3, bs = workloads.fp8_block_tensor(0)
    c, s = moe.fp8_block128_to_w2(dev(e4m3[None]), dev(bs[None]))
    torch.cuda.synchronize()
    wc, ws = requant.fp8_block128_to_w2(e4m3[None], bs[None])
    assert np.array_equal(s.cpu().numpy(), ws)
    assert np.array_equal(c.cpu().numpy(), wc)


def test_mxfp4_bit_exact_full_range_and_workload(gpu):
    rng = np.random.default_rng(22)
    n, R, C = 2, 128, 1024
    e2m1 = rng.integers(0, 256, size=(n, R, C // 2), dtype=np.uint8)
    ue8m0 = rng.integers(0, 255, size=(n, R, C // 32)).astype(np.uint8)   # the whole byte range but 255
    e2m1[1, 0, :16] = 0x88                                               # a -0 block
    for a, b in ((e2m1, ue8m0), tuple(t[None] for t in workloads.mxfp4_tensor(0))):
        c, s = moe.mxfp4_to_w2(dev(a), dev(b))
        torch.cuda.synchronize()
        wc, ws = requant.mxfp4_to_w2(a, b)
        assert np.array_equal(s.cpu().numpy(), ws)
        assert np.array_equal(c.cpu().numpy(), wc)


def test_fp8_and_mxfp4_nan_inputs_are_reported(gpu):
    e4m3 = np.full((1, 128, 128), 0x38, np.uint8)
    e4m3[0, 3, 5] = 0x7F
    with pytest.raises(moe.MoeW2Error) as ei:
        moe.fp8_block128_to_w2(dev(e4m3), dev(np.ones((1, 1, 1), np.float32)))
    assert ei.value.status == -8
    with pytest.raises(moe.MoeW2Error) as ei:
        moe.fp8_block128_to_w2(dev(np.full((1, 128, 128), 0x38, np.uint8)), dev(np.full((1, 1, 1), np.nan, np.float32)))
    assert ei.value.status == -8
    with pytest.raises(moe.MoeW2Error) as ei:
        moe.mxfp4_to_w2(dev(np.zeros((1, 1, 16), np.uint8)), dev(np.full((1, 1, 1), 255, np.uint8)))
    assert ei.value.status == -8
