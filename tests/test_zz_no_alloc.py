"""moe_w2_forward_noalloc (the forward with the library's own per-GPU scratch as workspace, for
callers that cannot allocate) against moe_w2_forward with a caller workspace: bit-identical
outputs on successive calls of decreasing size over every kernel organisation (grouped GEMM,
sorted decode with split groups, routed decode, tiny-batch direct), and calls whose workspace
would exceed the scratch refused on the host."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
import workloads

from gpu_helpers import dev, dev_bf16, pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer(gpu):
    rng = np.random.default_rng(41)
    planes = workloads.draw_planes(rng, 64, 1024, 512)
    h = pack(planes)
    yield h
    h.free()


def _inputs(T, top_k, E, K, seed):
    rng = np.random.default_rng(seed)
    x = workloads.draw_x(rng, T, K)
    ids, w = workloads.uniform_routing(rng, T, E, top_k)
    return dev_bf16(x), dev(ids), dev(w)


@pytest.mark.parametrize("out_dtype", [moe.OUT_F32, moe.OUT_BF16])
def test_noalloc_matches_forward_on_shrinking_calls(layer, out_dtype):
    K, E, top_k = 1024, 64, 8
    dt = torch.float32 if out_dtype == moe.OUT_F32 else torch.bfloat16
    # GEMM organisation (P = 768), sorted decode with split groups (P = 512, ~8 pairs per expert),
    # routed decode (P = 256), direct (P = 8), routed decode again (P = 40)
    for i, T in enumerate((96, 64, 32, 1, 5)):
        x, ids, w = _inputs(T, top_k, E, K, 100 + i)
        want = moe.moe_w2_forward(layer, x, ids, w, out_dtype=out_dtype)
        y = torch.full((T, K), float("nan"), dtype=dt, device="cuda")
        got = moe.moe_w2_forward_noalloc(layer, x, ids, w, y, out_dtype=out_dtype)
        torch.cuda.synchronize()
        print(f"noalloc T={T} out_dtype={out_dtype}", flush=True)
        assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_noalloc_forced_paths_and_repeat(layer):
    """Both kernel families forced on one batch, each called twice in a row: bit-identical to the
    workspace entry point."""
    K, E, top_k = 1024, 64, 8
    x, ids, w = _inputs(24, top_k, E, K, 7)
    for path in (moe.PATH_GEMM, moe.PATH_DECODE, moe.PATH_DECODE_SORTED):
        want = moe.moe_w2_forward(layer, x, ids, w, out_dtype=moe.OUT_F32, path=path)
        for _ in range(2):
            y = torch.empty((24, K), dtype=torch.float32, device="cuda")
            moe.moe_w2_forward_noalloc(layer, x, ids, w, y, out_dtype=moe.OUT_F32, path=path)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), want.view(torch.int32))


def test_noalloc_streamed_down_gemm(gpu):
    """I = 2048 with K a multiple of 512: the GEMM organisation's down stage is the streamed kernel
    (one workgroup per compute unit); two calls in a row, the second smaller, bit-identical to the
    workspace entry point."""
    rng = np.random.default_rng(43)
    K, I, E, top_k = 512, 2048, 32, 4
    h = pack(workloads.draw_planes(rng, E, K, I))
    try:
        for i, T in enumerate((300, 150)):   # 1200 and 600 pairs
            x, ids, w = _inputs(T, top_k, E, K, 200 + i)
            want = moe.moe_w2_forward(h, x, ids, w, out_dtype=moe.OUT_F32, path=moe.PATH_GEMM)
            y = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
            moe.moe_w2_forward_noalloc(h, x, ids, w, y, out_dtype=moe.OUT_F32, path=moe.PATH_GEMM)
            torch.cuda.synchronize()
            print(f"noalloc streamed down T={T}", flush=True)
            assert torch.equal(y.view(torch.int32), want.view(torch.int32))
    finally:
        h.free()


def test_noalloc_rejects_calls_beyond_the_scratch(layer):
    """A call whose workspace exceeds MOE_W2_NOALLOC_SCRATCH_BYTES returns EUNSUPPORTED on the host."""
    K, top_k = 1024, 8
    T = 4096
    assert moe.moe_w2_workspace_bytes(layer, T, top_k) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeW2Error) as ei:
        moe.moe_w2_forward_noalloc(layer, x, ids, w, y)
    assert ei.value.status == -2
