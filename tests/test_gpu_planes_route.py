"""GPU: moe_w2_pack / unpack round trip, pack-time validation, and the routing pass against the
oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import forward as oracle_fwd
import workloads

from gpu_helpers import dev, pack

pytestmark = pytest.mark.gpu


def _planes(E, K, I, seed):
    return workloads.draw_planes(np.random.default_rng(seed), E, K, I)


@pytest.mark.parametrize("shape", [(8, 256, 512), (3, 768, 256), (2, 512, 1024)])
def test_pack_unpack_roundtrip_is_exact(gpu, shape):
    E, K, I = shape
    p = _planes(E, K, I, 5)
    # include extreme scale bytes (0 and 252) in both matrices
    p["dn_scales"][0] = 30
    p["dn_scales"][1, :, :] = np.arange(I // 32, dtype=np.uint8)[None, :] % 30 + 200
    p["gu_scales"][0, 0, 0] = 252
    p["gu_scales"][0, 1, 0] = 0
    p["dn_scales"][2 % E, 0, 0] = 252
    h = pack(p)
    out = [t.cpu().numpy() for t in moe.moe_w2_unpack(h)]
    torch.cuda.synchronize()
    for name, got in zip(("gu_codes", "gu_scales", "dn_codes", "dn_scales"), out):
        assert np.array_equal(got, p[name]), name


def test_pack_rejects_bad_scales(gpu):
    p = _planes(2, 256, 256, 6)
    q = dict(p, gu_scales=p["gu_scales"].copy())
    q["gu_scales"][1, 3, 2] = 253
    with pytest.raises(moe.MoeW2Error) as ei:
        pack(q)
    assert ei.value.status == -3
    q = dict(p, dn_scales=p["dn_scales"].copy())
    q["dn_scales"][0, 5, 1] = 255
    with pytest.raises(moe.MoeW2Error) as ei:
        pack(q)
    assert ei.value.status == -3
    q = dict(p, dn_scales=p["dn_scales"].copy())
    q["dn_scales"][0, 5, 1] = 253      # 4 * 2^126 is not finite in fp32
    with pytest.raises(moe.MoeW2Error) as ei:
        pack(q)
    assert ei.value.status == -3
    q["dn_scales"][0, 5, 1] = 252      # the largest accepted byte
    q["dn_scales"][0, 7, 0] = 0        # and the smallest, in the same row as 252: any spread
    q["dn_scales"][0, 7, 1] = 252
    pack(q)


ROUTE_CASES = [(1, 256, 8), (8, 256, 8), (32, 256, 8), (64, 256, 8), (4, 8, 2), (600, 64, 8),
               (1000, 256, 8), (8192, 256, 8), (5000, 1024, 4), (77, 3, 3)]


@pytest.mark.parametrize("T,E,top_k", ROUTE_CASES)
def test_route_matches_oracle_exactly(gpu, T, E, top_k):
    rng = np.random.default_rng(T * 7 + E)
    ids = rng.integers(0, E, size=(T, top_k)).astype(np.int32)
    ids[rng.random((T, top_k)) < 0.02] = -1
    ids[rng.random((T, top_k)) < 0.01] = E + 3
    off, perm = moe.moe_w2_route(dev(ids), E)
    torch.cuda.synchronize()
    want_off, want_perm = oracle_fwd.route(ids, E)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy(), want_perm)


def test_route_zipf_prefill_shape(gpu):
    inst = workloads.zipf_instances(8192, 1, seed=3, K=16, E=256, top_k=8)[0]
    off, perm = moe.moe_w2_route(dev(inst["topk_ids"]), 256)
    torch.cuda.synchronize()
    want_off, want_perm = oracle_fwd.route(inst["topk_ids"], 256)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy(), want_perm)
