"""FP4 (MXFP4) expert planes (moe_w4_pack / moe_w4_unpack / moe_w4_forward) through the C ABI,
against the f64 oracle with e2m1 weights (README bullet "FP4 recovery - used surgically"; bullet
"The kernels": the FP4 GEMM beside the 2-bit one). Bar: max |y_gpu - y_oracle| <= 1e-2 *
rms(y_oracle) on the fp32 output, on both kernel families, with several tiles and ragged tails;
pack/unpack exact; the full decode shape on every token."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import formats, forward as oracle_fwd
import workloads

from gpu_helpers import dev, dev_bf16, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-2


def pack4(planes):
    return moe.moe_w4_pack(dev(planes["gu_codes"]), dev(planes["gu_scales"]), dev(planes["dn_codes"]),
                           dev(planes["dn_scales"]))


def _case(T, K, I, E, top_k, seed, zipf=False):
    rng = np.random.default_rng(seed)
    planes = workloads.draw_planes_fp4(rng, E, K, I)
    x = workloads.draw_x(rng, T, K)
    if zipf:
        ids, w = workloads.zipf_routing(rng, T, E, top_k, rank_perm=rng.permutation(E))
    else:
        ids, w = workloads.uniform_routing(rng, T, E, top_k)
    return dict(planes, x=x, topk_ids=ids, topk_w=w)


def _oracle(c, tokens=None):
    return oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), c["topk_ids"], c["topk_w"], c["gu_codes"],
                                  c["gu_scales"], c["dn_codes"], c["dn_scales"], tokens=tokens, fp4=True)


def _fwd(h, c, path, ws=None):
    y = moe.moe_w4_forward(h, dev_bf16(c["x"]), dev(c["topk_ids"]), dev(c["topk_w"]), out_dtype=moe.OUT_F32,
                           path=path, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("shape", [(8, 256, 512), (3, 512, 768), (16, 768, 256)])
def test_w4_pack_unpack_roundtrip_is_exact(gpu, shape):
    E, K, I = shape
    planes = workloads.draw_planes_fp4(np.random.default_rng(E + K), E, K, I)
    back = moe.moe_w4_unpack(pack4(planes))
    for name, t in zip(("gu_codes", "gu_scales", "dn_codes", "dn_scales"), back):
        assert np.array_equal(t.cpu().numpy(), planes[name]), name


CASES = [
    (4, 256, 512, 8, 2, 40, False, moe.PATH_DECODE),
    (3, 512, 512, 8, 2, 41, False, moe.PATH_DECODE),        # direct tiny-batch kernels
    (37, 512, 768, 16, 4, 42, False, moe.PATH_DECODE),
    (128, 512, 256, 4, 4, 43, True, moe.PATH_DECODE),
    (60, 512, 512, 32, 8, 46, True, moe.PATH_DECODE_SORTED),
    (4, 256, 512, 8, 2, 40, False, moe.PATH_GEMM),
    (300, 768, 512, 8, 2, 44, False, moe.PATH_GEMM),
    (200, 1024, 256, 32, 8, 45, True, moe.PATH_GEMM),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}K{c[1]}I{c[2]}E{c[3]}k{c[4]}-p{c[7]}" for c in CASES])
def test_w4_parity(gpu, case):
    T, K, I, E, k, seed, zipf, path = case
    c = _case(T, K, I, E, k, seed, zipf)
    h = pack4(c)
    y = _fwd(h, c, path)
    err = rel_max_err(y, _oracle(c))
    print(f"w4 {case}: rel max err {err:.2e}")
    assert err <= TOL


def test_w4_paths_agree_and_repeat_bit_identically(gpu):
    c = _case(64, 512, 512, 8, 4, 46)
    h = pack4(c)
    a = _fwd(h, c, moe.PATH_DECODE)
    b = _fwd(h, c, moe.PATH_GEMM)
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2))
    assert np.max(np.abs(a - b)) <= 5e-3 * rms
    assert np.array_equal(a.view(np.int32), _fwd(h, c, moe.PATH_DECODE).view(np.int32))
    assert np.array_equal(b.view(np.int32), _fwd(h, c, moe.PATH_GEMM).view(np.int32))


def test_w4_invalid_ids_and_planes_checks(gpu):
    c = _case(16, 256, 256, 8, 4, 47)
    c["topk_ids"] = c["topk_ids"].copy()
    c["topk_ids"][3, 2] = -1
    c["topk_ids"][7, 0] = 99
    h = pack4(c)
    ws = moe.alloc_workspace(h, 16, 4)
    y = _fwd(h, c, moe.PATH_DECODE, ws)
    assert rel_max_err(y, _oracle(c)) <= TOL
    inv, _ = moe.moe_w2_read_counters(ws)
    assert inv == 2
    with pytest.raises(moe.MoeW2Error):       # 2-bit unpack of FP4 planes
        moe.moe_w2_unpack(h)
    bad = c["gu_scales"].copy()
    bad[1, 5, 0] = 253
    with pytest.raises(moe.MoeW2Error) as ex:
        pack4(dict(c, gu_scales=bad))
    assert ex.value.status == -3


@pytest.mark.parametrize("T", [1, 8, 32])
def test_w4_decode_full_shape_every_token(gpu, T):
    """K=4096, I=2048 (the decode shape) with E=64 experts and uniform top-8 routing, the AUTO
    path: every token against the f64 oracle; the GEMM family run on the same call agrees closely."""
    rng = np.random.default_rng(60 + T)
    K, I, E = 4096, 2048, 64
    planes = workloads.draw_planes_fp4(rng, E, K, I)
    x = workloads.draw_x(rng, T, K)
    ids, w = workloads.uniform_routing(rng, T, E, 8)
    c = dict(planes, x=x, topk_ids=ids, topk_w=w)
    h = pack4(c)
    y = _fwd(h, c, moe.PATH_AUTO)
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), c["topk_ids"], c["topk_w"], c["gu_codes"],
                                   c["gu_scales"], c["dn_codes"], c["dn_scales"], fp4=True, workers=4)
    err = rel_max_err(y, y_ref)
    print(f"w4 decode T={T}: every token rel max err {err:.2e}")
    assert err <= TOL
    yg = _fwd(h, c, moe.PATH_GEMM)
    assert np.max(np.abs(y - yg)) <= 5e-3 * np.sqrt(np.mean(y.astype(np.float64) ** 2))


def _random_cases(n=8, seed=4048):
    """Seeded random shapes as for the 2-bit planes: T in [1, 160], K and I multiples of 256 up to
    1280, E in [1, 96], top_k up to min(8, E), uniform or Zipf routing."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 97))
        top_k = int(rng.integers(1, min(8, E) + 1))
        out.append((int(rng.integers(1, 161)), 256 * int(rng.integers(1, 6)), 256 * int(rng.integers(1, 6)), E, top_k,
                    2000 + i, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"T{c[0]}K{c[1]}I{c[2]}E{c[3]}k{c[4]}{'z' if c[6] else 'u'}")
def test_w4_random_shapes_parity(gpu, case):
    T, K, I, E, top_k, seed, zipf = case
    c = _case(T, K, I, E, top_k, seed, zipf)
    h = pack4(c)
    y_ref = _oracle(c)
    for path in (moe.PATH_DECODE, moe.PATH_GEMM):
        if path == moe.PATH_DECODE and T * top_k > 512:
            continue
        err = rel_max_err(_fwd(h, c, path), y_ref)
        print(f"{case} path={path} rel max err {err:.2e}")
        assert err <= TOL, (case, path, err)
