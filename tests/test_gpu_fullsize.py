"""Parity at the full sizes of the measured workloads, in the launch configuration bench.py times:
moe_w2_forward with the path chosen by the library (decode kernels up to 512 pairs, the grouped
GEMMs above), and nvfp4_to_w2 over all 256 tensors in one call.

The f64 oracle recomputes sampled outputs one by one (every pair of a sampled token, every block
of a sampled row); properties that hold at any size cover the rest: the bf16 output is the RNE
of the fp32 output everywhere, and the two kernel families agree on every output.
Bar: max |y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) over the sampled tokens; codes and scales
bit-exact."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import formats, forward as oracle_fwd, requant
import workloads

from gpu_helpers import bf16_rne_bits, dev, forward, pack, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _oracle(planes, inst, tokens):
    x = formats.bf16_bits_to_f64(inst["x"])
    return oracle_fwd.moe_forward(x, inst["topk_ids"], inst["topk_w"], planes["gu_codes"], planes["gu_scales"],
                                  planes["dn_codes"], planes["dn_scales"], tokens=tokens)


def _check_sampled(h, planes, inst, tokens, label):
    y = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_F32).cpu().numpy()
    err = rel_max_err(y[tokens], _oracle(planes, inst, tokens))
    print(f"{label}: tokens {list(tokens)} rel max err {err:.2e}", flush=True)
    assert err <= TOL
    return y


def _check_bf16_and_paths(h, inst, y32, label):
    y16 = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_BF16)
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne_bits(y32))
    other = moe.PATH_GEMM
    if inst["topk_ids"].size <= 512:         # the library picks the decode kernels here
        y_o = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_F32, path=other).cpu().numpy()
        d = rel_max_err(y_o, y32.astype(np.float64))
        print(f"{label}: decode vs GEMM kernels rel max diff {d:.2e}", flush=True)
        assert d <= TOL


@pytest.fixture(scope="module")
def decode_layer(gpu):
    planes = workloads.decode_layer()
    h = pack(planes)
    yield planes, h
    h.free()


@pytest.mark.parametrize("T,tokens", [(1, [0]), (8, [0, 5, 7]), (32, [0, 13, 31])])
def test_decode_layer_full_size(decode_layer, T, tokens):
    """K=4096 I=2048 E=256 top-8, uniform routing, routing instance 0 of the bench."""
    planes, h = decode_layer
    inst = workloads.decode_instances(T, 1)[0]
    y = _check_sampled(h, planes, inst, np.array(tokens), f"decode T={T}")
    _check_bf16_and_paths(h, inst, y, f"decode T={T}")


@pytest.fixture(scope="module")
def zipf_layer(gpu):
    c = workloads.PREFILL
    planes = workloads.zipf_layer(c["seed"], c["K"], c["I"], c["E"])
    h = pack(planes)
    yield planes, h
    h.free()


def _zipf_tokens(ids, E):
    """Token 0, the last token, a token routed to the most loaded expert, one routed to the least
    loaded active expert (its pairs sit in a ragged last tile) and three seeded random tokens."""
    counts = np.bincount(ids.ravel(), minlength=E)
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
    t_hot = int(np.nonzero((ids == hot).any(axis=1))[0][0])
    t_cold = int(np.nonzero((ids == cold).any(axis=1))[0][-1])
    extra = np.random.default_rng(7).integers(0, ids.shape[0], size=3)
    return np.unique(np.concatenate([[0, ids.shape[0] - 1, t_hot, t_cold], extra]))


def test_zipf_decode_batch_full_size(zipf_layer):
    """T=64 K=6144 I=2048 E=256 top-8, Zipf(1.1) routing (planes of the K=6144 layer)."""
    planes, h = zipf_layer
    c = workloads.DECODE_ZIPF
    inst = workloads.zipf_instances(c["T"], 1, c["seed"], c["K"], c["E"], c["top_k"])[0]
    tokens = _zipf_tokens(inst["topk_ids"], c["E"])
    y = _check_sampled(h, planes, inst, tokens, "zipf T=64")
    _check_bf16_and_paths(h, inst, y, "zipf T=64")


def test_prefill_full_size(zipf_layer):
    """T=8192 K=6144 I=2048 E=256 top-8, Zipf(1.1) routing: every expert active, groups of very
    uneven size through the grouped GEMMs."""
    planes, h = zipf_layer
    c = workloads.PREFILL
    inst = workloads.zipf_instances(c["T"], 1, c["seed"], c["K"], c["E"], c["top_k"])[0]
    tokens = _zipf_tokens(inst["topk_ids"], c["E"])
    y = _check_sampled(h, planes, inst, tokens, "prefill T=8192")
    y16 = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_BF16)
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne_bits(y))
    # any-size property: the routing permutation of this batch is the oracle's, bit for bit
    offsets, perm = moe.moe_w2_route(dev(inst["topk_ids"]), c["E"])
    w_off, w_perm = oracle_fwd.route(inst["topk_ids"], c["E"])
    assert np.array_equal(offsets.cpu().numpy(), w_off)
    assert np.array_equal(perm.cpu().numpy(), w_perm)


def test_requant_full_size(gpu):
    """nvfp4_to_w2 over 256 tensors of [2048, 6144] in one call; sampled rows of sampled tensors
    recomputed by the exact oracle, bit for bit."""
    c = workloads.REQUANT
    n, R, C = c["n"], c["R"], c["C"]
    e2m1 = torch.empty((n, R, C // 2), dtype=torch.uint8, device="cuda")
    e4m3 = torch.empty((n, R, C // 16), dtype=torch.uint8, device="cuda")
    s2 = np.zeros(n, np.float32)
    host = {}
    sample = [0, 1, 97, 200, n - 1]
    for i in range(n):
        a, b, s = workloads.nvfp4_tensor(i)
        e2m1[i].copy_(torch.from_numpy(a))
        e4m3[i].copy_(torch.from_numpy(b))
        s2[i] = s
        if i in sample:
            host[i] = (a, b, s)
    codes, scales = moe.nvfp4_to_w2(e2m1, e4m3, dev(s2))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for i in sample:
        a, b, s = host[i]
        rows = np.unique(np.concatenate([[0, R - 1], rng.integers(0, R, size=6)]))
        wc, ws = requant.requant_rows(a[rows], b[rows], s)
        gc = codes[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        gs = scales[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        print(f"requant tensor {i}: rows {list(rows)}", flush=True)
        assert np.array_equal(gs, ws)
        assert np.array_equal(gc, wc)
