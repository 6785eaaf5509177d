"""Parity at the full sizes of the measured workloads, in the launch configuration bench.py times:
moe_w2_forward with the path chosen by the library (decode kernels up to 512 pairs, the grouped
GEMMs above), and nvfp4_to_w2 over all 256 tensors in one call.

Decode batches (T = 1, 8, 32 and the Zipf T=64 batch) are compared with the f64 oracle on every
token. The 8192-token prefill is compared on 256 seeded random tokens plus edge tokens, and on
every pair of eight whole expert groups (the largest, the second largest, the smallest, the
smallest with more than one 64-row tile, and four seeded random experts): a forward whose router
weights are 1 on that expert's pairs and 0 elsewhere returns each of its pairs' down rows as y,
through the same routing and tiles as the full batch. The bf16 output is the RNE of the fp32
output everywhere, and on the decode shapes the two kernel families agree on every output.
nvfp4_to_w2 is compared with the exact oracle on all 256 tensors through SHA-256 digests of the
oracle's codes and scales (tests/golden/requant_nvfp4_full.txt, written by
tests/golden/make_requant_digests.py from oracle/ alone).
Bar: max |y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) over the compared outputs; codes and scales
bit-exact."""
import hashlib
import os

import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import formats, forward as oracle_fwd, requant
import workloads

from gpu_helpers import bf16_rne_bits, dev, forward, pack, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-2


WORKERS = max(1, min(4, os.cpu_count() or 1))   # oracle experts computed at a time (CPU threads)


def _oracle(planes, inst, tokens, ids=None, w=None):
    x = formats.bf16_bits_to_f64(inst["x"])
    ids = inst["topk_ids"] if ids is None else ids
    w = inst["topk_w"] if w is None else w
    return oracle_fwd.moe_forward(x, ids, w, planes["gu_codes"], planes["gu_scales"],
                                  planes["dn_codes"], planes["dn_scales"], tokens=tokens, workers=WORKERS)


def _check_sampled(h, planes, inst, tokens, label):
    y = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_F32).cpu().numpy()
    err = rel_max_err(y[tokens], _oracle(planes, inst, tokens))
    shown = list(tokens) if len(tokens) <= 8 else f"{len(tokens)} tokens"
    print(f"{label}: {shown} rel max err {err:.2e}", flush=True)
    assert err <= TOL
    return y


def _check_expert_groups(h, planes, inst, experts, label):
    """Every pair of each listed expert: router weights 1 on the expert's pairs and 0 elsewhere
    make y[t] that pair's down row (each token routes to an expert at most once here)."""
    ids = inst["topk_ids"]
    for e in experts:
        mask = ids == e
        assert mask.sum(axis=1).max() <= 1
        w1 = mask.astype(np.float32)
        tokens = np.nonzero(mask.any(axis=1))[0]
        y = forward(h, inst["x"], ids, w1, moe.OUT_F32).cpu().numpy()
        ref = _oracle(planes, inst, tokens, ids=np.where(mask, ids, -1).astype(np.int32), w=w1)
        err = rel_max_err(y[tokens], ref)
        # tokens that do not route to e get exactly zero
        rest = np.ones(ids.shape[0], bool)
        rest[tokens] = False
        print(f"{label}: expert {e}, all {len(tokens)} pairs, rel max err {err:.2e}", flush=True)
        assert err <= TOL
        assert not np.any(y[rest])


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


@pytest.mark.parametrize("T", [1, 8, 32])
def test_decode_layer_full_size(decode_layer, T):
    """K=4096 I=2048 E=256 top-8, uniform routing, routing instance 0 of the bench: every token."""
    planes, h = decode_layer
    inst = workloads.decode_instances(T, 1)[0]
    y = _check_sampled(h, planes, inst, np.arange(T), f"decode T={T}")
    _check_bf16_and_paths(h, inst, y, f"decode T={T}")


@pytest.fixture(scope="module")
def zipf_layer(gpu):
    c = workloads.PREFILL
    planes = workloads.zipf_layer(c["seed"], c["K"], c["I"], c["E"])
    h = pack(planes)
    yield planes, h
    h.free()


def _zipf_tokens(ids, E):
    """Token 0, the last token, the first and last tokens routed to the most loaded expert, the
    last one routed to the least loaded active expert (its pairs sit in a ragged last tile) and
    256 seeded random tokens."""
    counts = np.bincount(ids.ravel(), minlength=E)
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
    t_hot = np.nonzero((ids == hot).any(axis=1))[0]
    t_cold = int(np.nonzero((ids == cold).any(axis=1))[0][-1])
    extra = np.random.default_rng(7).choice(ids.shape[0], size=256, replace=False)
    return np.unique(np.concatenate([[0, ids.shape[0] - 1, t_hot[0], t_hot[-1], t_cold], extra]))


def _prefill_experts(ids, E):
    """The largest, second largest and smallest active groups, the smallest group with more than
    one 64-row M-tile (a ragged tile after a full one), and four seeded random active experts."""
    counts = np.bincount(ids.ravel(), minlength=E)
    order = np.argsort(-counts, kind="stable")
    active = order[counts[order] > 0]
    multi = active[counts[active] > 64]
    rng = np.random.default_rng(8)
    picks = [int(active[0]), int(active[1]), int(active[-1]), int(multi[-1])]
    picks += [int(e) for e in rng.choice(active[2:-1], size=4, replace=False)]
    return list(dict.fromkeys(picks))


def test_zipf_decode_batch_full_size(zipf_layer):
    """T=64 K=6144 I=2048 E=256 top-8, Zipf(1.1) routing (planes of the K=6144 layer): every token."""
    planes, h = zipf_layer
    c = workloads.DECODE_ZIPF
    inst = workloads.zipf_instances(c["T"], 1, c["seed"], c["K"], c["E"], c["top_k"])[0]
    y = _check_sampled(h, planes, inst, np.arange(c["T"]), "zipf T=64")
    _check_bf16_and_paths(h, inst, y, "zipf T=64")


def test_prefill_full_size(zipf_layer):
    """T=8192 K=6144 I=2048 E=256 top-8, Zipf(1.1) routing: every expert active, groups of very
    uneven size through the grouped GEMMs."""
    planes, h = zipf_layer
    c = workloads.PREFILL
    inst = workloads.zipf_instances(c["T"], 1, c["seed"], c["K"], c["E"], c["top_k"])[0]
    tokens = _zipf_tokens(inst["topk_ids"], c["E"])
    y = _check_sampled(h, planes, inst, tokens, "prefill T=8192")
    _check_expert_groups(h, planes, inst, _prefill_experts(inst["topk_ids"], c["E"]), "prefill T=8192")
    y16 = forward(h, inst["x"], inst["topk_ids"], inst["topk_w"], moe.OUT_BF16)
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne_bits(y))
    # any-size property: the routing permutation of this batch is the oracle's, bit for bit
    offsets, perm = moe.moe_w2_route(dev(inst["topk_ids"]), c["E"])
    w_off, w_perm = oracle_fwd.route(inst["topk_ids"], c["E"])
    assert np.array_equal(offsets.cpu().numpy(), w_off)
    assert np.array_equal(perm.cpu().numpy(), w_perm)


GOLDEN_REQUANT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "requant_nvfp4_full.txt")


def _requant_digests():
    out = {}
    with open(GOLDEN_REQUANT) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                i, dc, ds = line.split()
                out[int(i)] = (dc, ds)
    return out


def test_requant_full_size(gpu):
    """nvfp4_to_w2 over 256 tensors of [2048, 6144] in one call, every tensor's codes and scale
    bytes bit-exact against the exact oracle (digests of its output). On a mismatch the oracle
    recomputes that tensor to name the first differing row."""
    c = workloads.REQUANT
    n, R, C = c["n"], c["R"], c["C"]
    golden = _requant_digests()
    assert sorted(golden) == list(range(n))
    e2m1 = torch.empty((n, R, C // 2), dtype=torch.uint8, device="cuda")
    e4m3 = torch.empty((n, R, C // 16), dtype=torch.uint8, device="cuda")
    s2 = np.zeros(n, np.float32)
    for i in range(n):
        a, b, s = workloads.nvfp4_tensor(i)
        e2m1[i].copy_(torch.from_numpy(a))
        e4m3[i].copy_(torch.from_numpy(b))
        s2[i] = s
    codes, scales = moe.nvfp4_to_w2(e2m1, e4m3, dev(s2))
    torch.cuda.synchronize()
    bad = []
    for i in range(n):
        gc = codes[i].cpu().numpy()
        gs = scales[i].cpu().numpy()
        if (hashlib.sha256(gc.tobytes()).hexdigest(), hashlib.sha256(gs.tobytes()).hexdigest()) != golden[i]:
            bad.append(i)
            if len(bad) == 1:
                a, b, s = workloads.nvfp4_tensor(i)
                wc, ws = requant.requant_rows(a, b, s)
                rows = np.nonzero((wc != gc).any(axis=1) | (ws != gs).any(axis=1))[0]
                print(f"requant tensor {i}: {len(rows)} rows differ from the oracle, first {rows[:4]}", flush=True)
    print(f"requant: {n - len(bad)} of {n} tensors bit-exact", flush=True)
    assert not bad, f"tensors differing from the oracle: {bad[:16]}"
