"""Pins for oracle.forward: routing against a hand-worked fixture and invariants; the forward
against a library routine in its dense special case (E=1, top-1), hand-derived closed forms and
exact invariants."""
import os

import numpy as np
import pytest
import torch

from oracle import formats, forward
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_route_example():
    d = {}
    with open(os.path.join(GOLDEN, "route_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            d[key] = rest
    ids = np.array([[int(v) for v in tok.split()] for tok in d["ids"].split("|")], dtype=np.int32)
    return ids, np.array(d["offsets"].split(), dtype=np.int32), np.array(d["perm"].split(), dtype=np.int32)


def test_route_hand_example():
    ids, offsets, perm = _read_route_example()
    got_o, got_p = forward.route(ids, E=4)
    assert np.array_equal(got_o, offsets)
    assert np.array_equal(got_p, perm)


def test_route_invariants():
    rng = np.random.default_rng(3)
    for T, E, k in [(1, 256, 8), (37, 16, 4), (500, 256, 8), (64, 8, 8)]:
        ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
        offsets, perm = forward.route(ids, E)
        flat = ids.reshape(-1)
        assert sorted(perm.tolist()) == list(range(T * k))            # a permutation
        assert offsets[0] == 0 and np.all(np.diff(offsets) >= 0)
        valid = (flat >= 0) & (flat < E)
        assert offsets[E] == valid.sum()
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)  # stable
        tail = perm[offsets[E]:]
        assert np.all(~valid[tail]) and np.all(np.diff(tail) > 0)


def _dense_weights_independent(packed, scale_bytes):
    """Dequantize with torch's float8_e8m0fnu for the scale and the printed codebook."""
    book = {}
    with open(os.path.join(GOLDEN, "codebook.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                book[int(c)] = float(v)
    p = np.asarray(packed)
    rows, nb = p.shape
    vals = np.zeros((rows, nb * 4))
    for sh in range(4):
        codes = (p >> (2 * sh)) & 3
        vals[:, sh::4] = np.vectorize(book.get)(codes)
    s = torch.from_numpy(np.ascontiguousarray(scale_bytes, dtype=np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return vals * np.repeat(s, 32, axis=1)


def test_single_expert_top1_is_dense_silu_mlp():
    """E = 1, top-1, weight 1: the layer is the dense gated MLP D (silu(G x) * (U x)), computed
    here with torch's silu and matmul in float64 on independently dequantized weights."""
    rng = np.random.default_rng(12)
    T, K, I = 6, 64, 96
    planes = workloads.draw_planes(rng, 1, K, I)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    y = forward.moe_forward(x, ids, w, **planes)
    wgu = torch.from_numpy(_dense_weights_independent(planes["gu_codes"][0], planes["gu_scales"][0]))
    wdn = torch.from_numpy(_dense_weights_independent(planes["dn_codes"][0], planes["dn_scales"][0]))
    xt = torch.from_numpy(x)
    ref = torch.matmul(torch.nn.functional.silu(torch.matmul(xt, wgu[:I].T)) * torch.matmul(xt, wgu[I:].T), wdn.T)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(ref.numpy()).max())


def test_hand_case_all_plus_one():
    """T=1, K=I=32, E=1: every code +1 (code 2), every scale byte 127 (2^0), x = 1. Then each gate
    and up output is 32, a = 32 * sigmoid(32) * 32 for all 32 intermediate units, and every output
    is 32 * a, scaled by the router weight 0.5."""
    K = I = 32
    gu = np.full((1, 2 * I, K // 4), 0xAA, np.uint8)       # 0b10101010 = four codes 2
    gus = np.full((1, 2 * I, 1), 127, np.uint8)
    dn = np.full((1, K, I // 4), 0xAA, np.uint8)
    dns = np.full((1, K, 1), 127, np.uint8)
    x = np.ones((1, K))
    y = forward.moe_forward(x, np.zeros((1, 1), np.int32), np.full((1, 1), 0.5, np.float32), gu, gus, dn, dns)
    a = 32.0 * 32.0 / (1.0 + np.exp(-32.0))
    np.testing.assert_allclose(y, np.full((1, K), 0.5 * 32.0 * a), rtol=1e-15)


def test_gate_and_up_are_not_swapped():
    """Gate rows (0..I-1) all -1 and up rows (I..2I-1) all +1 with x = 20/32 per element give
    g = -20, u = +20: a = silu(-20) * 20 ~ -4e-8. Swapping gate and up would give silu(20)*(-20)
    = -400."""
    K = I = 32
    gu = np.concatenate([np.full((1, I, K // 4), 0x55, np.uint8),     # code 1 = -1
                         np.full((1, I, K // 4), 0xAA, np.uint8)], axis=1)  # code 2 = +1
    gus = np.full((1, 2 * I, 1), 127, np.uint8)
    a = forward.moe_forward_act(np.full((1, K), 20.0 / 32.0), np.zeros((1, 1), np.int32), gu, gus)
    want = -20.0 / (1.0 + np.exp(20.0)) * 20.0
    np.testing.assert_allclose(a[0, 0], np.full(I, want), rtol=1e-13)


def _tiny_inputs(seed=0):
    d = workloads.tiny(seed)
    x = formats.bf16_bits_to_f64(d["x"])
    return d, x


def test_linear_in_router_weights_and_invalid_ids_contribute_nothing():
    d, x = _tiny_inputs()
    P = dict(gu_codes=d["gu_codes"], gu_scales=d["gu_scales"], dn_codes=d["dn_codes"], dn_scales=d["dn_scales"])
    w1 = d["topk_w"]
    w2 = np.random.default_rng(1).uniform(-1, 1, w1.shape).astype(np.float32)
    y1 = forward.moe_forward(x, d["topk_ids"], w1, **P)
    y2 = forward.moe_forward(x, d["topk_ids"], w2, **P)
    y12 = forward.moe_forward(x, d["topk_ids"], w1.astype(np.float64) + w2, **P)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12 * np.abs(y1).max())
    bad = d["topk_ids"].copy()
    bad[:, 1] = -1
    yb = forward.moe_forward(x, bad, w1, **P)
    only0 = forward.moe_forward(x, d["topk_ids"][:, :1], w1[:, :1], **P)
    assert np.array_equal(yb, only0)


def test_duplicate_ids_sum_their_weights():
    d, x = _tiny_inputs()
    P = dict(gu_codes=d["gu_codes"], gu_scales=d["gu_scales"], dn_codes=d["dn_codes"], dn_scales=d["dn_scales"])
    ids = np.stack([d["topk_ids"][:, 0]] * 2, axis=1)
    w = np.array([[0.25, 0.5]] * d["T"], np.float32)
    y = forward.moe_forward(x, ids, w, **P)
    y1 = forward.moe_forward(x, ids[:, :1], np.full((d["T"], 1), 0.75, np.float32), **P)
    np.testing.assert_allclose(y, y1, rtol=1e-13, atol=1e-14 * np.abs(y1).max())


def test_down_scale_and_sign_invariants_are_exact():
    """Down scale bytes + 1 double y exactly; down codes c -> 3 - c negate y exactly (f64)."""
    d, x = _tiny_inputs()
    P = dict(gu_codes=d["gu_codes"], gu_scales=d["gu_scales"], dn_codes=d["dn_codes"], dn_scales=d["dn_scales"])
    y = forward.moe_forward(x, d["topk_ids"], d["topk_w"], **P)
    P2 = dict(P, dn_scales=(d["dn_scales"] + 1).astype(np.uint8))
    assert np.array_equal(forward.moe_forward(x, d["topk_ids"], d["topk_w"], **P2), 2 * y)
    P3 = dict(P, dn_codes=(~d["dn_codes"]).astype(np.uint8))    # NOT of every 2-bit field = 3 - c
    assert np.array_equal(forward.moe_forward(x, d["topk_ids"], d["topk_w"], **P3), -y)


def test_token_subset_matches_full():
    d, x = _tiny_inputs()
    P = dict(gu_codes=d["gu_codes"], gu_scales=d["gu_scales"], dn_codes=d["dn_codes"], dn_scales=d["dn_scales"])
    y = forward.moe_forward(x, d["topk_ids"], d["topk_w"], **P)
    ys = forward.moe_forward(x, d["topk_ids"], d["topk_w"], tokens=[3, 1], **P)
    # same arithmetic; BLAS may block a smaller batch differently, so allow f64 rounding
    np.testing.assert_allclose(ys, y[[3, 1]], rtol=1e-12, atol=1e-14 * np.abs(y).max())


def test_resident_forward_reductions_and_additivity():
    """Expert-cache reading (README paragraph on the base cache): non-resident experts' pairs
    contribute nothing. With every expert resident it is the full forward; with none it is zero;
    and two complementary resident sets add up to the full forward (each pair lands in exactly
    one of them), which a mask on the wrong index (slot vs expert, token vs pair) breaks."""
    d, x = _tiny_inputs(5)
    E = d["gu_codes"].shape[0]
    args = (d["gu_codes"], d["gu_scales"], d["dn_codes"], d["dn_scales"])
    full = forward.moe_forward(x, d["topk_ids"], d["topk_w"], *args)
    assert np.array_equal(forward.moe_forward_resident(x, d["topk_ids"], d["topk_w"], *args, np.ones(E, bool)), full)
    assert not np.any(forward.moe_forward_resident(x, d["topk_ids"], d["topk_w"], *args, np.zeros(E, bool)))
    rng = np.random.default_rng(6)
    for _ in range(4):
        res = rng.random(E) < 0.5
        a = forward.moe_forward_resident(x, d["topk_ids"], d["topk_w"], *args, res)
        b = forward.moe_forward_resident(x, d["topk_ids"], d["topk_w"], *args, ~res)
        assert np.max(np.abs(a + b - full)) <= 1e-12 * np.max(np.abs(full))
        assert not np.array_equal(a, full) or res.all() or not np.isin(d["topk_ids"], np.nonzero(~res)[0]).any()


def test_resident_ids_hand_example():
    """Misses are pairs with a valid id whose expert is not resident; invalid ids stay invalid and
    are not misses."""
    ids = np.array([[0, 3], [2, -1], [5, 1]], dtype=np.int32)   # E = 4: id 5 and -1 are invalid
    resident = np.array([True, False, True, False])
    got, miss = forward.resident_ids(ids, 4, resident)
    assert np.array_equal(got, np.array([[0, -1], [2, -1], [-1, -1]], dtype=np.int32))
    assert miss == 2   # ids 3 and 1


def test_unpack_e2m1_hand_bytes():
    """FP4 packing: element 2i in the low nibble of byte i. 0x8A -> nibbles 0xA (-1.0), 0x8 (-0.0);
    0x21 -> 0x1 (0.5), 0x2 (1.0)."""
    n = formats.unpack_e2m1(np.array([[0x8A, 0x21]], np.uint8))
    assert n.tolist() == [[0xA, 0x8, 0x1, 0x2]]
    vals = [formats.e2m1_value(v) for v in n[0]]
    assert vals == [-1.0, -0.0, 0.5, 1.0] and np.signbit(vals[1])


def _dense_fp4_independent(packed, scale_bytes):
    """FP4 weights from the e2m1 bit-field definition, element by element, and torch's
    float8_e8m0fnu for the scales."""
    p = np.asarray(packed)
    rows, nb = p.shape
    vals = np.zeros((rows, nb * 2))
    for r in range(rows):
        for i in range(nb):
            vals[r, 2 * i] = formats.e2m1_value(int(p[r, i]) & 15)
            vals[r, 2 * i + 1] = formats.e2m1_value(int(p[r, i]) >> 4)
    s = torch.from_numpy(np.ascontiguousarray(scale_bytes, dtype=np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return vals * np.repeat(s, 32, axis=1)


def test_fp4_single_expert_top1_is_dense_silu_mlp():
    """FP4 experts (README bullet "FP4 recovery - used surgically"), E = 1, top-1: the dense gated
    MLP with torch's silu and matmul in float64 on independently dequantized e2m1 weights."""
    rng = np.random.default_rng(13)
    T, K, I = 5, 64, 64
    planes = workloads.draw_planes_fp4(rng, 1, K, I)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    y = forward.moe_forward(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), **planes, fp4=True)
    wgu = torch.from_numpy(_dense_fp4_independent(planes["gu_codes"][0], planes["gu_scales"][0]))
    wdn = torch.from_numpy(_dense_fp4_independent(planes["dn_codes"][0], planes["dn_scales"][0]))
    xt = torch.from_numpy(x)
    ref = torch.matmul(torch.nn.functional.silu(torch.matmul(xt, wgu[:I].T)) * torch.matmul(xt, wgu[I:].T), wdn.T)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(ref.numpy()).max())


def test_fp4_sign_and_scale_invariants_are_exact():
    """Flipping the sign bit of every down code negates y; one more down scale step doubles it;
    both exactly (power-of-two and sign changes are exact in f64)."""
    rng = np.random.default_rng(14)
    T, K, I, E = 7, 64, 64, 3
    planes = workloads.draw_planes_fp4(rng, E, K, I)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    ids, w = workloads.uniform_routing(rng, T, E, 2)
    y = forward.moe_forward(x, ids, w, **planes, fp4=True)
    neg = dict(planes, dn_codes=planes["dn_codes"] ^ np.uint8(0x88))
    assert np.array_equal(forward.moe_forward(x, ids, w, **neg, fp4=True), -y)
    dbl = dict(planes, dn_scales=planes["dn_scales"] + np.uint8(1))
    assert np.array_equal(forward.moe_forward(x, ids, w, **dbl, fp4=True), 2 * y)


def test_brute_force_tiny_multi_expert():
    """E=3 experts, top-2, T=3 tokens, K=I=32, by scalar loops per pair and per output element:
    each weight read straight from its packed byte and scale byte (codebook printed on the pages,
    tests/golden/codebook.txt; UE8M0 value 2^(b-127)), no matrix routine and no grouping by
    expert. Token 1 routes twice to one expert (summed like any pair), token 2 has an invalid id
    (contributes nothing). The oracle's grouped f64 forward must agree to rounding."""
    import math
    book = {}
    with open(os.path.join(GOLDEN, "codebook.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                book[int(c)] = float(v)
    rng = np.random.default_rng(21)
    E, T, K, I, top_k = 3, 3, 32, 32, 2
    gu_codes = rng.integers(0, 256, size=(E, 2 * I, K // 4), dtype=np.uint8)
    gu_scales = (127 + rng.integers(-4, 2, size=(E, 2 * I, K // 32))).astype(np.uint8)
    dn_codes = rng.integers(0, 256, size=(E, K, I // 4), dtype=np.uint8)
    dn_scales = (127 + rng.integers(-4, 2, size=(E, K, I // 32))).astype(np.uint8)
    x_bits = workloads.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    x = formats.bf16_bits_to_f64(x_bits)
    ids = np.array([[2, 0], [1, 1], [0, 7]], np.int32)
    w = np.array([[0.625, 0.375], [0.5, 0.25], [0.75, 0.125]], np.float32)

    def weight(codes, scales, e, r, k):
        code = (int(codes[e, r, k // 4]) >> (2 * (k % 4))) & 3
        return book[code] * 2.0 ** (int(scales[e, r, k // 32]) - 127)

    y = [[0.0] * K for _ in range(T)]
    for t in range(T):
        for j in range(top_k):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            a = []
            for i in range(I):
                g = sum(weight(gu_codes, gu_scales, e, i, k) * float(x[t, k]) for k in range(K))
                u = sum(weight(gu_codes, gu_scales, e, I + i, k) * float(x[t, k]) for k in range(K))
                a.append(g / (1.0 + math.exp(-g)) * u)
            for n in range(K):
                o = sum(weight(dn_codes, dn_scales, e, n, i) * a[i] for i in range(I))
                y[t][n] += float(w[t, j]) * o
    want = np.array(y)
    got = forward.moe_forward(x, ids, w, gu_codes, gu_scales, dn_codes, dn_scales)
    rms = np.sqrt(np.mean(want ** 2))
    assert rms > 0
    assert np.max(np.abs(got - want)) <= 1e-12 * rms
    # a dropped term, a gate/up swap or a wrong expert would be off by orders of magnitude more
    assert np.max(np.abs(got[2] - float(w[2, 0]) * forward.pair_outputs(x, ids, gu_codes, gu_scales, dn_codes,
                                                                        dn_scales)[2, 0])) <= 1e-12 * rms


def _dense_nvfp4_independent(packed, scale_bytes, scale2):
    """NVFP4 weights from the e2m1 bit-field definition element by element, torch's float8_e4m3fn
    for the block-16 scales and an fp32 scale_2 (README opening paragraph; "The v0.24.0 port",
    section "Our hooks", modelopt.py bullet)."""
    p = np.asarray(packed)
    rows, nb = p.shape
    out = np.zeros((rows, nb * 2))
    sb = torch.from_numpy(np.ascontiguousarray(scale_bytes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    s = sb.to(torch.float64).numpy()
    for r in range(rows):
        for k in range(nb * 2):
            nib = (int(p[r, k // 2]) >> (4 * (k % 2))) & 15
            out[r, k] = formats.e2m1_value(nib) * s[r, k // 16] * float(np.float32(scale2))
    return out


def test_nvfp4_dequant_covers_every_finite_scale_encoding():
    """Every finite E4M3FN scale byte (both signs, zero, subnormals, 448) against torch's
    float8_e4m3fn decode, and NaN scale bytes / a non-finite scale_2 are refused."""
    rng = np.random.default_rng(31)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    scales = rng.permutation(np.concatenate([finite, finite])).reshape(4, 127)
    codes = rng.integers(0, 256, size=(4, 127 * 8), dtype=np.uint8)
    got = forward.dequant_rows_nvfp4(codes, scales, np.float32(3.0517578125e-05))
    assert np.array_equal(got, _dense_nvfp4_independent(codes, scales, np.float32(3.0517578125e-05)))
    for bad in (0x7F, 0xFF):
        s = scales.copy()
        s[3, 5] = bad
        with pytest.raises(ValueError):
            forward.dequant_rows_nvfp4(codes, s, 1.0)
    with pytest.raises(ValueError):
        forward.dequant_rows_nvfp4(codes, scales, np.inf)


def test_nvfp4_single_expert_top1_is_dense_silu_mlp():
    """NVFP4 experts, E = 1, top-1: the dense gated MLP with torch's silu and matmul in float64 on
    independently dequantized weights; gate, up and down carry different scale_2 values, so a
    swapped or shared scale_2 fails."""
    rng = np.random.default_rng(32)
    T, K, I = 5, 64, 64
    planes = workloads.draw_planes_nvfp4(rng, 1, K, I)
    planes["gu_scale2"] = np.array([[2.0 ** -14, 3.0 * 2.0 ** -13]], np.float32)
    planes["dn_scale2"] = np.array([5.0 * 2.0 ** -15], np.float32)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    y = forward.moe_forward(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), planes["gu_codes"],
                            planes["gu_scales"], planes["dn_codes"], planes["dn_scales"],
                            nvfp4=(planes["gu_scale2"], planes["dn_scale2"]))
    g = _dense_nvfp4_independent(planes["gu_codes"][0][:I], planes["gu_scales"][0][:I], planes["gu_scale2"][0, 0])
    u = _dense_nvfp4_independent(planes["gu_codes"][0][I:], planes["gu_scales"][0][I:], planes["gu_scale2"][0, 1])
    d = _dense_nvfp4_independent(planes["dn_codes"][0], planes["dn_scales"][0], planes["dn_scale2"][0])
    xt = torch.from_numpy(x)
    ref = torch.matmul(torch.nn.functional.silu(torch.matmul(xt, torch.from_numpy(g).T)) *
                       torch.matmul(xt, torch.from_numpy(u).T), torch.from_numpy(d).T).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_nvfp4_with_power_of_two_pair_scales_is_mxfp4():
    """Special case: when each 32-block's two E4M3 scales are the same power of two 2^(b-127)
    (byte ((b - 120) << 3)) and every scale_2 is 1, the NVFP4 forward is the MXFP4 forward with
    UE8M0 bytes b, exactly."""
    rng = np.random.default_rng(33)
    T, K, I, E = 6, 64, 96, 3
    fp4 = workloads.draw_planes_fp4(rng, E, K, I)
    for name in ("gu_scales", "dn_scales"):
        fp4[name] = (127 + rng.integers(-6, 8, size=fp4[name].shape)).astype(np.uint8)
    to_e4m3 = lambda b: np.repeat(((b.astype(np.int32) - 120) << 3).astype(np.uint8), 2, axis=-1)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    ids, w = workloads.uniform_routing(rng, T, E, 2)
    y4 = forward.moe_forward(x, ids, w, **fp4, fp4=True)
    ynv = forward.moe_forward(x, ids, w, fp4["gu_codes"], to_e4m3(fp4["gu_scales"]), fp4["dn_codes"],
                              to_e4m3(fp4["dn_scales"]), nvfp4=(np.ones((E, 2), np.float32), np.ones(E, np.float32)))
    assert np.array_equal(y4, ynv)


def test_nvfp4_down_scale2_and_scale_sign_invariants_are_exact():
    """Doubling every down scale_2 doubles y; flipping the sign bit of every down E4M3 scale
    negates y; both exactly."""
    rng = np.random.default_rng(34)
    T, K, I, E = 7, 64, 64, 3
    p = workloads.draw_planes_nvfp4(rng, E, K, I)
    x = formats.bf16_bits_to_f64(workloads.draw_x(rng, T, K))
    ids, w = workloads.uniform_routing(rng, T, E, 2)
    fwd = lambda dn_scales, dn_scale2: forward.moe_forward(x, ids, w, p["gu_codes"], p["gu_scales"], p["dn_codes"],
                                                          dn_scales, nvfp4=(p["gu_scale2"], dn_scale2))
    y = fwd(p["dn_scales"], p["dn_scale2"])
    assert np.array_equal(fwd(p["dn_scales"], 2 * p["dn_scale2"]), 2 * y)
    assert np.array_equal(fwd(p["dn_scales"] ^ np.uint8(0x80), p["dn_scale2"]), -y)
