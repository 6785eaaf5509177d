"""GPU parity of moe_w2_forward (decode and GEMM kernels) against the f64 oracle, plus exact
invariants of the GPU path. Bar: max |y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) on the fp32
output; the bf16 output must be the round-to-nearest-even of the fp32 output, bit for bit."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import formats, forward as oracle_fwd
import workloads

from gpu_helpers import bf16_rne_bits, dev, dev_bf16, forward, pack, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-2
PATHS = [moe.PATH_DECODE, moe.PATH_GEMM, moe.PATH_DECODE_SORTED]
DECODE_PATHS = (moe.PATH_DECODE, moe.PATH_DECODE_SORTED)


def _oracle(case, tokens=None):
    x = formats.bf16_bits_to_f64(case["x"])
    return oracle_fwd.moe_forward(x, case["topk_ids"], case["topk_w"], case["gu_codes"], case["gu_scales"],
                                  case["dn_codes"], case["dn_scales"], tokens=tokens)


def _case(T, K, I, E, top_k, seed, zipf=False):
    rng = np.random.default_rng(seed)
    planes = workloads.draw_planes(rng, E, K, I)
    x = workloads.draw_x(rng, T, K)
    if zipf:
        ids, w = workloads.zipf_routing(rng, T, E, top_k, rank_perm=rng.permutation(E))
    else:
        ids, w = workloads.uniform_routing(rng, T, E, top_k)
    return dict(planes, x=x, topk_ids=ids, topk_w=w)


@pytest.fixture(scope="module")
def tiny(gpu):
    d = workloads.tiny()
    return d, pack(d), _oracle(d)


@pytest.mark.parametrize("path", PATHS)
def test_tiny_layer_parity(tiny, path):
    d, h, y_ref = tiny
    y = forward(h, d["x"], d["topk_ids"], d["topk_w"], moe.OUT_F32, path).cpu().numpy()
    err = rel_max_err(y, y_ref)
    print(f"tiny path={path} rel max err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("path", PATHS)
def test_bf16_output_is_rne_of_f32(tiny, path):
    d, h, _ = tiny
    y32 = forward(h, d["x"], d["topk_ids"], d["topk_w"], moe.OUT_F32, path).cpu().numpy()
    y16 = forward(h, d["x"], d["topk_ids"], d["topk_w"], moe.OUT_BF16, path)
    bits = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, bf16_rne_bits(y32))


CASES = [
    # several tiles along every axis with ragged tails: (T, K, I, E, top_k, seed, zipf)
    (37, 512, 768, 16, 4, 21, False),
    (300, 768, 512, 8, 2, 22, False),
    (200, 1024, 256, 32, 8, 23, True),
    (3, 256, 256, 4, 4, 24, False),     # top_k == E
    (3, 512, 512, 8, 3, 25, False),     # 9 pairs: the fewest the routed decode organisation takes
    (128, 512, 256, 4, 4, 26, True),    # 512 pairs: the most the decode kernels take
    (20, 512, 1024, 64, 8, 27, False),  # >= 32 groups, I/256 a multiple of 4: two row pairs per wave in down
    (24, 768, 768, 48, 6, 28, True),    # >= 32 groups, I/256 = 3: one row pair per wave, 4 per workgroup
    (40, 256, 256, 1024, 8, 29, True),  # E = 1024, the most experts a layer may have
    # I = 2048 with K a multiple of 512: the down GEMM streams k-tiles across the tiles a workgroup
    # walks (one workgroup per compute unit)
    (256, 1024, 2048, 256, 8, 30, False),  # ~8 rows per expert: 512 down tiles, 2 per workgroup, ragged
    (512, 2048, 2048, 16, 8, 31, True),    # Zipf groups of several M-tiles: 320 down tiles
    (65, 512, 2048, 8, 8, 34, False),      # 520 pairs, one N-block: 16 down tiles (8 of one valid row), most workgroups idle
    (150, 768, 2048, 8, 4, 35, True),      # I = 2048 but K not a multiple of 512: the tile-at-a-time down GEMM
    (300, 1024, 512, 32, 4, 36, True),     # I = 512 (2 k-tiles per tile): the streamed down GEMM's short form
    # K = 3072 and 6144 (12 and 24 k-tiles) over many experts of few rows: several gate_up tiles per
    # row of workgroups
    (256, 3072, 512, 256, 8, 32, False),   # ~8 rows per expert: ~520 gate_up tiles
    (512, 6144, 256, 256, 8, 33, False),   # ~16 rows per expert, 24 k-tiles per tile
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}K{c[1]}I{c[2]}E{c[3]}k{c[4]}" for c in CASES])
@pytest.mark.parametrize("path", PATHS)
def test_mid_size_parity(gpu, case, path):
    T, K, I, E, top_k, seed, zipf = case
    c = _case(T, K, I, E, top_k, seed, zipf)
    h = pack(c)
    if path == moe.PATH_DECODE and T * top_k > 512:
        # the routed decode organisation stops at 512 pairs (the sorted one takes any number)
        with pytest.raises(moe.MoeW2Error) as exc:
            forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path)
        assert exc.value.status == -2
        return
    y_ref = _oracle(c)
    y = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    err = rel_max_err(y, y_ref)
    print(f"{case} path={path} rel max err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("path", PATHS)
def test_wide_dynamic_range_inputs(gpu, path):
    """The A operand is split into e4m3 parts per 32-value block: x blocks holding one large value
    and values 2^-6 .. 2^-24 of it, gated intermediates of widely different size (scale bytes
    40 .. 200 spread over rows and blocks; gate_up bytes 110 .. 125 keep |a| within fp16), and a
    block whose x is all zero stay within the bar."""
    c = _case(40, 512, 512, 8, 4, 51)
    rng = np.random.default_rng(52)
    xf = rng.standard_normal((40, 512)).astype(np.float32) * np.exp2(-rng.integers(6, 25, size=(40, 512)))
    xf[:, ::32] = np.where(rng.random((40, 16)) < 0.5, 8.0, -8.0)
    xf[3, 64:96] = 0.0
    c["x"] = workloads.f32_to_bf16_bits(xf)
    c["gu_scales"] = rng.integers(110, 126, size=c["gu_scales"].shape).astype(np.uint8)
    c["dn_scales"] = rng.integers(40, 200, size=c["dn_scales"].shape).astype(np.uint8)
    y_ref = _oracle(c)
    h = pack(c)
    y = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    err = rel_max_err(y, y_ref)
    print(f"wide dynamic range path={path} rel max err {err:.2e}")
    assert np.all(np.isfinite(y))
    assert err <= TOL


def test_paths_agree_closely(gpu):
    """The two kernel families on one layer. They feed the matrix instruction differently: the
    decode kernels split x and the fp16 gated intermediate exactly into e4m3 parts, the GEMM
    kernels into three e2m3 parts whose sum is within 2^-13 of the block maximum per element. So
    they agree to a few 1e-3 of rms (each is also held to the oracle bar on its own)."""
    c = _case(64, 512, 512, 8, 4, 31)
    h = pack(c)
    a = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, moe.PATH_DECODE).cpu().numpy()
    b = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, moe.PATH_GEMM).cpu().numpy()
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2))
    rel = float(np.max(np.abs(a - b)) / rms)
    print(f"decode vs GEMM path: max|diff| / rms = {rel:.2e}")
    assert rel <= 5e-3


@pytest.mark.parametrize("path", PATHS)
def test_repeats_are_bit_identical(gpu, path):
    c = _case(64, 512, 512, 16, 8, 41, zipf=True)
    h = pack(c)
    ws = moe.alloc_workspace(h, 64, 8)
    ys = [forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path, ws).cpu().numpy() for _ in range(6)]
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))


@pytest.mark.parametrize("path", PATHS)
def test_down_scale_doubling_is_exact_and_negation_nearly(gpu, path):
    c = _case(40, 512, 512, 8, 2, 51)
    y = forward(pack(c), c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    c2 = dict(c, dn_scales=(c["dn_scales"] + 1).astype(np.uint8))
    y2 = forward(pack(c2), c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    assert np.array_equal(y2, 2 * y)
    c3 = dict(c, dn_codes=(~c["dn_codes"]).astype(np.uint8))
    y3 = forward(pack(c3), c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    # The matrix cores' fp32 accumulation is not sign-symmetric in its last bit, so negating the
    # down weights negates y up to last-bit rounding (exact would need symmetric rounding).
    d = np.abs(y3.astype(np.float64) + y)
    ulp = np.spacing(np.abs(y).astype(np.float32)).astype(np.float64)
    print(f"negation: {np.count_nonzero(d)} of {d.size} entries differ, max {np.max(d / ulp):.1f} ulp")
    assert np.max(d) <= 1e-5 * np.sqrt(np.mean(y.astype(np.float64) ** 2))


@pytest.mark.parametrize("path", PATHS)
def test_invalid_ids_contribute_nothing_and_are_counted(gpu, path):
    c = _case(20, 256, 512, 8, 4, 61)
    ids = c["topk_ids"].copy()
    ids[::3, 1] = -1
    ids[1::5, 3] = 8       # == E, out of range
    n_bad = int(((ids < 0) | (ids >= 8)).sum())
    h = pack(c)
    ws = moe.alloc_workspace(h, 20, 4)
    y = forward(h, c["x"], ids, c["topk_w"], moe.OUT_F32, path, ws).cpu().numpy()
    inv, ovf = moe.moe_w2_read_counters(ws)
    assert inv == n_bad and ovf == 0
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), ids, c["topk_w"], c["gu_codes"], c["gu_scales"],
                                   c["dn_codes"], c["dn_scales"])
    assert rel_max_err(y, y_ref) <= TOL


@pytest.mark.parametrize("path", PATHS)
def test_duplicate_ids_are_summed(gpu, path):
    c = _case(16, 256, 256, 4, 2, 71)
    ids = np.stack([c["topk_ids"][:, 0]] * 2, axis=1).astype(np.int32)
    y = forward(pack(c), c["x"], ids, c["topk_w"], moe.OUT_F32, path).cpu().numpy()
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), ids, c["topk_w"], c["gu_codes"], c["gu_scales"],
                                   c["dn_codes"], c["dn_scales"])
    assert rel_max_err(y, y_ref) <= TOL


def test_zero_tokens_is_a_noop(gpu):
    c = _case(4, 256, 256, 4, 2, 81)
    h = pack(c)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    y = moe.moe_w2_forward(h, x, ids, w, out_dtype=moe.OUT_F32)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_workspace_too_small_is_rejected(gpu):
    c = _case(4, 256, 256, 4, 2, 82)
    h = pack(c)
    ws = torch.empty(moe.moe_w2_workspace_bytes(h, 4, 2) - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeW2Error) as ei:
        forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, moe.PATH_AUTO, ws)
    assert ei.value.status == -6


def test_down_rows_with_large_exponent_spread(gpu):
    """Down rows whose scale bytes lie far from 127 and spread over up to 30 exponents."""
    c = _case(24, 256, 512, 4, 2, 91)
    rng = np.random.default_rng(92)
    base = rng.integers(20, 220, size=(4, 256, 1))
    c["dn_scales"] = (base + rng.integers(0, 30, size=(4, 256, 16))).astype(np.uint8)
    y_ref = _oracle(c)
    h = pack(c)
    for path in PATHS:
        y = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
        assert rel_max_err(y, y_ref) <= TOL


@pytest.mark.parametrize("T", [1, 2])
def test_tiny_batch_direct_path(gpu, T):
    """P = T*top_k <= 8 runs without a routing pass; invalid and duplicate ids included."""
    c = _case(T, 512, 512, 16, 4, 101 + T)
    ids = c["topk_ids"].copy()
    ids[0, 1] = -1
    ids[0, 2] = ids[0, 3]           # duplicate expert within a token
    h = pack(c)
    ws = moe.alloc_workspace(h, T, 4)
    for path in (moe.PATH_AUTO, moe.PATH_DECODE):
        y = forward(h, c["x"], ids, c["topk_w"], moe.OUT_F32, path, ws).cpu().numpy()
        y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), ids, c["topk_w"], c["gu_codes"],
                                       c["gu_scales"], c["dn_codes"], c["dn_scales"])
        assert rel_max_err(y, y_ref) <= TOL
        inv, ovf = moe.moe_w2_read_counters(ws)
        assert inv == 1 and ovf == 0


def test_all_ids_invalid_gives_zero(gpu):
    for T in (1, 16):
        c = _case(T, 256, 256, 4, 2, 111)
        ids = np.full((T, 2), -1, np.int32)
        y = forward(pack(c), c["x"], ids, c["topk_w"], moe.OUT_F32, moe.PATH_AUTO).cpu().numpy()
        assert np.all(y == 0)


@pytest.mark.parametrize("T,path", [(2, moe.PATH_DECODE), (16, moe.PATH_DECODE), (16, moe.PATH_GEMM)],
                         ids=["direct", "routed-decode", "gemm"])
def test_act_overflow_is_counted(gpu, T, path):
    """Gate/up scales that push part of silu(g) * u past the fp16 range: the counter equals the
    oracle's count of |a| >= 65520 (rounds to inf in fp16), up to entries within 1% of that bound."""
    c = _case(T, 256, 512, 8, 4, 121)
    rng = np.random.default_rng(122)
    c["gu_scales"] = rng.integers(127, 132, size=c["gu_scales"].shape).astype(np.uint8)
    a = np.abs(oracle_fwd.moe_forward_act(formats.bf16_bits_to_f64(c["x"]), c["topk_ids"], c["gu_codes"],
                                          c["gu_scales"]))
    lo, hi = int(np.sum(a >= 65520 * 1.01)), int(np.sum(a >= 65520 * 0.99))
    h = pack(c)
    ws = moe.alloc_workspace(h, T, 4)
    forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path, ws)
    inv, ovf = moe.moe_w2_read_counters(ws)
    print(f"T={T} path={path}: act_overflow {ovf}, oracle {lo}..{hi} of {a.size}")
    assert lo > 0 and inv == 0 and lo <= ovf <= hi


def _random_cases(n=14, seed=2024):
    """Shapes drawn once from a fixed seed: T in [1, 160], K and I multiples of 256 up to 1280 (so
    I/256 takes values that do and do not divide the decode ring), E in [1, 96], top_k up to
    min(8, E), uniform or Zipf routing - a spread of group counts, chunk splits and ragged tiles."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 97))
        top_k = int(rng.integers(1, min(8, E) + 1))
        out.append((int(rng.integers(1, 161)), 256 * int(rng.integers(1, 6)), 256 * int(rng.integers(1, 6)), E, top_k,
                    1000 + i, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"T{c[0]}K{c[1]}I{c[2]}E{c[3]}k{c[4]}{'z' if c[6] else 'u'}")
def test_random_shapes_parity(gpu, case):
    """Both kernel families against the oracle (the routed decode organisation only where
    T*top_k <= 512)."""
    T, K, I, E, top_k, seed, zipf = case
    c = _case(T, K, I, E, top_k, seed, zipf)
    h = pack(c)
    y_ref = _oracle(c)
    for path in PATHS:
        if path == moe.PATH_DECODE and T * top_k > 512:
            continue
        y = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path).cpu().numpy()
        err = rel_max_err(y, y_ref)
        print(f"{case} path={path} rel max err {err:.2e}")
        assert err <= TOL, (case, path, err)


@pytest.mark.parametrize("path", DECODE_PATHS, ids=["routed", "sorted"])
@pytest.mark.parametrize("out_dtype", [moe.OUT_F32, moe.OUT_BF16], ids=["f32", "bf16"])
def test_decode_routed_edge_tokens(gpu, out_dtype, path):
    """The routed and sorted decode organisations with two row pairs per wave in down (2-bit
    planes, >= 32 active groups, I/256 a multiple of 4): tokens with invalid ids, one with a
    duplicate id and one with no valid id (a zero row). Three forwards on one workspace are
    bit-identical, fp32 matches the oracle and bf16 is its round-to-nearest-even, and a stage
    sequence that runs the down stage twice gives the same y."""
    T, K, I, E, top_k = 24, 512, 1024, 64, 8
    c = _case(T, K, I, E, top_k, 71)
    ids = c["topk_ids"].copy()
    ids[::4, 2] = -1
    ids[1::6, 5] = E
    ids[3, 1] = ids[3, 0]
    ids[7, :] = -1
    h = pack(c)
    ws = moe.alloc_workspace(h, T, top_k)
    ys = [forward(h, c["x"], ids, c["topk_w"], out_dtype, path, ws) for _ in range(3)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    y32 = forward(h, c["x"], ids, c["topk_w"], moe.OUT_F32, path, ws).cpu().numpy()
    assert np.all(y32[7] == 0)
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), ids, c["topk_w"], c["gu_codes"], c["gu_scales"],
                                   c["dn_codes"], c["dn_scales"])
    assert rel_max_err(y32, y_ref) <= TOL
    if out_dtype == moe.OUT_BF16:   # bf16 output = RNE of the same path's fp32 result
        bits = ys[0].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits, bf16_rne_bits(y32))
    inv, _ = moe.moe_w2_read_counters(ws)
    assert inv == int(((ids < 0) | (ids >= E)).sum())
    # stages one at a time, the down stage twice
    x_d, ids_d, w_d = dev_bf16(c["x"]), dev(ids), dev(np.asarray(c["topk_w"], np.float32))
    y2 = torch.full_like(ys[0], 7.0)
    for st in (moe.STAGE_ROUTE, moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        moe.moe_w2_forward_stage(st, h, x_d, ids_d, w_d, y2, ws, out_dtype, path)
    torch.cuda.synchronize()
    assert torch.equal(y2, ys[0])


@pytest.mark.parametrize("T,path,zipf", [(1, moe.PATH_DECODE, False), (40, moe.PATH_DECODE, False),
                                         (40, moe.PATH_DECODE_SORTED, True),
                                         (12, moe.PATH_GEMM, False), (300, moe.PATH_GEMM, True)],
                         ids=["direct", "routed-decode", "sorted-decode-zipf", "gemm-single-row-tiles", "gemm-zipf"])
def test_stages_in_order_equal_forward(gpu, T, path, zipf):
    """ROUTE, GATE_UP, DOWN, COMBINE called one at a time on one workspace give moe_w2_forward's y
    bit for bit, for each organisation; at T=12 on the GEMM kernels nearly every M-tile holds a
    single valid row (the gate_up epilogue writes only that row's split records)."""
    K, I, E, top_k = 512, 1024, 64, 8
    c = _case(T, K, I, E, top_k, 81 + T, zipf=zipf)
    h = pack(c)
    ws = moe.alloc_workspace(h, T, top_k)
    y = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, path, ws)
    x_d, ids_d = dev_bf16(c["x"]), dev(np.asarray(c["topk_ids"], np.int32))
    w_d = dev(np.asarray(c["topk_w"], np.float32))
    y2 = torch.full_like(y, 7.0)
    for st in (moe.STAGE_ROUTE, moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        moe.moe_w2_forward_stage(st, h, x_d, ids_d, w_d, y2, ws, moe.OUT_F32, path)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(c["x"]), c["topk_ids"], c["topk_w"], c["gu_codes"],
                                   c["gu_scales"], c["dn_codes"], c["dn_scales"])
    assert rel_max_err(y.cpu().numpy(), y_ref) <= TOL


@pytest.mark.parametrize("T,zipf", [(2, False), (5, True), (24, False), (48, True), (64, True), (64, False)])
def test_sorted_and_routed_decode_agree(gpu, T, zipf):
    """The two decode organisations process the same 4-row chunks of each expert with the same
    per-row arithmetic where no expert has more than 4 pairs (only the workgroup order differs):
    their outputs agree bit for bit. Where an expert has more, the sorted organisation passes its
    weights once per 16 rows, splitting the gate_up reduction into slices summed afterwards, so
    the two agree to rounding (within 2e-3 of rms) and each meets the oracle bar (K=1024, I=512,
    E=64, top-8, up to the 512-pair limit of the routed organisation)."""
    K, I, E, top_k = 1024, 512, 64, 8
    c = _case(T, K, I, E, top_k, 300 + T, zipf=zipf)
    h = pack(c)
    a = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, moe.PATH_DECODE)
    b = forward(h, c["x"], c["topk_ids"], c["topk_w"], moe.OUT_F32, moe.PATH_DECODE_SORTED)
    largest = int(np.bincount(np.asarray(c["topk_ids"]).ravel(), minlength=E).max())
    if largest <= 4:
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        return
    d = rel_max_err(b.cpu().numpy(), a.cpu().numpy().astype(np.float64))
    print(f"T={T} zipf={zipf}: largest group {largest}, routed vs sorted rel max diff {d:.2e}")
    assert d <= 2e-3
    y_ref = _oracle(c)
    assert rel_max_err(a.cpu().numpy(), y_ref) <= TOL and rel_max_err(b.cpu().numpy(), y_ref) <= TOL


GROUPS = [5, 8, 9, 15, 16, 17, 31, 33, 64, 1, 2, 3, 4]


@pytest.mark.parametrize("E,fmt", [(24, "w2"), (96, "w2"), (96, "w4"), (96, "nvfp4")],
                         ids=["few-groups-w2", "w2", "w4", "nvfp4"])
def test_sorted_wide_groups(gpu, E, fmt):
    """The sorted organisation's split groups: experts with 5, 8, 9, 15, 16, 17, 31, 33 and 64
    pairs (groups of 16 rows split into 2 to 4 reduction slices, and ragged last groups of 1 to 4
    rows that run unsplit) next to experts with 1 to 4 pairs, on workgroups of one row pair
    (fewer than 32 groups) and of four; all three weight formats against the f64 oracle, the
    forward's stages one at a time bit-identical to the forward, repeats bit-identical."""
    T, K, I, top_k = 64, 768, 512, 8
    rng = np.random.default_rng(500 + E)
    if fmt == "w2":
        planes = workloads.draw_planes(rng, E, K, I)
    elif fmt == "w4":
        planes = workloads.draw_planes_fp4(rng, E, K, I)
    else:
        planes = workloads.draw_planes_nvfp4(rng, E, K, I)
    x = workloads.draw_x(rng, T, K)
    sizes = GROUPS if E > 24 else GROUPS[:9]
    ids, w = workloads.grouped_routing(rng, T, E, top_k, sizes)
    if fmt == "w2":
        h = pack(planes)
        fwd = moe.moe_w2_forward
    elif fmt == "w4":
        h = moe.moe_w4_pack(*[dev(planes[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")])
        fwd = moe.moe_w4_forward
    else:
        h = moe.moe_w4_pack_nvfp4(*[dev(planes[k]) for k in ("gu_codes", "gu_scales", "gu_scale2", "dn_codes",
                                                              "dn_scales", "dn_scale2")])
        fwd = moe.moe_w4_forward
    x_d, ids_d, w_d = dev_bf16(x), dev(ids), dev(w)
    ws = moe.alloc_workspace(h, T, top_k)
    y = fwd(h, x_d, ids_d, w_d, out_dtype=moe.OUT_F32, path=moe.PATH_DECODE_SORTED, workspace=ws)
    y_again = fwd(h, x_d, ids_d, w_d, out_dtype=moe.OUT_F32, path=moe.PATH_DECODE_SORTED, workspace=ws)
    y2 = torch.full_like(y, 7.0)
    for st in (moe.STAGE_ROUTE, moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        moe.moe_w2_forward_stage(st, h, x_d, ids_d, w_d, y2, ws, moe.OUT_F32, moe.PATH_DECODE_SORTED)
    torch.cuda.synchronize()
    assert torch.equal(y, y_again) and torch.equal(y2, y)
    nv = (planes["gu_scale2"], planes["dn_scale2"]) if fmt == "nvfp4" else None
    y_ref = oracle_fwd.moe_forward(formats.bf16_bits_to_f64(x), ids, w, planes["gu_codes"], planes["gu_scales"],
                                   planes["dn_codes"], planes["dn_scales"], fp4=fmt == "w4", nvfp4=nv)
    err = rel_max_err(y.cpu().numpy(), y_ref)
    print(f"E={E} {fmt}: rel max err {err:.2e}")
    assert err <= TOL
