"""GPU moe_w2_codebook_sweep (sign-bias diagnostic) against the oracle.

Block decisions are taken in the same float64 order on both sides, so a tensor of one block gives
bit-identical sse / err; tensor sums over many blocks are added in different orders and are
compared to 1e-12 (sse: a sum of non-negative terms, relative; err: relative to the Cauchy-Schwarz
bound sqrt(N sse) of the sum of |v - x|).
"""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import sweep
import workloads

from gpu_helpers import dev

pytestmark = pytest.mark.gpu

SYM = np.array([-4, -1, 1, 4], np.float32)


def _gpu(x, cbs):
    st, mo, best = moe.moe_w2_codebook_sweep(dev(x), cbs)
    torch.cuda.synchronize()
    return st.cpu().numpy(), mo.cpu().numpy(), best.cpu().numpy()


def _codebooks(seed, k):
    rng = np.random.default_rng(seed)
    fam = workloads.codebook_family()
    pick = fam[np.sort(rng.choice(len(fam), size=k, replace=False))]
    extra = np.array([SYM, [-6, -1, 1, 6], [-2, -1, 0, 1], [-1, 0, 1, 2], [-3, -1, 1, 3]], np.float32)
    return np.concatenate([pick, extra])


def _check_close(st, mo, best, st_o, mo_o, best_o, N):
    sse, sse_o = st[..., 0], st_o[..., 0]
    assert np.all(np.abs(sse - sse_o) <= 1e-12 * sse_o + 1e-300)
    bound = np.sqrt(N * sse_o) + 1e-300
    assert np.all(np.abs(st[..., 1] - st_o[..., 1]) <= 1e-12 * bound)
    assert np.allclose(st[..., 2], st_o[..., 2], rtol=1e-12, atol=0)
    assert np.all(np.abs(st[..., 3] - st_o[..., 3]) <= 1e-12 * np.abs(st_o[..., 2]) + 1e-300)
    assert np.allclose(mo[:, 0], mo_o[:, 0], rtol=1e-12, atol=0)
    assert np.all(np.abs(mo[:, 1] - mo_o[:, 1]) <= 1e-12 * np.sqrt(N * mo_o[:, 0]))
    for t in range(best.shape[0]):
        for k in range(2):
            if best[t, k] != best_o[t, k]:   # a near-tie between two codebooks' tensor sums
                a, b = st_o[t, best[t, k], 0], st_o[t, best_o[t, k], 0]
                assert abs(a - b) <= 1e-12 * b, (t, k)


@pytest.mark.parametrize("shape", [(3, 16, 256), (2, 37, 96), (1, 1, 32), (5, 64, 1024)])
def test_parity_small(gpu, shape):
    """Several tensors; block counts that leave ragged workgroups (37*96/32 = 111 blocks)."""
    n, R, C = shape
    x = np.stack([workloads.sweep_tensor(i, R=R, C=C) for i in range(n)])
    cbs = _codebooks(1, 60)
    st, mo, best = _gpu(x, cbs)
    st_o, mo_o, best_o = sweep.codebook_sweep(x, cbs)
    _check_close(st, mo, best, st_o, mo_o, best_o, R * C)


def test_single_blocks_bit_identical(gpu):
    """One block per tensor: the GPU's sse and err are the block's own, bit for bit, over blocks with
    zeros of both signs, ties at code midpoints, fp32 subnormals, huge values and all-zero blocks."""
    rng = np.random.default_rng(3)
    tiny = np.float32(2.0 ** -149)
    fixed = [
        np.zeros(32), -np.zeros(32), np.array([0.0, -0.0] * 16), np.array([tiny, -tiny] * 16),
        np.array([3.0e38, -3.0e38, 1.0, -1.0] * 8), np.array([2.5, -2.5, 0.0, -0.0, 1.0, 4.0, -1.0, -4.0] * 4),
        np.array([0.5, -0.5, 1.5, -1.5, 0.0, -0.0, 3.0, -3.0] * 4), np.concatenate([[1.0], np.zeros(31)]),
        np.concatenate([[-0.0], np.full(31, 1e-30)]),
    ]
    rand = [rng.integers(-16, 17, 32) * 0.25 * 2.0 ** rng.integers(-3, 4) for _ in range(40)]
    rand += [rng.standard_normal(32) * 2.0 ** rng.integers(-30, 30) for _ in range(40)]
    x = np.stack([np.asarray(b, np.float32) for b in fixed + rand])[:, None, :]
    cbs = _codebooks(2, 40)
    st, mo, best = _gpu(x, cbs)
    for t in range(x.shape[0]):
        for m in range(len(cbs)):
            _, sse, err = sweep.block_choice_c(x[t, 0], cbs[m])
            assert st[t, m, 0] == sse, (t, m)
            assert st[t, m, 1] == err or (st[t, m, 1] == 0 and err == 0), (t, m)


def test_full_family_workload_shape_sampled(gpu):
    """The bench workload: 8 tensors of [2048, 6144] against all 1239 candidate codebooks, in one
    call. Sampled check: tensor 0 and 7 under the symmetric codebook, the GPU's best symmetric and
    asymmetric ones and a few more, recomputed by the oracle."""
    n, R, C = 8, 2048, 6144
    fam = workloads.codebook_family()
    x = np.stack([workloads.sweep_tensor(i) for i in range(n)])
    print(f"sweep {n} x [{R}, {C}] x {len(fam)} codebooks", flush=True)
    st, mo, best = _gpu(x, fam)
    i_sym = int(np.where((fam == SYM).all(1))[0][0])
    for t in (0, n - 1):
        ms = sorted({i_sym, int(best[t, 0]), int(best[t, 1]), 0, len(fam) - 1, 617})
        st_o, mo_o, _ = sweep.codebook_sweep(x[t:t + 1], fam[ms])
        _check_close(st[t:t + 1, ms], mo[t:t + 1], np.zeros((1, 2), np.int32), st_o, mo_o,
                     np.zeros((1, 2), np.int32), R * C)
    # best indices are argmins of the returned sse over each kind
    sym = (fam[:, 0] == -fam[:, 3]) & (fam[:, 1] == -fam[:, 2])
    for t in range(n):
        assert best[t, 0] == np.where(sym)[0][np.argmin(st[t, sym, 0])]
        assert best[t, 1] == np.where(~sym)[0][np.argmin(st[t, ~sym, 0])]


def test_deterministic(gpu):
    x = np.stack([workloads.sweep_tensor(i, R=128, C=512) for i in range(3)])
    cbs = _codebooks(4, 30)
    a = _gpu(x, cbs)
    b = _gpu(x, cbs)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_errors_and_empty(gpu):
    x = np.stack([workloads.sweep_tensor(0, R=4, C=64)])
    bad = x.copy()
    bad[0, 1, 5] = np.nan
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(bad, SYM[None])
    assert ei.value.status == -8
    bad[0, 1, 5] = np.inf
    with pytest.raises(moe.MoeW2Error):
        _gpu(bad, SYM[None])
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(x, np.array([[-1, 1, 1, 4]], np.float32))            # not strictly ascending
    assert ei.value.status == -1
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(x, np.array([[-1, 1, 2, np.inf]], np.float32))
    assert ei.value.status == -1
    with pytest.raises(moe.MoeW2Error) as ei:
        _gpu(np.zeros((1, 2, 48), np.float32), SYM[None])         # C % 32 != 0
    assert ei.value.status == -2
    st, mo, best = _gpu(np.zeros((2, 0, 64), np.float32), np.array([SYM, [-2, -1, 0, 1]], np.float32))
    assert np.all(st == 0) and np.all(mo == 0) and best.tolist() == [[0, 1], [0, 1]]


def test_most_codebooks_allowed(gpu):
    """4096 candidate codebooks (the maximum) on a small tensor: every statistic against the oracle."""
    rng = np.random.default_rng(17)
    cbs = np.sort(rng.uniform(-8, 8, size=(4096, 4)), axis=1).astype(np.float32)
    cbs[:, 1] += np.float32(1e-3)          # keep each row strictly ascending after rounding
    cbs[:, 2] += np.float32(2e-3)
    cbs[:, 3] += np.float32(3e-3)
    cbs = np.sort(cbs, axis=1)
    assert np.all(np.diff(cbs, axis=1) > 0)
    x = np.stack([workloads.sweep_tensor(i, R=4, C=64) for i in range(2)])
    st, mo, best = _gpu(x, cbs)
    st_o, mo_o, best_o = sweep.codebook_sweep(x, cbs)
    _check_close(st, mo, best, st_o, mo_o, best_o, 4 * 64)
