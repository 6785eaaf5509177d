"""Expert slots (moe_w2_planes_create / moe_w2_pack_slot / moe_w2_forward_slots) through the C ABI.
The pages' expert cache (README paragraph on the base cache; "The v0.24.0 port", BASE cache
bullet): a missing expert's contribution is zeroed and an in-graph miss counter bumped; after the
missing experts are fetched, the replayed step is bit-identical to a fully resident forward.
Checked here on both kernel families: a full slot map gives exactly the plain forward's bits;
misses are counted exactly, give exactly the plain forward with those pairs' ids invalid, and
match the f64 oracle over the resident experts within 1e-2 * rms; a captured graph replayed
after the missing experts are packed and the device map updated gives the fully resident bits."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
from oracle import formats, forward as oracle_fwd
import workloads

from gpu_helpers import dev, dev_bf16, pack, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-2
# (T, path); top_k = 4. The sorted decode case (Zipf routing over 16 experts, ~12 pairs each) has
# split groups in both stages.
CASES = [(48, moe.PATH_DECODE), (48, moe.PATH_DECODE_SORTED), (300, moe.PATH_GEMM)]


def _layer(T, seed, K=512, I=256, E=16, top_k=4):
    rng = np.random.default_rng(seed)
    planes = workloads.draw_planes(rng, E, K, I)
    x = workloads.draw_x(rng, T, K)
    ids, w = workloads.zipf_routing(rng, T, E, top_k, rank_perm=rng.permutation(E))
    ids = ids.copy()
    ids[0, 1] = -1          # one invalid pair: not a miss, still counted as invalid
    return planes, x, ids, w, rng


def _fill(h, planes, slot_of_expert, experts):
    for e in experts:
        moe.moe_w2_pack_slot(h, int(slot_of_expert[e]), dev(planes["gu_codes"][e]), dev(planes["gu_scales"][e]),
                             dev(planes["dn_codes"][e]), dev(planes["dn_scales"][e]))


def _bits(t):
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("T,path", CASES)
def test_full_slot_map_is_bit_identical_to_forward(gpu, T, path):
    planes, x, ids, w, rng = _layer(T, 70 + T)
    E = planes["gu_codes"].shape[0]
    xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
    ref = moe.moe_w2_forward(pack(planes), xd, idd, wd, out_dtype=moe.OUT_F32, path=path)
    slot_of = rng.permutation(E).astype(np.int32)
    h = moe.moe_w2_planes_create(E, planes["gu_codes"].shape[2] * 4, planes["gu_codes"].shape[1] // 2)
    _fill(h, planes, slot_of, range(E))
    ws = moe.alloc_workspace(h, T, ids.shape[1])
    y = moe.moe_w2_forward_slots(h, dev(slot_of), xd, idd, wd, out_dtype=moe.OUT_F32, workspace=ws, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(ref))
    inv, _ = moe.moe_w2_read_counters(ws)
    assert moe.moe_w2_read_miss_counter(ws) == 0 and inv == 1


@pytest.mark.parametrize("T,path", CASES)
def test_misses_contribute_nothing_and_are_counted(gpu, T, path):
    planes, x, ids, w, rng = _layer(T, 80 + T)
    E, K, I = planes["gu_codes"].shape[0], planes["gu_codes"].shape[2] * 4, planes["gu_codes"].shape[1] // 2
    S = 10
    resident = np.zeros(E, bool)
    resident[rng.permutation(E)[:S]] = True
    slot_of = np.full(E, -1, np.int32)
    slot_of[resident] = rng.permutation(S)
    slot_of[~resident] = rng.choice([-1, S, 1 << 20], size=int((~resident).sum()))   # outside [0, S)
    h = moe.moe_w2_planes_create(S, K, I)
    _fill(h, planes, slot_of, np.nonzero(resident)[0])
    xd, wd = dev_bf16(x), dev(w)
    ws = moe.alloc_workspace(h, T, ids.shape[1])
    y = moe.moe_w2_forward_slots(h, dev(slot_of), xd, dev(ids), wd, out_dtype=moe.OUT_F32, workspace=ws, path=path)
    torch.cuda.synchronize()
    masked, n_miss = oracle_fwd.resident_ids(ids, E, resident)
    assert n_miss > 0
    assert moe.moe_w2_read_miss_counter(ws) == n_miss
    inv, _ = moe.moe_w2_read_counters(ws)
    assert inv == n_miss + 1
    # exactly the plain forward on fully packed planes with the missing experts' pairs invalid
    ref = moe.moe_w2_forward(pack(planes), xd, dev(masked), wd, out_dtype=moe.OUT_F32, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(ref))
    y_or = oracle_fwd.moe_forward_resident(formats.bf16_bits_to_f64(x), ids, w, planes["gu_codes"], planes["gu_scales"],
                                           planes["dn_codes"], planes["dn_scales"], resident)
    err = rel_max_err(y.cpu().numpy(), y_or)
    print(f"T={T} path={path}: {n_miss} misses, rel max err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("T,path", CASES)
def test_graph_replay_after_fetch_is_bit_identical_to_resident(gpu, T, path):
    planes, x, ids, w, rng = _layer(T, 90 + T)
    E, K, I = planes["gu_codes"].shape[0], planes["gu_codes"].shape[2] * 4, planes["gu_codes"].shape[1] // 2
    xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
    full = moe.moe_w2_forward(pack(planes), xd, idd, wd, out_dtype=moe.OUT_F32, path=path).clone()
    slots = rng.permutation(E).astype(np.int32)           # the slot each expert will get
    first = rng.permutation(E)[:E // 2]                    # resident before the step
    slot_map = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    slot_map[torch.from_numpy(first).cuda()] = dev(slots[first])
    h = moe.moe_w2_planes_create(E, K, I)
    _fill(h, planes, slots, first)
    ws = moe.alloc_workspace(h, T, ids.shape[1])
    y = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_w2_forward_slots(h, slot_map, xd, idd, wd, out_dtype=moe.OUT_F32, workspace=ws, path=path, y=y)
    g.replay()
    torch.cuda.synchronize()
    missing = np.setdiff1d(np.unique(ids[(ids >= 0) & (ids < E)]), first)
    res = np.zeros(E, bool)
    res[first] = True
    _, n_miss = oracle_fwd.resident_ids(ids, E, res)
    assert moe.moe_w2_read_miss_counter(ws) == n_miss > 0
    # fetch: pack the missing experts into their slots, update the device map, replay the graph
    _fill(h, planes, slots, missing)
    slot_map[torch.from_numpy(missing).cuda()] = dev(slots[missing])
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(full)), rep
        assert moe.moe_w2_read_miss_counter(ws) == 0


def test_pack_slot_rejects_bad_arguments(gpu):
    rng = np.random.default_rng(1)
    planes = workloads.draw_planes(rng, 2, 256, 256)
    h = moe.moe_w2_planes_create(2, 256, 256)
    with pytest.raises(moe.MoeW2Error):
        moe.moe_w2_pack_slot(h, 2, dev(planes["gu_codes"][0]), dev(planes["gu_scales"][0]),
                             dev(planes["dn_codes"][0]), dev(planes["dn_scales"][0]))
    bad = planes["gu_scales"][0].copy()
    bad[3, 1] = 253
    with pytest.raises(moe.MoeW2Error) as ex:
        moe.moe_w2_pack_slot(h, 1, dev(planes["gu_codes"][0]), dev(bad), dev(planes["dn_codes"][0]),
                             dev(planes["dn_scales"][0]))
    assert ex.value.status == -3
