"""Routing and the f64 forward of the 2-bit routed-expert MoE layer (test infrastructure; see
oracle/__init__). Plain definitions, no blocking or fusion beyond what the definition states;
numpy's matmul is the only library step.

Definition (reading of the pages; the plain reading is stated where they are silent):
* weights: W[r, k] = CODEBOOK[code[r, k]] * 2**(scale[r, k // 32] - 127)
  (README bullet "2-bit expert planes - the sign-bias finding" for the codebook; "The v0.24.0
  port", section "Our hooks", modelopt.py bullet for UE8M0 block-32 scales).
* NVFP4 experts (README opening paragraph and bullet "FP4 recovery - used surgically"; "The
  v0.24.0 port", section "Our hooks", modelopt.py bullet for the format):
  W[r, k] = e2m1(code[r, k]) * e4m3(scale[r, k // 16]) * scale_2, with one fp32 scale_2 per
  tensor: the gate rows, the up rows and the down matrix of an expert each have their own
  (reading: the checkpoint quantizes gate and up as separate tensors; the pages do not say).
* gate_up[e] holds 2I rows: rows 0..I-1 are the gate projection, rows I..2I-1 the up projection
  (the pages are silent on the order; this is the usual fused w13 layout).
* per pair (t, j) with expert e = ids[t, j]:  g = G_e x_t,  u = U_e x_t,
  a = silu(g) * u with silu(z) = z / (1 + exp(-z)),  o = D_e a   (gated MLP; the pages name the
  SiLU-gated product only through the method statement, not a formula).
* y[t] = sum over j = 0..top_k-1 in ascending order of w[t, j] * o_(t, j)  ("Deterministic
  unpermute" bullet: bijective per-pair placement, fixed-order sum). Pairs whose id is outside
  [0, E) contribute nothing (reading; the pages' miss path zeroes a missing expert's
  contribution - "The v0.24.0 port", BASE cache bullet).
* routing: offsets = exclusive scan of per-expert pair counts; perm = the pair indices
  p = t*top_k + j stably sorted by expert id, invalid ids last ("Deterministic unpermute" bullet:
  valid sorted ids form a permutation of token*top_k+j).
"""
import numpy as np

from .formats import CODEBOOK, E2M1_MAGNITUDE, e4m3_value, unpack_codes, unpack_e2m1

_CODEBOOK = np.array(CODEBOOK, dtype=np.float64)
_E2M1 = np.array([m for m in E2M1_MAGNITUDE] + [-m for m in E2M1_MAGNITUDE], dtype=np.float64)


def dequant_rows(packed, scale_bytes):
    """Packed codes [rows, n/4] + UE8M0 scale bytes [rows, n/32] -> f64 weights [rows, n]."""
    codes = unpack_codes(packed)
    vals = _CODEBOOK[codes]
    sb = np.asarray(scale_bytes).astype(np.int64)
    if sb.size and (sb.max() > 254 or sb.min() < 0):
        raise ValueError("UE8M0 scale byte out of range")
    s = np.ldexp(1.0, sb - 127)
    return vals * np.repeat(s, 32, axis=-1)


def dequant_rows_fp4(packed, scale_bytes):
    """FP4 experts (README bullet "FP4 recovery - used surgically": hot experts kept at FP4):
    packed e2m1 codes [rows, n/2] + UE8M0 scale bytes [rows, n/32] -> f64 weights [rows, n],
    W = e2m1(code) * 2**(b - 127)."""
    vals = _E2M1[unpack_e2m1(packed)]
    sb = np.asarray(scale_bytes).astype(np.int64)
    if sb.size and (sb.max() > 254 or sb.min() < 0):
        raise ValueError("UE8M0 scale byte out of range")
    return vals * np.repeat(np.ldexp(1.0, sb - 127), 32, axis=-1)


def _e4m3_table():
    t = np.full(256, np.nan)
    for b in range(256):
        try:
            t[b] = e4m3_value(b)
        except ValueError:
            pass
    return t


_E4M3 = _e4m3_table()


def dequant_rows_nvfp4(packed, scale_bytes, scale2):
    """NVFP4 rows: packed e2m1 codes [rows, n/2] + E4M3FN scale bytes [rows, n/16] + the fp32
    scale_2 -> f64 weights [rows, n], W = e2m1(code) * e4m3(scale byte) * scale_2 (exact in f64:
    at most 2 + 4 + 24 significant bits). NaN scale bytes or a non-finite scale_2 raise."""
    vals = _E2M1[unpack_e2m1(packed)]
    s = _E4M3[np.asarray(scale_bytes, dtype=np.uint8)]
    if np.isnan(s).any():
        raise ValueError("E4M3 NaN scale byte")
    s2 = float(np.float32(scale2))
    if not np.isfinite(s2):
        raise ValueError("non-finite scale_2")
    return vals * np.repeat(s, 16, axis=-1) * s2


def _dequant(fp4):
    return dequant_rows_fp4 if fp4 else dequant_rows


def route(topk_ids, E):
    """Stable expert sort of the pairs p = t*top_k + j.

    Returns (offsets int32 [E+1], perm int32 [T*top_k]). offsets[E] counts the valid pairs;
    perm[offsets[E]:] lists the invalid pairs (id outside [0, E)) in ascending order.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    key = np.where(valid, ids, E)
    perm = np.argsort(key, kind="stable")
    return offsets.astype(np.int32), perm.astype(np.int32)


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)) in f64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def pair_outputs(x, topk_ids, gu_codes, gu_scales, dn_codes, dn_scales, tokens=None, fp4=False, workers=1,
                 nvfp4=None):
    """Per-pair down-projection outputs o[(t, j)] in f64.

    x: [T, K] f64 (the bf16 activations' exact values). Returns an array [len(tokens), top_k, K];
    rows of invalid pairs are zero. ``tokens`` restricts the computation to a subset of tokens
    (for spot checks of large workloads); default all tokens. fp4: the planes hold e2m1 codes
    (two per byte) instead of 2-bit codes. ``workers`` > 1 computes that many experts at a time
    in threads; every pair's arithmetic is the same either way (each pair belongs to one expert).
    nvfp4: (gu_scale2 [E, 2], dn_scale2 [E]) for NVFP4 planes (e2m1 codes, E4M3 block-16 scales).
    """
    dq = _dequant(fp4)
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, K = x.shape
    E, two_i, _ = gu_codes.shape
    I = two_i // 2
    top_k = ids.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), top_k, K), dtype=np.float64)
    sel = ids[tokens]  # [n_tok, top_k]

    def weights(e):
        if nvfp4 is None:
            return dq(gu_codes[e], gu_scales[e]), dq(dn_codes[e], dn_scales[e])
        gs2, ds2 = np.asarray(nvfp4[0], np.float32), np.asarray(nvfp4[1], np.float32)
        w_gu = np.concatenate([dequant_rows_nvfp4(gu_codes[e][:I], gu_scales[e][:I], gs2[e, 0]),
                               dequant_rows_nvfp4(gu_codes[e][I:], gu_scales[e][I:], gs2[e, 1])])
        return w_gu, dequant_rows_nvfp4(dn_codes[e], dn_scales[e], ds2[e])

    def expert(e):
        rows, js = np.nonzero(sel == e)
        w_gu, w_dn = weights(e)               # [2I, K], [K, I]
        xe = x[tokens[rows]]                              # [n_e, K]
        g = xe @ w_gu[:I].T                               # [n_e, I]
        u = xe @ w_gu[I:].T
        a = silu(g) * u
        out[rows, js] = a @ w_dn.T                        # [n_e, K]

    experts = [int(e) for e in np.unique(sel) if 0 <= e < E]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(expert, experts))
    else:
        for e in experts:
            expert(e)
    return out


def moe_forward(x, topk_ids, topk_w, gu_codes, gu_scales, dn_codes, dn_scales, tokens=None, fp4=False, workers=1,
                nvfp4=None):
    """y[t] = sum_j (ascending) w[t, j] * o_(t, j); f64 [len(tokens), K]."""
    o = pair_outputs(x, topk_ids, gu_codes, gu_scales, dn_codes, dn_scales, tokens, fp4, workers, nvfp4)
    w = np.asarray(topk_w, dtype=np.float64)
    tokens = np.arange(o.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    w = w[tokens]
    y = np.zeros((o.shape[0], o.shape[2]), dtype=np.float64)
    for j in range(o.shape[1]):
        y += w[:, j:j + 1] * o[:, j]
    return y


def moe_forward_act(x, topk_ids, gu_codes, gu_scales, tokens=None):
    """The gated intermediate a = silu(G x) * (U x) per pair, f64 [len(tokens), top_k, I]
    (for localising a disagreement; not part of the layer's output)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    E, two_i, _ = gu_codes.shape
    I = two_i // 2
    tokens = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), ids.shape[1], I), dtype=np.float64)
    sel = ids[tokens]
    for e in np.unique(sel):
        if e < 0 or e >= E:
            continue
        rows, js = np.nonzero(sel == e)
        w_gu = dequant_rows(gu_codes[e], gu_scales[e])
        xe = x[tokens[rows]]
        out[rows, js] = silu(xe @ w_gu[:I].T) * (xe @ w_gu[I:].T)
    return out


def resident_ids(topk_ids, E, resident):
    """Expert-cache reading of a forward (README paragraph on the base cache; "The v0.24.0 port",
    BASE cache bullet): a pair whose expert is not resident contributes nothing and counts as a
    miss. resident: bool [E]. Returns (ids with the non-resident experts' pairs set to -1, number
    of misses); ids already outside [0, E) stay invalid and are not misses."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    res = np.asarray(resident, dtype=bool)
    valid = (ids >= 0) & (ids < E)
    hit = np.zeros_like(valid)
    hit[valid] = res[ids[valid]]
    miss = valid & ~hit
    return np.where(hit, ids, -1).astype(np.int32), int(miss.sum())


def moe_forward_resident(x, topk_ids, topk_w, gu_codes, gu_scales, dn_codes, dn_scales, resident, tokens=None):
    """The forward with only the resident experts (resident: bool [E]); f64 [len(tokens), K]."""
    E = gu_codes.shape[0]
    ids, _ = resident_ids(topk_ids, E, resident)
    return moe_forward(x, ids, topk_w, gu_codes, gu_scales, dn_codes, dn_scales, tokens)
