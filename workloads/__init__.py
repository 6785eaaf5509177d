"""Seeded synthetic inputs for the 2-bit routed-expert MoE layer and the NVFP4 re-quantizer.

This module only draws inputs; it holds none of the method's arithmetic, and both the oracle
side and the GPU side (tests, bench) take their inputs from it. Every generator uses NumPy's
PCG64 (``np.random.default_rng``) with the seed and draw order written in its docstring.

Shapes and distributions follow the workloads named for the method: a tiny layer (T=4, K=256,
I=512, E=8, top-2), decode batches T in {1, 8, 32} at K=4096/I=2048/E=256/top-8 with uniform
routing, a K=6144 decode batch T=64 with Zipf(1.1) routing, an 8192-token K=6144 prefill with
Zipf(1.1) routing, and 256 NVFP4 expert tensors [2048, 6144] for the re-quantizer. Codes are
uniform over the four 2-bit values; UE8M0 scale exponents are uniform in [-10, -6];
activations are bf16 N(0, 1).
"""
import numpy as np

TINY = dict(T=4, K=256, I=512, E=8, top_k=2, seed=0)
DECODE = dict(K=4096, I=2048, E=256, top_k=8, seed=1, Ts=(1, 8, 32))
DECODE_ZIPF = dict(T=64, K=6144, I=2048, E=256, top_k=8, seed=2)
PREFILL = dict(T=8192, K=6144, I=2048, E=256, top_k=8, seed=3)
REQUANT = dict(n=256, R=2048, C=6144, seed=4)


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (round to nearest even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def draw_planes(rng, E, K, I):
    """Canonical 2-bit planes of one layer, drawn in this order:
    gate_up codes [E, 2I, K/4] (uniform bytes = four independent uniform 2-bit codes),
    gate_up scale bytes [E, 2I, K/32] = 127 + U{-10..-6},
    down codes [E, K, I/4], down scale bytes [E, K, I/32] = 127 + U{-10..-6}."""
    gu_codes = rng.integers(0, 256, size=(E, 2 * I, K // 4), dtype=np.uint8)
    gu_scales = (127 + rng.integers(-10, -5, size=(E, 2 * I, K // 32))).astype(np.uint8)
    dn_codes = rng.integers(0, 256, size=(E, K, I // 4), dtype=np.uint8)
    dn_scales = (127 + rng.integers(-10, -5, size=(E, K, I // 32))).astype(np.uint8)
    return dict(gu_codes=gu_codes, gu_scales=gu_scales, dn_codes=dn_codes, dn_scales=dn_scales)


def draw_planes_fp4(rng, E, K, I):
    """Canonical FP4 (MXFP4) planes of one layer, drawn in this order: gate_up codes [E, 2I, K/2]
    (uniform bytes = two independent uniform e2m1 nibbles), gate_up scale bytes [E, 2I, K/32] =
    127 + U{-10..-6}, down codes [E, K, I/2], down scale bytes [E, K, I/32] = 127 + U{-10..-6}."""
    gu_codes = rng.integers(0, 256, size=(E, 2 * I, K // 2), dtype=np.uint8)
    gu_scales = (127 + rng.integers(-10, -5, size=(E, 2 * I, K // 32))).astype(np.uint8)
    dn_codes = rng.integers(0, 256, size=(E, K, I // 2), dtype=np.uint8)
    dn_scales = (127 + rng.integers(-10, -5, size=(E, K, I // 32))).astype(np.uint8)
    return dict(gu_codes=gu_codes, gu_scales=gu_scales, dn_codes=dn_codes, dn_scales=dn_scales)


def draw_planes_nvfp4(rng, E, K, I):
    """Canonical NVFP4 planes of one layer, drawn in this order: gate_up codes [E, 2I, K/2]
    (uniform bytes = two independent uniform e2m1 nibbles), gate_up E4M3FN scale bytes
    [E, 2I, K/16] uniform in 0x28..0x7E (the positive normal values 2^-2 .. 448, the range a
    block scale amax/6/scale_2 takes), gate_up scale_2 [E, 2] = fp32(U[2e-5, 1e-4]) (gate, up),
    down codes [E, K, I/2], down scale bytes [E, K, I/16] as above, down scale_2 [E] as above."""
    gu_codes = rng.integers(0, 256, size=(E, 2 * I, K // 2), dtype=np.uint8)
    gu_scales = rng.integers(0x28, 0x7F, size=(E, 2 * I, K // 16), dtype=np.uint8)
    gu_scale2 = rng.uniform(2e-5, 1e-4, size=(E, 2)).astype(np.float32)
    dn_codes = rng.integers(0, 256, size=(E, K, I // 2), dtype=np.uint8)
    dn_scales = rng.integers(0x28, 0x7F, size=(E, K, I // 16), dtype=np.uint8)
    dn_scale2 = rng.uniform(2e-5, 1e-4, size=(E,)).astype(np.float32)
    return dict(gu_codes=gu_codes, gu_scales=gu_scales, gu_scale2=gu_scale2, dn_codes=dn_codes,
                dn_scales=dn_scales, dn_scale2=dn_scale2)


def _softmax_f32(logits):
    z = logits.astype(np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=-1, keepdims=True)).astype(np.float32)


def draw_x(rng, T, K):
    """bf16 activations N(0,1): float32 normal draws rounded to bf16; returns uint16 bits."""
    return f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))


def tiny(seed=TINY["seed"]):
    """Tiny layer. Draw order: x [T,K]; router logits N(0,1) [T,E] -> softmax -> top-2
    (descending probability) -> renormalised (fp32); then the planes."""
    c = TINY
    rng = np.random.default_rng(seed)
    x = draw_x(rng, c["T"], c["K"])
    logits = rng.standard_normal((c["T"], c["E"]), dtype=np.float32)
    p = _softmax_f32(logits)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :c["top_k"]].astype(np.int32)
    w = np.take_along_axis(p, ids, axis=1).astype(np.float64)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    planes = draw_planes(rng, c["E"], c["K"], c["I"])
    return dict(x=x, topk_ids=ids, topk_w=w, **planes, **{k: c[k] for k in ("T", "K", "I", "E", "top_k")})


def uniform_routing(rng, T, E, top_k):
    """ids = the first top_k entries of an independent permutation of the E experts per token;
    weights = softmax of top_k N(0,1) logits (fp32)."""
    ids = np.stack([rng.permutation(E)[:top_k] for _ in range(T)]).astype(np.int32).reshape(T, top_k)
    w = _softmax_f32(rng.standard_normal((T, top_k), dtype=np.float32))
    return ids, w


def zipf_routing(rng, T, E, top_k, s=1.1, rank_perm=None):
    """Zipf(s) expert popularity: p_r ~ r^-s for rank r = 1..E, ranks mapped to experts by the
    permutation ``rank_perm``; each token samples top_k distinct experts without replacement
    (Gumbel-top-k of log p, in descending perturbed score); weights as in uniform_routing."""
    r = np.arange(1, E + 1, dtype=np.float64)
    logp_rank = -s * np.log(r)
    logp = np.empty(E)
    logp[rank_perm] = logp_rank
    g = logp[None, :] + rng.gumbel(size=(T, E))
    ids = np.argsort(-g, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    w = _softmax_f32(rng.standard_normal((T, top_k), dtype=np.float32))
    return ids, w


def grouped_routing(rng, T, E, top_k, sizes):
    """Routing with prescribed group sizes: expert i (i < len(sizes)) gets sizes[i] pairs, the
    remaining pairs go to experts len(sizes) .. E-1 in turn; the pair positions are a random
    permutation of the T*top_k pairs (a token may route to one expert more than once). Weights as
    in uniform_routing. sum(sizes) <= T*top_k."""
    P = T * top_k
    flat = []
    for i, n in enumerate(sizes):
        flat += [i] * int(n)
    rest = P - len(flat)
    if rest < 0:
        raise ValueError("more pairs in the groups than the batch has")
    others = max(1, E - len(sizes))
    flat += [len(sizes) + (k % others) for k in range(rest)]
    ids = np.asarray(flat, dtype=np.int32)[rng.permutation(P)].reshape(T, top_k)
    w = _softmax_f32(rng.standard_normal((T, top_k), dtype=np.float32))
    return ids, w


def decode_layer(seed=DECODE["seed"], K=DECODE["K"], I=DECODE["I"], E=DECODE["E"]):
    """Planes of the K=4096 decode layer (draw_planes with the given seed)."""
    return draw_planes(np.random.default_rng(seed), E, K, I)


def decode_instances(T, R, seed=DECODE["seed"], K=DECODE["K"], E=DECODE["E"], top_k=DECODE["top_k"]):
    """R routing instances of T tokens with uniform routing, drawn after the planes' stream with
    seed (seed, T): per instance x [T, K] then (ids, w)."""
    rng = np.random.default_rng([seed, T])
    out = []
    for _ in range(R):
        x = draw_x(rng, T, K)
        ids, w = uniform_routing(rng, T, E, top_k)
        out.append(dict(x=x, topk_ids=ids, topk_w=w))
    return out


def zipf_layer(seed, K, I, E):
    """Planes of a K=6144 layer for the Zipf workloads."""
    return draw_planes(np.random.default_rng(seed), E, K, I)


def zipf_instances(T, R, seed, K, E, top_k, s=1.1):
    """R Zipf-routed instances of T tokens. Stream seed (seed, T): first the rank->expert
    permutation (shared by all instances), then per instance x [T, K] and (ids, w)."""
    rng = np.random.default_rng([seed, T])
    rank_perm = rng.permutation(E)
    out = []
    for _ in range(R):
        x = draw_x(rng, T, K)
        ids, w = zipf_routing(rng, T, E, top_k, s, rank_perm)
        out.append(dict(x=x, topk_ids=ids, topk_w=w))
    return out


def nvfp4_tensor(i, seed=REQUANT["seed"], R=REQUANT["R"], C=REQUANT["C"]):
    """NVFP4 expert tensor i with stream seed (seed, i): e2m1 bytes [R, C/2] uniform over 0..255
    (two uniform nibbles, low nibble = even element), e4m3 bytes [R, C/16] uniform in 0x18..0x58
    (the positive normal E4M3 values in [2^-4, 2^4]), scale_2 = fp32(U[1e-3, 1e-2])."""
    rng = np.random.default_rng([seed, i])
    e2m1 = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    e4m3 = rng.integers(0x18, 0x59, size=(R, C // 16), dtype=np.uint8)
    scale2 = np.float32(rng.uniform(1e-3, 1e-2))
    return e2m1, e4m3, scale2


def fp8_block_tensor(i, R=2048, C=6144, seed=REQUANT["seed"]):
    """FP8 block-quant tensor i: E4M3FN bytes uniform over the 254 finite encodings [R, C] (so
    zeros, subnormals, both signs and the whole exponent range occur), then fp32 scales per
    128 x 128 block, 2^U(-12, -2) [R/128, C/128]; seeded by (seed, 1000 + i)."""
    rng = np.random.default_rng([seed, 1000 + i])
    b = rng.integers(0, 254, size=(R, C), dtype=np.uint16).astype(np.uint8)
    b = np.where(b >= 0x7F, b + 1, b).astype(np.uint8)          # skip 0x7F; 0xFF is never drawn
    scales = np.exp2(rng.uniform(-12.0, -2.0, size=(R // 128, C // 128))).astype(np.float32)
    return b, scales


def mxfp4_tensor(i, R=2048, C=6144, seed=REQUANT["seed"]):
    """MXFP4 tensor i: e2m1 nibbles uniform over all 16 values, packed low nibble first [R, C/2],
    UE8M0 scale bytes 127 + U{-12..2} [R, C/32]; seeded by (seed, 2000 + i)."""
    rng = np.random.default_rng([seed, 2000 + i])
    e2m1 = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    ue8m0 = (127 + rng.integers(-12, 3, size=(R, C // 32))).astype(np.uint8)
    return e2m1, ue8m0


SWEEP = dict(n=180, R=2048, C=6144, seed=5)


def codebook_family():
    """Candidate 2-bit codebooks for the sign-bias sweep: every set of 4 distinct values from the
    15 e2m1 values {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} whose largest magnitude is 3, 4 or 6
    (one representative per power-of-two scaling, which the block exponent absorbs), ascending,
    in lexicographic order: float32 [1239, 4]. Holds {-4,-1,1,4} and the other symmetric sets."""
    import itertools
    mags = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = sorted([-m for m in mags] + [0.0] + mags)
    out = [c for c in itertools.combinations(vals, 4) if max(abs(c[0]), abs(c[3])) in (3.0, 4.0, 6.0)]
    return np.array(out, dtype=np.float32)


def sweep_tensor(i, R=SWEEP["R"], C=SWEEP["C"], seed=SWEEP["seed"]):
    """Synthetic expert weight tensor i for the sign-bias sweep, float32 [R, C], stream seed
    (seed, i): standard normal values, 5% of them (uniform draw < 0.05) widened x3 for heavier
    tails, then each row scaled by 2^U(-9, -5) (per-output-channel spread). Symmetric in sign."""
    rng = np.random.default_rng([seed, i])
    z = rng.standard_normal((R, C), dtype=np.float32)
    wide = rng.random((R, C), dtype=np.float32) < 0.05
    np.multiply(z, np.float32(3.0), out=z, where=wide)
    z *= np.exp2(rng.uniform(-9.0, -5.0, size=(R, 1))).astype(np.float32)
    return z
