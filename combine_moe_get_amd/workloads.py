"""Seeded synthetic inputs for MoE dispatch/combine.

This module only draws inputs.  It holds none of the method's arithmetic
(no layout, quantization or combine), so the CPU oracle and the HIP path can
both be fed from it.  All draws use numpy's PCG64 via
``np.random.default_rng([seed, config_id, tensor_id])``, which is platform
independent.  bf16 tensors are returned as uint16 bit patterns, rounded from
float32 to nearest-even.

The five named workloads stand in for the token batches the pages run:
DeepEP's decode test (128 tokens per rank, hidden 7168, top-8, the issue
"#84 Questions on Profiling dispatch_t ..."), DeepEP's prefill benchmark
(4096 tokens, hidden 7168, top-8, quoted in "Wide-EP / DBO / DeepEP hardware
cliff", section "What the published DeepEP tables are really telling you")
and the CANN "low_latency_dispatch" examples (zero/copy/constant experts).
No dataset or trained weights are involved.
"""
import numpy as np

# tensor ids of the rng streams
_X, _TOPK, _W, _MASK, _SMOOTH, _Y, _A1, _A2, _V, _FUZZ = range(10)

CONFIGS = {
    1: dict(name="tiny", T=128, H=1024, K=4, E=16, P=4, Z=0, C=0, Kc=0, num_max=0,
            quant_mode=0, smooth=False, routing="uniform", mask_p=None,
            desc="T=128 H=1024 E=16 top-4 uniform distinct, softmax weights, P=4, bf16 passthrough"),
    2: dict(name="ll_decode", T=4096, H=7168, K=8, E=256, P=32, Z=0, C=0, Kc=0, num_max=128,
            quant_mode=2, smooth=True, routing="uniform", mask_p=None,
            desc="128 tokens/rank x P=32 (T=4096), H=7168, E=256 top-8 uniform distinct, "
                 "dynamic int8 with per-channel smooth scales U(0.5,1.5)"),
    3: dict(name="ht_prefill", T=4096, H=7168, K=8, E=256, P=64, Z=0, C=0, Kc=0, num_max=0,
            quant_mode=0, smooth=False, routing="zipf", mask_p=None,
            desc="T=4096 H=7168 E=256 top-8 Zipf(s=1) popularity, P=64, bf16 passthrough"),
    4: dict(name="special", T=8192, H=4096, K=8, E=128, P=16, Z=2, C=2, Kc=2, num_max=0,
            quant_mode=0, smooth=False, routing="uniform_all", mask_p=None,
            desc="T=8192 H=4096 E=128 routed + 2 zero + 2 copy + 2 constant experts, top-8 "
                 "uniform distinct over all 134 ids, expert outputs N(0,1), P=16"),
    5: dict(name="grouped_masked", T=16384, H=7168, K=8, E=256, P=64, Z=0, C=0, Kc=0, num_max=256,
            quant_mode=2, smooth=False, routing="grouped", mask_p=0.9,
            desc="T=16384 H=7168 E=256 in 8 groups, top-4 groups then top-8 experts, "
                 "active mask Bernoulli(0.9), dynamic int8 without smooth scales, P=64"),
}


def rng_for(seed, config_id, tensor_id):
    return np.random.default_rng([int(seed), int(config_id), int(tensor_id)])


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng, shape, chunk_rows=4096):
    """N(0,1) drawn as float32, rounded to bf16; drawn in row chunks to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.uint16)
    if len(shape) == 0 or out.size == 0:
        return out
    rows = shape[0]
    flat = out.reshape(rows, -1)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        flat[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32))
    return out


def _softmax(z):
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _uniform_distinct(rng, T, n_ids, K):
    return np.argsort(rng.random((T, n_ids)), axis=1, kind="stable")[:, :K].astype(np.int32)


def _zipf_distinct(rng, T, E, K, s=1.0):
    # expert popularity p_e proportional to 1/rank^s over a seeded permutation;
    # K distinct experts per token by Gumbel-top-K (weighted sampling without replacement)
    perm = rng.permutation(E)
    p = np.empty(E)
    p[perm] = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    g = -np.log(-np.log(rng.random((T, E))))
    keys = np.log(p)[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def _grouped(rng, T, E, K, n_groups=8, top_groups=4):
    logits = rng.standard_normal((T, E))
    gs = E // n_groups
    gscore = logits.reshape(T, n_groups, gs).max(axis=2)
    keep = np.argsort(-gscore, axis=1, kind="stable")[:, :top_groups]
    allowed = np.zeros((T, n_groups), bool)
    np.put_along_axis(allowed, keep, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), logits, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :K].astype(np.int32)
    chosen = np.take_along_axis(logits, idx, axis=1)
    return idx, _softmax(chosen).astype(np.float32)


def make_inputs(config_id, seed=0, with_expert_out=False, T=None, P=None):
    """Inputs of a named workload.  ``T`` (a multiple of P) may shrink the token
    count for quick runs and ``P`` (dividing E) change the simulated rank count;
    every other size stays as named."""
    c = dict(CONFIGS[config_id])
    if P is not None:
        assert c["E"] % P == 0
        c["P"] = P
        c["num_max"] = 0
    if T is not None:
        assert T % c["P"] == 0
        c["T"] = T
    Tn, H, K, E, P = c["T"], c["H"], c["K"], c["E"], c["P"]
    Z, C, Kc = c["Z"], c["C"], c["Kc"]
    x = normal_bf16(rng_for(seed, config_id, _X), (Tn, H))
    rt = rng_for(seed, config_id, _TOPK)
    weights = None
    if c["routing"] == "uniform":
        topk = _uniform_distinct(rt, Tn, E, K)
    elif c["routing"] == "uniform_all":
        topk = _uniform_distinct(rt, Tn, E + Z + C + Kc, K)
    elif c["routing"] == "zipf":
        topk = _zipf_distinct(rt, Tn, E, K)
    elif c["routing"] == "grouped":
        topk, weights = _grouped(rt, Tn, E, K)
    else:
        raise ValueError(c["routing"])
    if weights is None:
        weights = _softmax(rng_for(seed, config_id, _W).standard_normal((Tn, K))).astype(np.float32)
    mask = None
    if c["mask_p"] is not None:
        mask = (rng_for(seed, config_id, _MASK).random(Tn) < c["mask_p"]).astype(np.uint8)
    smooth = None
    if c["smooth"]:
        smooth = rng_for(seed, config_id, _SMOOTH).uniform(0.5, 1.5, H).astype(np.float32)
    out = dict(cfg=c, config_id=config_id, seed=seed, x=x, topk_idx=np.ascontiguousarray(topk),
               topk_weights=np.ascontiguousarray(weights, np.float32), mask=mask, smooth=smooth,
               ori_x=None, alpha1=None, alpha2=None, const_v=None)
    if Kc > 0:
        out["alpha1"] = f32_to_bf16_bits(rng_for(seed, config_id, _A1).uniform(0, 1, (Kc, H)).astype(np.float32))
        out["alpha2"] = f32_to_bf16_bits(rng_for(seed, config_id, _A2).uniform(0, 1, (Kc, H)).astype(np.float32))
        out["const_v"] = normal_bf16(rng_for(seed, config_id, _V), (Kc, H))
    if C + Kc > 0:
        out["ori_x"] = x
    return out


def expert_out_normal(rows, H, seed=0, config_id=0):
    """Stand-in expert outputs: N(0,1) rows [rows, H] in bf16."""
    return normal_bf16(rng_for(seed, config_id, _Y), (max(int(rows), 0), H))


def fuzz_world(seed, T=None, H=None, K=None, E=None, P=None, Z=None, C=None, Kc=None,
               p_drop=0.1, p_dup=0.05, p_bad=0.0, p_mask=0.2):
    """A small random world with dropped (-1) slots, duplicate ids in a token,
    special experts, inactive tokens and (optionally) out-of-range ids."""
    r = rng_for(seed, 99, _FUZZ)
    P = P or int(r.choice([1, 2, 3, 4, 8]))
    L = int(r.integers(1, 5))
    E = E or P * L
    Z = int(r.integers(0, 3)) if Z is None else Z
    C = int(r.integers(0, 3)) if C is None else C
    Kc = int(r.integers(0, 3)) if Kc is None else Kc
    etot = E + Z + C + Kc
    K = K or int(r.integers(1, min(16, etot) + 1))
    BS = int(r.integers(1, 40))
    T = P * BS if T is None else T
    H = H or 8 * int(r.integers(1, 80))
    topk = r.integers(0, etot, size=(T, K)).astype(np.int32)
    topk[r.random((T, K)) < p_drop] = -1
    if K > 1:
        dup = r.random(T) < p_dup
        topk[dup, 1] = topk[dup, 0]
    if p_bad > 0:
        bad = r.random((T, K)) < p_bad
        topk[bad] = r.choice([-7, -2, etot, etot + 5], size=int(bad.sum()))
    mask = (r.random(T) >= p_mask).astype(np.uint8)
    x = f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    smooth = r.uniform(0.5, 1.5, H).astype(np.float32)
    a1 = f32_to_bf16_bits(r.uniform(-1, 1, (Kc, H)).astype(np.float32))
    a2 = f32_to_bf16_bits(r.uniform(-1, 1, (Kc, H)).astype(np.float32))
    v = f32_to_bf16_bits(r.standard_normal((Kc, H)).astype(np.float32))
    return dict(T=T, H=H, K=K, E=E, P=P, Z=Z, C=C, Kc=Kc, x=x, topk_idx=topk, topk_weights=w,
                mask=mask, smooth=smooth, alpha1=a1, alpha2=a2, const_v=v, ori_x=x)
