"""Seeded synthetic inputs for the QUADS rollout hot path.

Shared by the tests, the benchmark and the oracle checks.  It holds input
synthesis only -- random draws, bf16 rounding of the draws and routing
tables -- and none of the method's arithmetic.

The pages (QUADS, arXiv 2607.15810) measure on a 25B-A2.8B MoE model whose
weights and shapes are not public, during RL rollout on maths and code
prompts.  These seeded tensors stand in for them.  Their value structure
follows section 3.3, Fig. 4(a): a few persistent high-magnitude channels
over a light- or heavy-tailed body, so the quantization residual forms
vertical bands.

Recipe (numpy PCG64; SeedSequence(seed).spawn(4) gives independent streams
for [activations, outlier choice, weights, routing]):
  * activations are drawn in fp32 (N(0,1) or Student-t), whole outlier
    columns are multiplied by their factor, and the result is rounded to
    bf16 (nearest, ties to even) and kept as uint16 bit patterns;
  * weights are N(0, 0.02) per expert, rounded to bf16 the same way;
  * routing tables are int32 expert ids [T, top_k] with fp32 weights.
"""

import numpy as np

SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005}


def streams(seed):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest, ties to even); finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def activations(rng_a, rng_o, m, k, body="normal", nu=3.0, n_outlier=0, factor=1.0):
    """bf16 bits [m, k]: N(0,1) or Student-t(nu) body, n_outlier columns scaled."""
    if body == "normal":
        x = rng_a.standard_normal((m, k), dtype=np.float32)
    elif body == "student_t":
        x = rng_a.standard_t(nu, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(body)
    cols = np.sort(rng_o.choice(k, size=n_outlier, replace=False)) if n_outlier else \
        np.zeros(0, np.int64)
    if n_outlier:
        x[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(x), cols


def weights(rng_w, e, n, k, std=0.02):
    """bf16 bits [e, n, k], N(0, std), drawn one expert at a time."""
    out = np.empty((e, n, k), dtype=np.uint16)
    for i in range(e):
        out[i] = f32_to_bf16_bits(rng_w.standard_normal((n, k), dtype=np.float32)
                                  * np.float32(std))
    return out


def _softmax(z):
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


def routing_softmax_topk(rng, t, e, topk):
    """Router logits N(0,1); top-k by logit (ties to the lower id); weights are
    the full-softmax probabilities of the chosen experts, not renormalized."""
    logits = rng.standard_normal((t, e))
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    w = np.take_along_axis(_softmax(logits), ids, axis=1)
    return ids.astype(np.int32), w.astype(np.float32)


def routing_zipf(rng, t, e, topk, s=1.2):
    """topk distinct experts per token drawn without replacement with
    p(e) proportional to (e+1)^-s; weights = softmax of topk N(0,1) draws."""
    p = (np.arange(1, e + 1, dtype=np.float64)) ** -s
    p /= p.sum()
    ids = np.stack([rng.choice(e, size=topk, replace=False, p=p) for _ in range(t)])
    w = _softmax(rng.standard_normal((t, topk)))
    return ids.astype(np.int32), w.astype(np.float32)


def routing_uniform(rng, t, e, topk):
    """topk distinct experts per token, uniformly (argsort of uniform keys);
    weights = softmax of topk N(0,1) draws."""
    ids = np.argsort(rng.random((t, e)), axis=1)[:, :topk]
    w = _softmax(rng.standard_normal((t, topk)))
    return ids.astype(np.int32), w.astype(np.float32)


# The five workloads (sizes as stated for the measured configurations).
CONFIGS = {
    1: dict(kind="dense", m=32, k_dim=256, n=128, body="normal", n_outlier=4,
            factor=16.0, rac_k=16),
    2: dict(kind="dense", m=4096, k_dim=4096, n=4096, body="student_t", nu=3.0,
            n_outlier=41, factor=20.0, rac_k=128),
    3: dict(kind="moe", t=4096, e=128, h=2048, i=768, topk=8, body="normal",
            n_outlier=20, factor=20.0, routing="softmax", rac_k=64),
    4: dict(kind="moe", t=64, e=128, h=2048, i=768, topk=8, body="normal",
            n_outlier=20, factor=20.0, routing="zipf", rac_k=64),
    5: dict(kind="moe", t=16384, e=64, h=4096, i=1536, topk=8, body="student_t",
            nu=2.5, n_outlier=82, factor=32.0, routing="uniform", rac_k=64),
}


def make_dense(seed, m, k_dim, n, body="normal", nu=3.0, n_outlier=0, factor=1.0,
               rac_k=0, **_):
    ra, ro, rw, _rr = streams(seed)
    x, cols = activations(ra, ro, m, k_dim, body, nu, n_outlier, factor)
    w = weights(rw, 1, n, k_dim)
    return dict(x=x, outlier_cols=cols, w=w, rac_k=rac_k)


def make_moe(seed, t, e, h, i, topk, body="normal", nu=3.0, n_outlier=0, factor=1.0,
             routing="softmax", rac_k=0, with_weights=True, **_):
    ra, ro, rw, rr = streams(seed)
    x, cols = activations(ra, ro, t, h, body, nu, n_outlier, factor)
    if routing == "softmax":
        ids, tw = routing_softmax_topk(rr, t, e, topk)
    elif routing == "zipf":
        ids, tw = routing_zipf(rr, t, e, topk)
    elif routing == "uniform":
        ids, tw = routing_uniform(rr, t, e, topk)
    else:
        raise ValueError(routing)
    out = dict(x=x, outlier_cols=cols, topk_ids=ids, topk_w=tw, rac_k=rac_k)
    if with_weights:
        out["w13"] = weights(rw, e, 2 * i, h)
        out["w2"] = weights(rw, e, h, i)
    return out


def make(cfg_id, **overrides):
    """Inputs of workload cfg_id (1..5); keyword overrides change sizes."""
    c = dict(CONFIGS[cfg_id])
    c.update(overrides)
    seed = c.pop("seed", SEEDS[cfg_id])
    if c["kind"] == "dense":
        return make_dense(seed, **c)
    return make_moe(seed, **c)
