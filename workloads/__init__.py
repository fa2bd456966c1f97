"""Seeded synthetic inputs shaped like the FP8 linear layers the pages discuss.

This module only draws random numbers and rounds them to bf16 bit patterns; it
holds none of the FP8 method's arithmetic. The tests feed the same bytes to the
HIP library and to the CPU oracle; the benchmark uses it for its inputs.

Every workload draws from numpy.random.default_rng(seed) in the order written
here, in float32, then rounds to bf16 with round-to-nearest-even.

Workloads (full sizes; every function accepts smaller shapes for tests):
  c1  rowwise FP8 linear, X [256 x 512] ~ N(0,1) with two rows scaled by 50,
      W [512 x 512] ~ N(0, 0.02^2)
  c2  Llama3-8B FFN up-projection, X [8192 x 4096] Student-t(4)/sqrt(2)
      (unit variance, heavy tails), W [14336 x 4096] ~ N(0, 0.02^2)
  c3  Flux-12B MLP linear with tensorwise delayed scaling: W [12288 x 3072]
      ~ N(0, 0.02^2) drawn first, then 16 steps of X_t [4608 x 3072] =
      c_t N(0,1) with c_0 = 1 and c_t = c_{t-1} u_t, u_t ~ U(0.5, 2)
  c4  DeepSeek-V3 MoE layer, one GPU's share: 32 experts with Zipf(1.1)
      token counts over 16384 tokens (three experts forced empty),
      tokens [16384 x 7168] ~ N(0,1) sorted by expert,
      W_e [32 x 2048 x 7168] ~ N(0, 0.006^2)
  c5  backward of c2: c2's X and W, then dY [8192 x 14336] ~ N(0, 1e-3^2)
  c6  DeepSeek-V3 MoE layer forward, one GPU's share: 2048 tokens
      [2048 x 7168] ~ N(0,1), each routed to 8 of 32 experts (Zipf(1.1)
      popularity, drawn without replacement), router weights a softmax of
      N(0,1) logits over the 8; per expert gate|up W1 [4096 x 7168] and down
      W2 [7168 x 2048], both ~ N(0, 0.006^2)
"""
import numpy as np


def bf16_bits(a):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return rounded


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def c1(m=256, n=512, k=512, seed=0, outlier_rows=2, outlier_factor=50.0):
    """Rowwise linear with outlier rows. Returns dict(x [m x k], w [n x k]) as bf16 bits."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (m, k))
    rows = rng.choice(m, min(outlier_rows, m), replace=False)
    x[rows] *= np.float32(outlier_factor)
    w = _normal(rng, (n, k), 0.02)
    return {"x": bf16_bits(x), "w": bf16_bits(w), "outlier_rows": np.sort(rows)}


def _c2_draw(rng, m, n, k):
    x = (rng.standard_t(4, size=(m, k)) / np.sqrt(2.0)).astype(np.float32)
    w = _normal(rng, (n, k), 0.02)
    return {"x": bf16_bits(x), "w": bf16_bits(w)}


def c2(m=8192, n=14336, k=4096, seed=0):
    """Llama3-8B FFN up-proj. Returns dict(x [m x k], w [n x k]) as bf16 bits."""
    return _c2_draw(np.random.default_rng(seed), m, n, k)


def c3(m=4608, n=12288, k=3072, steps=16, seed=0):
    """Delayed-scaling linear. Returns dict(w [n x k], x_steps) where x_steps() yields
    (c_t, X_t bf16 bits) for the 16 steps; call it once, after using w."""
    rng = np.random.default_rng(seed)
    w = bf16_bits(_normal(rng, (n, k), 0.02))

    def x_steps():
        c = 1.0
        for t in range(steps):
            if t >= 1:
                c = c * float(rng.uniform(0.5, 2.0))
            yield c, bf16_bits(_normal(rng, (m, k)) * np.float32(c))

    return {"w": w, "x_steps": x_steps}


def zipf_counts(rng, total, groups, exponent=1.1, forced_empty=3):
    """Tokens per expert: a random rank per expert, probability ~ (rank+1)^-exponent,
    multinomial draw; the experts ranked last `forced_empty` get no tokens and
    theirs go to the top-ranked expert (total preserved)."""
    ranks = rng.permutation(groups)
    p = (ranks + 1.0) ** (-exponent)
    p /= p.sum()
    counts = rng.multinomial(total, p).astype(np.int64)
    if forced_empty:
        empty = ranks >= groups - forced_empty
        top = int(np.argmin(ranks))
        counts[top] += counts[empty].sum()
        counts[empty] = 0
    return counts


def c4(tokens=16384, experts=32, n=2048, k=7168, seed=0, forced_empty=3):
    """MoE grouped GEMM. Returns dict(x [tokens x k] sorted by expert, w [experts x n x k],
    counts [experts], offsets int64 [experts + 1])."""
    rng = np.random.default_rng(seed)
    counts = zipf_counts(rng, tokens, experts, forced_empty=forced_empty)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    x = bf16_bits(_normal(rng, (tokens, k)))
    w = bf16_bits(_normal(rng, (experts, n, k), 0.006))
    return {"x": x, "w": w, "counts": counts, "offsets": offsets}


def c4b(tokens=16384, experts=32, n=2048, k=7168, seed=0, forced_empty=3):
    """Backward of c4's expert layer: c4's draws, then the output gradient
    dY [tokens x n] ~ 1e-3 N(0,1) (same scale as c5's)."""
    rng = np.random.default_rng(seed)
    counts = zipf_counts(rng, tokens, experts, forced_empty=forced_empty)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    x = bf16_bits(_normal(rng, (tokens, k)))
    w = bf16_bits(_normal(rng, (experts, n, k), 0.006))
    dy = bf16_bits(_normal(rng, (tokens, n), 1e-3))
    return {"x": x, "w": w, "dy": dy, "counts": counts, "offsets": offsets}


def c5(m=8192, n=14336, k=4096, seed=0):
    """Backward of c2: X [m x k], W [n x k] as in c2, then dY [m x n]."""
    rng = np.random.default_rng(seed)
    d = _c2_draw(rng, m, n, k)
    d["dy"] = bf16_bits(_normal(rng, (m, n), 1e-3))
    return d


def topk_routing(rng, tokens, experts, topk, exponent=1.1):
    """Expert choices per token, distinct, drawn without replacement with
    Zipf(exponent) popularity (a random rank per expert; Gumbel top-k over
    log-probabilities), and router weights: a softmax over topk N(0,1) logits.
    Returns (idx int32 [tokens x topk], weights float32 [tokens x topk])."""
    ranks = rng.permutation(experts)
    logp = -exponent * np.log(ranks + 1.0)
    keys = logp[None, :] + rng.gumbel(size=(tokens, experts))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :topk].astype(np.int32)
    logits = rng.standard_normal((tokens, topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


def c6(tokens=2048, experts=32, topk=8, hidden=7168, inter=2048, seed=0):
    """MoE layer forward. Returns dict(x [tokens x hidden], idx, weights
    [tokens x topk], w1 [experts x 2 inter x hidden] (gate rows, then up rows),
    w2 [experts x hidden x inter])."""
    rng = np.random.default_rng(seed)
    idx, weights = topk_routing(rng, tokens, experts, topk)
    x = bf16_bits(_normal(rng, (tokens, hidden)))
    w1 = bf16_bits(_normal(rng, (experts, 2 * inter, hidden), 0.006))
    w2 = bf16_bits(_normal(rng, (experts, hidden, inter), 0.006))
    return {"x": x, "idx": idx, "weights": weights, "w1": w1, "w2": w2}
