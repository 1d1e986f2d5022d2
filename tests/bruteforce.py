"""Pure-Python recomputation without any cache, used to pin the oracle.

"Part 47 | Inference basics: KV Cache, batching, sampling" (chengxuchu.com),
section 2.1, describes the naive path: every generation step recomputes
attention over the whole prefix from scratch.  These loops do exactly that on
tiny inputs, with math.fsum and math.exp, from contiguous per-position K/V
lists -- no block table, no numpy, nothing shared with the oracle.
"""
import math


def attend_one(q, keys, values, sigma):
    """softmax(sigma * q . k_t) weighted sum of v_t for one query row over lists of rows."""
    if not keys:
        return [0.0] * len(values[0]) if values else []
    xs = [sigma * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    mu = max(xs)
    ws = [math.exp(x - mu) for x in xs]
    z = math.fsum(ws)
    dim = len(values[0])
    return [math.fsum(w * v[d] for w, v in zip(ws, values)) / z for d in range(dim)]


def naive_generation(qs, ks, vs, sigma):
    """Step t recomputes attention of query t over positions 0..t (causal, inclusive).

    qs, ks, vs: lists over positions of per-position vectors.  Returns one
    output vector per step.
    """
    outs = []
    for t in range(len(qs)):
        outs.append(attend_one(qs[t], ks[:t + 1], vs[:t + 1], sigma))
    return outs
