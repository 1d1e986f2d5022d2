"""Plain, slow CPU oracle for attention over a paged KV cache (float64, numpy).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What it computes, and where the pages define it:

* Scaled dot-product attention, softmax(Q K^T / sqrt(d)) V: "Part 47 |
  Inference basics: KV Cache, batching, sampling" (chengxuchu.com), section
  2.1.  The query of position t dots the keys of positions 1..t (causal,
  inclusive).
* Decode: one new token per request; its K/V are appended to the cache first,
  then its query reads the whole cache (same page, section 2.2).
* Paging only changes where K/V live: a block table maps a sequence's logical
  blocks of 16 tokens to physical blocks anywhere in the pool (the
  ainews.alishangtian.com article, section "PagedAttention"; same page as
  above, section 5.2; caffein.top essay, section on paging).  So the oracle
  gathers each sequence's blocks into a contiguous [L, kv_heads, head_dim]
  array -- the per-layer slice of the contiguous cache shape of section 2.3 --
  and applies the plain definition to it.
* Chunked prefill: a prompt is cut into chunks; each chunk row attends
  causally to everything cached before it and to the chunk rows up to itself
  (caffein.top essay, section "Chunked Prefill"; serving deep-dive page,
  paragraph on chunked prefill).
* Grouped-query attention: fewer kv heads than query heads (section 2.3 of the
  chengxuchu.com page); consecutive query heads share a kv head.

Readings taken where the pages are silent (each is listed in the design notes):
cache layout [num_blocks, kv_heads, 16, head_dim]; slot = block * 16 + offset;
a negative slot skips its row; scale is applied as the float32 value the GPU
receives; an empty context gives a zero output; chunk c has
context_lens[c] - chunk_start[c] valid rows and later rows stay NaN here.

Arithmetic: every value is widened exactly to float64 (bf16 bits << 16 as a
float32, then to float64); products, the max shift, exp and the normalisation
are all float64.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


# ---------------------------------------------------------------- helpers

def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of raw cache/query data (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        wide = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """kv head read by query head h: consecutive query heads share one kv head."""
    return h // (num_q_heads // num_kv_heads)


def slot_location(slot: int) -> tuple:
    """(physical block, offset in block) of a flat cache slot."""
    return slot // BLOCK_SIZE, slot % BLOCK_SIZE


def token_location(table_row: np.ndarray, t: int) -> tuple:
    """(physical block, offset) of logical token t of a sequence."""
    return int(table_row[t // BLOCK_SIZE]), t % BLOCK_SIZE


def causal_key_count(chunk_start: int, row: int) -> int:
    """Number of keys visible to chunk row `row`: positions 0 .. chunk_start+row inclusive."""
    return chunk_start + row + 1


def exact_scale(scale) -> float:
    """The scale as the float32 the GPU receives, widened to float64."""
    return float(np.float32(scale))


# ---------------------------------------------------------------- cache write

def kv_write(k_cache, v_cache, new_k, new_v, slot_mapping):
    """Return copies of the caches with row i of new_k/new_v stored at slot_mapping[i].

    A raw copy of the bit patterns: no arithmetic touches the values.  Rows with a
    negative slot are skipped.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        b, o = slot_location(int(s))
        kc[b, :, o, :] = new_k[i]
        vc[b, :, o, :] = new_v[i]
    return kc, vc


# ---------------------------------------------------------------- gather

def copy_blocks(k_cache, v_cache, src_blocks, dst_blocks):
    """Copy-on-write of whole blocks.

    ainews.alishangtian.com article on inference engines, section
    "PagedAttention": a physical block shared by several sequences is copied
    to a block of its own before one of them modifies it.  Returns new caches
    in which block dst[i] holds the bits of block src[i] (every kv head, all
    slots); pairs naming an id outside [0, num_blocks) are skipped.  Raw bits
    are copied, so NaN payloads survive.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    nb = k_cache.shape[0]
    for s, d in zip(np.asarray(src_blocks).tolist(), np.asarray(dst_blocks).tolist()):
        if 0 <= s < nb and 0 <= d < nb:
            kc[d] = k_cache[s]
            vc[d] = v_cache[s]
    return kc, vc


def gather(cache, table_row, length: int) -> np.ndarray:
    """Contiguous [length, kv_heads, head_dim] copy (raw) of a sequence's cached rows."""
    out = np.empty((length,) + cache.shape[1:2] + cache.shape[3:], dtype=cache.dtype)
    for t in range(length):
        b, o = token_location(table_row, t)
        out[t] = cache[b, :, o, :]
    return out


def gather_fast(cache, table_row, length: int) -> np.ndarray:
    """Same result as gather(), built block by block (used for long contexts)."""
    nb = -(-length // BLOCK_SIZE)
    if nb == 0:
        return np.empty((0,) + cache.shape[1:2] + cache.shape[3:], dtype=cache.dtype)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = cache[ids]  # [nb, Hkv, 16, D]
    seq = blocks.transpose(0, 2, 1, 3).reshape(nb * BLOCK_SIZE, cache.shape[1], cache.shape[3])
    return seq[:length]


# ---------------------------------------------------------------- attention

def attend(qg: np.ndarray, keys: np.ndarray, values: np.ndarray, sigma: float,
           key_counts=None) -> np.ndarray:
    """softmax(sigma * q k^T) v for a group of query rows over one kv head, float64.

    qg [R, D]; keys, values [L, D]; key_counts[r] (optional) limits row r to the
    first key_counts[r] keys.  A row that sees no key returns zeros.
    """
    R, L = qg.shape[0], keys.shape[0]
    out = np.zeros((R, values.shape[1]), dtype=np.float64)
    if L == 0:
        return out
    x = sigma * (qg @ keys.T)  # [R, L]
    if key_counts is not None:
        cols = np.arange(L)[None, :]
        visible = cols < np.asarray(key_counts)[:, None]
        x = np.where(visible, x, -np.inf)
    mu = x.max(axis=1, keepdims=True)
    seen = np.isfinite(mu[:, 0])
    w = np.exp(x[seen] - mu[seen])
    out[seen] = (w @ values) / w.sum(axis=1, keepdims=True)
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype, gather_fn=None):
    """Decode attention: out[s, h] = softmax(scale q[s,h] K_s^T) V_s over the first context_lens[s] tokens.

    q [B, Hq, D]; caches [NB, Hkv, 16, D]; returns float64 [B, Hq, D].
    """
    gather_fn = gather_fn or gather_fast
    q64 = to_f64(q, dtype)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    sigma = exact_scale(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        K = to_f64(gather_fn(k_cache, block_tables[s], L), dtype)
        V = to_f64(gather_fn(v_cache, block_tables[s], L), dtype)
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            out[s, heads] = attend(q64[s, heads], K[:, g], V[:, g], sigma)
    return out


def decode_shared_prefix(q, k_cache, v_cache, prefix_blocks, block_tables, context_lens, scale, dtype):
    """Decode for sequences that all start with one prompt prefix stored once.

    ainews.alishangtian.com article on inference engines, section
    "PagedAttention": requests with a common prefix reference the same physical
    blocks.  Sequence s's context is the prefix -- the 16-token blocks
    prefix_blocks, in order -- followed by its own context_lens[s] tokens listed
    in block_tables[s]; the result is plain attention over that whole context
    (decode above), whatever order the work is done in.
    """
    prefix_blocks = np.asarray(prefix_blocks, dtype=np.int64).reshape(-1)
    tables = np.asarray(block_tables)
    n_pre = prefix_blocks.shape[0]
    full = np.empty((tables.shape[0], n_pre + tables.shape[1]), dtype=np.int64)
    full[:, :n_pre] = prefix_blocks
    full[:, n_pre:] = tables
    lens = np.asarray(context_lens, dtype=np.int64) + n_pre * BLOCK_SIZE
    return decode(q, k_cache, v_cache, full, lens, scale, dtype)


def prefill_chunk(q_chunk, chunk_start, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                  gather_fn=None):
    """Causal attention of each prefill chunk's rows over its cached context.

    q_chunk [Nc, Cmax, Hq, D]; chunk c has n_c = context_lens[c] - chunk_start[c]
    rows; row i sits at position chunk_start[c] + i and sees keys 0..that position.
    Returns float64 [Nc, Cmax, Hq, D]; rows i >= n_c are NaN (not computed).
    """
    gather_fn = gather_fn or gather_fast
    q64 = to_f64(q_chunk, dtype)
    Nc, Cmax, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    sigma = exact_scale(scale)
    out = np.full((Nc, Cmax, Hq, D), np.nan, dtype=np.float64)
    for c in range(Nc):
        P0, L = int(chunk_start[c]), int(context_lens[c])
        n = L - P0
        if n <= 0:
            continue
        K = to_f64(gather_fn(k_cache, block_tables[c], L), dtype)
        V = to_f64(gather_fn(v_cache, block_tables[c], L), dtype)
        counts = [causal_key_count(P0, i) for i in range(n)]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[c, :n, h] = attend(q64[c, :n, h], K[:, g], V[:, g], sigma, key_counts=counts)
    return out


# ---------------------------------------------------------------- split context + LSE merge

def partition_partials(qg: np.ndarray, keys: np.ndarray, values: np.ndarray, sigma: float,
                       partition_tokens: int):
    """Per-partition (m, l, o) of a group of query rows: running max, sum of
    exp(x - m) and the unnormalised sum of exp(x - m) * v, each partition covering
    partition_tokens consecutive keys."""
    L = keys.shape[0]
    parts = []
    for a in range(0, L, partition_tokens):
        b = min(L, a + partition_tokens)
        x = sigma * (qg @ keys[a:b].T)
        m = x.max(axis=1)
        w = np.exp(x - m[:, None])
        parts.append((m, w.sum(axis=1), w @ values[a:b]))
    return parts


def lse_merge(parts):
    """Combine partition partials: M = max m_p, out = sum e^(m_p-M) o_p / sum e^(m_p-M) l_p."""
    ms = np.stack([p[0] for p in parts])  # [P, R]
    M = ms.max(axis=0)
    scale = np.exp(ms - M[None, :])
    lam = sum(scale[i] * parts[i][1] for i in range(len(parts)))
    num = sum(scale[i][:, None] * parts[i][2] for i in range(len(parts)))
    return num / lam[:, None]


def decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                       partition_tokens: int = 2048):
    """Decode computed as split-context partitions merged by log-sum-exp.

    Equal to decode() in exact arithmetic; kept to show the merge is exact.
    """
    q64 = to_f64(q, dtype)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    sigma = exact_scale(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        K = to_f64(gather_fast(k_cache, block_tables[s], L), dtype)
        V = to_f64(gather_fast(v_cache, block_tables[s], L), dtype)
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            parts = partition_partials(q64[s, heads], K[:, g], V[:, g], sigma, partition_tokens)
            out[s, heads] = lse_merge(parts)
    return out


# ---------------------------------------------------------------- comparisons

def max_rownorm_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = last axis)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max()) if got.size else 0.0

