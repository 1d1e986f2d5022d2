"""Byte and FLOP accounting for the paged-attention hot path.

These are the algorithmic amounts of work, the quantities a roofline divides
by time: what the method must move or compute, not what an implementation
happens to move.

The KV ledger follows "Part 47 | Inference basics: KV Cache, batching,
sampling" (chengxuchu.com), section 2.3: layers x 2 (K and V) x batch x
kv_heads x sequence_length x head_dim x bytes_per_element.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def kv_ledger_bytes(layers: int, batch: int, kv_heads: int, seq_len: int, head_dim: int,
                    bytes_per_elem: int) -> int:
    """KV cache size of a contiguous cache, the page's shape formula."""
    return layers * 2 * batch * kv_heads * seq_len * head_dim * bytes_per_elem


def decode_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 elem_bytes: int, block_tables=None, dedupe_shared: bool = False, q_bytes: int = None,
                 scale_bytes: int = 0) -> dict:
    """Algorithmic bytes of one decode call.

    kv:     every (sequence, token) K and V row, or, with dedupe_shared, every
            distinct physical slot once (a prefix shared by many block tables is
            read once); a quantised cache adds its per-(slot, kv head) K and V
            scales (scale_bytes each);
    qo:     the queries read and the outputs written (q_bytes per element,
            default elem_bytes);
    tables: the block-table entries read and the context lengths.
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    row = num_kv_heads * (head_dim * elem_bytes + scale_bytes) * 2  # K + V bytes per token
    if dedupe_shared:
        assert block_tables is not None
        slots = set()
        for s, L in enumerate(lens):
            nb = -(-int(L) // BLOCK_SIZE)
            for j in range(nb):
                p = int(block_tables[s][j])
                n = min(BLOCK_SIZE, int(L) - j * BLOCK_SIZE)
                slots.update(p * BLOCK_SIZE + o for o in range(n))
        kv = len(slots) * row
    else:
        kv = int(lens.sum()) * row
    qo = 2 * len(lens) * num_q_heads * head_dim * (elem_bytes if q_bytes is None else q_bytes)
    tables = int(sum(-(-int(L) // BLOCK_SIZE) for L in lens)) * 4 + 4 * len(lens)
    return {"kv": kv, "qo": qo, "tables": tables, "total": kv + qo + tables}


def write_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Algorithmic bytes of one cache write: K and V rows read, the same written, slots read."""
    rows = 2 * num_tokens * num_kv_heads * head_dim * elem_bytes
    return 2 * rows + 4 * num_tokens


def copy_bytes(num_pairs: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Algorithmic bytes of a block copy: each pair's K and V block read and written, the two ids read."""
    block = num_kv_heads * BLOCK_SIZE * head_dim * elem_bytes
    return num_pairs * (2 * 2 * block + 8)


def prefill_flops(chunk_start, context_lens, num_q_heads: int, head_dim: int) -> int:
    """FLOPs of the causal (query, key) pairs of a set of prefill chunks (QK^T and PV, 2 each)."""
    pairs = 0
    for p0, L in zip(np.asarray(chunk_start).tolist(), np.asarray(context_lens).tolist()):
        n = L - p0
        pairs += p0 * n + n * (n + 1) // 2
    return 4 * head_dim * num_q_heads * pairs


def prefill_bytes(chunk_start, context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  elem_bytes: int) -> int:
    """Algorithmic bytes of a prefill-chunk call: each chunk's cached K/V once, q in, out written."""
    kv = int(np.asarray(context_lens, dtype=np.int64).sum()) * num_kv_heads * head_dim * 2 * elem_bytes
    rows = int((np.asarray(context_lens) - np.asarray(chunk_start)).sum())
    qo = 2 * rows * num_q_heads * head_dim * elem_bytes
    return kv + qo
