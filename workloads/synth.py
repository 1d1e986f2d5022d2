"""Seeded synthetic inputs for attention over a paged KV cache.

This module only builds inputs.  It plays the part of the serving runtime's
KV manager: it draws context lengths, hands out physical block ids from a
shuffled pool, fills the cache that an earlier prefill would have left behind,
and lists the slots that this step's new tokens go to.  It computes no
attention, no softmax and no cache write; both the GPU library and the CPU
oracle receive exactly the arrays made here.

Source for the cache organisation: the ainews.alishangtian.com article on
inference engines, section "PagedAttention" (fixed blocks of usually 16
tokens, allocated on demand, chained by a block table; shared prefixes stored
once and referenced by many requests), and the caffein.top essay on modern LLM
inference runtimes, section on paging (logically contiguous tokens mapped to
non-contiguous physical blocks, e.g. request A -> blocks 1, 4, 7).

Conventions used throughout:
  * values are N(0, 1) float32, rounded to bfloat16 by round-to-nearest-even
    for bf16 workloads and carried as raw uint16 bit patterns;
  * every cache slot that no sequence may read, and every slot that this
    step's writes will fill, holds NaN (bf16 0x7FC0) so that a wrong read
    shows up as NaN instead of plausible numbers;
  * context_lens count the tokens written in this step, so a decode query sits
    at position context_len - 1 and its own K/V are written first;
  * unused block-table entries point at an unused (NaN) block.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)
SEED_BASE = 295000


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs stay below 0xFF800000, so the uint32 sum cannot wrap
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class SeqSpec:
    """One sequence of the batch.

    length: tokens resident in the cache after this step's writes.
    n_new:  tokens written by this step (1 for a decode, the chunk length for a
            prefill chunk); they sit at positions [length - n_new, length).
    kind:   "decode" (one query at position length-1) or "chunk" (n_new query
            rows at positions [length - n_new, length)).
    shared_prefix: the first blocks of its table are the batch's shared prefix.
    """

    length: int
    n_new: int = 1
    kind: str = "decode"
    shared_prefix: bool = False


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    dtype: str  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: np.float32
    # cache state before this step's writes: [num_blocks, Hkv, 16, D]
    k_cache: np.ndarray
    v_cache: np.ndarray
    # the step's new K/V rows and where they go
    new_k: np.ndarray  # [T, Hkv, D]
    new_v: np.ndarray
    slot_mapping: np.ndarray  # int32 [T]
    # decode part
    q: np.ndarray  # [B, Hq, D]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    context_lens: np.ndarray  # int32 [B]
    # prefill-chunk part
    q_chunk: np.ndarray  # [Nc, Cmax, Hq, D]; rows past each chunk are NaN
    chunk_start: np.ndarray  # int32 [Nc]
    chunk_tables: np.ndarray  # int32 [Nc, max_blocks_c]
    chunk_context_lens: np.ndarray  # int32 [Nc]
    # bookkeeping
    pad_block: int = 0
    shared_blocks: Optional[np.ndarray] = None
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_chunks(self) -> int:
        return int(self.chunk_start.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def np_store_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32


def pool_size_for(total_blocks: int, fill: float = 0.9) -> int:
    """Smallest pool whose occupancy by total_blocks does not exceed `fill`."""
    return int(math.ceil(total_blocks / fill - 1e-9))


def _draw_values(rng, shape, dtype) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    return v


def _draw_pool(rng, num_blocks, hkv, d, dtype, chunk_blocks=1024) -> np.ndarray:
    """N(0,1) values for every slot of a pool.

    Chunk i of `chunk_blocks` blocks draws from its own PCG64 stream seeded by
    (one 63-bit draw of `rng`, i), so the result does not depend on how many
    threads fill it.
    """
    store = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((num_blocks, hkv, BLOCK_SIZE, d), dtype=store)
    base = int(rng.integers(2 ** 63))

    def fill(i):
        b0 = i * chunk_blocks
        b1 = min(num_blocks, b0 + chunk_blocks)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([base, i])))
        out[b0:b1] = _draw_values(g, (b1 - b0, hkv, BLOCK_SIZE, d), dtype)

    n = -(-num_blocks // chunk_blocks)
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(n)))
    return out


def build(
    name: str,
    seed: int,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    seqs: list,
    *,
    num_blocks: Optional[int] = None,
    fill: float = 0.9,
    shared_prefix_blocks: int = 0,
    max_blocks: Optional[int] = None,
    max_blocks_chunk: Optional[int] = None,
    chunk_len_max: Optional[int] = None,
    scale: Optional[float] = None,
    rng: Optional[np.random.Generator] = None,
    poison: bool = True,
    description: str = "",
) -> Workload:
    """Lay out a batch of sequences in a shuffled block pool and draw its values.

    Draw order (after any lengths the caller drew from the same generator):
    block permutation, decode q, chunk q, K pool, V pool, new K rows, new V rows.
    """
    assert dtype in ("f32", "bf16")
    assert num_q_heads % num_kv_heads == 0
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    bs = BLOCK_SIZE
    nblk = [int(math.ceil(s.length / bs)) for s in seqs]
    sp = shared_prefix_blocks
    for s, n in zip(seqs, nblk):
        if s.shared_prefix:
            assert n >= sp and s.length - s.n_new >= sp * bs, "writes must not touch shared blocks"
        assert 0 <= s.n_new <= s.length
    private = sum(n - (sp if s.shared_prefix else 0) for s, n in zip(seqs, nblk))
    total = private + sp
    if num_blocks is None:
        num_blocks = pool_size_for(total, fill)
    assert num_blocks >= total, "pool too small"

    perm = rng.permutation(num_blocks).astype(np.int32)
    shared = perm[:sp].copy()
    cursor = sp
    tables = []
    for s, n in zip(seqs, nblk):
        if s.shared_prefix:
            own = perm[cursor:cursor + n - sp]
            cursor += n - sp
            tables.append(np.concatenate([shared, own]))
        else:
            tables.append(perm[cursor:cursor + n].copy())
            cursor += n
    pad_block = int(perm[cursor]) if cursor < num_blocks else 0

    dec = [i for i, s in enumerate(seqs) if s.kind == "decode"]
    chk = [i for i, s in enumerate(seqs) if s.kind == "chunk"]

    def table_array(idx, width):
        if width is None:
            width = max([nblk[i] for i in idx], default=1)
            width = max(width, 1)
        t = np.full((len(idx), width), pad_block, dtype=np.int32)
        for r, i in enumerate(idx):
            assert nblk[i] <= width
            t[r, :nblk[i]] = tables[i]
        return t

    block_tables = table_array(dec, max_blocks)
    chunk_tables = table_array(chk, max_blocks_chunk)
    context_lens = np.array([seqs[i].length for i in dec], dtype=np.int32)
    chunk_context_lens = np.array([seqs[i].length for i in chk], dtype=np.int32)
    chunk_start = np.array([seqs[i].length - seqs[i].n_new for i in chk], dtype=np.int32)
    if chunk_len_max is None:
        chunk_len_max = max([seqs[i].n_new for i in chk], default=1)

    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    q = _draw_values(rng, (len(dec), hq, d), dtype)
    q_chunk = _draw_values(rng, (len(chk), chunk_len_max, hq, d), dtype)
    nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    if poison:
        for r, i in enumerate(chk):
            q_chunk[r, seqs[i].n_new:] = nan

    k_cache = _draw_pool(rng, num_blocks, hkv, d, dtype)
    v_cache = _draw_pool(rng, num_blocks, hkv, d, dtype)

    # slots holding context that existed before this step
    valid = np.zeros((num_blocks, bs), dtype=bool)
    for s, tab in zip(seqs, tables):
        old = s.length - s.n_new
        full, rem = divmod(old, bs)
        valid[tab[:full], :] = True
        if rem:
            valid[tab[full], :rem] = True
    if poison:
        inv_b, inv_o = np.nonzero(~valid)
        k_cache[inv_b, :, inv_o, :] = nan
        v_cache[inv_b, :, inv_o, :] = nan

    # the step's new rows: decode tokens first, then chunk rows, in batch order
    slots = []
    for i in dec + chk:
        s = seqs[i]
        tab = tables[i]
        for pos in range(s.length - s.n_new, s.length):
            slots.append(int(tab[pos // bs]) * bs + pos % bs)
    slot_mapping = np.array(slots, dtype=np.int32)
    new_k = _draw_values(rng, (len(slots), hkv, d), dtype)
    new_v = _draw_values(rng, (len(slots), hkv, d), dtype)

    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(
        name=name, seed=seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        num_blocks=num_blocks, scale=np.float32(scale), k_cache=k_cache, v_cache=v_cache,
        new_k=new_k, new_v=new_v, slot_mapping=slot_mapping, q=q, block_tables=block_tables,
        context_lens=context_lens, q_chunk=q_chunk, chunk_start=chunk_start,
        chunk_tables=chunk_tables, chunk_context_lens=chunk_context_lens, pad_block=pad_block,
        shared_blocks=shared if sp else None, description=description,
    )


def fp8_pool(w: Workload, seed: Optional[int] = None) -> dict:
    """An fp8 (E4M3) version of workload w's cache pool, drawn afresh.

    Codes are uniform over the 254 finite E4M3 bytes (0x7F and 0xFF, the NaN
    codes, excluded) and scales uniform in [2^-12, 2^-6) as float32, one per
    (slot, kv head).  Slots that w poisons with NaN (no context has reached
    them) get the NaN code 0x7F and a NaN scale.  Returns uint8 caches
    [NB, Hkv, 16, D] and float32 scales [NB, Hkv, 16] for K and for V.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed + 7000 if seed is None else seed))
    shape = w.k_cache.shape
    out = {}
    for name, ref in (("k", w.k_cache), ("v", w.v_cache)):
        r = rng.integers(0, 254, size=shape, dtype=np.uint8)
        codes = r + (r >= 0x7F).astype(np.uint8)  # skip 0x7F; the top draw 253 maps to 0xFE
        scales = rng.uniform(2.0 ** -12, 2.0 ** -6, size=shape[:3]).astype(np.float32)
        raw = ref[:, :, :, 0]
        poisoned = (raw == BF16_NAN) if w.dtype == "bf16" else np.isnan(raw)
        codes[poisoned] = 0x7F
        scales[poisoned] = np.nan
        out[name + "_cache"], out[name + "_scale"] = codes, scales
    return out


# --------------------------------------------------------------------------
# The five serving mixes.  Integer ranges are inclusive.

def tiny_f32(seed: Optional[int] = None) -> Workload:
    """4 sequences (17, 40, 64, 200 tokens), 8 q = 8 kv heads x 64, fp32, pool of 32 blocks."""
    seed = SEED_BASE + 1 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [17, 40, 64, 200]
    return build("tiny-decode-f32", seed, "f32", 8, 8, 64, [SeqSpec(L) for L in lens],
                 num_blocks=32, rng=rng, scale=0.125,
                 description="4 seqs, L={17,40,64,200}, 8q/8kv x 64, fp32, 32-block pool")


def llama8b_decode(seed: Optional[int] = None, batch: int = 64, lo: int = 128, hi: int = 4096) -> Workload:
    """Llama-3-8B-shaped decode step: 64 seqs, L ~ U{128..4096}, 32 q / 8 kv heads x 128, bf16."""
    seed = SEED_BASE + 2 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi + 1, size=batch)
    return build("llama3-8b-decode-bf16", seed, "bf16", 32, 8, 128, [SeqSpec(int(L)) for L in lens],
                 max_blocks=hi // BLOCK_SIZE, rng=rng,
                 description=f"{batch} seqs, L~U{{{lo}..{hi}}}, 32q/8kv x 128, bf16, 90% pool fill")


def mixed_step(seed: Optional[int] = None) -> Workload:
    """48 decode seqs (L ~ U{256..8192}) + prefill chunks of 512 at 0 and 1536 of 4096-token prompts."""
    seed = SEED_BASE + 3 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(256, 8192 + 1, size=48)
    seqs = [SeqSpec(int(L)) for L in lens]
    for start in (0, 1536):
        seqs.append(SeqSpec(start + 512, n_new=512, kind="chunk"))
    return build("mixed-step-bf16", seed, "bf16", 32, 8, 128, seqs, max_blocks=8192 // BLOCK_SIZE,
                 max_blocks_chunk=4096 // BLOCK_SIZE, chunk_len_max=512, rng=rng,
                 description="48 decode seqs L~U{256..8192} + 2x512-token chunks at 0 and 1536, "
                             "32q/8kv x 128, bf16")


def shared_prefix(seed: Optional[int] = None, batch: int = 256) -> Workload:
    """256 seqs sharing 128 physical prefix blocks (2048 tokens) + private suffixes U{16..512}."""
    seed = SEED_BASE + 4 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    suffix = rng.integers(16, 512 + 1, size=batch)
    seqs = [SeqSpec(2048 + int(x), shared_prefix=True) for x in suffix]
    return build("shared-prefix-bf16", seed, "bf16", 32, 8, 128, seqs, shared_prefix_blocks=128,
                 max_blocks=(2048 + 512) // BLOCK_SIZE, rng=rng,
                 description=f"{batch} seqs, 2048-token shared prefix (128 blocks) + suffix U{{16..512}}, "
                             "32q/8kv x 128, bf16")


def long_context(seed: Optional[int] = None, batch: int = 8, lo: int = 32768, hi: int = 131072) -> Workload:
    """Long-context decode: 8 seqs, L ~ U{32768..131072}, 64 q / 8 kv heads x 128, bf16."""
    seed = SEED_BASE + 5 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi + 1, size=batch)
    return build("long-context-decode-bf16", seed, "bf16", 64, 8, 128, [SeqSpec(int(L)) for L in lens],
                 max_blocks=hi // BLOCK_SIZE, rng=rng,
                 description=f"{batch} seqs, L~U{{{lo}..{hi}}}, 64q/8kv x 128, bf16, 90% pool fill")


def spec_verify(seed: Optional[int] = None, batch: int = 64, k: int = 4, lo: int = 128,
                hi: int = 4096) -> Workload:
    """Speculative-decoding verify step: 64 seqs with accepted contexts L ~ U{128..4096}
    (the last accepted token included) and k = 4 draft tokens each, so k + 1 = 5 new
    causal rows per sequence; 32 q / 8 kv heads x 128, bf16.  Not one of the five
    serving mixes: the verify pass is the prefill-chunk call with 5-row chunks."""
    seed = SEED_BASE + 6 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi + 1, size=batch)
    seqs = [SeqSpec(int(L) + k, n_new=k + 1, kind="chunk") for L in lens]
    return build(f"spec-verify-k{k}-bf16" if batch == 64 else f"spec-verify-k{k}-b{batch}-bf16", seed, "bf16", 32, 8, 128, seqs, max_blocks_chunk=-(-(hi + k) // BLOCK_SIZE),
                 chunk_len_max=k + 1, rng=rng,
                 description=f"{batch} seqs, accepted L~U{{{lo}..{hi}}} + {k} drafts ({k + 1} causal rows each), "
                             "32q/8kv x 128, bf16")


def prefill_large(seed: Optional[int] = None, chunks: int = 16, rows: int = 512, start: int = 3584) -> Workload:
    """Large chunked prefill: 16 chunks of 512 rows at position 3584 of 4096-token prompts,
    32 q / 8 kv heads x 128, bf16.  Not one of the five serving mixes: a prefill big
    enough that the matrix cores, not the launch, set its time."""
    seed = SEED_BASE + 7 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    seqs = [SeqSpec(start + rows, n_new=rows, kind="chunk") for _ in range(chunks)]
    return build("prefill-large-bf16", seed, "bf16", 32, 8, 128, seqs,
                 max_blocks_chunk=-(-(start + rows) // BLOCK_SIZE), chunk_len_max=rows, rng=rng,
                 description=f"{chunks} chunks x {rows} rows at position {start}, 32q/8kv x 128, bf16")


CONFIGS = {
    1: tiny_f32,
    2: llama8b_decode,
    3: mixed_step,
    4: shared_prefix,
    5: long_context,
}


# Supplementary workloads for the rows beyond the five mixes, by name.
SUPPLEMENTARY = {
    "spec-verify": spec_verify,
    "spec-verify-b8": lambda seed=None: spec_verify(seed, batch=8),
    "prefill-large": prefill_large,
}


def make(cfg_id, **kw) -> Workload:
    """A serving mix by number (1..5) or a supplementary workload by name."""
    if isinstance(cfg_id, str):
        return SUPPLEMENTARY[cfg_id](**kw)
    return CONFIGS[cfg_id](**kw)
