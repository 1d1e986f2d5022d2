"""Host-side checks of the seeded serving mixes (no GPU)."""
import numpy as np
import pytest

import workloads
from workloads import accounting, synth


def _owned_slots(tables, lens):
    out = []
    for s, L in enumerate(lens):
        for t in range(int(L)):
            out.append(int(tables[s][t // 16]) * 16 + t % 16)
    return out


def test_seeded_reproducible():
    a = workloads.make(1)
    b = workloads.make(1)
    for f in ("k_cache", "v_cache", "q", "block_tables", "slot_mapping", "new_k"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    c = workloads.make(1, seed=7)
    assert not np.array_equal(a.q, c.q)


def test_tiny_config_shape():
    w = workloads.make(1)
    assert w.dtype == "f32" and w.num_blocks == 32
    assert list(w.context_lens) == [17, 40, 64, 200]
    assert w.block_tables.shape == (4, 13)
    used = {int(w.block_tables[s, j]) for s, L in enumerate(w.context_lens) for j in range(-(-L // 16))}
    assert len(used) == 22
    assert w.scale == np.float32(0.125)


@pytest.mark.parametrize("cfg", [1, 2, 3, "spec-verify-b8", "prefill-large"])
def test_tables_slots_and_poison(cfg):
    w = workloads.make(cfg)
    bs = 16
    seq_tables = list(w.block_tables) + list(w.chunk_tables)
    seq_lens = list(w.context_lens) + list(w.chunk_context_lens)
    ids = [int(t[j]) for t, L in zip(seq_tables, seq_lens) for j in range(-(-int(L) // bs))]
    assert len(ids) == len(set(ids)), "private blocks must not repeat"
    assert all(0 <= i < w.num_blocks for i in ids)
    assert w.pad_block not in ids
    if cfg in (2, 3):
        assert len(ids) / w.num_blocks <= 0.9 + 1e-9
        assert len(ids) / (w.num_blocks - 1) > 0.9 - 1e-9
    # new-token slots are the last n_new positions of each sequence, decode rows first
    expect = []
    for t, L in zip(w.block_tables, w.context_lens):
        expect.append(int(t[(L - 1) // bs]) * bs + (L - 1) % bs)
    for t, L, p0 in zip(w.chunk_tables, w.chunk_context_lens, w.chunk_start):
        expect += [int(t[p // bs]) * bs + p % bs for p in range(p0, L)]
    assert list(w.slot_mapping) == expect
    # poison: every slot not holding prior context is NaN, the others finite
    val = w.k_cache.astype(np.float32) if w.dtype == "f32" else synth.bf16_bits_to_f32(w.k_cache)
    finite = np.isfinite(val).all(axis=(1, 3))  # [NB, 16]
    owned = set(_owned_slots(seq_tables, seq_lens)) - set(expect)
    flat = {b * bs + o for b, o in zip(*np.nonzero(finite))}
    assert flat == owned


def test_shared_prefix_layout():
    w = workloads.make(4)
    assert w.block_tables.shape == (256, 160)
    assert (w.block_tables[:, :128] == w.shared_blocks[None, :]).all()
    assert ((w.context_lens >= 2048 + 16) & (w.context_lens <= 2048 + 512)).all()
    # writes never touch a shared block
    assert not set(int(s) // 16 for s in w.slot_mapping) & set(int(b) for b in w.shared_blocks)


def test_mixed_step_chunks():
    w = workloads.make(3)
    assert list(w.chunk_start) == [0, 1536]
    assert list(w.chunk_context_lens) == [512, 2048]
    assert w.q_chunk.shape == (2, 512, 32, 128)
    assert len(w.slot_mapping) == 48 + 1024


def test_prefill_large_chunks():
    w = workloads.make("prefill-large")
    assert w.num_seqs == 0 and w.num_chunks == 16
    assert (w.chunk_start == 3584).all() and (w.chunk_context_lens == 4096).all()
    assert w.q_chunk.shape == (16, 512, 32, 128)
    assert len(w.slot_mapping) == 16 * 512
    # 4 D Hq per causal (row, key) pair: 16 chunks of 512 rows at positions 3584..4095
    assert accounting.prefill_flops(w.chunk_start, w.chunk_context_lens, 32, 128) == \
        4 * 128 * 32 * 16 * (3584 * 512 + 512 * 513 // 2)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], np.float32)
    b = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert list(synth.bf16_bits_to_f32(b)[:3]) == [1.0, 1.0, 1.015625]
    assert synth.bf16_bits_to_f32(b)[3] == -2.5


def test_accounting_formulas():
    lens = np.array([16, 17, 1])
    d = accounting.decode_bytes(lens, 4, 2, 8, 2)
    assert d["kv"] == 34 * 2 * 8 * 2 * 2
    assert d["tables"] == (1 + 2 + 1) * 4 + 3 * 4
    # shared slots counted once
    tables = np.array([[5, 6], [5, 7]])
    dd = accounting.decode_bytes(np.array([20, 18]), 4, 2, 8, 2, block_tables=tables, dedupe_shared=True)
    assert dd["kv"] == (16 + 4 + 2) * 2 * 8 * 2 * 2
    assert accounting.prefill_flops([0], [3], 1, 1) == 4 * (3 * 4 // 2)
    assert accounting.write_bytes(2, 1, 4, 2) == 2 * (2 * 2 * 4 * 2) + 8
