"""The read probe reads exactly the rows a decode reads (GPU).

Each wavefront folds the 32-bit words it loaded with XOR; the host computes the
same fold from the cache arrays with the same even split of the batch's
(sequence, kv head, block) list over the wavefronts, over the rows before each
context length only.  Equal words mean every valid row of every tile was read
by the right wavefront (rows past a context come back as zeros and fold to
nothing, so reading a poisoned slot would show).
"""
import numpy as np
import pytest

import oracle
import paged_kv_cache_295_amd as pkv
import workloads
from tests.gpu_util import DeviceWorkload, torch
from workloads import SeqSpec, build

pytestmark = pytest.mark.gpu


def expected_words(k_cache, v_cache, tables, lens, waves):
    hkv = k_cache.shape[1]
    words_k = np.ascontiguousarray(k_cache).view(np.uint32).reshape(k_cache.shape[0], hkv, 16, -1)
    words_v = np.ascontiguousarray(v_cache).view(np.uint32).reshape(k_cache.shape[0], hkv, 16, -1)
    tiles = []
    for s, L in enumerate(np.asarray(lens).tolist()):
        nb = -(-L // 16)
        for g in range(hkv):
            for j in range(nb):
                p = int(tables[s, j])
                rows = min(16, L - 16 * j)
                x = np.bitwise_xor.reduce(words_k[p, g, :rows].ravel()) ^ np.bitwise_xor.reduce(
                    words_v[p, g, :rows].ravel())
                tiles.append(int(x))
    T = len(tiles)
    out = np.zeros(waves, np.uint32)
    for w in range(waves):
        acc = 0
        for t in range(w * T // waves, (w + 1) * T // waves):
            acc ^= tiles[t]
        out[w] = acc
    return out


def run_probe(dw, waves):
    t = torch()
    out = t.zeros(waves, dtype=t.int32, device="cuda:0")
    pkv.paged_kv_read_probe(dw.k_cache, dw.v_cache, dw.tables, dw.lens, waves, out)
    t.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("waves", [1024, 7])
def test_probe_reads_the_decode_rows_llama3_8b(waves):
    w = workloads.make(2)
    dw = DeviceWorkload(w)
    pkv.paged_kv_write(dw.new_k, dw.new_v, dw.slots, dw.k_cache, dw.v_cache)
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    got = run_probe(dw, waves)
    assert np.array_equal(got, expected_words(rk, rv, w.block_tables, w.context_lens, waves))


@pytest.mark.parametrize("dtype,hkv,d", [("f32", 8, 64), ("bf16", 2, 64), ("f32", 4, 128)])
def test_probe_ragged_and_empty_contexts(dtype, hkv, d):
    rng = np.random.Generator(np.random.PCG64(61))
    lens = [0, 1, 15, 16, 17, 0, 300, 33]
    w = build(f"probe-{dtype}", 61, dtype, hkv * 4, hkv, d, [SeqSpec(L, n_new=1 if L else 0) for L in lens], rng=rng)
    dw = DeviceWorkload(w)
    pkv.paged_kv_write(dw.new_k, dw.new_v, dw.slots, dw.k_cache, dw.v_cache)
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    for waves in (1, 5, 64, 300):  # more wavefronts than blocks: some read nothing
        got = run_probe(dw, waves)
        assert np.array_equal(got, expected_words(rk, rv, w.block_tables, w.context_lens, waves)), waves
