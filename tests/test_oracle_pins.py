"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Every check here compares the oracle with something other than itself:
closed forms, a textbook special case, values the pages print, invariants the
pages state, or a pure-Python recomputation without a cache.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import bruteforce
from tests.paged_fixtures import place, relabel
from workloads import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, *shape):
    return rng.standard_normal(size=shape).astype(np.float32)


# ------------------------------------------------------------ page-printed values

def test_kv_ledger_matches_page():
    """The chengxuchu.com page, section 2.3, prints 8.00 GiB for its ledger example."""
    g = json.load(open(os.path.join(GOLDEN, "kv_ledger.json")))
    i = g["inputs"]
    b = accounting.kv_ledger_bytes(i["layers"], i["batch"], i["kv_heads"], i["sequence_length"],
                                   i["head_dim"], i["bytes_per_element"])
    assert f"{b / 1024 ** 3:.2f}" == f"{g['printed_gib']:.2f}"
    assert b == 8 * 1024 ** 3  # exactly


def test_toykv_code_semantics():
    """ToyKV (chengxuchu.com, section 6.1): one-hot tokens, key = token, value = 2 token, no scale.

    Decode step i over the paged cache must give the closed forms of the page's
    code; the printed rows under it are garbled and must NOT be reproduced.
    """
    g = json.load(open(os.path.join(GOLDEN, "toykv_printed.json")))
    e = math.e
    expected = [
        [2.0, 0.0, 0.0, 0.0],
        [2 / (1 + e), 2 * e / (1 + e), 0.0, 0.0],
        [2 / (2 + e), 2 / (2 + e), 2 * e / (2 + e), 0.0],
    ]
    eye = np.eye(4, dtype=np.float32)
    ks = eye[:3, None, :]  # [3, Hkv=1, 4]
    vs = 2 * eye[:3, None, :]
    rng = np.random.default_rng(0)
    for step in range(3):
        kc, vc, tab, lens = place([ks[:step + 1]], [vs[:step + 1]], 4, rng)
        q = eye[step][None, None, :]
        out = oracle.decode(q, kc, vc, tab, lens, 1.0, "f32")[0, 0]
        np.testing.assert_allclose(out, expected[step], rtol=1e-15, atol=1e-15)
        assert not np.allclose(np.round(out, 3), g["printed_output"][step])


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_returns_value_exactly(dtype):
    rng = np.random.default_rng(1)
    hq, hkv, d = 8, 2, 16
    k = rand(rng, 1, hkv, d)
    v = rand(rng, 1, hkv, d)
    kc, vc, tab, lens = place([k], [v], 3, rng)
    q = rand(rng, 1, hq, d)
    if dtype == "bf16":
        to = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncate: any bits do
        kc, vc, q = to(kc), to(vc), to(q)
    out = oracle.decode(q, kc, vc, tab, lens, 0.25, dtype)
    vv = oracle.to_f64(vc, dtype)[tab[0, 0], :, 0, :]
    for h in range(hq):
        assert np.array_equal(out[0, h], vv[h // (hq // hkv)])


def test_uniform_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    L, d = 37, 8
    k = np.repeat(rand(rng, 1, 1, d), L, axis=0)
    v = rand(rng, L, 1, d)
    kc, vc, tab, lens = place([k], [v], 4, rng)
    q = rand(rng, 1, 1, d)
    out = oracle.decode(q, kc, vc, tab, lens, 0.3, "f32")[0, 0]
    mean = [math.fsum(float(v[t, 0, j]) for t in range(L)) / L for j in range(d)]
    np.testing.assert_allclose(out, mean, rtol=1e-14, atol=1e-15)


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(3)
    L, d = 21, 8
    k, v = rand(rng, L, 1, d), rand(rng, L, 1, d)
    kc, vc, tab, lens = place([k], [v], 3, rng)
    out = oracle.decode(rand(rng, 1, 1, d), kc, vc, tab, lens, 0.0, "f32")[0, 0]
    mean = [math.fsum(float(v[t, 0, j]) for t in range(L)) / L for j in range(d)]
    np.testing.assert_allclose(out, mean, rtol=1e-14, atol=1e-15)


def test_two_tokens_logistic():
    rng = np.random.default_rng(4)
    d = 8
    k, v = rand(rng, 2, 1, d), rand(rng, 2, 1, d)
    kc, vc, tab, lens = place([k], [v], 2, rng)
    q = rand(rng, 1, 1, d)
    sig = float(np.float32(0.7))
    x0 = sig * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], k[0, 0]))
    x1 = sig * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], k[1, 0]))
    w0 = 1.0 / (1.0 + math.exp(x1 - x0))
    w1 = 1.0 / (1.0 + math.exp(x0 - x1))
    ref = [w0 * float(v[0, 0, j]) + w1 * float(v[1, 0, j]) for j in range(d)]
    out = oracle.decode(q, kc, vc, tab, lens, 0.7, "f32")[0, 0]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value():
    """One logit above the rest by ~1000: every other weight underflows to exactly 0."""
    L, d = 30, 32
    rng = np.random.default_rng(5)
    k = np.zeros((L, 1, d), np.float32)
    for t in range(L):
        k[t, 0, t] = 1.0
    v = rand(rng, L, 1, d)
    star = 17
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, star] = 1000.0
    kc, vc, tab, lens = place([k], [v], 3, rng)
    out = oracle.decode(q, kc, vc, tab, lens, 1.0, "f32")[0, 0]
    assert np.array_equal(out, v[star, 0].astype(np.float64))
    assert np.isfinite(out).all()


def test_empty_context_is_zero():
    rng = np.random.default_rng(6)
    kc = np.full((2, 1, 16, 4), np.nan, np.float32)
    out = oracle.decode(rand(rng, 1, 2, 4), kc, kc, np.zeros((1, 1), np.int32),
                        np.zeros(1, np.int32), 0.5, "f32")
    assert np.array_equal(out, np.zeros_like(out))


# ------------------------------------------------------------ brute force without a cache

@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_naive_recompute(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3]))
    hq, d = hkv * G, int(rng.choice([3, 4, 8]))
    lens = [int(rng.integers(1, 41)) for _ in range(B)]
    ks = [rand(rng, L, hkv, d) for L in lens]
    vs = [rand(rng, L, hkv, d) for L in lens]
    kc, vc, tab, lens_a = place(ks, vs, sum(-(-L // 16) for L in lens) + 2, rng)
    q = rand(rng, B, hq, d)
    scale = float(rng.uniform(0.1, 1.0))
    sig = float(np.float32(scale))
    out = oracle.decode(q, kc, vc, tab, lens_a, scale, "f32")
    for s in range(B):
        for h in range(hq):
            g = h // G
            qs = [[0.0] * d] * (lens[s] - 1) + [[float(x) for x in q[s, h]]]
            kk = [[float(x) for x in ks[s][t, g]] for t in range(lens[s])]
            vv = [[float(x) for x in vs[s][t, g]] for t in range(lens[s])]
            ref = bruteforce.naive_generation(qs, kk, vv, sig)[-1]
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_prefill_matches_naive_recompute(seed):
    """Every chunk row equals the naive step over positions 0..its own (inclusive)."""
    rng = np.random.default_rng(200 + seed)
    hkv, G, d = 2, 2, 4
    hq = hkv * G
    prompt = int(rng.integers(5, 45))
    p0 = int(rng.integers(0, prompt))
    k, v = rand(rng, prompt, hkv, d), rand(rng, prompt, hkv, d)
    kc, vc, tab, lens = place([k], [v], 6, rng)
    cmax = prompt - p0 + 2
    qc = np.full((1, cmax, hq, d), np.nan, np.float32)
    qc[0, :prompt - p0] = rand(rng, prompt - p0, hq, d)
    out = oracle.prefill_chunk(qc, np.array([p0], np.int32), kc, vc, tab, lens, 0.5, "f32")
    sig = 0.5
    for h in range(hq):
        g = h // G
        kk = [[float(x) for x in k[t, g]] for t in range(prompt)]
        vv = [[float(x) for x in v[t, g]] for t in range(prompt)]
        qs = [[0.0] * d] * p0 + [[float(x) for x in qc[0, i, h]] for i in range(prompt - p0)]
        refs = bruteforce.naive_generation(qs, kk, vv, sig)
        for i in range(prompt - p0):
            np.testing.assert_allclose(out[0, i, h], refs[p0 + i], rtol=1e-12, atol=1e-13)
    assert np.isnan(out[0, prompt - p0:]).all()


# ------------------------------------------------------------ invariants the pages state

def _random_batch(rng, B=3, hkv=2, G=2, d=8, maxlen=70, shared=None):
    lens = [int(rng.integers(1, maxlen)) + (shared or 0) for _ in range(B)]
    base_k = rand(rng, shared or 0, hkv, d)
    base_v = rand(rng, shared or 0, hkv, d)
    ks = [np.concatenate([base_k, rand(rng, L - (shared or 0), hkv, d)]) for L in lens]
    vs = [np.concatenate([base_v, rand(rng, L - (shared or 0), hkv, d)]) for L in lens]
    return ks, vs, rand(rng, B, hkv * G, d)


def test_block_permutation_invariance_bitwise():
    rng = np.random.default_rng(7)
    ks, vs, q = _random_batch(rng)
    kc, vc, tab, lens = place(ks, vs, 20, rng)
    a = oracle.decode(q, kc, vc, tab, lens, 0.4, "f32")
    for _ in range(3):
        kc2, vc2, tab2 = relabel(kc, vc, tab, rng)
        b = oracle.decode(q, kc2, vc2, tab2, lens, 0.4, "f32")
        assert np.array_equal(a, b)


def test_prefix_sharing_equals_private_copies_bitwise():
    rng = np.random.default_rng(8)
    ks, vs, q = _random_batch(rng, shared=32)
    kc_s, vc_s, tab_s, lens = place(ks, vs, 40, rng, shared=32)
    assert len({tuple(tab_s[s, :2]) for s in range(len(ks))}) == 1  # really shared
    kc_p, vc_p, tab_p, lens_p = place(ks, vs, 40, rng)
    a = oracle.decode(q, kc_s, vc_s, tab_s, lens, 0.4, "f32")
    b = oracle.decode(q, kc_p, vc_p, tab_p, lens_p, 0.4, "f32")
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_replicated_kv_heads():
    rng = np.random.default_rng(9)
    hkv, G, d = 2, 3, 8
    ks, vs, q = _random_batch(rng, hkv=hkv, G=G, d=d)
    kc, vc, tab, lens = place(ks, vs, 20, rng)
    a = oracle.decode(q, kc, vc, tab, lens, 0.4, "f32")
    kr = [np.repeat(k, G, axis=1) for k in ks]  # kv head h//G for query head h
    vr = [np.repeat(v, G, axis=1) for v in vs]
    kc2, vc2, tab2, lens2 = place(kr, vr, 20, rng)
    b = oracle.decode(q, kc2, vc2, tab2, lens2, 0.4, "f32")
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def test_chunking_does_not_change_results():
    """A prompt prefilled as one chunk equals any split into chunks (chunking only reschedules)."""
    rng = np.random.default_rng(10)
    hkv, G, d, n = 2, 2, 8, 53
    k, v = rand(rng, n, hkv, d), rand(rng, n, hkv, d)
    qrows = rand(rng, n, hkv * G, d)
    kc, vc, tab, lens = place([k], [v], 6, rng)
    whole = oracle.prefill_chunk(qrows[None], np.array([0], np.int32), kc, vc, tab, lens, 0.3, "f32")[0]
    for cut in (1, 16, 17, 40, 52):
        first = oracle.prefill_chunk(qrows[None, :cut], np.array([0], np.int32), kc, vc, tab,
                                     np.array([cut], np.int32), 0.3, "f32")[0]
        second = oracle.prefill_chunk(qrows[None, cut:], np.array([cut], np.int32), kc, vc, tab,
                                      np.array([n], np.int32), 0.3, "f32")[0]
        np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-13, atol=1e-14)


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(11)
    hkv, G, d, n = 2, 4, 8, 45
    k, v = rand(rng, n, hkv, d), rand(rng, n, hkv, d)
    qrows = rand(rng, n, hkv * G, d)
    kc, vc, tab, lens = place([k], [v], 6, rng)
    pf = oracle.prefill_chunk(qrows[None], np.array([0], np.int32), kc, vc, tab, lens, 0.3, "f32")
    dec = oracle.decode(qrows[None, -1], kc, vc, tab, lens, 0.3, "f32")
    np.testing.assert_allclose(dec[0], pf[0, -1], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("part", [16, 32, 48, 2048])
def test_partitioned_lse_merge_equals_plain(part):
    rng = np.random.default_rng(12)
    ks, vs, q = _random_batch(rng, maxlen=150)
    kc, vc, tab, lens = place(ks, vs, 40, rng)
    a = oracle.decode(q, kc, vc, tab, lens, 0.4, "f32")
    b = oracle.decode_partitioned(q, kc, vc, tab, lens, 0.4, "f32", partition_tokens=part)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ cache write and gather

def test_write_round_trip_and_untouched_slots():
    rng = np.random.default_rng(13)
    nb, hkv, d = 10, 2, 8
    kc = rand(rng, nb, hkv, 16, d)
    vc = rand(rng, nb, hkv, 16, d)
    kc[3] = np.nan  # poisoned block must survive bit for bit
    slots = np.array([5 * 16 + 2, 0, 7 * 16 + 15, -1, 9 * 16 + 8], np.int32)
    nk, nv = rand(rng, len(slots), hkv, d), rand(rng, len(slots), hkv, d)
    kc2, vc2 = oracle.kv_write(kc, vc, nk, nv, slots)
    touched = np.zeros((nb, 16), bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        touched[s // 16, s % 16] = True
        assert np.array_equal(kc2[s // 16, :, s % 16].view(np.uint32), nk[i].view(np.uint32))
        assert np.array_equal(vc2[s // 16, :, s % 16].view(np.uint32), nv[i].view(np.uint32))
    for b in range(nb):
        for o in range(16):
            if not touched[b, o]:
                assert np.array_equal(kc2[b, :, o].view(np.uint32), kc[b, :, o].view(np.uint32))
                assert np.array_equal(vc2[b, :, o].view(np.uint32), vc[b, :, o].view(np.uint32))
    # inputs not modified
    assert np.isnan(kc[3]).all()


def test_write_then_gather_returns_rows():
    """gather(write(x)) == x, bit for bit, for a sequence laid out in a random table."""
    rng = np.random.default_rng(14)
    nb, hkv, d, L = 12, 2, 4, 37
    table = rng.permutation(nb)[:3].astype(np.int32)
    slots = np.array([table[t // 16] * 16 + t % 16 for t in range(L)], np.int32)
    rows_k, rows_v = rand(rng, L, hkv, d), rand(rng, L, hkv, d)
    kc = np.full((nb, hkv, 16, d), np.nan, np.float32)
    kc2, vc2 = oracle.kv_write(kc, kc.copy(), rows_k, rows_v, slots)
    for fn in (oracle.gather, oracle.gather_fast):
        assert np.array_equal(fn(kc2, table, L).view(np.uint32), rows_k.view(np.uint32))
        assert np.array_equal(fn(vc2, table, L).view(np.uint32), rows_v.view(np.uint32))


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049], np.uint16)
    ref = [1.0, -1.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 3.140625]
    assert list(oracle.to_f64(bits, "bf16")) == ref


def test_shared_prefix_decode_brute_force():
    """Shared-prefix decode against a per-sequence recompute over the concatenated
    context (prefix tokens, then the sequence's own), from contiguous lists."""
    rng = np.random.default_rng(21)
    hkv, G, d, pre = 2, 2, 8, 32
    suffix = [0, 5, 17, 40]
    base_k, base_v = rand(rng, pre, hkv, d), rand(rng, pre, hkv, d)
    own_k = [rand(rng, n, hkv, d) for n in suffix]
    own_v = [rand(rng, n, hkv, d) for n in suffix]
    q = rand(rng, len(suffix), hkv * G, d)
    # the pool: prefix blocks once, then each sequence's own blocks
    full_k = [np.concatenate([base_k, k]) for k in own_k]
    full_v = [np.concatenate([base_v, v]) for v in own_v]
    kc, vc, tab, lens = place(full_k, full_v, 24, rng, shared=pre)
    prefix_blocks = tab[0, :pre // 16].copy()
    own_tables = np.zeros((len(suffix), tab.shape[1]), dtype=np.int32)
    own_tables[:, :tab.shape[1] - pre // 16] = tab[:, pre // 16:]
    got = oracle.decode_shared_prefix(q, kc, vc, prefix_blocks, own_tables, np.array(suffix), 0.35, "f32")
    for s in range(len(suffix)):
        for h in range(hkv * G):
            g = h // G
            keys = [list(map(float, full_k[s][t, g])) for t in range(pre + suffix[s])]
            vals = [list(map(float, full_v[s][t, g])) for t in range(pre + suffix[s])]
            ref = bruteforce.attend_one(list(map(float, q[s, h])), keys, vals, oracle.exact_scale(0.35))
            np.testing.assert_allclose(got[s, h], ref, rtol=1e-12, atol=1e-13)


def test_copy_blocks_element_loop_and_invariance():
    """Block copy against an element-by-element loop; decode through copied blocks
    equals decode through the originals; invalid pairs are skipped; NaN payloads survive."""
    rng = np.random.default_rng(23)
    nb, hkv, d = 12, 2, 4
    kc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    kc[3, 1, 5, 2] = np.float32(np.nan)
    src = np.array([3, 0, 7, 99, 4], dtype=np.int32)
    dst = np.array([9, 10, 11, 2, -1], dtype=np.int32)
    k2, v2 = oracle.copy_blocks(kc, vc, src, dst)
    ek, ev = kc.copy(), vc.copy()
    for s, t in zip(src, dst):
        if 0 <= s < nb and 0 <= t < nb:
            for h in range(hkv):
                for o in range(16):
                    for e in range(d):
                        ek[t, h, o, e] = kc[s, h, o, e]
                        ev[t, h, o, e] = vc[s, h, o, e]
    assert k2.view(np.uint32).tobytes() == ek.view(np.uint32).tobytes()
    assert v2.view(np.uint32).tobytes() == ev.view(np.uint32).tobytes()
    assert np.isnan(k2[9, 1, 5, 2])
    q = rng.standard_normal((1, hkv, d)).astype(np.float32)
    a = oracle.decode(q, k2, v2, np.array([[0, 7]], dtype=np.int32), np.array([30]), 0.5, "f32")
    b = oracle.decode(q, k2, v2, np.array([[10, 11]], dtype=np.int32), np.array([30]), 0.5, "f32")
    assert np.array_equal(a, b)


# ------------------------------------------------------------ the comparison helpers every GPU verdict uses

def test_comparison_helpers_against_hand_computed_values():
    """max_abs_err and max_rownorm_rel_err on values worked out by hand.

    Rows are the last axis.  Row 0: errors (0.5, 0, 0), largest |ref| 4 -> 0.125.
    Row 1: errors (0, 0.05, 0), largest |ref| 0.5 -> 0.1.  Row 2: a zero
    reference row divides by 1 (its relative error is its absolute error, 0.1).
    So the largest absolute error (0.5, row 0) and the largest relative one
    (0.125, also row 0) come from the same row here; a second case separates them.
    """
    ref = np.array([[1.0, -4.0, 2.0], [0.5, 0.25, -0.5], [0.0, 0.0, 0.0]])
    got = np.array([[1.5, -4.0, 2.0], [0.5, 0.30, -0.5], [0.0, 0.1, 0.0]])
    assert oracle.max_abs_err(got, ref) == pytest.approx(0.5, abs=1e-15)
    assert oracle.max_rownorm_rel_err(got, ref) == pytest.approx(0.125, abs=1e-15)
    # large absolute error on a large row, small on a small row: the relative
    # maximum is the small row's (0.01 / 0.02 = 0.5 against 1 / 100 = 0.01)
    ref2 = np.array([[[100.0, 0.0]], [[0.02, -0.01]]])  # [2, 1, 2]: rows over the last axis
    got2 = np.array([[[101.0, 0.0]], [[0.02, -0.02]]])
    assert oracle.max_abs_err(got2, ref2) == pytest.approx(1.0, abs=1e-12)
    assert oracle.max_rownorm_rel_err(got2, ref2) == pytest.approx(0.5, abs=1e-12)
    # symmetric in sign, zero for identical inputs, empty input gives 0
    assert oracle.max_abs_err(-got, -ref) == oracle.max_abs_err(got, ref)
    assert oracle.max_rownorm_rel_err(ref, ref) == 0.0 and oracle.max_abs_err(ref, ref) == 0.0
    assert oracle.max_abs_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    assert oracle.max_rownorm_rel_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_comparison_helpers_never_pass_a_nan():
    """A NaN output makes both errors NaN, which fails every `err <= bar` check."""
    ref = np.ones((2, 3))
    got = ref.copy()
    got[1, 2] = np.nan
    a, r = oracle.max_abs_err(got, ref), oracle.max_rownorm_rel_err(got, ref)
    assert math.isnan(a) and math.isnan(r)
    assert not (a <= 1.0) and not (r <= 1.0)
