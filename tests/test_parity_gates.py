"""The parity bars can tell a right answer from a wrong one (CPU only, no GPU).

On the long-context batch (8 sequences of 32k-131k tokens, 64 query / 8 kv
heads) every output is small (|o| ~ 0.01-0.04): the 2e-2 absolute bar for
bf16 is about as large as the outputs themselves.  These tests take the
oracle's own result, change it the way a plausible kernel mistake would, and
check that the bars of tests/tolerances.py reject it -- while they accept a
result that carries exactly the roundings the bf16 kernels are documented to
make (softmax weights rounded to bf16 before the value product, output rounded
to bf16).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.tolerances import BF16_ABS, BF16_REL, attn_errors, within_bar


def bf16_round(x):
    """float64 -> nearest bf16 value (ties to even), as float64."""
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


@pytest.fixture(scope="module", params=[5, 2], ids=["long-context", "llama3-8b-decode"])
def case(request):
    w = workloads.make(request.param)
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    B, hq, d = w.q.shape
    hkv = w.num_kv_heads
    G = hq // hkv
    q = oracle.to_f64(w.q, w.dtype)
    sigma = oracle.exact_scale(w.scale)
    ref = oracle.decode(w.q, rk, rv, w.block_tables, w.context_lens, w.scale, w.dtype)
    # partitions of 2048 tokens as the long-context batch is configured; 64 (four blocks) for the
    # batch of contexts from 128 tokens, so that every context has more than one
    part = 2048 if w.max_context_len > 8192 else 64
    rounded = np.zeros_like(ref)      # the kernels' two documented roundings
    no_part = np.zeros_like(ref)      # one partition left out of the merge
    no_new = oracle.decode(w.q, rk, rv, w.block_tables, w.context_lens - 1, w.scale, w.dtype)  # newest token unread
    for s in range(B):
        L = int(w.context_lens[s])
        K = oracle.to_f64(oracle.gather_fast(rk, w.block_tables[s], L), w.dtype)
        V = oracle.to_f64(oracle.gather_fast(rv, w.block_tables[s], L), w.dtype)
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            x = sigma * (q[s, hs] @ K[:, g].T)
            p = np.exp(x - x.max(axis=1, keepdims=True))
            rounded[s, hs] = bf16_round((bf16_round(p) @ V[:, g]) / p.sum(axis=1, keepdims=True))
            parts = oracle.partition_partials(q[s, hs], K[:, g], V[:, g], sigma, part)
            drop = len(parts) // 2  # a middle partition
            no_part[s, hs] = oracle.lse_merge(parts[:drop] + parts[drop + 1:])
    return w, ref, rounded, no_part, no_new


def test_bar_accepts_the_documented_roundings(case):
    w, ref, rounded, _, _ = case
    a, r = attn_errors(rounded, ref)
    assert r > 2.0 ** -9  # the roundings are visible...
    assert within_bar(rounded, ref, "bf16"), (a, r)  # ...and inside the bar


def test_bar_rejects_a_dropped_partition(case):
    w, ref, _, no_part, _ = case
    a, r = attn_errors(no_part, ref)
    assert r > BF16_REL and not within_bar(no_part, ref, "bf16"), (a, r)


def test_bar_rejects_an_unread_newest_token(case):
    w, ref, _, _, no_new = case
    a, r = attn_errors(no_new, ref)
    assert r > BF16_REL and not within_bar(no_new, ref, "bf16"), (a, r)


def test_absolute_bar_alone_misses_long_context_mistakes(case):
    """Why the relative bar exists: at long contexts the absolute one passes both mistakes."""
    w, ref, _, no_part, no_new = case
    if w.max_context_len < 32768:
        pytest.skip("short contexts: the absolute bar catches these mistakes too")
    assert attn_errors(no_part, ref)[0] <= BF16_ABS
    assert attn_errors(no_new, ref)[0] <= BF16_ABS
