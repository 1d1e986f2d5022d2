"""The decode entry point that allocates nothing, against the one with a workspace (GPU).

paged_attn_decode_noalloc keeps the split decode's partial states in a buffer
inside the library.  It runs the same kernels as paged_attn_decode, so on the
same inputs both give the same bits; both are also held to the bf16 bar
against the oracle.  Two calls in a row, the second with a smaller batch
(fewer, shorter sequences, a larger GQA group), check that what the first
call leaves in the buffer does not leak into the second.
"""
import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_cache_295_amd as pkv
import workloads
from tests.gpu_util import DeviceWorkload, bits, empty_like_q, torch, values
from tests.tolerances import BF16_ABS, BF16_REL, attn_errors, record
from workloads import SeqSpec, build

pytestmark = pytest.mark.gpu


def decode_both(w, dw, partition_tokens=0):
    ws_out = empty_like_q(w.q.shape, w.dtype)
    na_out = empty_like_q(w.q.shape, w.dtype)
    pkv.paged_attn_decode(dw.q, dw.k_cache, dw.v_cache, dw.tables, dw.lens, float(w.scale), ws_out,
                          max_context_len=w.max_context_len, partition_tokens=partition_tokens)
    pkv.paged_attn_decode_noalloc(dw.q, dw.k_cache, dw.v_cache, dw.tables, dw.lens, float(w.scale), na_out,
                                  max_context_len=w.max_context_len, partition_tokens=partition_tokens)
    torch().cuda.synchronize()
    return ws_out, na_out


def check_same(w, dw, what, partition_tokens=0):
    ws_out, na_out = decode_both(w, dw, partition_tokens)
    assert np.array_equal(bits(na_out), bits(ws_out)), f"{what}: the two entry points differ"
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    ref = oracle.decode(w.q, rk, rv, w.block_tables, w.context_lens, w.scale, w.dtype)
    a, r = attn_errors(values(na_out), ref)
    record(f"no-alloc decode: {what}", w.dtype, a, r)
    print(f"{what}: abs {a:.3e} rel {r:.3e}", flush=True)
    assert a <= BF16_ABS and r <= BF16_REL


def test_two_calls_in_a_row_second_smaller():
    w1 = workloads.make(2)  # 64 sequences, 32q/8kv: 1024 waves' partials
    dw1 = DeviceWorkload(w1)
    pkv.paged_kv_write(dw1.new_k, dw1.new_v, dw1.slots, dw1.k_cache, dw1.v_cache)
    check_same(w1, dw1, "Llama-3-8B batch (64 sequences)")
    rng = np.random.Generator(np.random.PCG64(77))
    lens = [int(x) for x in rng.integers(1, 1500, size=7)]
    w2 = build("noalloc-small", 77, "bf16", 64, 8, 128, [SeqSpec(L) for L in lens], rng=rng)
    dw2 = DeviceWorkload(w2)
    pkv.paged_kv_write(dw2.new_k, dw2.new_v, dw2.slots, dw2.k_cache, dw2.v_cache)
    check_same(w2, dw2, "7 sequences, 64q/8kv")
    # fixed partitions through the same buffer
    check_same(w2, dw2, "7 sequences, partitions of 256", partition_tokens=256)


def test_oversized_fixed_partitions_fail_before_launch():
    lib = pkv.load_library()
    assert lib.paged_attn_decode_noalloc_scratch_bytes() == 2048 * 2 * 8 * 130 * 4
    desc = pkv.CacheDesc(64, 16, 8, 128, 1)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call fails on the host first
    st = lib.paged_attn_decode_noalloc(fake, 4096, 32, fake, fake, ctypes.byref(desc), fake, 8192, fake, 131072,
                                       0.1, fake, 16, None)
    assert st == -8 and b"scratch" in lib.pkv_status_string(st)
