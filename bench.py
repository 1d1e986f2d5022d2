#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

Default workload: the Llama-3-8B-shaped decode step (64 sequences, context
lengths uniform in [128, 4096], 32 query / 8 kv heads x 128, bf16, 16-token
blocks in a shuffled pool at 90% fill).  One step = the cache write of the 64
new tokens + the paged decode attention of the 64 sequences (+ the prefill
chunks for the mixed workload), on inputs already resident in HBM.

Prints one JSON line.  `value` is the KV bytes the decode step reads per
second of step time (GB/s, whole job), over exactly `--steps` steps timed with
the host clock between two device synchronisations.  The line also carries
seq-tokens/s; the roofline of the decode call, whose headline is the call with
the last-level caches cold (a 512 MB overwrite before each call, outside its
HIP events; mean and p50/p95/p99 of per-call events on the stream the library
launches on), beside the same call back to back with warm caches
(`roofline_llc_warm`); HBM traffic from rocprofv3 counters taken on the same
kernels; what the access pattern allows (`achievable`: the read probe, the
decode's K/V loads with no arithmetic, timed the same way); and the CPU oracle
timed on the host's cores as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cold] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV HBM GB/s (% of peak) + seq-tokens/s, 8B-shaped batch"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

# HBM traffic of one decode call, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch summed over the call's two
# kernels), scaled by what the same counters read for kernels of known bytes in
# the same runs: the read probe, which reads exactly the call's K/V rows with the
# decode's own 16-byte non-temporal buffer loads (FETCH_SIZE x 1.998), and a
# 256 MiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); factors 2.0 and 1.0
# are used.  Keyed by (workload, --kv-dtype).  Valid only for the decode kernel
# sources it was measured on: reported as null once their hash differs.
TRAFFIC = {
    ("llama3-8b-decode-bf16", "model"): {"read_bytes": 510129357, "write_bytes": 3504538,
                                        "sources_sha256": "bd0ec6e61032a96c49195e1b207ae8d2f37821d2ca75cc7bb74bea203cec1065"},
    ("llama3-8b-decode-bf16", "fp8"): {"read_bytes": 273598669, "write_bytes": 3508634,
                                      "sources_sha256": "bd0ec6e61032a96c49195e1b207ae8d2f37821d2ca75cc7bb74bea203cec1065"},
}
CSRC = os.path.join(ROOT, "paged_kv_cache_295_amd", "csrc")
DECODE_SOURCES = ("decode.hip", "pkv_device.hpp", "pkv_internal.hpp")


def verify_balanced(w) -> bool:
    """Which kernels paged_attn_spec_verify runs for this batch (for the report only; the library decides):
    the balanced split when a bf16 cache at head dim 128 gives each wave 4 or 8 query heads whose rows fit 32
    matrix-core columns, over at least 128 (sequence, kv head, head subgroup) streams."""
    g = w.num_q_heads // w.num_kv_heads
    gb = 8 if g % 8 == 0 else 4 if g % 4 == 0 else 0
    rows = w.q_chunk.shape[1]
    return (w.dtype == "bf16" and w.head_dim == 128 and gb > 0 and gb * rows <= 32
            and w.num_chunks * w.num_q_heads // gb >= 128)


def sources_sha256() -> str:
    """Hash of the sources the decode kernels are built from."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


WORKLOADS = {
    "llama3-8b-decode": 2,
    "tiny-decode-f32": 1,
    "mixed-step": 3,
    "shared-prefix": 4,
    "long-context": 5,
    "spec-verify": "spec-verify",  # supplementary: speculative-decoding verify (5-row chunks)
    "spec-verify-b8": "spec-verify-b8",  # the same with 8 sequences (keys split over the GPU)
    "prefill-large": "prefill-large",  # supplementary: 16 chunks x 512 rows at 3584 keys (matrix-core bound)
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama3-8b-decode", choices=sorted(WORKLOADS))
    p.add_argument("--streams", type=int, default=2, choices=[1, 2],
                   help="mixed step: 2 runs the prefill chunks on a second stream beside the decode")
    p.add_argument("--partition", type=int, default=0,
                   help="decode partition tokens (0 = balanced split over a fixed number of wavefronts)")
    p.add_argument("--cold", action="store_true", help="read 512 MB before every step (LLC-cold timing)")
    p.add_argument("--no-cascade", action="store_true",
                   help="shared-prefix workload: plain decode over the full tables instead of the shared-prefix call")
    p.add_argument("--kv-dtype", choices=["model", "fp8"], default="model",
                   help="fp8: the cache held as E4M3 codes with per-(slot, kv head) scales (decode workloads)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold-check", action="store_true",
                   help="skip the supplementary timing of the attention call with cold last-level caches")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    p.add_argument("--copy-pairs", type=int, default=512,
                   help="block pairs of the supplementary copy-on-write measurement (0: skip)")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="after timing, run one device copy of this many MiB (calibrates HBM byte counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(how the path would shard across GPUs is described in the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_295_amd as pkv
    import workloads
    from workloads import accounting

    cfg = WORKLOADS[args.workload]
    w = workloads.make(cfg)
    # the CPU oracle first, before anything touches the GPU (its worker processes are forked)
    fp8 = args.kv_dtype == "fp8"
    prefill_only = cfg == "prefill-large"
    cpu = None if args.no_cpu_baseline or fp8 or prefill_only else cpu_baseline(w, args.cpu_seconds)

    pkv.load_library()
    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.int32:
            return torch.from_numpy(a).to(dev)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if fp8:
        if w.dtype != "bf16" or w.num_chunks or w.shared_blocks is not None:
            raise SystemExit("--kv-dtype fp8 takes the bf16 decode workloads without chunks or a shared prefix")
        pool = workloads.fp8_pool(w)
        kc, vc = (torch.from_numpy(pool["k_cache"]).to(dev), torch.from_numpy(pool["v_cache"]).to(dev))
        ksc, vsc = (torch.from_numpy(pool["k_scale"]).to(dev), torch.from_numpy(pool["v_scale"]).to(dev))
    else:
        kc, vc = to_dev(w.k_cache), to_dev(w.v_cache)
    nk, nv, slots = to_dev(w.new_k), to_dev(w.new_v), to_dev(w.slot_mapping)
    q, tables, lens = to_dev(w.q), to_dev(w.block_tables), to_dev(w.context_lens)
    out = torch.empty_like(q)
    has_chunks = w.num_chunks > 0
    if has_chunks:
        qc, cstart, ctables, clens = (to_dev(w.q_chunk), to_dev(w.chunk_start), to_dev(w.chunk_tables),
                                      to_dev(w.chunk_context_lens))
        oc = torch.empty_like(qc)
    part = args.partition  # 0: balanced split
    cascade = w.shared_blocks is not None and not args.no_cascade and part == 0
    if cascade:  # the shared prefix once, then each sequence's own blocks
        n_pre = len(w.shared_blocks)
        assert (w.block_tables[:, :n_pre] == w.shared_blocks).all()
        prefix = to_dev(w.shared_blocks.astype(np.int32))
        own_tables = to_dev(np.ascontiguousarray(w.block_tables[:, n_pre:]).astype(np.int32))
        own_lens = to_dev((w.context_lens - n_pre * 16).astype(np.int32))
        ws_bytes = pkv.shared_prefix_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                     n_pre * 16)
    else:
        ws_bytes = pkv.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                              w.max_context_len, part)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # Evicting the caches: a read of 512 MB (twice the MI355X's 256 MB Infinity
    # Cache plus the L2s).  A read, not a write: writing the buffer would leave
    # the caches full of dirty lines whose write-back the next call would pay for.
    flush_buf = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) if args.cold else None
    flush = (lambda: flush_buf.sum()) if args.cold else None
    scale = float(w.scale)

    def write():
        if fp8:
            pkv.paged_kv_write_fp8(nk, nv, slots, kc, vc, ksc, vsc)
        else:
            pkv.paged_kv_write(nk, nv, slots, kc, vc)

    def decode():
        if fp8:
            pkv.paged_attn_decode_fp8(q, kc, vc, ksc, vsc, tables, lens, scale, out, max_context_len=w.max_context_len,
                                      partition_tokens=part, workspace=ws)
        elif cascade:
            pkv.paged_attn_decode_shared_prefix(q, kc, vc, prefix, own_tables, own_lens, scale, out, workspace=ws)
        else:
            pkv.paged_attn_decode(q, kc, vc, tables, lens, scale, out, max_context_len=w.max_context_len,
                                  partition_tokens=part, workspace=ws)

    verify = w.num_seqs == 0 and has_chunks  # chunk rows only: the verify pass, or the large prefill
    if verify:
        vws = torch.empty(max(1, pkv.spec_verify_workspace_bytes(w.num_chunks, w.q_chunk.shape[1], w.num_q_heads,
                                                                w.num_kv_heads, w.head_dim, w.chunk_tables.shape[1])),
                          dtype=torch.uint8, device=dev)

    elif has_chunks:
        pws = torch.empty(max(1, pkv.prefill_chunk_workspace_bytes(w.num_chunks, w.q_chunk.shape[1], w.num_q_heads,
                                                                  w.num_kv_heads, w.head_dim,
                                                                  w.chunk_tables.shape[1])),
                          dtype=torch.uint8, device=dev)

    def prefill():
        if verify and not prefill_only:
            pkv.paged_attn_spec_verify(qc, cstart, kc, vc, ctables, clens, scale, oc, workspace=vws)
        elif prefill_only:
            pkv.paged_attn_prefill_chunk_ws(qc, cstart, kc, vc, ctables, clens, scale, oc, workspace=vws)
        else:
            pkv.paged_attn_prefill_chunk_ws(qc, cstart, kc, vc, ctables, clens, scale, oc, workspace=pws)

    # Mixed step on two streams: the prefill chunks do not depend on the decode,
    # so after the cache write they run on a second stream (default priority)
    # beside it -- the decode is bound by HBM, the chunks by the matrix cores.
    two_streams = args.streams == 2 and w.num_seqs > 0 and has_chunks
    side = torch.cuda.Stream() if two_streams else None
    written = torch.cuda.Event() if two_streams else None

    def step():
        write()
        if two_streams:
            written.record()
            side.wait_event(written)
            decode()
            with torch.cuda.stream(side):
                prefill()
            torch.cuda.current_stream().wait_stream(side)
            return
        if w.num_seqs:
            decode()
        if has_chunks:
            prefill()

    for _ in range(args.warmup):
        if flush is not None:
            flush()
        step()
    torch.cuda.synchronize()

    def timed(fn, n):
        """n calls of fn back to back; HIP events around the region on the current stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            if flush is not None:
                flush()
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def per_call(fn, n, before=None):
        """n calls of fn, each bracketed by its own pair of HIP events (before() runs outside the pair)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            if before is not None:
                before()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) for e0, e1 in evs])

    def stats(ms):
        return {"mean": round(float(ms.mean()), 5), "p50": round(float(np.percentile(ms, 50)), 5),
                "p95": round(float(np.percentile(ms, 95)), 5), "p99": round(float(np.percentile(ms, 99)), 5),
                "min": round(float(ms.min()), 5), "max": round(float(ms.max()), 5), "samples": int(ms.size)}

    # the K timed steps
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        if flush is not None:
            flush()
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    # the parts of the step, each in a timed region of its own (events around
    # the region; with --cold the 512 MB overwrite before each call is included)
    write_ms = timed(write, K)
    dec_ms = timed(decode, K) if w.num_seqs else 0.0
    pre_ms = timed(prefill, K) if has_chunks else 0.0
    flush_ms = timed(lambda: None, K) if flush is not None else 0.0
    if flush is not None:  # the overwrite is not part of the calls
        write_ms, dec_ms, pre_ms = write_ms - flush_ms, dec_ms - flush_ms, (pre_ms - flush_ms if has_chunks else 0.0)
        ms_per_step = max(ms_per_step - flush_ms, 1e-6)

    # The attention call, call by call: with warm caches (back to back) and
    # with the last-level caches cold -- a 512 MB read (twice the MI355X's
    # 256 MB Infinity Cache) before every call, outside the call's own events.
    # The cold figure is the headline: it is bound by HBM alone, while warm
    # repeated calls can find part of the batch's K/V still in that cache.
    main_call = decode if w.num_seqs else prefill
    n_calls = max(50, K)
    warm_calls = per_call(main_call, n_calls)
    cold_calls = None
    buf = None
    if not args.no_cold_check:
        buf = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        evict = lambda: buf.sum()  # noqa: E731
        for _ in range(3):  # first touches of the new buffer
            evict()
            main_call()
        cold_calls = per_call(main_call, n_calls, before=evict)
    warm_region_ms = dec_ms if w.num_seqs else pre_ms

    eb = w.elem_bytes
    if verify:
        pb = accounting.prefill_bytes(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.num_kv_heads,
                                      w.head_dim, eb)
        kv_bytes = int(w.chunk_context_lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * 2 * eb
        dec = {"kv": kv_bytes, "total": pb}
        n_seq = w.num_chunks
    else:
        dec = accounting.decode_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 1 if fp8 else eb,
                                      block_tables=w.block_tables, dedupe_shared=(cfg == 4), q_bytes=eb,
                                      scale_bytes=4 if fp8 else 0)
        kv_bytes = dec["kv"]
        n_seq = w.num_seqs
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    seq_tok_s = n_seq / (ms_per_step * 1e-3)
    tr = TRAFFIC.get((w.name, args.kv_dtype))
    traffic = None
    if tr is not None and tr["sources_sha256"] == sources_sha256() and part == 0 and not args.cold and not verify:
        traffic = tr["read_bytes"] + tr["write_bytes"]
    head_ms = float(cold_calls.mean()) if cold_calls is not None else warm_region_ms
    if prefill_only:  # matrix-core bound: causal-pair FLOPs of the call against the dense bf16 peak
        fl = accounting.prefill_flops(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.head_dim)
        work, unit, peak, bound = fl, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma"
        rate = lambda ms: fl / (ms * 1e-3) / 1e12  # noqa: E731
    else:
        work, unit, peak, bound = dec["total"], "GB/s", HBM_PEAK_GBS, "hbm"
        rate = lambda ms: dec["total"] / (ms * 1e-3) / 1e9  # noqa: E731
    kernel = ("paged_attn_prefill_chunk_ws: prefill_mfma_kernel<chunk>" if prefill_only else
              ("paged_attn_spec_verify: decode_balanced_kernel<verify rows> + decode_balanced_merge_kernel"
               if verify_balanced(w) else
               "paged_attn_spec_verify: prefill_mfma_kernel<split> + prefill_split_merge_kernel") if verify else
              ("paged_attn_decode_shared_prefix: prefill_mfma_kernel<prefix> + prefix_merge_kernel + "
               "decode_balanced_kernel + decode_balanced_merge_kernel") if cascade else
              ("paged_attn_decode_fp8: decode_balanced_kernel<fp8> + decode_balanced_merge_kernel"
               if fp8 and part == 0 else
               "paged_attn_decode: decode_balanced_kernel + decode_balanced_merge_kernel"
               if part == 0 else "paged_attn_decode: decode_partition_kernel + decode_merge_kernel"))
    roofline = {"bound": bound, "achieved": round(rate(head_ms), 1), "peak": peak, "unit": unit,
                "frac": round(rate(head_ms) / peak, 4), "traffic": traffic,
                "llc": "cold" if cold_calls is not None else "warm",
                "kernel": kernel, "launch_ms_mean": round(head_ms, 5),
                "per_call_ms": stats(cold_calls) if cold_calls is not None else stats(warm_calls)}
    if prefill_only:
        roofline["algorithmic_flops_per_launch"] = fl
    else:
        roofline["algorithmic_bytes_per_launch"] = dec["total"]
        roofline["traffic_read_write_bytes"] = [tr["read_bytes"], tr["write_bytes"]] if traffic else None
    roofline_warm = {"launch_ms_mean": round(warm_region_ms, 5), "achieved": round(rate(warm_region_ms), 1),
                     "frac": round(rate(warm_region_ms) / peak, 4), "per_call_ms": stats(warm_calls),
                     "note": "back-to-back calls: the mean from events around the whole run of calls, the "
                             "percentiles from events around each call"}

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 kv, bf16 q/out" if fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "seed": w.seed, "num_seqs": n_seq,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": 16, "num_blocks": w.num_blocks,
                   "context_tokens": int((w.chunk_context_lens if verify else w.context_lens).sum()),
                   "max_context_len": w.max_context_len,
                   "split": "one workgroup per (chunk, kv head, 128-row tile)" if prefill_only else
                            ("balanced over 1024 wavefronts, heads x rows of a (sequence, kv head) as matrix-core "
                             "columns" if verify_balanced(w) else
                             "keys of each (sequence, kv head) cut into pieces" if w.num_chunks * w.num_kv_heads < 256
                             else "one workgroup per (sequence, kv head)") if verify else
                            f"fixed partitions of {part} tokens" if part else
                            (f"shared prefix of {len(w.shared_blocks) * 16} tokens attended once, then " if cascade
                             else "") +
                            f"balanced over {pkv.decode_split_waves(w.num_q_heads, w.num_kv_heads)} wavefronts",
                   "kv_bytes_per_step": kv_bytes, "llc": "cold (512 MB read before each step)" if args.cold else "warm",
                   "kv_cache": "E4M3 codes + float32 scale per (slot, kv head)" if fp8 else w.dtype,
                   "streams": 2 if two_streams else 1,
                   "layers_per_step": 1},
        "seq_tokens_per_s": round(seq_tok_s, 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "write_ms_mean": round(write_ms, 5),
        "decode_ms_mean": round(dec_ms, 5),
        "roofline": roofline,
        "roofline_llc_warm": roofline_warm,
    }
    if has_chunks:
        flops = accounting.prefill_flops(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.head_dim)
        pm = pre_ms
        res["prefill"] = {"ms_mean": round(pm, 5), "flops": flops,
                          "tflops": round(flops / (pm * 1e-3) / 1e12, 2),
                          "mfma_frac_of_bf16_peak": round(flops / (pm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    if w.num_seqs and not cascade and part == 0:
        # What this access pattern allows: the read probe loads every K/V row the
        # decode call reads, with its loads, over the same wavefront count, and
        # computes nothing (paged_kv_read_probe).
        # (an fp8 cache runs twice the bf16 count unless a wave takes four or eight heads at D = 128)
        gb = next(x for x in (8, 4, 2, 1) if (w.num_q_heads // w.num_kv_heads) % x == 0)
        fp8_twice = fp8 and not (gb in (4, 8) and w.head_dim == 128)
        waves = pkv.decode_split_waves(w.num_q_heads, w.num_kv_heads) * (2 if fp8_twice else 1)
        pwords = torch.empty(waves, dtype=torch.int32, device=dev)
        probe = (lambda: pkv.paged_kv_read_probe(kc, vc, tables, lens, waves, pwords, k_scale=ksc, v_scale=vsc)) \
            if fp8 else (lambda: pkv.paged_kv_read_probe(kc, vc, tables, lens, waves, pwords))
        for _ in range(3):
            probe()
        probe_warm = timed(probe, n_calls)
        probe_cold = per_call(probe, n_calls, before=evict) if buf is not None else None
        # the K/V rows it reads (an fp8 cache's codes; its scales are not read)
        pbytes = int(np.sum(w.context_lens, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * (1 if fp8 else eb)
        p_ms = float(probe_cold.mean()) if probe_cold is not None else probe_warm
        res["achievable"] = {
            "kernel": f"paged_kv_read_probe over {waves} wavefronts (the decode's K/V loads, no arithmetic)",
            "bytes_per_launch": pbytes, "llc": "cold" if probe_cold is not None else "warm",
            "launch_ms_mean": round(p_ms, 5), "gbs": round(pbytes / (p_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(pbytes / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "warm_launch_ms_mean": round(probe_warm, 5),
            "decode_over_probe": round(p_ms / head_ms, 4)}
    if buf is not None:
        del buf

    if args.copy_pairs and not verify and not fp8:
        # supplementary: copy-on-write block copies, cached blocks into blocks no table holds
        held = set(np.asarray(w.block_tables).ravel().tolist()) | set(np.asarray(w.chunk_tables).ravel().tolist())
        free = np.array([b for b in range(w.num_blocks) if b not in held], dtype=np.int32)
        n_pairs = min(args.copy_pairs, len(free))
        rng = np.random.default_rng(w.seed)
        src_blocks = to_dev(rng.choice(np.array(sorted(held), dtype=np.int32), n_pairs, replace=False))
        dst_blocks = to_dev(free[:n_pairs])
        copy_ms = timed(lambda: pkv.paged_kv_copy_blocks(src_blocks, dst_blocks, kc, vc), K)
        cb = accounting.copy_bytes(n_pairs, w.num_kv_heads, w.head_dim, eb)
        res["copy_blocks"] = {"pairs": n_pairs, "algorithmic_bytes": cb, "ms_mean": round(copy_ms, 5),
                              "gbs": round(cb / (copy_ms * 1e-3) / 1e9, 1),
                              "frac_of_hbm_peak": round(cb / (copy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if args.copy_probe_mb:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = {"read": n * 4, "write": n * 4}
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


_W = None  # the workload and its written cache, for the baseline's worker processes
_RK = _RV = None


def _oracle_item(s):
    import oracle
    w = _W
    if w.num_seqs == 0:
        oracle.prefill_chunk(w.q_chunk[s:s + 1], w.chunk_start[s:s + 1], _RK, _RV, w.chunk_tables[s:s + 1],
                             w.chunk_context_lens[s:s + 1], w.scale, w.dtype)
    else:
        oracle.decode(w.q[s:s + 1], _RK, _RV, w.block_tables[s:s + 1], w.context_lens[s:s + 1], w.scale, w.dtype)
    return s


def cpu_baseline(w, seconds):
    """The fp64 oracle (write + attention of the same step) timed on all of the host's cores.

    The oracle itself is unchanged: the cache write runs once, then the batch's
    sequences (or verify chunks) go to a pool of one worker process per core,
    each calling the oracle on one sequence with single-threaded BLAS; whole
    passes over the batch repeat until about `seconds` of wall time.  Called
    before anything touches the GPU, so the forked workers hold no GPU state.
    """
    import multiprocessing

    from threadpoolctl import threadpool_limits

    import oracle

    global _W, _RK, _RV
    cores = len(os.sched_getaffinity(0))
    verify = w.num_seqs == 0
    n_items = w.num_chunks if verify else w.num_seqs
    lens = w.chunk_context_lens if verify else w.context_lens
    passes = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        _W = w
        _RK, _RV = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
        with multiprocessing.get_context("fork").Pool(cores) as pool:
            while n_items and (passes == 0 or time.perf_counter() - t0 < seconds):
                list(pool.imap_unordered(_oracle_item, range(n_items)))
                passes += 1
        wall = time.perf_counter() - t0
    _W = _RK = _RV = None
    row = w.num_kv_heads * w.head_dim * 2 * w.elem_bytes
    tokens = passes * int(np.asarray(lens, dtype=np.int64).sum())
    what = "verify chunks" if verify else "decode"
    return {"value": round(tokens * row / wall / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seq_tokens_per_s": round(passes * n_items / wall, 2),
            "sample": f"fp64 numpy oracle, one process per core ({cores}): cache write of the step's "
                      f"{len(w.slot_mapping)} rows + {passes} passes of {what} over the batch's {n_items} "
                      f"sequences ({tokens} context tokens), {wall:.1f} s wall"}


if __name__ == "__main__":
    main()
