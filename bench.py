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
seq-tokens/s, the roofline of the decode call (its average duration from HIP
events around a second timed region of back-to-back decode calls on the
stream the library launches on; HBM traffic from rocprofv3 counters taken on
the same kernels) and the CPU oracle timed on the host as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cold] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV HBM GB/s (% of peak) + seq-tokens/s, 8B-shaped batch"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

# HBM traffic of one decode call, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch summed over the call's two
# kernels), scaled by what the same counters read for a device copy of 256 MiB
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Keyed by (workload, --kv-dtype).  Valid
# only for the decode kernel sources it was measured on: reported as null once
# their hash differs.
TRAFFIC = {
    ("llama3-8b-decode-bf16", "model"): {"read_bytes": 530040320, "write_bytes": 3422147,
                                        "sources_sha256": "2262b5bf93b717dec9a5f08df814efd21811532944d60e19fcd16b1bde5ecf7d"},
    ("llama3-8b-decode-bf16", "fp8"): {"read_bytes": 284962795, "write_bytes": 5462576,
                                      "sources_sha256": "2262b5bf93b717dec9a5f08df814efd21811532944d60e19fcd16b1bde5ecf7d"},
}
CSRC = os.path.join(ROOT, "paged_kv_cache_295_amd", "csrc")
DECODE_SOURCES = ("decode.hip", "pkv_device.hpp", "pkv_internal.hpp")


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
    p.add_argument("--cold", action="store_true", help="overwrite 512 MB before every step (LLC-cold timing)")
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

    pkv.load_library()
    dev = torch.device("cuda:0")
    cfg = WORKLOADS[args.workload]
    w = workloads.make(cfg)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.int32:
            return torch.from_numpy(a).to(dev)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    fp8 = args.kv_dtype == "fp8"
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
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) if args.cold else None
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
    prefill_only = cfg == "prefill-large"
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
            flush.zero_()
        step()
    torch.cuda.synchronize()

    def timed(fn, n):
        """n calls of fn back to back; HIP events around the region on the current stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            if flush is not None:
                flush.zero_()
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # the K timed steps
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        if flush is not None:
            flush.zero_()
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

    # The same attention call with the last-level caches cold: a 512 MB
    # overwrite (twice the MI355X's 256 MB Infinity Cache) before every call,
    # its own time subtracted.  Warm repeated calls can find part of the batch's
    # K/V still in that cache; this figure is the one bound by HBM alone.
    cold_ms = None
    main_call = decode if w.num_seqs else (prefill if verify else None)
    if main_call is not None and flush is None and not args.no_cold_check:
        buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

        def flushed():
            buf.zero_()
            main_call()
        for _ in range(3):  # first touches of the new buffer are not part of either region
            flushed()
        n_cold = max(10, K // 4)
        flush_only = timed(lambda: buf.zero_(), n_cold)
        cold_ms = timed(flushed, n_cold) - flush_only
        del buf

    eb = w.elem_bytes
    if verify:
        pb = accounting.prefill_bytes(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.num_kv_heads,
                                      w.head_dim, eb)
        kv_bytes = int(w.chunk_context_lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * 2 * eb
        dec = {"kv": kv_bytes, "total": pb}
        n_seq, launch_ms = w.num_chunks, pre_ms
    else:
        dec = accounting.decode_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 1 if fp8 else eb,
                                      block_tables=w.block_tables, dedupe_shared=(cfg == 4), q_bytes=eb,
                                      scale_bytes=4 if fp8 else 0)
        kv_bytes = dec["kv"]
        n_seq, launch_ms = w.num_seqs, dec_ms
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    seq_tok_s = n_seq / (ms_per_step * 1e-3)
    achieved = dec["total"] / (launch_ms * 1e-3) / 1e9 if launch_ms > 0 else 0.0
    tr = TRAFFIC.get((w.name, args.kv_dtype))
    traffic = None
    if tr is not None and tr["sources_sha256"] == sources_sha256() and part == 0 and not args.cold and not verify:
        traffic = tr["read_bytes"] + tr["write_bytes"]
    if prefill_only:  # matrix-core bound: causal-pair FLOPs of the call against the dense bf16 peak
        fl = accounting.prefill_flops(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.head_dim)
        tf = fl / (launch_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "paged_attn_prefill_chunk_ws: prefill_mfma_kernel<chunk>",
                    "algorithmic_flops_per_launch": fl, "launch_ms_mean": round(launch_ms, 5)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "paged_attn_spec_verify: prefill_mfma_kernel<split> + prefill_split_merge_kernel"
                    if verify else
                              ("paged_attn_decode_shared_prefix: prefill_mfma_kernel<prefix> + prefix_merge_kernel + "
                               "decode_balanced_kernel + decode_balanced_merge_kernel") if cascade else
                              ("paged_attn_decode_fp8: decode_balanced_kernel<fp8> + decode_balanced_merge_kernel"
                               if fp8 and part == 0 else
                               "paged_attn_decode: decode_balanced_kernel + decode_balanced_merge_kernel"
                               if part == 0 else "paged_attn_decode: decode_partition_kernel + decode_merge_kernel"),
                    "algorithmic_bytes_per_launch": dec["total"], "launch_ms_mean": round(launch_ms, 5),
                    "traffic_read_write_bytes": [tr["read_bytes"], tr["write_bytes"]] if traffic else None}

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
                            ("keys of each (sequence, kv head) cut into pieces" if w.num_chunks * w.num_kv_heads < 256
                             else "one workgroup per (sequence, kv head)") if verify else
                            f"fixed partitions of {part} tokens" if part else
                            (f"shared prefix of {len(w.shared_blocks) * 16} tokens attended once, then " if cascade
                             else "") +
                            f"balanced over {pkv.decode_split_waves(w.num_q_heads, w.num_kv_heads)} wavefronts",
                   "kv_bytes_per_step": kv_bytes, "llc": "cold (512 MB overwrite per step)" if args.cold else "warm",
                   "kv_cache": "E4M3 codes + float32 scale per (slot, kv head)" if fp8 else w.dtype,
                   "streams": 2 if two_streams else 1,
                   "layers_per_step": 1},
        "seq_tokens_per_s": round(seq_tok_s, 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "write_ms_mean": round(write_ms, 5),
        "decode_ms_mean": round(dec_ms, 5),
        "roofline": roofline,
        "roofline_llc_cold": None if cold_ms is None else {
            "launch_ms_mean": round(cold_ms, 5),
            "achieved": round(roofline["algorithmic_flops_per_launch"] / (cold_ms * 1e-3) / 1e12, 1) if prefill_only
            else round(dec["total"] / (cold_ms * 1e-3) / 1e9, 1),
            "frac": round(roofline["algorithmic_flops_per_launch"] / (cold_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
            if prefill_only else round(dec["total"] / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "the same call after a 512 MB overwrite of the caches, the overwrite's time subtracted"},
    }
    if has_chunks:
        flops = accounting.prefill_flops(w.chunk_start, w.chunk_context_lens, w.num_q_heads, w.head_dim)
        pm = pre_ms
        res["prefill"] = {"ms_mean": round(pm, 5), "flops": flops,
                          "tflops": round(flops / (pm * 1e-3) / 1e12, 2),
                          "mfma_frac_of_bf16_peak": round(flops / (pm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

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
    if not args.no_cpu_baseline and not fp8 and not prefill_only:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, cfg)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, seconds, cfg):
    """The fp64 oracle (write + attention of the same step) timed on one host thread."""
    from threadpoolctl import threadpool_limits

    import oracle

    # sample: whole sequences (decode) or chunks (verify rows) of the batch, in
    # order, until ~`seconds` of CPU work
    verify = w.num_seqs == 0
    n_items = w.num_chunks if verify else w.num_seqs
    lens = w.chunk_context_lens if verify else w.context_lens
    done_seqs, done_tokens, t_total = 0, 0, 0.0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
        t_total += time.perf_counter() - t0
        while n_items and t_total < seconds:
            for s in range(n_items):
                t0 = time.perf_counter()
                if verify:
                    oracle.prefill_chunk(w.q_chunk[s:s + 1], w.chunk_start[s:s + 1], rk, rv, w.chunk_tables[s:s + 1],
                                         w.chunk_context_lens[s:s + 1], w.scale, w.dtype)
                else:
                    oracle.decode(w.q[s:s + 1], rk, rv, w.block_tables[s:s + 1], w.context_lens[s:s + 1], w.scale,
                                  w.dtype)
                t_total += time.perf_counter() - t0
                done_seqs += 1
                done_tokens += int(lens[s])
                if t_total >= seconds:
                    break
    row = w.num_kv_heads * w.head_dim * 2 * w.elem_bytes
    what = "verify chunks" if verify else "decode"
    return {"value": round(done_tokens * row / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seq_tokens_per_s": round(done_seqs / t_total, 2),
            "sample": f"fp64 numpy oracle, one thread: cache write of the step's {len(w.slot_mapping)} rows + "
                      f"{what} of {done_seqs} sequences taken in batch order ({done_tokens} context tokens), "
                      f"{t_total:.1f} s"}


if __name__ == "__main__":
    main()
