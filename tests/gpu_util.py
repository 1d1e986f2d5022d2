"""Helpers for the GPU tests: move seeded numpy inputs to the device and results back.

Only plumbing: bf16 data travels as raw uint16 bits, so the device receives
exactly the bits the oracle reads.
"""
import numpy as np

from workloads import synth


def torch():
    import torch as t
    return t


def device():
    t = torch()
    if not t.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return t.device("cuda:0")


def to_dev(arr, dtype: str):
    """numpy raw data (uint16 bf16 bits or float32, or int32) -> device tensor."""
    t = torch()
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.int32:
        return t.from_numpy(arr).to(device())
    if dtype == "bf16":
        return t.from_numpy(arr.view(np.int16)).view(t.bfloat16).to(device())
    return t.from_numpy(arr.astype(np.float32, copy=False)).to(device())


def bits(x) -> np.ndarray:
    """Device tensor -> numpy raw bits (uint16 for bf16, uint32 for float32)."""
    t = torch()
    x = x.detach().contiguous()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.view(t.int32).cpu().numpy().view(np.uint32)


def values(x) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = torch()
    if x.dtype == t.bfloat16:
        return synth.bf16_bits_to_f32(bits(x)).astype(np.float64)
    return x.detach().float().cpu().numpy().astype(np.float64)


def empty_like_q(shape, dtype: str, fill_nan=True):
    t = torch()
    td = t.bfloat16 if dtype == "bf16" else t.float32
    out = t.empty(shape, dtype=td, device=device())
    if fill_nan:
        out.fill_(float("nan"))
    return out


class DeviceWorkload:
    """A Workload's arrays on the device."""

    def __init__(self, w):
        self.w = w
        dt = w.dtype
        self.k_cache = to_dev(w.k_cache, dt)
        self.v_cache = to_dev(w.v_cache, dt)
        self.new_k = to_dev(w.new_k, dt)
        self.new_v = to_dev(w.new_v, dt)
        self.slots = to_dev(w.slot_mapping, dt)
        self.q = to_dev(w.q, dt)
        self.tables = to_dev(w.block_tables, dt)
        self.lens = to_dev(w.context_lens, dt)
        self.q_chunk = to_dev(w.q_chunk, dt)
        self.chunk_start = to_dev(w.chunk_start, dt)
        self.chunk_tables = to_dev(w.chunk_tables, dt)
        self.chunk_lens = to_dev(w.chunk_context_lens, dt)
