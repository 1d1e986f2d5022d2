"""Attention over a paged KV cache on AMD Instinct MI355X (gfx950).

Thin ctypes binding of libpagedkv.so (include/pagedkv.h).  It only marshals
arguments -- tensor pointers, sizes read from tensor shapes, the current HIP
stream -- and raises PagedKVError on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback, so a
missing library is an error.

PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PagedKVError", "load_library", "paged_kv_write", "paged_attn_decode", "paged_attn_prefill_chunk",
    "decode_workspace_bytes", "decode_split_waves", "library_path", "BLOCK_SIZE",
    "paged_attn_decode_shared_prefix", "shared_prefix_workspace_bytes", "paged_kv_copy_blocks", "BlockPool",
    "paged_kv_write_fp8", "paged_attn_decode_fp8", "paged_kv_copy_blocks_fp8",
    "paged_attn_spec_verify", "spec_verify_workspace_bytes", "paged_attn_prefill_chunk_ws",
    "prefill_chunk_workspace_bytes", "paged_attn_lse_merge", "paged_attn_decode_noalloc", "noalloc_scratch_bytes",
    "paged_kv_read_probe",
]

BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpagedkv.so"
_lib = None

PKV_DTYPE_F32 = 0
PKV_DTYPE_BF16 = 1
PKV_DTYPE_FP8_E4M3 = 2


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib.pkv_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("PAGEDKV_LIB", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libpagedkv.so (built in-tree by paged_kv_cache_295_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_295_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    cdp = ctypes.POINTER(CacheDesc)
    lib.paged_kv_write.argtypes = [vp, vp, vp, i64, vp, vp, cdp, vp]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_kv_copy_blocks.argtypes = [vp, vp, cdp, vp, vp, i64, vp]
    lib.paged_kv_copy_blocks.restype = ctypes.c_int
    lib.paged_attn_decode_split_waves.argtypes = [i32, i32]
    lib.paged_attn_decode_split_waves.restype = i32
    lib.paged_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attn_decode_workspace_bytes.restype = sz
    lib.paged_attn_decode.argtypes = [vp, i32, i32, vp, vp, cdp, vp, i32, vp, i32, f32, vp, i32, vp, sz, vp]
    lib.paged_attn_decode.restype = ctypes.c_int
    lib.paged_attn_decode_shared_prefix_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.paged_attn_decode_shared_prefix_workspace_bytes.restype = sz
    lib.paged_attn_decode_shared_prefix.argtypes = [vp, i32, i32, vp, vp, cdp, vp, i32, vp, i32, vp, f32, vp, vp, sz,
                                                    vp]
    lib.paged_attn_decode_shared_prefix.restype = ctypes.c_int
    fp = ctypes.c_void_p
    lib.paged_kv_write_fp8.argtypes = [vp, vp, i32, vp, i64, vp, vp, fp, fp, cdp, vp]
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    lib.paged_attn_decode_fp8.argtypes = [vp, i32, i32, vp, vp, fp, fp, cdp, vp, i32, vp, i32, f32, vp, i32, vp, sz,
                                          vp]
    lib.paged_attn_decode_fp8.restype = ctypes.c_int
    lib.paged_kv_copy_blocks_fp8.argtypes = [vp, vp, fp, fp, cdp, vp, vp, i64, vp]
    lib.paged_kv_copy_blocks_fp8.restype = ctypes.c_int
    lib.paged_attn_prefill_chunk.argtypes = [vp, i32, i32, i32, vp, vp, vp, cdp, vp, i32, vp, f32, vp, vp]
    lib.paged_attn_prefill_chunk.restype = ctypes.c_int
    ip = ctypes.POINTER(i32)
    lib.paged_block_fork.argtypes = [ip, i32, ip, ip, i32]
    lib.paged_block_fork.restype = ctypes.c_int
    lib.paged_block_append_slot.argtypes = [ip, i32, i32, ip, i32, ip, ip, ip, ip, ip, ip]
    lib.paged_block_append_slot.restype = ctypes.c_int
    lib.paged_block_release.argtypes = [ip, i32, ip, i32, ip, ip]
    lib.paged_block_release.restype = ctypes.c_int
    lib.paged_attn_prefill_chunk_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attn_prefill_chunk_workspace_bytes.restype = sz
    lib.paged_attn_prefill_chunk_ws.argtypes = [vp, i32, i32, i32, vp, vp, vp, cdp, vp, i32, vp, f32, vp, vp, sz, vp]
    lib.paged_attn_prefill_chunk_ws.restype = ctypes.c_int
    lib.paged_attn_spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attn_spec_verify_workspace_bytes.restype = sz
    lib.paged_attn_spec_verify.argtypes = [vp, i32, i32, i32, vp, vp, vp, cdp, vp, i32, vp, f32, vp, vp, sz, vp]
    lib.paged_attn_spec_verify.restype = ctypes.c_int
    lib.paged_attn_decode_noalloc.argtypes = [vp, i32, i32, vp, vp, cdp, vp, i32, vp, i32, f32, vp, i32, vp]
    lib.paged_attn_decode_noalloc.restype = ctypes.c_int
    lib.paged_attn_decode_noalloc_scratch_bytes.argtypes = []
    lib.paged_attn_decode_noalloc_scratch_bytes.restype = sz
    lib.paged_kv_read_probe.argtypes = [vp, vp, cdp, vp, i32, i32, vp, i32, vp, vp]
    lib.paged_kv_read_probe.restype = ctypes.c_int
    lib.paged_attn_lse_merge.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp]
    lib.paged_attn_lse_merge.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_abi_version.argtypes = []
    lib.pkv_abi_version.restype = i32
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PKV_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _on_one_gpu(*tensors):
    """Every tensor argument must live on one GPU: the kernels dereference these
    addresses, and a host tensor's address read on the GPU is a wild pointer.
    Checked before the library is called, so a misplaced tensor never reaches a kernel."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"tensor arguments must be on the GPU, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensor arguments must be on one GPU, got {dev} and {t.device}")
    return dev


def _ptr(t) -> int:
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _i32(t, name):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t)


def _same_dtype(*ts):
    d = ts[0].dtype
    for t in ts[1:]:
        if t.dtype != d:
            raise TypeError("q/out/k/v/caches must share one dtype")


def _stream(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _cache_desc(k_cache) -> CacheDesc:
    if k_cache.dim() != 4 or k_cache.shape[2] != BLOCK_SIZE:
        raise ValueError("caches must be [num_blocks, num_kv_heads, 16, head_dim]")
    nb, hkv, _, d = k_cache.shape
    return CacheDesc(nb, BLOCK_SIZE, hkv, d, _dtype_code(k_cache))


def _fp8_desc(k_cache, v_cache, k_scale, v_scale) -> CacheDesc:
    """Descriptor of an E4M3 cache (uint8 or float8_e4m3fn tensors) with float32 scales [NB, Hkv, 16]."""
    torch = _torch()
    fp8_types = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if k_cache.dtype not in fp8_types or v_cache.dtype != k_cache.dtype:
        raise TypeError("fp8 caches must be uint8 (E4M3 codes) or float8_e4m3fn")
    if k_cache.dim() != 4 or k_cache.shape[2] != BLOCK_SIZE or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, num_kv_heads, 16, head_dim]")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or \
            k_scale.shape != k_cache.shape[:3] or v_scale.shape != k_cache.shape[:3]:
        raise ValueError("scales must be float32 [num_blocks, num_kv_heads, 16]")
    nb, hkv, _, d = k_cache.shape
    return CacheDesc(nb, BLOCK_SIZE, hkv, d, PKV_DTYPE_FP8_E4M3)


def _check(status: int, what: str):
    if status != 0:
        raise PagedKVError(status, what)


def paged_kv_write(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """Store row i of k/v ([T, Hkv, D]) at cache slot slot_mapping[i] (int32 [T])."""
    _on_one_gpu(k, v, slot_mapping, k_cache, v_cache)
    lib = load_library()
    _same_dtype(k, v, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    if k.shape[1:] != (desc.num_kv_heads, desc.head_dim) or v.shape != k.shape or v_cache.shape != k_cache.shape:
        raise ValueError("k, v must be [T, num_kv_heads, head_dim] matching the caches")
    if slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be [T]")
    st = lib.paged_kv_write(_ptr(k), _ptr(v), _i32(slot_mapping, "slot_mapping"), k.shape[0], _ptr(k_cache),
                            _ptr(v_cache), ctypes.byref(desc), _stream(stream))
    _check(st, "paged_kv_write")


def paged_kv_copy_blocks(src_blocks, dst_blocks, k_cache, v_cache, stream=None):
    """Copy block src_blocks[i] to block dst_blocks[i] in both caches (int32 [N] each)."""
    _on_one_gpu(src_blocks, dst_blocks, k_cache, v_cache)
    lib = load_library()
    _same_dtype(k_cache, v_cache)
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if src_blocks.dim() != 1 or dst_blocks.shape != src_blocks.shape:
        raise ValueError("src_blocks and dst_blocks must be [N]")
    st = lib.paged_kv_copy_blocks(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _i32(src_blocks, "src_blocks"),
                                  _i32(dst_blocks, "dst_blocks"), src_blocks.shape[0], _stream(stream))
    _check(st, "paged_kv_copy_blocks")


def paged_kv_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream=None):
    """Quantise row i of k/v ([T, Hkv, D], bf16 or f32) into E4M3 codes + scales at slot slot_mapping[i]."""
    _on_one_gpu(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale)
    lib = load_library()
    desc = _fp8_desc(k_cache, v_cache, k_scale, v_scale)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if k.shape[1:] != (desc.num_kv_heads, desc.head_dim) or v.shape != k.shape:
        raise ValueError("k, v must be [T, num_kv_heads, head_dim] matching the caches")
    if slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be [T]")
    st = lib.paged_kv_write_fp8(_ptr(k), _ptr(v), _dtype_code(k), _i32(slot_mapping, "slot_mapping"), k.shape[0],
                                _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), ctypes.byref(desc),
                                _stream(stream))
    _check(st, "paged_kv_write_fp8")


def paged_kv_copy_blocks_fp8(src_blocks, dst_blocks, k_cache, v_cache, k_scale, v_scale, stream=None):
    """Copy block src_blocks[i] to dst_blocks[i]: codes of both caches and their scales."""
    _on_one_gpu(src_blocks, dst_blocks, k_cache, v_cache, k_scale, v_scale)
    lib = load_library()
    desc = _fp8_desc(k_cache, v_cache, k_scale, v_scale)
    if src_blocks.dim() != 1 or dst_blocks.shape != src_blocks.shape:
        raise ValueError("src_blocks and dst_blocks must be [N]")
    st = lib.paged_kv_copy_blocks_fp8(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                      ctypes.byref(desc), _i32(src_blocks, "src_blocks"),
                                      _i32(dst_blocks, "dst_blocks"), src_blocks.shape[0], _stream(stream))
    _check(st, "paged_kv_copy_blocks_fp8")


def decode_split_waves(num_q_heads: int, num_kv_heads: int) -> int:
    """Wavefronts the balanced decode split (partition_tokens=0) divides a batch's work over."""
    return int(load_library().paged_attn_decode_split_waves(num_q_heads, num_kv_heads))


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                           partition_tokens=0) -> int:
    return int(load_library().paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                                max_context_len, partition_tokens))


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                      partition_tokens=0, workspace=None, stream=None):
    """out[s, h] = softmax(scale q[s, h] K_s^T) V_s over the first context_lens[s] cached tokens.

    max_context_len: host-side bound on context_lens (defaults to the block
    table's capacity, 16 * block_tables.shape[1]).  partition_tokens: 0 for the
    balanced split, else fixed partitions of that many tokens.  workspace:
    optional uint8 device tensor (16-byte aligned, as torch allocations are);
    allocated here when needed and not given.
    """
    _on_one_gpu(q, k_cache, v_cache, block_tables, context_lens, out, workspace)
    lib = load_library()
    _same_dtype(q, out, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    B, hq, d = q.shape
    if out.shape != q.shape or d != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables [B, max_blocks], context_lens [B]")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * BLOCK_SIZE
    need = decode_workspace_bytes(B, hq, desc.num_kv_heads, d, max_context_len, partition_tokens)
    if need and workspace is None:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.paged_attn_decode(_ptr(q), B, hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                               _i32(block_tables, "block_tables"), max_blocks, _i32(context_lens, "context_lens"),
                               int(max_context_len), float(scale), _ptr(out), int(partition_tokens), ws_ptr,
                               ws_bytes, _stream(stream))
    _check(st, "paged_attn_decode")
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of the partial-state buffer paged_attn_decode_noalloc keeps on each GPU."""
    return int(load_library().paged_attn_decode_noalloc_scratch_bytes())


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                              partition_tokens=0, stream=None):
    """paged_attn_decode without a workspace: the partial states live in the library's own buffer
    (noalloc_scratch_bytes() per GPU), so the call allocates nothing.  Calls that may overlap on one
    GPU share that buffer and race."""
    _on_one_gpu(q, k_cache, v_cache, block_tables, context_lens, out)
    lib = load_library()
    _same_dtype(q, out, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    B, hq, d = q.shape
    if out.shape != q.shape or d != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables [B, max_blocks], context_lens [B]")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * BLOCK_SIZE
    torch = _torch()
    with torch.cuda.device(q.device):  # the library finds its buffer on the current GPU
        st = lib.paged_attn_decode_noalloc(_ptr(q), B, hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                                           _i32(block_tables, "block_tables"), max_blocks,
                                           _i32(context_lens, "context_lens"), int(max_context_len), float(scale),
                                           _ptr(out), int(partition_tokens), _stream(stream))
    _check(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, out,
                          max_context_len=None, partition_tokens=0, workspace=None, stream=None):
    """paged_attn_decode over an E4M3 cache with per-(slot, kv head) scales; q and out bfloat16."""
    _on_one_gpu(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out, workspace)
    lib = load_library()
    torch = _torch()
    desc = _fp8_desc(k_cache, v_cache, k_scale, v_scale)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("q and out must be bfloat16")
    B, hq, d = q.shape
    if out.shape != q.shape or d != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables [B, max_blocks], context_lens [B]")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * BLOCK_SIZE
    need = decode_workspace_bytes(B, hq, desc.num_kv_heads, d, max_context_len, partition_tokens)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.paged_attn_decode_fp8(_ptr(q), B, hq, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                   ctypes.byref(desc), _i32(block_tables, "block_tables"), max_blocks,
                                   _i32(context_lens, "context_lens"), int(max_context_len), float(scale), _ptr(out),
                                   int(partition_tokens), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "paged_attn_decode_fp8")
    return out


def shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, prefix_len) -> int:
    return int(load_library().paged_attn_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                                              head_dim, prefix_len))


def paged_attn_decode_shared_prefix(q, k_cache, v_cache, prefix_blocks, block_tables, context_lens, scale, out,
                                    workspace=None, stream=None):
    """Decode for sequences that share the prefix held in prefix_blocks (int32 [P]; P*16 tokens):
    sequence s attends to the prefix and then to its own context_lens[s] tokens in block_tables[s]."""
    _on_one_gpu(q, k_cache, v_cache, prefix_blocks, block_tables, context_lens, out, workspace)
    lib = load_library()
    _same_dtype(q, out, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    B, hq, d = q.shape
    if out.shape != q.shape or d != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables [B, max_blocks], context_lens [B]")
    if prefix_blocks.dim() != 1:
        raise ValueError("prefix_blocks [num_prefix_blocks]")
    prefix_len = prefix_blocks.shape[0] * BLOCK_SIZE
    need = shared_prefix_workspace_bytes(B, hq, desc.num_kv_heads, d, prefix_len)
    if workspace is None:
        workspace = _torch().empty(max(need, 1), dtype=_torch().uint8, device=q.device)
    pb = _i32(prefix_blocks, "prefix_blocks") if prefix_len else None
    st = lib.paged_attn_decode_shared_prefix(_ptr(q), B, hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), pb,
                                             prefix_len, _i32(block_tables, "block_tables"), block_tables.shape[1],
                                             _i32(context_lens, "context_lens"), float(scale), _ptr(out),
                                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream))
    _check(st, "paged_attn_decode_shared_prefix")
    return out


def paged_attn_prefill_chunk(q_chunk, chunk_start, k_cache, v_cache, block_tables, context_lens, scale, out,
                             stream=None):
    """Causal attention of each chunk's rows (q_chunk [Nc, Cmax, Hq, D]) over its cached context."""
    _on_one_gpu(q_chunk, chunk_start, k_cache, v_cache, block_tables, context_lens, out)
    lib = load_library()
    _same_dtype(q_chunk, out, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    nc, cmax, hq, d = q_chunk.shape
    if out.shape != q_chunk.shape or d != desc.head_dim:
        raise ValueError("q_chunk/out must be [Nc, Cmax, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != nc or chunk_start.shape != (nc,) \
            or context_lens.shape != (nc,):
        raise ValueError("block_tables [Nc, max_blocks], chunk_start [Nc], context_lens [Nc]")
    st = lib.paged_attn_prefill_chunk(_ptr(q_chunk), nc, cmax, hq, _i32(chunk_start, "chunk_start"),
                                      _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                                      _i32(block_tables, "block_tables"), block_tables.shape[1],
                                      _i32(context_lens, "context_lens"), float(scale), _ptr(out),
                                      _stream(stream))
    _check(st, "paged_attn_prefill_chunk")
    return out


class BlockPool:
    """Host block bookkeeping for copy-on-write sharing (paged_block_* calls).

    Holds the per-block holder counts and the free-list stack as int32 numpy
    arrays; block tables are int32 numpy arrays the caller owns.  All decisions
    are the library's; this class only passes the arrays.
    """

    def __init__(self, num_blocks: int):
        import numpy as np
        self.num_blocks = int(num_blocks)
        self.ref_counts = np.zeros(self.num_blocks, dtype=np.int32)
        # popped from the end: block 0 first
        self.free_list = np.arange(self.num_blocks - 1, -1, -1, dtype=np.int32)
        self._free_count = ctypes.c_int32(self.num_blocks)

    @property
    def free_count(self) -> int:
        return int(self._free_count.value)

    @staticmethod
    def _p(a, name):
        import numpy as np
        if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
            raise TypeError(f"{name} must be a contiguous int32 numpy array")
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def fork(self, parent_table, num_table_blocks: int, child_table):
        """child_table[:n] = parent_table[:n]; each shared block gains a holder."""
        lib = load_library()
        _check(lib.paged_block_fork(self._p(parent_table, "parent_table"), int(num_table_blocks),
                                    self._p(child_table, "child_table"), self._p(self.ref_counts, "ref_counts"),
                                    self.num_blocks), "paged_block_fork")

    def append_slot(self, table, context_len: int):
        """Slot of the token at position context_len; (src, dst) block copy to run first, or None."""
        lib = load_library()
        slot, src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.paged_block_append_slot(self._p(table, "table"), int(table.shape[-1]), int(context_len),
                                           self._p(self.ref_counts, "ref_counts"), self.num_blocks,
                                           self._p(self.free_list, "free_list"), ctypes.byref(self._free_count),
                                           ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst), ctypes.byref(n)),
               "paged_block_append_slot")
        return int(slot.value), ((int(src.value), int(dst.value)) if n.value else None)

    def release(self, table, num_table_blocks: int):
        """Each of the table's first num_table_blocks blocks loses a holder; unheld blocks are freed."""
        lib = load_library()
        _check(lib.paged_block_release(self._p(table, "table"), int(num_table_blocks),
                                       self._p(self.ref_counts, "ref_counts"), self.num_blocks,
                                       self._p(self.free_list, "free_list"), ctypes.byref(self._free_count)),
               "paged_block_release")


def prefill_chunk_workspace_bytes(num_chunks, chunk_len_max, num_q_heads, num_kv_heads, head_dim,
                                  max_blocks_per_seq) -> int:
    return int(load_library().paged_attn_prefill_chunk_workspace_bytes(num_chunks, chunk_len_max, num_q_heads,
                                                                       num_kv_heads, head_dim, max_blocks_per_seq))


def spec_verify_workspace_bytes(num_seqs, rows_max, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq) -> int:
    return int(load_library().paged_attn_spec_verify_workspace_bytes(num_seqs, rows_max, num_q_heads, num_kv_heads,
                                                                     head_dim, max_blocks_per_seq))


def _chunks_with_workspace(fn, size_fn, what, q, starts, k_cache, v_cache, block_tables, context_lens, scale, out,
                           workspace, stream):
    _on_one_gpu(q, starts, k_cache, v_cache, block_tables, context_lens, out, workspace)
    lib = load_library()
    torch = _torch()
    _same_dtype(q, out, k_cache, v_cache)
    desc = _cache_desc(k_cache)
    nb_, rows, hq, d = q.shape
    if out.shape != q.shape or d != desc.head_dim:
        raise ValueError("q/out must be [B, rows, Hq, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != nb_ or starts.shape != (nb_,) \
            or context_lens.shape != (nb_,):
        raise ValueError("block_tables [B, max_blocks], starts [B], context_lens [B]")
    need = size_fn(nb_, rows, hq, desc.num_kv_heads, d, block_tables.shape[1])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = getattr(lib, fn)(_ptr(q), nb_, rows, hq, _i32(starts, "starts"), _ptr(k_cache), _ptr(v_cache),
                          ctypes.byref(desc), _i32(block_tables, "block_tables"), block_tables.shape[1],
                          _i32(context_lens, "context_lens"), float(scale), _ptr(out), ws_ptr, ws_bytes,
                          _stream(stream))
    _check(st, what)
    return out


def paged_attn_prefill_chunk_ws(q_chunk, chunk_start, k_cache, v_cache, block_tables, context_lens, scale, out,
                                workspace=None, stream=None):
    """paged_attn_prefill_chunk with a workspace, which lets the keys of long row tiles be split over the GPU."""
    return _chunks_with_workspace("paged_attn_prefill_chunk_ws", prefill_chunk_workspace_bytes,
                                  "paged_attn_prefill_chunk_ws", q_chunk, chunk_start, k_cache, v_cache,
                                  block_tables, context_lens, scale, out, workspace, stream)


def paged_attn_spec_verify(q, row_start, k_cache, v_cache, block_tables, context_lens, scale, out, workspace=None,
                           stream=None):
    """Verify pass of speculative decoding: q [B, R, Hq, D] holds each sequence's new rows
    (last accepted token + drafts) at positions row_start[s] + i; causal attention over the cache."""
    return _chunks_with_workspace("paged_attn_spec_verify", spec_verify_workspace_bytes, "paged_attn_spec_verify",
                                  q, row_start, k_cache, v_cache, block_tables, context_lens, scale, out, workspace,
                                  stream)


def paged_attn_lse_merge(part_o, part_ml, out, stream=None):
    """Log-sum-exp merge of split-context partials: part_o float32 [R, P, D] (unnormalised
    outputs), part_ml float32 [R, P, 2] ((max in log2 units, sum of 2^(y - max))), out [R, D]
    float32 or bfloat16 = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p."""
    _on_one_gpu(part_o, part_ml, out)
    lib = load_library()
    torch = _torch()
    if part_o.dtype != torch.float32 or part_ml.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if part_o.dim() != 3 or part_ml.shape != part_o.shape[:2] + (2,) or out.shape != (part_o.shape[0], part_o.shape[2]):
        raise ValueError("part_o [R, P, D], part_ml [R, P, 2], out [R, D]")
    R, P, D = part_o.shape
    st = lib.paged_attn_lse_merge(_ptr(part_o), _ptr(part_ml), R, P, D, _dtype_code(out), _ptr(out), _stream(stream))
    _check(st, "paged_attn_lse_merge")
    return out


def paged_kv_read_probe(k_cache, v_cache, block_tables, context_lens, num_waves, out_words=None, stream=None,
                        k_scale=None, v_scale=None):
    """Measurement aid: read the K/V rows a decode over this batch reads, with its loads, over num_waves
    wavefronts; returns out_words (uint32-valued int32 [num_waves]), wavefront w's XOR of the words it read.
    fp8 caches pass their scales only to identify the cache (the scales are not read)."""
    torch = _torch()
    if out_words is None:
        out_words = torch.empty(num_waves, dtype=torch.int32, device=k_cache.device)
    _on_one_gpu(k_cache, v_cache, block_tables, context_lens, out_words)
    lib = load_library()
    desc = _fp8_desc(k_cache, v_cache, k_scale, v_scale) if k_scale is not None else _cache_desc(k_cache)
    if block_tables.dim() != 2 or context_lens.shape != (block_tables.shape[0],) or out_words.shape != (num_waves,):
        raise ValueError("block_tables [B, max_blocks], context_lens [B], out_words [num_waves]")
    st = lib.paged_kv_read_probe(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _i32(block_tables, "block_tables"),
                                 block_tables.shape[0], block_tables.shape[1], _i32(context_lens, "context_lens"),
                                 int(num_waves), _i32(out_words, "out_words"), _stream(stream))
    _check(st, "paged_kv_read_probe")
    return out_words
