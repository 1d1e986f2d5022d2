"""Oracle for the fp8-quantised KV cache (float64 / float32 numpy, CPU).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

"Part 47 | Inference basics: KV Cache, batching, sampling" (chengxuchu.com),
section 2.4: when the cache outgrows memory a server may keep it quantised.
The page fixes no format, so the readings here are:

* Codes: the OCP 8-bit floating-point E4M3 format -- sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals
  m / 8 * 2^-6; no infinities; exponent 15 with mantissa 7 is NaN; the
  largest finite magnitude is 448.
* One float32 scale per (cache slot, kv head): the row of head_dim values a
  token writes for one kv head is stored as codes c_d with
  x_d ~ value(c_d) * scale.  A write never touches another slot's codes or
  scale, so blocks filled one token at a time never need requantising.
* The integer decisions are taken in float32, step by step:
      amax  = max_d |x_d|                    (exact)
      scale = fl32(amax / 448)
      inv   = fl32(448 / amax), 0 when amax == 0
      y_d   = clamp(fl32(x_d * inv), -448, 448)
      c_d   = the E4M3 code nearest to y_d, ties to the even code (mantissa
              bit 0 clear)
  so the element of largest magnitude always becomes +-448.
* Attention over the quantised cache is the plain attention of the other
  oracle module applied to the dequantised values value(c) * scale (exact in
  float64).
"""
from __future__ import annotations

import numpy as np

from .paged_attention import BLOCK_SIZE, attend, exact_scale, kv_head_of, to_f64

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (NaN for the two NaN codes), from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code to each float32 y with |y| <= 448 (ties to the even code).

    Brute force over the 127 finite non-negative codes; the sign is the input's
    sign bit (so -0.0 gives 0x80).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64)).reshape(-1)
    if np.isnan(a).any() or (a > E4M3_MAX).any():
        raise ValueError("e4m3_encode takes finite values of magnitude <= 448")
    pos = E4M3_TABLE[:0x7F]  # codes 0x00 .. 0x7E, increasing
    out = np.empty(a.shape, dtype=np.uint8)
    for i0 in range(0, a.size, 1 << 16):
        v = a[i0:i0 + (1 << 16), None]
        d = np.abs(pos[None, :] - v)
        lo = np.argmin(d, axis=1)  # the lower of two equally near codes
        hi = np.minimum(lo + 1, 0x7E)
        r = np.arange(len(lo))
        tie = (hi != lo) & (d[r, hi] == d[r, lo])
        out[i0:i0 + len(lo)] = np.where(tie & (lo % 2 == 1), hi, lo)
    sign = (np.signbit(y).reshape(-1)).astype(np.uint8) << 7
    return (out | sign).reshape(y.shape)


def quantize_row(x) -> tuple:
    """(codes uint8 [D], scale float32) of one row of float32 values, as in the module header."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    f448 = np.float32(E4M3_MAX)
    scale = np.float32(amax / f448)
    inv = np.float32(f448 / amax) if amax != 0 else np.float32(0)
    y = np.clip(x * inv, -f448, f448).astype(np.float32)
    return e4m3_encode(y), scale


def kv_write_fp8(k_cache, v_cache, k_scale, v_scale, new_k, new_v, slot_mapping, in_dtype="bf16"):
    """Quantise and store row i of new_k / new_v ([T, Hkv, D], bf16 bits or float32) at slot_mapping[i].

    Caches are uint8 [NB, Hkv, 16, D], scales float32 [NB, Hkv, 16]; returns
    new copies.  A negative slot, or one past the pool, skips its row.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks, vs = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    nk = to_f64(new_k, in_dtype).astype(np.float32)  # exact: bf16 / float32 values
    nv = to_f64(new_v, in_dtype).astype(np.float32)
    nb = kc.shape[0]
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= nb * BLOCK_SIZE:
            continue
        b, o = s // BLOCK_SIZE, s % BLOCK_SIZE
        for g in range(kc.shape[1]):
            kc[b, g, o], ks[b, g, o] = quantize_row(nk[i, g])
            vc[b, g, o], vs[b, g, o] = quantize_row(nv[i, g])
    return kc, vc, ks, vs


def dequantize(cache, scale) -> np.ndarray:
    """float64 values value(code) * scale of a uint8 cache [NB, Hkv, 16, D] with scales [NB, Hkv, 16]."""
    return E4M3_TABLE[np.asarray(cache, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)[..., None]


def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, q_dtype="bf16"):
    """Decode attention (one query per sequence) over the dequantised fp8 cache; float64 [B, Hq, D]."""
    q64 = to_f64(q, q_dtype)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    sigma = exact_scale(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        nb = -(-L // BLOCK_SIZE)
        ids = np.asarray(block_tables[s][:nb], dtype=np.int64)
        K = dequantize(k_cache[ids], k_scale[ids])  # [nb, Hkv, 16, D]
        V = dequantize(v_cache[ids], v_scale[ids])
        K = K.transpose(0, 2, 1, 3).reshape(nb * BLOCK_SIZE, Hkv, D)[:L]
        V = V.transpose(0, 2, 1, 3).reshape(nb * BLOCK_SIZE, Hkv, D)[:L]
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            out[s, heads] = attend(q64[s, heads], K[:, g], V[:, g], sigma)
    return out
