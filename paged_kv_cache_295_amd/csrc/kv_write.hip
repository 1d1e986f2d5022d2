// Cache write: scatter each new token's K and V rows into its block slot.
//
// "Part 47 | Inference basics: KV Cache, batching, sampling" (chengxuchu.com),
// section 2.2: the new K/V are written at a given position of preallocated
// pages (no reallocation).  Slot s names block s / 16, offset s % 16; the
// cache layout [num_blocks][num_kv_heads][16][head_dim] puts one head's row of
// a slot at a contiguous head_dim run.
//
// One workgroup per new token: its threads copy the token's K and V rows in
// 16-byte chunks (num_kv_heads * head_dim * elem / 16 chunks per row, 128 for
// bf16 8 x 128).  A raw copy of the bits: bit-exact by construction.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

template <int kChunksPerHead>
__global__ __launch_bounds__(128) void kv_write_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                       const int32_t* __restrict__ slots, int64_t num_tokens,
                                                       uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                       int32_t num_blocks, int32_t num_kv_heads) {
  const int64_t row_chunks = (int64_t)num_kv_heads * kChunksPerHead;
  for (int64_t row = blockIdx.x; row < num_tokens; row += gridDim.x) {
    const int32_t slot = slots[row];
    if (slot < 0 || slot >= num_blocks * kBlock) continue;  // skipped rows
    const int64_t blk = slot >> 4;
    const int64_t off = slot & 15;
    for (int64_t j = threadIdx.x; j < row_chunks; j += blockDim.x) {
      const int64_t h = j / kChunksPerHead;
      const int64_t c = j - h * kChunksPerHead;
      const int64_t dst = ((blk * num_kv_heads + h) * kBlock + off) * kChunksPerHead + c;
      const int64_t src = row * row_chunks + j;
      const uint4 kv = k[src];
      const uint4 vv = v[src];
      k_cache[dst] = kv;
      v_cache[dst] = vv;
    }
  }
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  const int elem = a.dtype == 1 ? 2 : 4;
  const int cph = a.head_dim * elem / 16;
  const int64_t grid64 = a.num_tokens < 65536 ? a.num_tokens : 65536;
  const dim3 grid((unsigned)grid64), block(128);
  auto k = reinterpret_cast<const uint4*>(a.k);
  auto v = reinterpret_cast<const uint4*>(a.v);
  auto kc = reinterpret_cast<uint4*>(a.k_cache);
  auto vc = reinterpret_cast<uint4*>(a.v_cache);
  switch (cph) {
    case 8:
      hipLaunchKernelGGL(kv_write_kernel<8>, grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc, vc,
                         a.num_blocks, a.num_kv_heads);
      break;
    case 16:
      hipLaunchKernelGGL(kv_write_kernel<16>, grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc, vc,
                         a.num_blocks, a.num_kv_heads);
      break;
    case 32:
      hipLaunchKernelGGL(kv_write_kernel<32>, grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc, vc,
                         a.num_blocks, a.num_kv_heads);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp8 cache write: quantise each new token's K and V row of one kv head to
// OCP E4M3 codes with one float scale for the row ("Part 47", section 2.4: a
// server may keep the cache quantised; the format and the per-(slot, kv head)
// scale are this library's choice).  Every decision is taken in float32 in a
// fixed order, so the codes are reproducible bit for bit:
//   amax = max |x|, scale = amax / 448, inv = 448 / amax (0 if amax == 0),
//   y = clamp(x * inv, -448, 448), code = nearest E4M3 value, ties to even.
// One wave per (token, kv head); lane i holds dims i * NPL .. i * NPL + NPL - 1.

// E4M3 code of y, |y| <= 448, rounded to nearest with ties to the even code.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) {  // below 2^-6: the subnormal codes m * 2^-9, m = 0 .. 8 (8 is 2^-6 itself)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a = 2^e * (1 + f)
  float m = __builtin_rintf(ldexpf(a, 3 - e));               // 8 .. 16: implicit bit + 3 mantissa bits
  if (m == 16.0f) {
    ++e;
    m = 8.0f;
  }
  return sign | ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
}

template <int D, typename In>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(const In* __restrict__ k, const In* __restrict__ v,
                                                           const int32_t* __restrict__ slots, int64_t num_tokens,
                                                           uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                           float* __restrict__ k_scale, float* __restrict__ v_scale,
                                                           int32_t num_blocks, int32_t num_kv_heads) {
  constexpr int NPL = D / kWave;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= num_kv_heads) return;
  for (int64_t row = blockIdx.x; row < num_tokens; row += gridDim.x) {
    const int32_t slot = slots[row];
    if (slot < 0 || slot >= num_blocks * kBlock) continue;  // skipped rows
    const int64_t blk = slot >> 4, off = slot & 15;
    const int64_t srow = ((blk * num_kv_heads + h) * kBlock + off);  // scale index; codes at srow * D
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const In* src = (which ? v : k) + (row * num_kv_heads + h) * D + lane * NPL;
      float x[NPL];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        x[i] = (float)src[i];
        amax = fmaxf(amax, fabsf(x[i]));
      }
      amax = wave_max(amax);
      const float scale = amax / 448.0f;
      const float inv = amax != 0.0f ? 448.0f / amax : 0.0f;
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float y = fminf(fmaxf(x[i] * inv, -448.0f), 448.0f);
        packed |= e4m3_encode(y) << (8 * i);
      }
      uint8_t* dst = (which ? v_cache : k_cache) + srow * D + lane * NPL;
      if constexpr (NPL == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
      } else {
        *dst = (uint8_t)packed;
      }
      if (lane == 0) (which ? v_scale : k_scale)[srow] = scale;
    }
  }
}

hipError_t launch_kv_write_fp8(const WriteArgs& a, int32_t in_dtype, float* k_scale, float* v_scale,
                               hipStream_t stream) {
  const int64_t grid64 = a.num_tokens < 65536 ? a.num_tokens : 65536;
  const dim3 grid((unsigned)grid64, (unsigned)((a.num_kv_heads + 3) / 4)), block(256);
  auto kc = reinterpret_cast<uint8_t*>(a.k_cache);
  auto vc = reinterpret_cast<uint8_t*>(a.v_cache);
  if (in_dtype == 1) {
    auto k = reinterpret_cast<const __bf16*>(a.k);
    auto v = reinterpret_cast<const __bf16*>(a.v);
    if (a.head_dim == 128)
      hipLaunchKernelGGL((kv_write_fp8_kernel<128, __bf16>), grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc,
                         vc, k_scale, v_scale, a.num_blocks, a.num_kv_heads);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL((kv_write_fp8_kernel<64, __bf16>), grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc,
                         vc, k_scale, v_scale, a.num_blocks, a.num_kv_heads);
    else
      return hipErrorInvalidValue;
  } else if (in_dtype == 0) {
    auto k = reinterpret_cast<const float*>(a.k);
    auto v = reinterpret_cast<const float*>(a.v);
    if (a.head_dim == 128)
      hipLaunchKernelGGL((kv_write_fp8_kernel<128, float>), grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc,
                         vc, k_scale, v_scale, a.num_blocks, a.num_kv_heads);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL((kv_write_fp8_kernel<64, float>), grid, block, 0, stream, k, v, a.slots, a.num_tokens, kc,
                         vc, k_scale, v_scale, a.num_blocks, a.num_kv_heads);
    else
      return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Copy-on-write: copy whole blocks (every kv head, all 16 slots, K and V).
// ainews.alishangtian.com article on inference engines, section
// "PagedAttention": sequences share physical blocks, and a shared block that
// one of them must modify is first copied to a block of its own.  One
// workgroup per (src, dst) pair, 16-byte copies; pairs with an id outside
// [0, num_blocks) are skipped.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                             const int32_t* __restrict__ src_blocks,
                                                             const int32_t* __restrict__ dst_blocks,
                                                             int64_t num_pairs, int32_t num_blocks,
                                                             int64_t block_chunks) {
  for (int64_t i = blockIdx.x; i < num_pairs; i += gridDim.x) {
    const int32_t src = src_blocks[i], dst = dst_blocks[i];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) continue;
    const uint4* ks = k_cache + (int64_t)src * block_chunks;
    const uint4* vs = v_cache + (int64_t)src * block_chunks;
    uint4* kd = k_cache + (int64_t)dst * block_chunks;
    uint4* vd = v_cache + (int64_t)dst * block_chunks;
    // Every load of a thread's chunks is in flight before its stores, and the
    // stores carry the non-temporal hint (the copied blocks are not read again
    // in the call).  512 pairs of 2 x 32 KiB: 9.9 us against 11.2 us for one
    // load pair per iteration with plain stores; non-temporal loads as well
    // took 13.4 us.
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kUnroll = 8;
    for (int64_t j0 = threadIdx.x; j0 < block_chunks; j0 += (int64_t)blockDim.x * kUnroll) {
      u32x4 a[kUnroll], b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = j0 + (int64_t)u * blockDim.x;
        if (j < block_chunks) {
          a[u] = *reinterpret_cast<const u32x4*>(ks + j);
          b[u] = *reinterpret_cast<const u32x4*>(vs + j);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = j0 + (int64_t)u * blockDim.x;
        if (j < block_chunks) {
          __builtin_nontemporal_store(a[u], reinterpret_cast<u32x4*>(kd + j));
          __builtin_nontemporal_store(b[u], reinterpret_cast<u32x4*>(vd + j));
        }
      }
    }
  }
}

hipError_t launch_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                                 int64_t num_pairs, int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  const int64_t grid64 = num_pairs < 65536 ? num_pairs : 65536;
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3((unsigned)grid64), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache), src, dst, num_pairs,
                     num_blocks, block_bytes / 16);
  return hipGetLastError();
}

}  // namespace pkv
