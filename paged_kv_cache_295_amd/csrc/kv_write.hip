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
    for (int64_t j = threadIdx.x; j < block_chunks; j += blockDim.x) {
      const uint4 a = ks[j];
      const uint4 b = vs[j];
      kd[j] = a;
      vd[j] = b;
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
