// Chunked-prefill attention over the paged cache on gfx950 matrix cores (bf16).
//
// What is computed: the caffein.top essay on modern LLM inference runtimes
// (section on chunked prefill) cuts a long prompt into chunks interleaved with
// decode steps; each chunk row at position p attends to keys 0..p
// ("Part 47 | Inference basics: KV Cache, batching, sampling",
// chengxuchu.com, section 2.1: the query of position t dots the keys of
// positions 1..t).  The chunk's own K/V are already in the cache (written by
// the cache-write kernel), so every key comes through the block table.
//
// Design (one workgroup = 4 waves, 128 "M rows" = G query heads x 128/G chunk
// rows sharing one kv head):
//  * Key tiles of 64 tokens (4 cache blocks) are gathered through the block
//    table into LDS once per workgroup and shared by the G heads of the group:
//    K row-major [key][dim], V transposed [dim][key] (pairs of keys packed per
//    dword on the way in), both padded so the MFMA operand reads are free of
//    bank conflicts.  The next tile's global loads are in flight while the
//    current one is computed.
//  * Transposed formulation so that each lane owns one query row:
//      S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K (LDS), B = Q (registers)
//      O^T += V^T P^T   A = V^T (LDS), B = P (registers, from S^T's lanes)
//    In the 32x32 accumulator layout lane l holds column l % 32 (its query
//    row) and 16 of the 32 rows, the other 16 sit in lane l ^ 32; so the row
//    max needs one exchange with lane l ^ 32, and the softmax rescale of O^T
//    is a per-lane multiply.  P feeds the second product straight from the
//    registers of the first: the key order of the K dimension is permuted the
//    same way in A (two 8-byte V^T reads) and B, which leaves the sum unchanged.
//  * Online softmax in the log2 domain; causal mask by select (never by
//    multiplying, so NaN-filled unused slots cannot leak); P is rounded to bf16
//    for the matrix cores, accumulation stays float32.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKT = 64;       // keys per tile
constexpr int kMRows = 128;   // (head, row) pairs per workgroup
constexpr int kThreads = 256;

template <int D>
struct PrefillShape {
  static constexpr int kRC = D * 2 / 16;              // 16-byte chunks per key row
  static constexpr int kKStride = D * 2 + 16;         // LDS bytes per K row
  static constexpr int kVStride = kKT * 2 + 8;        // LDS bytes per V^T row
  static constexpr int kKBytes = kKT * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kKPerThread = kKT * kRC / kThreads;
  static constexpr int kVPairsPerThread = (kKT / 2) * kRC / kThreads;
  static constexpr int kKSteps = D / 16;  // QK^T steps of 16 head dims
  static constexpr int kND = D / 32;      // PV output blocks of 32 head dims
  static_assert(kKPerThread >= 1 && kVPairsPerThread >= 1, "tile too small for the workgroup");
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(const PrefillArgs a) {
  using S = PrefillShape<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::kKBytes + S::kVBytes];
  char* k_lds = smem;
  char* v_lds = smem + S::kKBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int QT = kMRows / G;
  const int n_mt = (a.chunk_len_max + QT - 1) / QT;
  const int npair = a.num_chunks * a.num_kv_heads;
  const int id = blockIdx.x;
  const int pair = id % npair;
  const int mt = n_mt - 1 - id / npair;  // the longest row tiles start first
  const int c = pair / a.num_kv_heads;
  const int g = pair - c * a.num_kv_heads;

  const int P0 = a.chunk_start[c];
  const int L = a.context_lens[c];
  const int n = L - P0;
  const bool bad_chunk = P0 < 0 || n < 0 || L > a.max_blocks_per_seq * kBlock || n > a.chunk_len_max;
  const int row0 = mt * QT;
  __bf16* __restrict__ out = reinterpret_cast<__bf16*>(a.out);
  if (bad_chunk) {
    const int rows = min(QT, a.chunk_len_max - row0);
    for (int idx = tid; idx < rows * G * D; idx += kThreads) {
      const int r = idx / (G * D), rem = idx - r * G * D;
      out[((int64_t)(c * a.chunk_len_max + row0 + r) * a.num_q_heads + g * G) * D + rem] =
          (__bf16)__builtin_nanf("");
    }
    return;
  }
  const int rows_here = min(QT, n - row0);
  if (rows_here <= 0) return;
  const int kend = P0 + row0 + rows_here;  // keys [0, kend) are visible to some row
  const int ntiles = (kend + kKT - 1) / kKT;

  // this lane's query row (column of S^T and O^T)
  const int mrow = wave * 32 + (lane & 31);
  const int hl = mrow / QT;
  const int qi = row0 + (mrow - hl * QT);
  const bool row_ok = hl < G && qi < n;
  const int qpos = P0 + qi;
  const int head = g * G + hl;

  bf16x8_t qop[S::kKSteps];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) +
                         ((int64_t)(c * a.chunk_len_max + qi) * a.num_q_heads + head) * D;
#pragma unroll
    for (int kk = 0; kk < S::kKSteps; ++kk) {
      if (row_ok) {
        const Chunk ch = load_chunk(qrow + kk * 16 + 8 * half);
        qop[kk] = as_bf16x8(ch.w[0], ch.w[1], ch.w[2], ch.w[3]);
      } else {
        qop[kk] = as_bf16x8(0u, 0u, 0u, 0u);
      }
    }
  }

  const int32_t* __restrict__ table = a.block_tables + (int64_t)c * a.max_blocks_per_seq;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache);
  const int64_t tile_bytes = (int64_t)kBlock * D * 2;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  int local_bad = 0;

  // byte offset in the cache of key position kpos of this kv head, or -1 past kend
  auto key_off = [&](int kpos) -> int64_t {
    if (kpos >= kend) return -1;
    int p = table[kpos >> 4];
    if (p < 0 || p >= a.num_blocks) {
      local_bad = 1;
      p = 0;
    }
    return (int64_t)p * blk_stride + (int64_t)g * tile_bytes + (int64_t)(kpos & 15) * D * 2;
  };
  auto gload_chunk = [&](const char* base, int64_t off, int ch) -> Chunk {
    if (off < 0) {
      Chunk z;
      z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0u;
      return z;
    }
    return load_chunk(base + off + ch * 16);
  };

  Chunk kreg[S::kKPerThread];
  Chunk vreg[S::kVPairsPerThread][2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int r = 0; r < S::kKPerThread; ++r) {
      const int q = tid + kThreads * r;
      const int key = q / S::kRC, ch = q % S::kRC;
      kreg[r] = gload_chunk(kc, key_off(kt * kKT + key), ch);
    }
#pragma unroll
    for (int r = 0; r < S::kVPairsPerThread; ++r) {
      const int q = tid + kThreads * r;
      const int kp = (q & 15) + 16 * (q / (16 * S::kRC));
      const int ch = (q >> 4) % S::kRC;
      vreg[r][0] = gload_chunk(vc, key_off(kt * kKT + 2 * kp), ch);
      vreg[r][1] = gload_chunk(vc, key_off(kt * kKT + 2 * kp + 1), ch);
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int r = 0; r < S::kKPerThread; ++r) {
      const int q = tid + kThreads * r;
      const int key = q / S::kRC, ch = q % S::kRC;
      store_chunk(k_lds + key * S::kKStride + ch * 16, kreg[r]);
    }
#pragma unroll
    for (int r = 0; r < S::kVPairsPerThread; ++r) {
      const int q = tid + kThreads * r;
      const int kp = (q & 15) + 16 * (q / (16 * S::kRC));
      const int ch = (q >> 4) % S::kRC;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = vreg[r][0].w[w], hi = vreg[r][1].w[w];
        const int dim = 8 * ch + 2 * w;
        *reinterpret_cast<uint32_t*>(v_lds + dim * S::kVStride + kp * 4) = (lo & 0xffffu) | (hi << 16);
        *reinterpret_cast<uint32_t*>(v_lds + (dim + 1) * S::kVStride + kp * 4) = (lo >> 16) | (hi & 0xffff0000u);
      }
    }
  };

  float m_run = kMaxInit, l_run = 0.0f;
  f32x16_t oacc[S::kND];
#pragma unroll
  for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[nd][v] = 0.0f;
  const float sl2 = a.scale_log2;

  gload(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    swrite();
    __syncthreads();
    if (kt + 1 < ntiles) gload(kt + 1);

    f32x16_t st[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[nb][v] = 0.0f;
      const char* krow = k_lds + (nb * 32 + (lane & 31)) * S::kKStride + 16 * half;
#pragma unroll
      for (int kk = 0; kk < S::kKSteps; ++kk) {
        const Chunk ch = load_chunk(krow + kk * 32);
        st[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ch.w[0], ch.w[1], ch.w[2], ch.w[3]), qop[kk],
                                                         st[nb], 0, 0, 0);
      }
    }

    // scale, causal mask (select), row max over this lane and lane ^ 32
    const bool diag = kt * kKT + kKT - 1 > P0 + row0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = st[nb][v] * sl2;
        if (diag) {
          const int kpos = kt * kKT + nb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          x = kpos > qpos ? -__builtin_inff() : x;
        }
        st[nb][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float mn = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - mn);
    m_run = mn;

    uint32_t pk[2][8];
    float ps = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float p0 = fast_exp2(st[nb][2 * u] - mn);
        const float p1 = fast_exp2(st[nb][2 * u + 1] - mn);
        ps += p0 + p1;
        pk[nb][u] = pack_bf16x2(p0, p1);
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[nd][v] *= alpha;

#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8_t bop = as_bf16x8(pk[nb][4 * s], pk[nb][4 * s + 1], pk[nb][4 * s + 2], pk[nb][4 * s + 3]);
        const int koff0 = nb * 32 + 16 * s + 4 * half;
#pragma unroll
        for (int nd = 0; nd < S::kND; ++nd) {
          const char* vrow = v_lds + (nd * 32 + (lane & 31)) * S::kVStride;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + koff0 * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (koff0 + 8) * 2);
          oacc[nd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo.x, lo.y, hi.x, hi.y), bop, oacc[nd], 0, 0,
                                                             0);
        }
      }
  }

  const int any_bad = __syncthreads_or(local_bad);
  const float l_tot = l_run + shfl_xor_f32(l_run, 32);
  if (!row_ok) return;
  const float inv = any_bad ? __builtin_nanf("") : 1.0f / l_tot;
  __bf16* orow = out + ((int64_t)(c * a.chunk_len_max + qi) * a.num_q_heads + head) * D;
#pragma unroll
  for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dim = nd * 32 + 8 * q4 + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(oacc[nd][4 * q4] * inv, oacc[nd][4 * q4 + 1] * inv);
      w.y = pack_bf16x2(oacc[nd][4 * q4 + 2] * inv, oacc[nd][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dim) = w;
    }
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G < 1 || G > kMRows) return hipErrorInvalidValue;
  const int QT = kMRows / G;
  const int64_t n_mt = (a.chunk_len_max + QT - 1) / QT;
  const int64_t grid = n_mt * a.num_chunks * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL(prefill_mfma_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(prefill_mfma_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
