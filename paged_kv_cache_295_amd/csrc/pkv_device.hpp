// Device helpers shared by the gfx950 kernels of libpagedkv: element access for
// float32 / bfloat16 16-byte chunks, wavefront (64-lane) reductions through DPP,
// and the exp2-based softmax constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;
// Running maxima start at the most negative finite float, so that an
// all-masked stream rescales by exp2(0) = 1 and never forms inf - inf.
constexpr float kMaxInit = -3.402823466e38f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

struct alignas(16) Chunk {  // 16 bytes: 8 bf16 or 4 float32
  uint32_t w[4];
};

__device__ __forceinline__ Chunk load_chunk(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  Chunk c;
  c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  return c;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming load: the non-temporal hint keeps K/V that is read once from
// displacing reusable lines and lets the memory system stream it (about
// 7 TB/s for plain reads on MI355X against about 6.2 TB/s without the hint).
__device__ __forceinline__ Chunk load_chunk_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Chunk c;
  c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  return c;
}

// A raw buffer resource over the `bytes` bytes at p (stride 0; the fourth
// descriptor word is the gfx9 one for untyped 32-bit data).  A load whose
// 16 bytes do not lie wholly inside [0, bytes) returns zeros and makes no
// memory access, so a size that stops at the last valid row masks the rest
// of a tile for free, and size 0 turns a load into a no-op.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Chunk as_chunk(i32x4_t v) {
  Chunk c;
  c.w[0] = (uint32_t)v.x; c.w[1] = (uint32_t)v.y; c.w[2] = (uint32_t)v.z; c.w[3] = (uint32_t)v.w;
  return c;
}

__device__ __forceinline__ void store_chunk(void* p, const Chunk& c) {
  *reinterpret_cast<uint4*>(p) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
}

// bf16 pair in one dword -> two floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kDtype = 0;
  // partial dot product of a query chunk with a key chunk, accumulated into acc
  __device__ __forceinline__ static float dot(const Chunk& q, const Chunk& k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q.w[i]), __uint_as_float(k.w[i]), acc);
    return acc;
  }
  __device__ __forceinline__ static float dot(const Chunk* q, const Chunk& k, float acc) { return dot(q[0], k, acc); }
  __device__ __forceinline__ static void widen(const Chunk& c, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c.w[i]);
  }
  __device__ __forceinline__ static Chunk narrow(const float (&f)[4]) {
    Chunk c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = __float_as_uint(f[i]);
    return c;
  }
};

template <>
struct Elem<__bf16> {
  static constexpr int kPerChunk = 8;
  static constexpr int kDtype = 1;
  __device__ __forceinline__ static float dot(const Chunk& q, const Chunk& k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w[i]),
                                            __builtin_bit_cast(bf16x2_t, k.w[i]), acc, false);
    return acc;
  }
  __device__ __forceinline__ static float dot(const Chunk* q, const Chunk& k, float acc) { return dot(q[0], k, acc); }
  __device__ __forceinline__ static void widen(const Chunk& c, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(c.w[i]);
      f[2 * i + 1] = bf16_hi(c.w[i]);
    }
  }
  __device__ __forceinline__ static Chunk narrow(const float (&f)[8]) {
    Chunk c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return c;
  }
};

// OCP E4M3 cache bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// largest finite 448; no infinities) with one float scale per (slot, kv head):
// value = e4m3(code) * scale.  Queries and outputs stay bfloat16.
struct Fp8E4M3 {};

// What a cache element type implies for the decode kernels: the query/output
// type Q, the bytes per cache element, and whether per-slot scales apply.
template <typename KV>
struct KvTraits {
  using Q = KV;
  static constexpr int kElemBytes = sizeof(KV);
  static constexpr bool kScaled = false;
};

template <>
struct KvTraits<Fp8E4M3> {
  using Q = __bf16;
  static constexpr int kElemBytes = 1;
  static constexpr bool kScaled = true;
};

// Two E4M3 codes (bytes 0-1 of w for hi == false, bytes 2-3 for hi == true)
// widened exactly to a bfloat16 pair (every E4M3 value is a bfloat16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <>
struct Elem<Fp8E4M3> {
  static constexpr int kPerChunk = 16;
  static constexpr int kDtype = 2;
  // q: the two bfloat16 chunks of the same 16 dims
  __device__ __forceinline__ static float dot(const Chunk* q, const Chunk& k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Chunk& qc = q[i >> 1];
      const int w = (i & 1) * 2;
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qc.w[w]),
                                            __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<false>(k.w[i])), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qc.w[w + 1]),
                                            __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<true>(k.w[i])), acc, false);
    }
    return acc;
  }
};

// ---- DPP lane exchanges inside a row of 16 lanes -------------------------
// quad_perm [1,0,3,2] = lane ^ 1, quad_perm [2,3,0,1] = lane ^ 2,
// row_half_mirror pairs lane i with 7 - i in each half row, row_mirror pairs
// lane i with 15 - i.  After the first two steps every lane of a quad holds
// the quad's value, so the mirrors complete an all-reduce over 8 and 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over groups of kLanes consecutive lanes (kLanes in {1,2,4,8,16}); every
// lane of a group receives the group's sum.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (kLanes >= 2) x += dpp_f32<0xB1>(x);
  if constexpr (kLanes >= 4) x += dpp_f32<0x4E>(x);
  if constexpr (kLanes >= 8) x += dpp_f32<0x141>(x);
  if constexpr (kLanes >= 16) x += dpp_f32<0x140>(x);
  static_assert(kLanes <= 16, "group_sum spans at most one DPP row");
  return x;
}

// Exchange across lane groups for an all-reduce: the value of lane l ^ MASK
// combined with the lane's own, for MASK in {8, 16, 32}.  8 is a DPP rotate by
// 8 inside each row of 16 lanes; 16 and 32 use the permlane16/32 swaps, which
// leave lane l's and lane (l ^ MASK)'s values in the two results.
template <int MASK>
__device__ __forceinline__ float xor_add(float x) {
  static_assert(MASK == 8 || MASK == 16 || MASK == 32, "xor_add: mask 8, 16 or 32");
  if constexpr (MASK == 8) {
    return x + dpp_f32<0x128>(x);  // row_ror:8
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = MASK == 16 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                              : __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  }
}

template <int MASK>
__device__ __forceinline__ float xor_max(float x) {
  static_assert(MASK == 8 || MASK == 16 || MASK == 32, "xor_max: mask 8, 16 or 32");
  if constexpr (MASK == 8) {
    return fmaxf(x, dpp_f32<0x128>(x));
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = MASK == 16 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                              : __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  }
}

// All-reduce over the lanes that differ only in the bits >= log2(FROM) of the
// lane id (the 64 / FROM lane groups of FROM consecutive lanes), FROM in
// {4, 8, 16, 32}.  For FROM = 4, ror:4 then ror:8 add the four lanes i, i+4,
// i+8, i+12 of a row (a cyclic group of rotations).
template <int FROM>
__device__ __forceinline__ float groups_add(float x) {
  if constexpr (FROM <= 4) x += dpp_f32<0x124>(x);  // row_ror:4, then the ror:8 step sums all four
  if constexpr (FROM <= 8) x = xor_add<8>(x);
  if constexpr (FROM <= 16) x = xor_add<16>(x);
  if constexpr (FROM <= 32) x = xor_add<32>(x);
  return x;
}

template <int FROM>
__device__ __forceinline__ float groups_max(float x) {
  if constexpr (FROM <= 4) x = fmaxf(x, dpp_f32<0x124>(x));
  if constexpr (FROM <= 8) x = xor_max<8>(x);
  if constexpr (FROM <= 16) x = xor_max<16>(x);
  if constexpr (FROM <= 32) x = xor_max<32>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, shfl_xor_f32(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += shfl_xor_f32(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Log-sum-exp merge of n partial states of one row, partial p at row index
// row0 + p * stride of part_ml (m in log2 units, l) and part_o (D floats,
// unnormalised).  Lane p loads partial p's (m, l), so every load is in flight
// at once; lane k ends with dims k, k + 64, ... of sum_p 2^(m_p - M) o_p in o
// and every lane with lam = sum_p 2^(m_p - M) l_p and M = max_p m_p.  nan:
// some m_p is NaN (the partial's inputs broke the contract).
template <int D>
__device__ __forceinline__ void merge_partials(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                               int64_t row0, int64_t stride, int n, float (&o)[D / kWave],
                                               float& M, float& lam, bool& nan) {
  constexpr int PER = D / kWave;
  const int lane = __lane_id();
  M = -__builtin_inff();
  nan = false;
  if (n <= kWave) {
    // one 8-byte load of (m, l) per lane serves both the max and the weights;
    // the outputs of the first kPre partials are loaded at the same time
    constexpr int kPre = 8;
    float pre[kPre][PER];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {  // past the n-th, partial 0 again (in bounds, unused)
      const float* src = part_o + (row0 + (int64_t)(j < n ? j : 0) * stride) * D + lane;
#pragma unroll
      for (int e = 0; e < PER; ++e) pre[j][e] = src[e * kWave];
    }
    float m = -__builtin_inff(), l = 0.0f;
    if (lane < n) {
      const float2 v = *reinterpret_cast<const float2*>(part_ml + (row0 + lane * stride) * 2);
      m = v.x;
      l = v.y;
    }
    nan = __builtin_amdgcn_ballot_w64(m != m) != 0;
    M = wave_max(m);
    const float f = lane < n ? fast_exp2(m - M) : 0.0f;
    lam = wave_sum(f * l);
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      if (j < n) {
        const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = fmaf(fj, pre[j][e], o[e]);
      }
    }
#pragma unroll 4
    for (int j = kPre; j < n; ++j) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
      const float* src = part_o + (row0 + (int64_t)j * stride) * D + lane;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(fj, src[e * kWave], o[e]);
    }
    return;
  }
  for (int p0 = 0; p0 < n; p0 += kWave) {
    const int p = p0 + lane;
    const float m = p < n ? part_ml[(row0 + p * stride) * 2] : -__builtin_inff();
    nan |= __builtin_amdgcn_ballot_w64(m != m) != 0;
    M = fmaxf(M, wave_max(m));
  }
  lam = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.0f;
  for (int p0 = 0; p0 < n; p0 += kWave) {
    const int p = p0 + lane;
    float f = 0.0f, l = 0.0f;
    if (p < n) {
      f = fast_exp2(part_ml[(row0 + p * stride) * 2] - M);
      l = part_ml[(row0 + p * stride) * 2 + 1];
    }
    lam += wave_sum(f * l);
    const int cnt = min(kWave, n - p0);
#pragma unroll 4
    for (int j = 0; j < cnt; ++j) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
      const float* src = part_o + (row0 + (int64_t)(p0 + j) * stride) * D + lane;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(fj, src[e * kWave], o[e]);
    }
  }
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return (T)__builtin_amdgcn_readfirstlane((int)v);
}

}  // namespace pkv
