// Paged decode attention for gfx950: split-context partitions + log-sum-exp merge.
//
// What is computed ("Part 47 | Inference basics: KV Cache, batching,
// sampling", chengxuchu.com, sections 2.1-2.2): for every query row and
// query head h, softmax(scale * q . K^T) V over the row's cached keys, where
// kv head h / G serves a group of G query heads (section 2.3, GQA).  The keys
// of token t live in physical block block_tables[seq][t / 16], offset t % 16
// (the ainews.alishangtian.com article, section "PagedAttention"; "Part 47",
// section 5.2: the kernel follows the block table to find K/V).
//
// Design (MI355X, wave64):
//  * One wave owns one work item (query row, kv head, head subgroup of GB
//    query heads, partition of P tokens).  The wave walks the partition's
//    blocks; each block's K tile and V tile for the kv head is one contiguous
//    16 x head_dim run, read with 16-byte loads so that every load
//    instruction covers a contiguous kilobyte (bf16, D = 128).
//  * Lane layout: LPT lanes share a token; lane (tg = lane / LPT,
//    li = lane % LPT) holds 16-byte chunk (c * LPT + li) of tokens
//    pass * (64 / LPT) + tg of each block.  The K/V values a lane loads stay in
//    its registers and serve all GB query heads of the group, so the K/V bytes
//    of a block are read from HBM once per kv head.
//  * Scores: per lane a partial dot product (v_dot2_f32_bf16 for bf16),
//    completed by an all-reduce over the LPT lanes of the token through DPP
//    row operations (quad_perm, row_half_mirror, row_mirror).
//  * Online softmax in the log2 domain (exp2, scale folded with log2 e); each
//    group of LPT lanes keeps its own running max / sum / output for its
//    tokens, so no cross-lane traffic is needed per block; the 64 / LPT
//    streams are merged once at the end of the partition.
//  * Block tables are read 64 entries at a time into a lane-indexed register
//    and broadcast with readlane; the next block's K/V loads are issued
//    before the current block is computed (register double buffering).
//  * A row whose context fits one partition writes its output directly;
//    otherwise each partition writes (m, l, unnormalised o) and the merge
//    kernel combines them: M = max m_p, out = sum 2^(m_p - M) o_p / sum
//    2^(m_p - M) l_p, exact in real arithmetic.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

struct RowInfo {
  int32_t seq;
  int32_t keys;  // keys visible to this query row
  bool bad;      // device-side contract broken: outputs become NaN
  bool skip;     // prefill row past the chunk's end: nothing to write
};

__device__ __forceinline__ RowInfo row_info(const DecodeArgs& a, int64_t row) {
  RowInfo r;
  r.seq = (int32_t)(row / a.rows_per_seq);
  const int32_t ri = (int32_t)(row - (int64_t)r.seq * a.rows_per_seq);
  const int32_t L = a.context_lens[r.seq];
  const int32_t cap = a.max_blocks_per_seq * kBlock;
  r.skip = false;
  if (a.chunk_start == nullptr) {
    r.keys = L;
    r.bad = L < 0 || L > cap || (int64_t)L > (int64_t)a.max_parts * a.partition_tokens;
  } else {
    const int32_t p0 = a.chunk_start[r.seq];
    const int32_t n = L - p0;
    r.bad = p0 < 0 || n < 0 || L > cap || n > a.rows_per_seq ||
            (int64_t)L > (int64_t)a.max_parts * a.partition_tokens;
    r.skip = !r.bad && ri >= n;
    r.keys = p0 + ri + 1;
  }
  return r;
}

template <typename T, int D, int GB, int LPT>
struct DecodeShape {
  using E = Elem<T>;
  static constexpr int kEPC = E::kPerChunk;       // elements per 16-byte chunk
  static constexpr int kRowChunks = D / kEPC;     // chunks per token row of one kv head
  static constexpr int kCPL = kRowChunks / LPT;   // chunks per lane per token
  static constexpr int kTPP = kWave / LPT;        // tokens covered by one load pass
  static constexpr int kNPass = kBlock / kTPP;    // tokens per lane per block
  static_assert(kRowChunks % LPT == 0 && kCPL >= 1, "LPT must divide the chunks of a row");
  static_assert(kBlock % kTPP == 0, "a block must be a whole number of passes");
};

template <typename T, int D, int GB, int LPT>
__global__ __launch_bounds__(64) void decode_partition_kernel(const DecodeArgs a) {
  using S = DecodeShape<T, D, GB, LPT>;
  using E = typename S::E;
  constexpr int EPC = S::kEPC, CPL = S::kCPL, TPP = S::kTPP, NP = S::kNPass;

  const int lane = __lane_id();
  const int tg = lane / LPT;
  const int li = lane % LPT;
  const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;

  int64_t t = blockIdx.x;
  const int part = (int)(t % a.max_parts);
  t /= a.max_parts;
  const int hs = (int)(t % hsubs);
  t /= hsubs;
  const int g = (int)(t % a.num_kv_heads);
  const int64_t row = t / a.num_kv_heads;
  if (row >= (int64_t)a.num_seqs * a.rows_per_seq) return;

  const RowInfo ri = row_info(a, row);
  if (ri.skip) return;
  const int h0 = g * (a.num_q_heads / a.num_kv_heads) + hs * GB;
  T* __restrict__ outp = reinterpret_cast<T*>(a.out) + (row * a.num_q_heads + h0) * (int64_t)D;

  if (ri.bad || ri.keys == 0) {
    if (part != 0) return;
    const float fill = ri.bad ? __builtin_nanf("") : 0.0f;
    for (int i = lane; i < GB * D; i += kWave) outp[i] = (T)fill;
    return;
  }
  const int P = a.partition_tokens;
  const int keys = ri.keys;
  const int start = part * P;
  if (start >= keys) return;
  const int end = min(keys, start + P);
  const int nparts = (keys + P - 1) / P;
  const int blk0 = start / kBlock;
  const int nblk = (end - start + kBlock - 1) / kBlock;

  // query chunks for the GB heads, in registers for the whole partition
  Chunk qv[GB][CPL];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + (row * a.num_q_heads + h0) * (int64_t)D;
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) qv[h][c] = load_chunk(qrow + h * D + (c * LPT + li) * EPC);
  }

  float m[GB], l[GB], acc[GB][CPL][EPC];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m[h] = kMaxInit;
    l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][c][e] = 0.0f;
  }

  const int32_t* __restrict__ table = a.block_tables + (int64_t)ri.seq * a.max_blocks_per_seq + blk0;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache);
  const int64_t tile_bytes = (int64_t)kBlock * D * sizeof(T);
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  // byte offset of this lane's chunk (pass p, chunk c) inside a tile
  auto lane_off = [&](int p, int c) -> int {
    return (p * TPP + tg) * (D * (int)sizeof(T)) + (c * LPT + li) * 16;
  };

  int tab_reg = 0;  // lane k holds table entry (window base + k)
  bool bad_block = false;
  auto block_ptr_off = [&](int jb) -> int64_t {
    if ((jb & 63) == 0) {
      const int n = nblk - jb;
      tab_reg = lane < n ? table[jb + lane] : 0;
    }
    int p = __builtin_amdgcn_readlane(tab_reg, jb & 63);
    if (p < 0 || p >= a.num_blocks) {
      bad_block = true;
      p = 0;
    }
    return (int64_t)p * blk_stride + (int64_t)g * tile_bytes;
  };

  Chunk kA[NP][CPL], vA[NP][CPL], kB[NP][CPL], vB[NP][CPL];
  auto load = [&](Chunk (&kk)[NP][CPL], Chunk (&vv)[NP][CPL], int64_t off) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < CPL; ++c) kk[p][c] = load_chunk(kc + off + lane_off(p, c));
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < CPL; ++c) vv[p][c] = load_chunk(vc + off + lane_off(p, c));
  };

  const float sl2 = a.scale_log2;
  auto compute = [&](Chunk (&kk)[NP][CPL], Chunk (&vv)[NP][CPL], int jb) {
    const int tok0 = (blk0 + jb) * kBlock + tg;  // this lane's token of pass 0
    const bool tail = (blk0 + jb + 1) * kBlock > end;
    if (tail) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (tok0 + p * TPP >= end)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) kk[p][c].w[w] = vv[p][c].w[w] = 0u;
    }
    float sc[NP][GB];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) d = E::dot(qv[h][c], kk[p][c], d);
        sc[p][h] = group_sum<LPT>(d) * sl2;
      }
    if (tail) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (tok0 + p * TPP >= end)
#pragma unroll
          for (int h = 0; h < GB; ++h) sc[p][h] = -__builtin_inff();
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int p = 1; p < NP; ++p) bm = fmaxf(bm, sc[p][h]);
      const float mn = fmaxf(m[h], bm);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      float ls = l[h] * alpha;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][c][e] *= alpha;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float pr = fast_exp2(sc[p][h] - mn);
        sc[p][h] = pr;
        ls += pr;
      }
      l[h] = ls;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float vf[EPC];
        E::widen(vv[p][c], vf);
#pragma unroll
        for (int h = 0; h < GB; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][c][e] = fmaf(sc[p][h], vf[e], acc[h][c][e]);
      }
  };

  load(kA, vA, block_ptr_off(0));
  for (int jb = 0; jb < nblk; jb += 2) {
    if (jb + 1 < nblk) load(kB, vB, block_ptr_off(jb + 1));
    compute(kA, vA, jb);
    if (jb + 1 >= nblk) break;
    if (jb + 2 < nblk) load(kA, vA, block_ptr_off(jb + 2));
    compute(kB, vB, jb + 1);
  }

  // merge the 64 / LPT per-token-group streams
#pragma unroll
  for (int mask = LPT; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float mo = shfl_xor_f32(m[h], mask);
      const float lo = shfl_xor_f32(l[h], mask);
      const float M = fmaxf(m[h], mo);
      const float fs = fast_exp2(m[h] - M), fo = fast_exp2(mo - M);
      l[h] = l[h] * fs + lo * fo;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float ao = shfl_xor_f32(acc[h][c][e], mask);
          acc[h][c][e] = acc[h][c][e] * fs + ao * fo;
        }
      m[h] = M;
    }
  }

  const float nan = __builtin_nanf("");
  if (nparts == 1) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (tg != h % TPP) continue;
      const float inv = bad_block ? nan : 1.0f / l[h];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float o[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[e] = acc[h][c][e] * inv;
        store_chunk(outp + h * D + (c * LPT + li) * EPC, E::narrow(o));
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (tg != h % TPP) continue;
      const int64_t pidx = (row * a.num_q_heads + h0 + h) * (int64_t)a.max_parts + part;
      float* po = a.part_o + pidx * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e4 = 0; e4 < EPC; e4 += 4) {
          float4 v4;
          v4.x = bad_block ? nan : acc[h][c][e4];
          v4.y = acc[h][c][e4 + 1];
          v4.z = acc[h][c][e4 + 2];
          v4.w = acc[h][c][e4 + 3];
          *reinterpret_cast<float4*>(po + (c * LPT + li) * EPC + e4) = v4;
        }
      if (li == 0) {
        a.part_ml[pidx * 2] = bad_block ? nan : m[h];
        a.part_ml[pidx * 2 + 1] = l[h];
      }
    }
  }
}

// Log-sum-exp merge of the partitions of every (query row, query head) whose
// context spans more than one partition.  One wave per (row, head); lane k
// owns output dims k, k + 64, ...
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int PER = D / kWave;
  const int lane = __lane_id();
  const int64_t item = blockIdx.x;
  const int64_t row = item / a.num_q_heads;
  const int h = (int)(item - row * a.num_q_heads);
  const RowInfo ri = row_info(a, row);
  const int P = a.partition_tokens;
  if (ri.skip || ri.bad || ri.keys <= P) return;
  const int nparts = (ri.keys + P - 1) / P;
  const int64_t base = (row * a.num_q_heads + h) * (int64_t)a.max_parts;
  const float* ml = a.part_ml + base * 2;

  float M = -__builtin_inff();
  for (int p = lane; p < nparts; p += kWave) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);

  float lam = 0.0f, o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.0f;
  const float* po = a.part_o + base * D;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    lam = fmaf(w, ml[2 * p + 1], lam);
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = fmaf(w, po[(int64_t)p * D + lane + k * kWave], o[k]);
  }
  const float inv = 1.0f / lam;
  T* outp = reinterpret_cast<T*>(a.out) + (row * a.num_q_heads + h) * (int64_t)D;
#pragma unroll
  for (int k = 0; k < PER; ++k) outp[lane + k * kWave] = (T)(o[k] * inv);
}

template <typename T, int D, int GB>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int LPT = (D * (int)sizeof(T) / 16) >= 16 ? 16 : (D * (int)sizeof(T) / 16);
  const int64_t rows = (int64_t)a.num_seqs * a.rows_per_seq;
  const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;
  const int64_t items = rows * a.num_kv_heads * hsubs * a.max_parts;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partition_kernel<T, D, GB, LPT>), dim3((unsigned)items), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t merges = rows * a.num_q_heads;
  if (merges > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)merges), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gb(const DecodeArgs& a, hipStream_t stream) {
  switch (heads_per_wave(a.num_q_heads / a.num_kv_heads)) {
    case 1: return launch_typed<T, D, 1>(a, stream);
    case 2: return launch_typed<T, D, 2>(a, stream);
    case 4: return launch_typed<T, D, 4>(a, stream);
    case 8: return launch_typed<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == 0) {
    if (a.head_dim == 64) return launch_gb<float, 64>(a, stream);
    if (a.head_dim == 128) return launch_gb<float, 128>(a, stream);
  } else if (a.dtype == 1) {
    if (a.head_dim == 64) return launch_gb<__bf16, 64>(a, stream);
    if (a.head_dim == 128) return launch_gb<__bf16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
