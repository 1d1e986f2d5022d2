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
//  * Block-table entries are read with scalar loads; the next block's K/V
//    loads are issued before the current block is computed (two register
//    stages).  The rescale of the running output is lazy: only when a score
//    exceeds the running max by more than 2^8.
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

#ifndef PKV_DECODE_STREAM_KV
#define PKV_DECODE_STREAM_KV 1
#endif
// K/V tiles are read with the non-temporal (streaming) hint.
constexpr bool kStreamKV = PKV_DECODE_STREAM_KV != 0;

// Probability-weighted sum of V rows for the tokens a lane holds:
// acc[h][c][e] += sum_p prob[p][h] * V[p][c][e].  float32 uses plain FMAs; bf16
// rounds the probabilities to bf16 and pairs two tokens per v_dot2_f32_bf16
// (the matrix-core prefill rounds P the same way), which halves the ALU work
// of the PV product.
template <typename T, int NP, int CPL, int GB>
struct PV;

template <int NP, int CPL, int GB>
struct PV<float, NP, CPL, GB> {
  __device__ __forceinline__ static void apply(const float (&prob)[NP][GB], const Chunk (&vv)[NP][CPL],
                                               float (&acc)[GB][CPL][4]) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int h = 0; h < GB; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[h][c][e] = fmaf(prob[p][h], __uint_as_float(vv[p][c].w[e]), acc[h][c][e]);
  }
};

template <int NP, int CPL, int GB>
struct PV<__bf16, NP, CPL, GB> {
  static_assert(NP % 2 == 0, "tokens are paired");
  __device__ __forceinline__ static void apply(const float (&prob)[NP][GB], const Chunk (&vv)[NP][CPL],
                                               float (&acc)[GB][CPL][8]) {
#pragma unroll
    for (int p = 0; p < NP; p += 2) {
      bf16x2_t pp[GB];
#pragma unroll
      for (int h = 0; h < GB; ++h) pp[h] = __builtin_bit_cast(bf16x2_t, pack_bf16x2(prob[p][h], prob[p + 1][h]));
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = vv[p][c].w[w], a1 = vv[p + 1][c].w[w];
          // (token p, token p+1) pairs of dims 2w and 2w+1
          const bf16x2_t ev = __builtin_bit_cast(bf16x2_t, (a0 & 0xffffu) | (a1 << 16));
          const bf16x2_t od = __builtin_bit_cast(bf16x2_t, (a0 >> 16) | (a1 & 0xffff0000u));
#pragma unroll
          for (int h = 0; h < GB; ++h) {
            acc[h][c][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], ev, acc[h][c][2 * w], false);
            acc[h][c][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], od, acc[h][c][2 * w + 1], false);
          }
        }
    }
  }
};

// All-reduce every score over the LPT lanes of its token, one DPP step at a
// time across all scores so that consecutive DPP reads never depend on the
// instruction right before them.
template <int LPT, int N>
__device__ __forceinline__ void group_sum_all(float (&x)[N]) {
  if constexpr (LPT >= 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<0xB1>(x[i]);
  }
  if constexpr (LPT >= 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x4E>(x[i]);
  }
  if constexpr (LPT >= 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x141>(x[i]);
  }
  if constexpr (LPT >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<0x140>(x[i]);
  }
}

// A running max is only moved (and the accumulators rescaled) when a new
// score exceeds it by more than this many powers of two; otherwise the stale
// max is kept, which bounds every probability by 2^kRescaleSlack and is exact
// after the final normalisation.
constexpr float kRescaleSlack = 8.0f;

template <typename T, int D, int GB, int LPT, int NS>
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
  const int nfull = (end - start) / kBlock;  // blocks with no token past `end`

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
  const int lane_base = tg * (D * (int)sizeof(T)) + li * 16;

  bool bad_block = false;
  auto block_off = [&](int jb) -> int64_t {
    int p = table[jb];  // uniform: a scalar load
    if (p < 0 || p >= a.num_blocks) {
      bad_block = true;
      p = 0;
    }
    return (int64_t)p * blk_stride + (int64_t)g * tile_bytes;
  };

  // Every block is loaded whole (rows past `end` in the last block are still
  // inside that block): one constant per-lane offset plus immediates, so no
  // address arithmetic sits between the loads of consecutive blocks.
  auto load = [&](Chunk (&kk)[NP][CPL], Chunk (&vv)[NP][CPL], int64_t off) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int o = lane_base + p * TPP * (D * (int)sizeof(T)) + c * LPT * 16;
        if constexpr (kStreamKV) {
          kk[p][c] = load_chunk_stream(kc + off + o);
          vv[p][c] = load_chunk_stream(vc + off + o);
        } else {
          kk[p][c] = load_chunk(kc + off + o);
          vv[p][c] = load_chunk(vc + off + o);
        }
      }
  };

  const float sl2 = a.scale_log2;
  auto compute = [&](const Chunk (&kk)[NP][CPL], const Chunk (&vv)[NP][CPL], int jb) {
    float x[NP * GB];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) d = E::dot(qv[h][c], kk[p][c], d);
        x[p * GB + h] = d;
      }
    group_sum_all<LPT>(x);
    float sc[NP][GB];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int h = 0; h < GB; ++h) sc[p][h] = x[p * GB + h] * sl2;
    {
      const int tok0 = (blk0 + jb) * kBlock + tg;
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int h = 0; h < GB; ++h) sc[p][h] = tok0 + p * TPP < end ? sc[p][h] : -__builtin_inff();
    }
    bool need = false;
    float bm[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      bm[h] = sc[0][h];
#pragma unroll
      for (int p = 1; p < NP; ++p) bm[h] = fmaxf(bm[h], sc[p][h]);
      need |= bm[h] > m[h] + kRescaleSlack;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const float mn = fmaxf(m[h], bm[h]);
        const float alpha = fast_exp2(m[h] - mn);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][c][e] *= alpha;
      }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float ls = l[h];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float pr = fast_exp2(sc[p][h] - m[h]);
        sc[p][h] = pr;
        ls += pr;
      }
      l[h] = ls;
    }
    // Rows past `end` (only in the last block) may hold NaN: a zero weight is
    // not enough (0 * NaN), so their V words are replaced by 0.  Done with
    // selects on every block so that there is a single code path.
    {
      const int tok0 = (blk0 + jb) * kBlock + tg;
      Chunk vz[NP][CPL];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const bool ok = tok0 + p * TPP < end;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) vz[p][c].w[w] = ok ? vv[p][c].w[w] : 0u;
      }
      PV<T, NP, CPL, GB>::apply(sc, vz, acc);
    }
  };

  // NS register stages: while block jb is computed, blocks jb+1 .. jb+NS-1
  // are in flight and block jb+NS is issued right after.  The prologue fills
  // every stage so that the loop is entered in its steady state; past the end
  // loads re-read the last block (an L2 hit), so no load is conditional.  The
  // body computes NS blocks and exits only at its end (a single exit keeps the
  // accumulators in place); blocks past the last one are wholly masked and add
  // exactly nothing.  Table entries are fetched one pass ahead.
  Chunk kS[NS][NP][CPL], vS[NS][NP][CPL];
  const int last = nblk - 1;
  int64_t offs[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    load(kS[st], vS[st], block_off(min(st, last)));
    // each stage's loads are issued before the next stage's: waits are in order
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int st = 0; st < NS; ++st) offs[st] = block_off(min(NS + st, last));
  for (int jb = 0;; jb += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      compute(kS[st], vS[st], jb + st);
      const int64_t next = block_off(min(jb + 2 * NS + st, last));
      load(kS[st], vS[st], offs[st]);
      offs[st] = next;
    }
    if (jb + NS >= nblk) break;
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
          v4.x = acc[h][c][e4];
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

// Lanes per token: fewer lanes per token means fewer DPP reduction steps and
// less redundant softmax work per block, at the price of more accumulator
// registers per lane (head_dim / LPT floats per head).  8 for up to four heads
// per wave, 16 for eight (whose accumulators would not fit otherwise).
#ifndef PKV_DECODE_LPT_SMALL_GROUP
#define PKV_DECODE_LPT_SMALL_GROUP 8
#endif
#ifndef PKV_DECODE_STAGES
#define PKV_DECODE_STAGES 2
#endif
template <typename T, int D, int GB>
constexpr int lanes_per_token() {
  constexpr int row_chunks = D * (int)sizeof(T) / 16;
  constexpr int want = GB >= 8 ? 16 : PKV_DECODE_LPT_SMALL_GROUP;
  return row_chunks < want ? row_chunks : want;
}
// Register stages of the K/V prefetch pipeline.
template <typename T, int D, int GB>
constexpr int pipeline_stages() {
  return PKV_DECODE_STAGES;
}

template <typename T, int D, int GB>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int LPT = lanes_per_token<T, D, GB>();
  constexpr int NS = pipeline_stages<T, D, GB>();
  const int64_t rows = (int64_t)a.num_seqs * a.rows_per_seq;
  const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;
  const int64_t items = rows * a.num_kv_heads * hsubs * a.max_parts;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partition_kernel<T, D, GB, LPT, NS>), dim3((unsigned)items), dim3(64), 0, stream, a);
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
