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
#include <type_traits>

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

template <typename KV, int D, int GB, int LPT>
struct DecodeShape {
  using E = Elem<KV>;
  using Q = typename KvTraits<KV>::Q;                   // query / output element
  static constexpr int kElemBytes = KvTraits<KV>::kElemBytes;
  static constexpr int kRowBytes = D * kElemBytes;      // one token row of one kv head
  static constexpr int kEPC = E::kPerChunk;             // cache elements per 16-byte chunk
  static constexpr int kQPC = kEPC * (int)sizeof(Q) / 16;  // query chunks holding the same dims
  static constexpr int kRowChunks = D / kEPC;           // chunks per token row of one kv head
  static constexpr int kCPL = kRowChunks / LPT;         // chunks per lane per token
  static constexpr int kTPP = kWave / LPT;              // tokens covered by one load pass
  static constexpr int kPPB = kBlock / kTPP;            // passes (tokens per lane) per block
  // Blocks per pipeline tile: two when a block gives a lane a single token, so
  // that every tile still gives each lane a pair of tokens for the PV product.
  static constexpr int kBPT = kPPB == 1 ? 2 : 1;
  static constexpr int kNPass = kPPB * kBPT;            // tokens per lane per tile
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
// of the PV product.  E4M3 codes are widened exactly to bf16 pairs first, and
// prob already carries each token's V scale.
template <typename KV, int NP, int CPL, int GB>
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

template <int NP, int CPL, int GB>
struct PV<Fp8E4M3, NP, CPL, GB> {
  __device__ __forceinline__ static void apply(const float (&prob)[NP][GB], const Chunk (&vv)[NP][CPL],
                                               float (&acc)[GB][CPL][16]) {
    if constexpr (NP % 2 == 0) {
#pragma unroll
      for (int p = 0; p < NP; p += 2) {
        bf16x2_t pp[GB];
#pragma unroll
        for (int h = 0; h < GB; ++h) pp[h] = __builtin_bit_cast(bf16x2_t, pack_bf16x2(prob[p][h], prob[p + 1][h]));
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // interleave the codes of the two tokens (byte permute: token p's bytes
            // are selectors 0-3, token p+1's 4-7), so that each widening of a byte
            // pair yields (token p, token p+1) of one dim, the operand order of P
            const uint32_t a0 = vv[p][c].w[w], a1 = vv[p + 1][c].w[w];
            const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // dims 4w, 4w+1
            const uint32_t hi = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // dims 4w+2, 4w+3
            const bf16x2_t d0 = __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<false>(lo));
            const bf16x2_t d1 = __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<true>(lo));
            const bf16x2_t d2 = __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<false>(hi));
            const bf16x2_t d3 = __builtin_bit_cast(bf16x2_t, fp8x2_to_bf16x2<true>(hi));
            const int e = 4 * w;
#pragma unroll
            for (int h = 0; h < GB; ++h) {
              acc[h][c][e] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], d0, acc[h][c][e], false);
              acc[h][c][e + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], d1, acc[h][c][e + 1], false);
              acc[h][c][e + 2] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], d2, acc[h][c][e + 2], false);
              acc[h][c][e + 3] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], d3, acc[h][c][e + 3], false);
            }
          }
      }
    } else {  // one token per lane per block: widened values, plain FMAs
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
              const uint32_t b = hi ? fp8x2_to_bf16x2<true>(vv[p][c].w[w]) : fp8x2_to_bf16x2<false>(vv[p][c].w[w]);
              const int e = 4 * w + 2 * hi;
#pragma unroll
              for (int h = 0; h < GB; ++h) {
                acc[h][c][e] = fmaf(prob[p][h], bf16_lo(b), acc[h][c][e]);
                acc[h][c][e + 1] = fmaf(prob[p][h], bf16_hi(b), acc[h][c][e + 1]);
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

// bf16 caches take the matrix-core segment only with a deep register
// pipeline: its longer chain per block (score products, lane exchanges, the
// softmax, the LDS copy of V, value products) is hidden by three or four
// blocks in flight but not by two (the shared-prefix suffixes, two stages,
// with the scores alone on the matrix cores: 98.9 us per call against 94.3;
// the Llama-3-8B batch, four stages: 93.1 against 94.7 us).
#ifndef PKV_DECODE_MFMA_BF16_MIN_STAGES
#define PKV_DECODE_MFMA_BF16_MIN_STAGES 3
#endif

// One wave's attention state for GB query heads of one kv head over a run of
// consecutive blocks of one sequence (a "segment"): the query chunks, and per
// token group the running max m (log2 units), sum l and unnormalised output.
template <typename KV, int D, int GB, int LPT, int NS, int CT = 1>
struct Segment {
  using S = DecodeShape<KV, D, GB, LPT>;
  using E = typename S::E;
  using T = typename S::Q;
  static constexpr int EPC = S::kEPC, CPL = S::kCPL, TPP = S::kTPP, NP = S::kNPass, QPC = S::kQPC;
  static constexpr int PPB = S::kPPB, BPT = S::kBPT;
  // token (relative to the tile's first token of this lane) of pass p
  static constexpr int tok_of(int p) { return (p / PPB) * kBlock + (p % PPB) * TPP; }
  static constexpr int RB = S::kRowBytes;
  static constexpr bool kScaled = KvTraits<KV>::kScaled;
  // The matrix-core segment (bf16 and E4M3 caches, D = 128, four or eight
  // query heads per wave).  Scores: S = K Q^T for the block's 16 tokens is one
  // chain of four v_mfma_f32_16x16x32_bf16 products over the head dims, tokens
  // as rows and heads as columns (4 or 8 of 16 used): lane l = 16 g + n loads K bytes
  // [64 j + 16 g, +16) of token n (so a load covers 64 contiguous bytes of 16
  // rows) and holds Q^T's same dims for head n, and ends with the scores of
  // tokens 4 g .. 4 g + 3 for head n.  The softmax runs there, one running max
  // per head for the whole block (the four lane groups agree on it through two
  // lane swaps), so every token of a head accumulates at the same scale.
  // Values: O^T += V^T P^T is eight v_mfma_f32_16x16x16_bf16 products, one per
  // 16 dims, with P^T (bf16) straight from the score lanes (lane 16 g + n holds
  // the weights of tokens 4 g .. 4 g + 3 for head n, the B operand) and V^T
  // read from the wave's LDS copy of the block with ds_read_b64_tr_b16 (lane
  // j of group g addresses token 4 g + j / 4, dims 4 (j % 4) of a 16-dim slice,
  // and lane i receives dim i of tokens 4 g .. 4 g + 3); the copy's 8-byte
  // units are XOR-swizzled by token so that those reads hit distinct banks.
  // No partial dot products, no score reductions, no token groups to merge.
  // Columns: with several query rows per sequence (the rows that verify draft
  // tokens), column c = 16 ct + n of column tile ct is row c / GB, head c % GB
  // of the group, with its own causal end; CT tiles share the K chunks of the
  // score products and the V^T reads of the value products.
  static constexpr bool kMfma =
      (std::is_same<KV, Fp8E4M3>::value || (std::is_same<KV, __bf16>::value && NS >= PKV_DECODE_MFMA_BF16_MIN_STAGES)) &&
      D == 128 && (GB == 4 || GB == 8);
  static constexpr int kKC = RB / 64;  // K chunks per lane per block
  static_assert(!kMfma || (BPT == 1 && NP * CPL == kKC && TPP * NP == kBlock), "one block per tile");
  static_assert(CT == 1 || kMfma, "column tiles are a matrix-core segment layout");
  // scales carried per stage (one dummy entry when there are none)
  static constexpr int NSC = kScaled ? (kMfma ? 4 : NP) : 1;

  Chunk qv[GB][CPL][QPC];
  // matrix-core segment, per column tile ct (lane l holds column 16 ct + l % 16):
  bf16x8_t qa[CT][4];        // Q^T, the B operand of the four score products
  float mh[CT], lh[CT];      // running max / sum of the column (this lane's tokens)
  f32x4_t oacc[CT][D / 16];  // O^T, dims 16 t + 4 (l / 16) + i of the column
  int ckeys[CT];             // keys the column attends to (0: no such column)
  int cols;                  // columns in use: GB times the rows
  float m[GB], l[GB], acc[GB][CPL][EPC];
  bool bad_block;
  int tg, li;
  int lane_base;  // byte offset of this lane's first chunk inside a tile
  const char* __restrict__ kc;
  const char* __restrict__ vc;
  const float* __restrict__ ksc;  // per-(slot, kv head) scales of scaled caches
  const float* __restrict__ vsc;
  float sl2;

  static constexpr int64_t kTileBytes = (int64_t)kBlock * RB;

  __device__ __forceinline__ explicit Segment(const DecodeArgs& a) {
    const int lane = __lane_id();
    tg = lane / LPT;
    li = lane % LPT;
    lane_base = tg * RB + li * 16;
    kc = reinterpret_cast<const char*>(a.k_cache);
    vc = reinterpret_cast<const char*>(a.v_cache);
    ksc = a.k_scale;
    vsc = a.v_scale;
    sl2 = a.scale_log2;
  }

  // The chunks of the GB query rows at qrow (head h0 of the row) this lane
  // multiplies.  Matrix-core segment: nrows rows rstride elements apart, row r
  // attending to keys [0, min(end, key0 + r)).
  __device__ __forceinline__ void load_q(const T* __restrict__ qrow, int64_t rstride, int nrows, int key0, int end) {
    if constexpr (kMfma) {
      const int lane = __lane_id();
      const int hm = lane & 15, q = lane >> 4;
      cols = GB * nrows;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + hm, r = c / GB, h = c % GB;
        const bool live = c < cols;
        ckeys[ct] = live ? min(end, key0 + r) : 0;
        const T* qc = qrow + r * rstride + h * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the dims product i takes from lane group q (bf16: chunk i; E4M3: half i % 2 of chunk i / 2)
          const int dim = std::is_same<KV, __bf16>::value ? 32 * i + 8 * q : 64 * (i >> 1) + 16 * q + 8 * (i & 1);
          const Chunk ch = live ? load_chunk(qc + dim) : Chunk{};
          qa[ct][i] = as_bf16x8(ch.w[0], ch.w[1], ch.w[2], ch.w[3]);
        }
      }
      return;
    }
    constexpr int QE = 16 / (int)sizeof(T);  // query elements per chunk
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < QPC; ++j) qv[h][c][j] = load_chunk(qrow + h * D + (c * LPT + li) * EPC + j * QE);
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      m[h] = kMaxInit;
      l[h] = 0.0f;

#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][c][e] = 0.0f;
    }
    bad_block = false;
    if constexpr (kMfma) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        mh[ct] = kMaxInit;
        lh[ct] = 0.0f;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) oacc[ct][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }

  // The K and V tiles (16 tokens of one kv head each) of the BPT blocks of a
  // pipeline tile, block b at byte offset off[b] of the caches, of which the
  // first nbytes[b] bytes (whole token rows) are read.  Each block is a
  // buffer resource of that size over its tile, so rows past the context and
  // the blocks past a segment's end (size 0) come back as zeros without a
  // memory access, while the load instructions stay unconditional: one
  // constant per-lane offset plus immediates, nothing computed per lane
  // between the loads of consecutive tiles.
  __device__ __forceinline__ void load_tile(Chunk (&kk)[NP][CPL], Chunk (&vv)[NP][CPL], float (&sk)[NSC],
                                            float (&sv)[NSC], const int64_t (&off)[BPT],
                                            const int (&nbytes)[BPT]) const {
    constexpr int kAux = kStreamKV ? 2 : 0;  // cache policy: bit 1 = non-temporal
    if constexpr (kMfma) {
      const int lane = __lane_id();
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + off[0], nbytes[0]);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vc + off[0], nbytes[0]);
      const int kbase = (lane & 15) * RB + 16 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < kKC; ++j)
        kk[j / CPL][j % CPL] = as_chunk(__builtin_amdgcn_raw_buffer_load_b128(kr, kbase + 64 * j, 0, kAux));
#pragma unroll
      for (int pp = 0; pp < PPB; ++pp)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          vv[pp][c] = as_chunk(
              __builtin_amdgcn_raw_buffer_load_b128(vr, lane_base + pp * TPP * RB + c * LPT * 16, 0, kAux));
      if constexpr (kScaled) {  // the scales of this lane's tokens 4 g .. 4 g + 3 (one 16-byte row piece)
        const int64_t so = off[0] / RB + 4 * (lane >> 4);
        const float4 k4 = *reinterpret_cast<const float4*>(ksc + so);
        const float4 v4 = *reinterpret_cast<const float4*>(vsc + so);
        sk[0] = k4.x; sk[1] = k4.y; sk[2] = k4.z; sk[3] = k4.w;
        sv[0] = v4.x; sv[1] = v4.y; sv[2] = v4.z; sv[3] = v4.w;
      }
      return;
    }
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + off[b], nbytes[b]);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vc + off[b], nbytes[b]);
#pragma unroll
      for (int pp = 0; pp < PPB; ++pp)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int p = b * PPB + pp;
          const int o = lane_base + pp * TPP * RB + c * LPT * 16;
          kk[p][c] = as_chunk(__builtin_amdgcn_raw_buffer_load_b128(kr, o, 0, kAux));
          vv[p][c] = as_chunk(__builtin_amdgcn_raw_buffer_load_b128(vr, o, 0, kAux));
        }
    }
    if constexpr (kScaled) {
      // a block's 16 scales sit at (block * kv heads + kv head) * 16, i.e. its offset / RB
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int64_t so = off[p / PPB] / RB + tg + (p % PPB) * TPP;
        sk[p] = __builtin_nontemporal_load(ksc + so);
        sv[p] = __builtin_nontemporal_load(vsc + so);
      }
    }
  }

  // Attend the query rows over one tile whose first token (of this lane's
  // pass 0) is tok0; tokens at or past `end` are masked.  (A branch to a
  // select-free variant for whole blocks was measured slower: the two code
  // paths cost the register pipeline its fixed placement.)
  __device__ __forceinline__ void compute(const Chunk (&kk)[NP][CPL], const Chunk (&vv)[NP][CPL],
                                          const float (&sk)[NSC], const float (&sv)[NSC], int tok0, int end) {
    if constexpr (kMfma) {
      compute_mfma(kk, vv, sk, sv, tok0 - tg);
      return;
    }
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
    for (int p = 0; p < NP; ++p) {
      // scaled caches: the token's K scale multiplies its dot products
      const float f = kScaled ? sk[kScaled ? p : 0] * sl2 : sl2;
#pragma unroll
      for (int h = 0; h < GB; ++h) sc[p][h] = tok0 + tok_of(p) < end ? x[p * GB + h] * f : -__builtin_inff();
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
    // Rows past `end` were not read (the tile's buffer size stops at the
    // context): their V words are 0 and their weights 0, so they add exactly
    // nothing.  (Reading them could return the NaN a free slot holds, and
    // 0 * NaN would poison the sum.)
    if constexpr (kScaled) {  // the V scale joins the weights (the sums l keep the plain ones)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float f = tok0 + tok_of(p) < end ? sv[kScaled ? p : 0] : 0.0f;
#pragma unroll
        for (int h = 0; h < GB; ++h) sc[p][h] *= f;
      }
    }
    PV<KV, NP, CPL, GB>::apply(sc, vv, acc);
  }

  // The matrix-core segment's block (tile = one block; its first token blk_tok).
  __device__ __forceinline__ void compute_mfma(const Chunk (&kk)[NP][CPL], const Chunk (&vv)[NP][CPL],
                                               const float (&sk)[NSC], const float (&sv)[NSC], int blk_tok) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    // one 16-token x 128-dim bf16 V tile per wave (the workgroup is the wave)
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kBlock * D];
    const int lane = __lane_id();
    const int n = lane & 15, g = lane >> 4;
    // 8-byte unit u (dims 4u .. 4u + 3) of token t sits at unit u ^ swz(t)
    auto swz = [](int t) { return 4 * (t & 3) ^ 16 * ((t >> 2) & 1); };

    // V tile -> LDS as bf16 (value lane (tg, li) holds tokens tg + TPP p)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = tg + TPP * p;
      char* row = reinterpret_cast<char*>(vt_lds) + t * (D * 2);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if constexpr (std::is_same<KV, __bf16>::value) {  // 8 dims: units 2 (8 c + li), +1
          const int u = 2 * (c * LPT + li);
          *reinterpret_cast<uint4*>(row + (u ^ swz(t)) * 8) =
              make_uint4(vv[p][c].w[0], vv[p][c].w[1], vv[p][c].w[2], vv[p][c].w[3]);
        } else {  // 16 codes (dims 16 (c LPT + li) .. + 15) widened: four units
          const Chunk& v = vv[p][c];
          const int u = 4 * (c * LPT + li);
          *reinterpret_cast<uint4*>(row + (u ^ swz(t)) * 8) =
              make_uint4(fp8x2_to_bf16x2<false>(v.w[0]), fp8x2_to_bf16x2<true>(v.w[0]),
                         fp8x2_to_bf16x2<false>(v.w[1]), fp8x2_to_bf16x2<true>(v.w[1]));
          *reinterpret_cast<uint4*>(row + ((u + 2) ^ swz(t)) * 8) =
              make_uint4(fp8x2_to_bf16x2<false>(v.w[2]), fp8x2_to_bf16x2<true>(v.w[2]),
                         fp8x2_to_bf16x2<false>(v.w[3]), fp8x2_to_bf16x2<true>(v.w[3]));
        }
      }
    }

    // scores S[token 4 g + i][column n] of each column tile
    f32x4_t d[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) d[ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8_t a;
      if constexpr (std::is_same<KV, __bf16>::value) {
        const Chunk& c = kk[i / CPL][i % CPL];
        a = as_bf16x8(c.w[0], c.w[1], c.w[2], c.w[3]);
      } else {  // E4M3: codes 8 (i % 2) .. 8 (i % 2) + 7 of chunk i / 2, widened exactly
        const Chunk& c = kk[(i >> 1) / CPL][(i >> 1) % CPL];
        const int w = (i & 1) * 2;
        a = as_bf16x8(fp8x2_to_bf16x2<false>(c.w[w]), fp8x2_to_bf16x2<true>(c.w[w]),
                      fp8x2_to_bf16x2<false>(c.w[w + 1]), fp8x2_to_bf16x2<true>(c.w[w + 1]));
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) d[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qa[ct][i], d[ct], 0, 0, 0);
    }
    s16x4_t pt[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float s[4], bm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = blk_tok + 4 * g + i < ckeys[ct];  // never for a column not in use
        s[i] = live ? d[ct][i] * (kScaled ? sk[kScaled ? i : 0] * sl2 : sl2) : -__builtin_inff();
        bm = fmaxf(bm, s[i]);
      }
      bm = xor_max<32>(xor_max<16>(bm));  // the block max of column n, in all four lane groups
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(bm > mh[ct] + kRescaleSlack) != 0, 0)) {
        const float mn = fmaxf(mh[ct], bm);
        const float alpha = fast_exp2(mh[ct] - mn);
        mh[ct] = mn;
        lh[ct] *= alpha;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) oacc[ct][t] *= alpha;
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = fast_exp2(s[i] - mh[ct]);  // 0 for a masked token or an unused column
        lh[ct] += pr;
        // scaled caches: the token's V scale joins the weight (the sum keeps the plain one)
        pv[i] = kScaled ? (s[i] > -__builtin_inff() ? pr * sv[kScaled ? i : 0] : 0.0f) : pr;
      }
      const uint32_t p01 = pack_bf16x2(pv[0], pv[1]), p23 = pack_bf16x2(pv[2], pv[3]);
      pt[ct] = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
    }

    // O^T[16 t .. 16 t + 15][column] += V^T P^T (one V^T read serves every column tile)
    const int tt = 4 * g + (n >> 2);  // the token this lane addresses for the transposing reads
    const char* rrow = reinterpret_cast<const char*>(vt_lds) + tt * (D * 2);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int u = 4 * t + (n & 3);
      const s16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(rrow + (u ^ swz(tt)) * 8));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        oacc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pt[ct], oacc[ct][t], 0, 0, 0);
    }
  }

  // Start from the attention state of a shared prefix: the a.init_splits
  // partials of rows [row, row + GB) (sequence * Hq + head) merged into token
  // group 0 (the other groups start empty; merge_groups combines them later).
  __device__ __forceinline__ void seed(const DecodeArgs& a, int64_t row) {
    if (tg != 0) return;
    // One partial per row (bf16 caches, the only ones the shared-prefix call
    // takes): the state is copied as it stands, every load of the GB rows in
    // flight together (the general loop below waits on each row's (m, l)
    // before it reads that row's output).
    if (std::is_same<KV, __bf16>::value && a.init_splits == 1) {
      static_assert(EPC % 4 == 0, "16-byte loads of the partial outputs");
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const float2 ml = *reinterpret_cast<const float2*>(a.init_ml + (row + h) * 2);
        m[h] = ml.x;
        l[h] = ml.y;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(a.init_o + (row + h) * D + (c * LPT + li) * EPC + e);
            acc[h][c][e] = v.x;
            acc[h][c][e + 1] = v.y;
            acc[h][c][e + 2] = v.z;
            acc[h][c][e + 3] = v.w;
          }
      }
#pragma unroll
      for (int h = 0; h < GB; ++h) bad_block |= m[h] != m[h];
      return;
    }
    const int64_t split_stride = (int64_t)a.num_seqs * a.num_q_heads;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float M = -__builtin_inff();
      for (int sp = 0; sp < a.init_splits; ++sp) {
        const float ms = a.init_ml[(sp * split_stride + row + h) * 2];
        bad_block |= ms != ms;
        M = fmaxf(M, ms);
      }
      float lam = 0.0f;
      for (int sp = 0; sp < a.init_splits; ++sp) {
        const int64_t r = sp * split_stride + row + h;
        const float f = fast_exp2(a.init_ml[r * 2] - M);
        lam = fmaf(f, a.init_ml[r * 2 + 1], lam);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][c][e] = fmaf(f, a.init_o[r * D + (c * LPT + li) * EPC + e], acc[h][c][e]);
      }
      m[h] = M;
      l[h] = lam;
    }
  }

  // Attend the GB query rows at qrow (head h0 of the row) over tokens
  // [16 * blk0, end) of one sequence, whose blocks blk0 .. blk0 + nblk - 1 are
  // listed at table[0 .. nblk - 1], for kv head g; seed_row >= 0 starts from
  // the shared-prefix state of that row (see seed).  Matrix-core segment with
  // several rows: nrows rows rstride elements apart, row r seeing the keys
  // before min(end, key0 + r).
  __device__ __forceinline__ void run(const DecodeArgs& a, const T* __restrict__ qrow,
                                      const int32_t* __restrict__ table, int g, int blk0, int nblk, int end,
                                      int64_t seed_row = -1, int64_t rstride = 0, int nrows = 1,
                                      int key0 = 0x7fffffff) {
    load_q(qrow, rstride, nrows, key0, end);
    reset();
    if (seed_row >= 0) {
      // The shared-prefix call runs the two-stage vector-ALU segment, which
      // takes a seed; the matrix-core segment has none and would drop the
      // prefix, so it marks the row bad (NaN) instead.
      if constexpr (kMfma)
        bad_block = true;
      else
        seed(a, seed_row);
    }
    const int64_t blk_stride = kTileBytes * a.num_kv_heads;
    const int num_blocks = a.num_blocks;
    // Table entries are uniform: scalar loads (the table is a read-only,
    // non-aliased argument), counted apart from the vector K/V loads.
    auto tile_off = [&](int p) -> int64_t {
      if (p < 0 || p >= num_blocks) {
        bad_block = true;
        p = 0;
      }
      return (int64_t)p * blk_stride + (int64_t)g * kTileBytes;
    };
    auto block_off = [&](int jb) -> int64_t { return tile_off(table[jb]); };
    // bytes of segment block jb that hold tokens before `end` (0 past the segment)
    auto block_bytes = [&](int jb) -> int {
      const int v = end - (blk0 + jb) * kBlock;
      return v <= 0 ? 0 : (v >= kBlock ? kBlock * RB : v * RB);
    };

    // NS register stages of BPT blocks each: while tile jt is computed, tiles
    // jt+1 .. jt+NS-1 are in flight and tile jt+NS is issued right after.  The
    // prologue fills every stage so that the loop is entered in its steady
    // state; past the end the loads have a buffer size of 0 (no memory access,
    // zeros), so no load is conditional.  The body computes NS tiles and exits
    // only at its end (a single exit keeps the accumulators in place); blocks
    // past the last one lie wholly past `end`, are masked and add exactly
    // nothing.  Table entries are fetched one pass ahead.
    constexpr int TB = NS * BPT;  // blocks per loop pass
    Chunk kS[NS][NP][CPL], vS[NS][NP][CPL];
    float skS[NS][NSC], svS[NS][NSC];
    const int last = nblk - 1;
    int64_t offs[NS][BPT];
    int nbs[NS][BPT];
    int first[2 * TB];  // the first 2 NS tiles' entries, fetched together
#pragma unroll
    for (int i = 0; i < 2 * TB; ++i) first[i] = table[min(i, last)];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      int64_t o[BPT];
      int nb[BPT];
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        o[b] = tile_off(first[st * BPT + b]);
        nb[b] = block_bytes(st * BPT + b);
      }
      load_tile(kS[st], vS[st], skS[st], svS[st], o, nb);
      // each stage's loads are issued before the next stage's: waits are in order
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        offs[st][b] = tile_off(first[TB + st * BPT + b]);
        nbs[st][b] = block_bytes(TB + st * BPT + b);
      }
    for (int jb = 0;; jb += TB) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        compute(kS[st], vS[st], skS[st], svS[st], (blk0 + jb + st * BPT) * kBlock + tg, end);
        int64_t next[BPT];
        int nextb[BPT];
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          next[b] = block_off(min(jb + 2 * TB + st * BPT + b, last));
          nextb[b] = block_bytes(jb + 2 * TB + st * BPT + b);
        }
        load_tile(kS[st], vS[st], skS[st], svS[st], offs[st], nbs[st]);
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          offs[st][b] = next[b];
          nbs[st][b] = nextb[b];
        }
      }
      if (jb + TB >= nblk) break;
    }
  }

  // The token groups' outputs are combined by a reduce-scatter: each halving
  // step across one lane bit that separates the groups (permlane32 / permlane16
  // swaps, a row rotate by 8) adds the partner's half of the values this lane
  // keeps and drops the other half, so that after the last step the lanes of
  // group tg hold the totals of flat values [tg * kR, (tg + 1) * kR) of the
  // [GB][CPL][EPC] output (head-major), and every group stores one piece.
  // Against an all-reduce of all GB * CPL * EPC values this moves and adds
  // kN (1/2 + 1/4 + 1/8) values instead of 3 kN.
  static constexpr int kGroups = kWave / LPT;
  static constexpr int kN = GB * CPL * EPC;
  static constexpr int kR = kN / kGroups;                     // values a lane keeps
  static constexpr int kRun = kR < EPC ? kR : EPC;            // contiguous dims of one store
  static constexpr bool kScatter = (LPT == 8 || LPT == 16) && kN % kGroups == 0 &&
                                   (kR <= EPC ? EPC % kR == 0 : kR % EPC == 0) && kRun % 4 == 0 &&
                                   (kRun * (int)sizeof(T)) % 16 == 0;

  // Flat value v of the [GB][CPL][EPC] outputs (v a constant once the loops
  // around a call are unrolled, so the array stays in registers).
  __device__ __forceinline__ float& at(int v) { return acc[v / (CPL * EPC)][(v / EPC) % CPL][v % EPC]; }
  __device__ __forceinline__ float at(int v) const { return acc[v / (CPL * EPC)][(v / EPC) % CPL][v % EPC]; }

  // Flat values [0, N) -> [0, N / 2): lanes whose bit 5 (k32) or bit 4 is
  // clear keep the totals of the first half, the others those of the second.
  template <int N, bool k32>
  __device__ __forceinline__ void halve_swap() {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint32_t a = __builtin_bit_cast(uint32_t, at(i)), b = __builtin_bit_cast(uint32_t, at(i + N / 2));
      const auto r = k32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                         : __builtin_amdgcn_permlane16_swap(a, b, false, false);
      at(i) = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }
  }
  // The same across lane bit 3 (lanes l and l ^ 8 of a row of 16: rotate by 8).
  template <int N>
  __device__ __forceinline__ void halve_ror8() {
    const bool upper = (__lane_id() & 8) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float send = upper ? at(i) : at(i + N / 2);
      const float mine = upper ? at(i + N / 2) : at(i);
      at(i) = mine + dpp_f32<0x128>(send);
    }
  }

  // Combine the 64 / LPT token-group streams: agree on the largest running
  // max and rescale to it; m and l are summed into every lane, the outputs too
  // where the reduce-scatter does not apply (else the store that follows
  // scatters them).
  __device__ __forceinline__ void merge_groups() {
    static_assert(LPT == 4 || LPT == 8 || LPT == 16, "token groups differ in lane bits 2..5, 3..5 or 4..5");
    bad_block = __builtin_amdgcn_ballot_w64(bad_block) != 0;
    if constexpr (kMfma) {  // one running max per column already; the sums of the four lane groups
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) lh[ct] = xor_add<32>(xor_add<16>(lh[ct]));
      return;
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float M = groups_max<LPT>(m[h]);
      const float f = fast_exp2(m[h] - M);
      m[h] = M;
      l[h] = groups_add<LPT>(l[h] * f);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][c][e] = kScatter ? acc[h][c][e] * f : groups_add<LPT>(acc[h][c][e] * f);
    }
  }

  // The reduce-scatter itself (the stores call it once, after merge_groups).
  __device__ __forceinline__ void scatter() {
    halve_swap<kN, true>();
    halve_swap<kN / 2, false>();
    if constexpr (LPT == 8) halve_ror8<kN / 4>();
  }

  // Which of the GB heads flat value tg * kR + r (this lane's kept range)
  // belongs to, and the output offset of its dims: head * D + (c * LPT + li) *
  // EPC + e.
  __device__ __forceinline__ int kept_offset(int r, int& head) const {
    const int v = tg * kR + r;
    head = v / (CPL * EPC);
    const int c = (v / EPC) % CPL, e = v % EPC;
    return head * D + (c * LPT + li) * EPC + e;
  }
  // Normalised output of the GB heads at outp (head h0 of the row; matrix-core
  // segment: row r of the columns at outp + r * rstride).
  __device__ __forceinline__ void store_out(T* __restrict__ outp, int64_t rstride = 0) {
    const float nan = __builtin_nanf("");
    if constexpr (kMfma) {  // lane 16 g + n: dims 16 t + 4 g .. + 3 of column 16 ct + n
      const int lane = __lane_id();
      const int n = lane & 15, g = lane >> 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + n, r = c / GB, h = c % GB;
        if (c >= cols) continue;
        const float inv = bad_block ? nan : 1.0f / lh[ct];
        T* o = outp + r * rstride + h * D;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          *reinterpret_cast<uint2*>(o + 16 * t + 4 * g) =
              make_uint2(pack_bf16x2(oacc[ct][t][0] * inv, oacc[ct][t][1] * inv),
                         pack_bf16x2(oacc[ct][t][2] * inv, oacc[ct][t][3] * inv));
      }
      return;
    }
    if constexpr (kScatter) {
      // normalise per head first (every head's sum is in every lane), then scatter
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const float inv = bad_block ? nan : 1.0f / l[h];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][c][e] *= inv;
      }
      scatter();
      constexpr int QE = 16 / (int)sizeof(T);  // output elements per 16-byte store
#pragma unroll
      for (int r = 0; r < kR; r += kRun) {
        int head;
        const int off = kept_offset(r, head);
#pragma unroll
        for (int j = 0; j < kRun; j += QE) {
          float o[QE];
#pragma unroll
          for (int e = 0; e < QE; ++e) o[e] = at(r + j + e);
          store_chunk(outp + off + j, Elem<T>::narrow(o));
        }
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (tg != h % TPP) continue;
      const float inv = bad_block ? nan : 1.0f / l[h];
      constexpr int QE = 16 / (int)sizeof(T);  // output elements per chunk
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < QPC; ++j) {
          float o[QE];
#pragma unroll
          for (int e = 0; e < QE; ++e) o[e] = acc[h][c][j * QE + e] * inv;
          store_chunk(outp + h * D + (c * LPT + li) * EPC + j * QE, Elem<T>::narrow(o));
        }
    }
  }

  // Partial (m, l, unnormalised o) of head h (matrix-core segment: column h)
  // at po + h * ostride (D floats) and pml + h * mlstride (2 floats).
  __device__ __forceinline__ void store_partial(float* __restrict__ po, int64_t ostride, float* __restrict__ pml,
                                                int64_t mlstride) {
    const float nan = __builtin_nanf("");
    if constexpr (kMfma) {
      const int lane = __lane_id();
      const int n = lane & 15, g = lane >> 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + n;
        if (c >= cols) continue;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          *reinterpret_cast<float4*>(po + c * ostride + 16 * t + 4 * g) =
              make_float4(oacc[ct][t][0], oacc[ct][t][1], oacc[ct][t][2], oacc[ct][t][3]);
        if (g == 0) {
          pml[c * mlstride] = bad_block ? nan : mh[ct];
          pml[c * mlstride + 1] = lh[ct];
        }
      }
      return;
    }
    if constexpr (kScatter) {
      scatter();
#pragma unroll
      for (int r = 0; r < kR; r += kRun) {
        int head;
        const int off = kept_offset(r, head);
        float* o = po + head * ostride + (off - head * D);
#pragma unroll
        for (int j = 0; j < kRun; j += 4) {
          float4 v4;
          v4.x = at(r + j);
          v4.y = at(r + j + 1);
          v4.z = at(r + j + 2);
          v4.w = at(r + j + 3);
          *reinterpret_cast<float4*>(o + j) = v4;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (tg != h % TPP) continue;
      if constexpr (!kScatter) {
        float* o = po + h * ostride;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e4 = 0; e4 < EPC; e4 += 4) {
            float4 v4;
            v4.x = acc[h][c][e4];
            v4.y = acc[h][c][e4 + 1];
            v4.z = acc[h][c][e4 + 2];
            v4.w = acc[h][c][e4 + 3];
            *reinterpret_cast<float4*>(o + (c * LPT + li) * EPC + e4) = v4;
          }
      }
      if (li == 0) {
        pml[h * mlstride] = bad_block ? nan : m[h];
        pml[h * mlstride + 1] = l[h];
      }
    }
  }
};

// Fixed partitions: one wave per (query row, kv head, head subgroup,
// partition of P tokens).  Also serves float32 prefill rows (one partition
// covering the whole table).
template <typename KV, int D, int GB, int LPT, int NS>
__global__ __launch_bounds__(64) void decode_partition_kernel(const DecodeArgs a, const int32_t* __restrict__ tables) {
  using T = typename KvTraits<KV>::Q;
  const int lane = __lane_id();
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

  Segment<KV, D, GB, LPT, NS> seg(a);
  const T* qrow = reinterpret_cast<const T*>(a.q) + (row * a.num_q_heads + h0) * (int64_t)D;
  seg.run(a, qrow, tables + (int64_t)ri.seq * a.max_blocks_per_seq + blk0, g, blk0, nblk, end);
  seg.merge_groups();
  if (nparts == 1) {
    seg.store_out(outp);
  } else {
    const int64_t pidx = (row * a.num_q_heads + h0) * (int64_t)a.max_parts + part;
    seg.store_partial(a.part_o + pidx * D, (int64_t)a.max_parts * D, a.part_ml + pidx * 2,
                      (int64_t)a.max_parts * 2);
  }
}

// Log-sum-exp merge of the partitions of every (query row, query head) whose
// context spans more than one partition.  One wave per (row, head); lane k
// owns output dims k, k + 64, ...  The partitions of a row are consecutive in
// the workspace ([row][head][max_parts]), so merge_partials reads them with
// stride 1, every (m, l) load in flight at once.
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
  float o[PER], M, lam;
  bool nan;
  merge_partials<D>(a.part_o, a.part_ml, (row * a.num_q_heads + h) * (int64_t)a.max_parts, 1, nparts, o, M, lam,
                    nan);
  const float inv = nan ? __builtin_nanf("") : 1.0f / lam;
  T* outp = reinterpret_cast<T*>(a.out) + (row * a.num_q_heads + h) * (int64_t)D;
#pragma unroll
  for (int k = 0; k < PER; ++k) outp[lane + k * kWave] = (T)(o[k] * inv);
}

// The merge on its own (paged_attn_lse_merge): row r's parts partials at
// [r][p] of part_o ([rows][parts][D]) and part_ml ([rows][parts][2]), the
// normalised result to out [rows][D].  One wave per row.
template <typename T, int D>
__global__ __launch_bounds__(64) void lse_merge_kernel(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml, int64_t rows, int parts,
                                                       T* __restrict__ out) {
  constexpr int PER = D / kWave;
  const int lane = __lane_id();
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  float o[PER], M, lam;
  bool nan;
  merge_partials<D>(part_o, part_ml, row * parts, 1, parts, o, M, lam, nan);
  const float inv = nan ? __builtin_nanf("") : 1.0f / lam;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[row * D + lane + k * kWave] = (T)(o[k] * inv);
}

template <typename T>
static hipError_t launch_lse_merge_typed(const float* part_o, const float* part_ml, int64_t rows, int parts,
                                         int head_dim, void* out, hipStream_t stream) {
  T* o = reinterpret_cast<T*>(out);
  if (head_dim == 64)
    hipLaunchKernelGGL((lse_merge_kernel<T, 64>), dim3((unsigned)rows), dim3(64), 0, stream, part_o, part_ml, rows,
                       parts, o);
  else if (head_dim == 128)
    hipLaunchKernelGGL((lse_merge_kernel<T, 128>), dim3((unsigned)rows), dim3(64), 0, stream, part_o, part_ml, rows,
                       parts, o);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int64_t rows, int parts, int head_dim,
                            int out_dtype, void* out, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (rows > 0x7fffffffLL || parts <= 0) return hipErrorInvalidValue;
  if (out_dtype == 0) return launch_lse_merge_typed<float>(part_o, part_ml, rows, parts, head_dim, out, stream);
  if (out_dtype == 1) return launch_lse_merge_typed<__bf16>(part_o, part_ml, rows, parts, head_dim, out, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- balanced split
//
// The work of a decode step is the list of streams (sequence s, stream k),
// k = (kv head, head subgroup), ordered by s then k.  A stream of nb blocks
// costs nb + kSegCost: one unit per K/V block plus a fixed charge, in block
// units, for what every segment pays once (reading q, filling the load
// pipeline, combining the token groups and storing).  With total cost C and W
// waves, wave w takes the cost interval [w C / W, (w+1) C / W); the first
// kSegCost units of a stream stand for its fixed charge and the next nb units
// are its blocks, so a wave that starts several short streams reads fewer
// blocks and every wave finishes at about the same time whatever the mix of
// context lengths.  A stream whose blocks lie wholly inside one wave's
// interval is finished there; a stream cut by an interval boundary leaves
// (m, l, o) partials -- a wave has at most two: its first segment (slot 0) and
// its last (slot 1) -- which the merge kernel combines.
//
// Sequences with a context outside [0, 16 * max_blocks] contribute no cost;
// the merge kernel writes NaN for them (and 0 for an empty context).
//
// The charge is 4 block units.  Measured on one box, cold caches, two
// rounds each (us per call; charge 2 / 3 / 4 / 5 / 6 / 8): Llama-3-8B batch
// 89.5 / 90.4 / 89.6 / 90.0 / 90.3 / 91.8; its fp8 cache 56.5 / 56.2 / 55.8 /
// 55.5 / 55.7 / 56.0; the shared-prefix call 95.9 / 94.3 / 93.2 / 93.6 / 93.2
// / 93.7; the verify pass (64 x 5 rows) 105.0 / 102.7 / 101.4 / 101.6 / - /
// 102.7; the mixed step's decode 137.3 / 137.6 / 137.3 / 137.7 / 137.8 /
// 138.4; the long-context batch is the same at 4, 6 and 8 (457-458).

#ifndef PKV_SEGMENT_COST
#define PKV_SEGMENT_COST 4
#endif
constexpr int kSegCost = PKV_SEGMENT_COST;

__device__ __forceinline__ int seq_blocks(int L, int cap) { return (L >= 0 && L <= cap) ? (L + kBlock - 1) / kBlock : 0; }

// Blocks a sequence's streams read.  Decode: its context.  The rows that
// verify draft tokens (starts != nullptr, up to R rows from position
// starts[s]): the keys of the last row, which are the whole context.  A
// sequence outside its contract, or with no rows, reads nothing (the merge
// kernel writes its NaN rows).
template <bool VR>
__device__ __forceinline__ int stream_blocks(int L, int P0, int cap, int R) {
  if constexpr (VR) {
    const int n = L - P0;
    return (P0 >= 0 && n >= 1 && n <= R && L <= cap) ? (L + kBlock - 1) / kBlock : 0;
  } else {
    return seq_blocks(L, cap);
  }
}

// Cost of all HH streams of a sequence with nb blocks.
__device__ __forceinline__ int64_t seq_cost(int nb, int HH) { return nb > 0 ? (int64_t)HH * (nb + kSegCost) : 0; }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// x + (x of the lane that DPP control kCtrl names), 0 where it names none.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int64_t dpp_add_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)x, kCtrl, kRowMask, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)((uint64_t)x >> 32), kCtrl, kRowMask, 0xF, false);
  return x + (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes (DPP: row_shr within rows of 16,
// then row_bcast:15 / row_bcast:31 across rows).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t x) {
  x = dpp_add_i64<0x111>(x);         // row_shr:1
  x = dpp_add_i64<0x112>(x);         // row_shr:2
  x = dpp_add_i64<0x114>(x);         // row_shr:4
  x = dpp_add_i64<0x118>(x);         // row_shr:8
  x = dpp_add_i64<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
  x = dpp_add_i64<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
  return x;
}

// Total cost over all sequences, and the cost of the sequences before s
// (every lane gets both); one pass over the lengths (and row starts).
template <bool VR>
__device__ __forceinline__ void cost_counts(const int32_t* __restrict__ lens, const int32_t* __restrict__ starts,
                                            int B, int s, int cap, int R, int HH, int64_t& total, int64_t& before) {
  total = 0;
  before = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int i = c0 + __lane_id();
    const int64_t incl =
        wave_incl_scan(i < B ? seq_cost(stream_blocks<VR>(lens[i], VR ? starts[i] : 0, cap, R), HH) : 0);
    const int64_t all = readlane64(incl, kWave - 1);
    total += all;
    if (s >= c0 + kWave) {
      before += all;
    } else if (s > c0) {
      before += readlane64(incl, s - c0 - 1);
    }
  }
  total = uniform64(total);
  before = uniform64(before);
}

// Total blocks of all sequences times HH (every lane gets it).
__device__ __forceinline__ void cost_counts_blocks(const int32_t* __restrict__ lens, int B, int cap, int HH,
                                                   int64_t& total, int64_t& unused) {
  total = 0;
  unused = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int i = c0 + __lane_id();
    const int64_t incl = wave_incl_scan(i < B ? (int64_t)seq_blocks(lens[i], cap) * HH : 0);
    total += readlane64(incl, kWave - 1);
  }
  total = uniform64(total);
}

__device__ __forceinline__ int64_t range_begin(int w, int W, int64_t U) { return (int64_t)w * U / W; }
// The wave whose range holds cost unit u.
__device__ __forceinline__ int wave_of(int64_t u, int W, int64_t U) { return (int)(((u + 1) * W + U - 1) / U) - 1; }

// VR: the rows that verify draft tokens (a.chunk_start: first row position
// per sequence, a.rows_per_seq rows at most), row r of a sequence seeing the
// keys before a.chunk_start[s] + r + 1; a stream's GB heads x rows are the
// columns of CT matrix-core column tiles, and a partial slot holds 16 CT
// columns.  Otherwise a decode (one row).
template <typename KV, int D, int GB, int LPT, int NS, int CT = 1, bool VR = false>
__global__ __launch_bounds__(64) void decode_balanced_kernel(const DecodeArgs a, const int32_t* __restrict__ tables,
                                                              const int32_t* __restrict__ lens) {
  using T = typename KvTraits<KV>::Q;
  constexpr int kSlotCols = VR ? 16 * CT : GB;  // columns of a partial slot
  const int lane = __lane_id();
  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int B = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hsubs = G / GB;
  const int HH = a.num_kv_heads * hsubs;  // streams per sequence
  const int cap = a.max_blocks_per_seq * kBlock;
  const int R = VR ? a.rows_per_seq : 1;
  const int32_t* __restrict__ starts = a.chunk_start;

  // A batch of at most 64 sequences keeps every length in a lane: one load
  // gives the total cost, this wave's first sequence and every later length
  // (the start of the kernel is one dependent load shorter, and moving to the
  // next sequence needs none).
  const bool small = B <= kWave;
  const int Llane = small && lane < B ? lens[lane] : 0;
  const int Plane = VR && small && lane < B ? starts[lane] : 0;
  int64_t U;
  int s = 0;
  int64_t cum = 0;
  int L, P0 = 0;
  int64_t u0, u1;
  if (small) {
    const int64_t c = lane < B ? seq_cost(stream_blocks<VR>(Llane, Plane, cap, R), HH) : 0;
    const int64_t incl = wave_incl_scan(c);
    U = uniform64(readlane64(incl, kWave - 1));
    u0 = range_begin(w, W, U);
    u1 = range_begin(w + 1, W, U);
    if (u0 >= u1) return;
    // the sequence s whose cost interval [cum, cum + cost) holds u0 (one exists: u0 < U)
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && incl > u0);
    s = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
    cum = uniform64(readlane64(incl - c, s));
    L = __builtin_amdgcn_readlane(Llane, s);
    if constexpr (VR) P0 = __builtin_amdgcn_readlane(Plane, s);
  } else {
    int64_t unused;
    cost_counts<VR>(lens, starts, B, 0, cap, R, HH, U, unused);
    u0 = range_begin(w, W, U);
    u1 = range_begin(w + 1, W, U);
    if (u0 >= u1) return;
    // locate u0: the sequence s whose cost interval [cum, cum + cost) holds it
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int i = c0 + lane;
      const int64_t c = i < B ? seq_cost(stream_blocks<VR>(lens[i], VR ? starts[i] : 0, cap, R), HH) : 0;
      const int64_t incl = wave_incl_scan(c);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(i < B && cum + incl > u0);
      if (hit) {
        const int ln = __builtin_ctzll(hit);
        s = c0 + ln;
        cum += readlane64(incl - c, ln);
        break;
      }
      cum += readlane64(incl, kWave - 1);
    }
    s = __builtin_amdgcn_readfirstlane(s);
    cum = uniform64(cum);
    L = lens[s];
    if constexpr (VR) P0 = starts[s];
  }

  Segment<KV, D, GB, LPT, NS, CT> seg(a);
  int nb = stream_blocks<VR>(L, P0, cap, R);
  bool first = true;
  for (int64_t u = u0;;) {
    const int64_t span = nb + kSegCost;  // cost of one stream of sequence s
    const int k = (int)((u - cum) / span);
    const int64_t sb = cum + (int64_t)k * span + kSegCost;  // the stream's first block
    const int64_t ub = u > sb ? u : sb;
    if (ub >= u1) break;  // the rest of the range is the stream's fixed charge
    const int64_t seg_end = min(u1, sb + nb);
    const int j = (int)(ub - sb), jn = (int)(seg_end - sb);
    const int g = k / hsubs, hs = k - g * hsubs;
    const int h0 = g * G + hs * GB;
    const int64_t row0 = ((int64_t)s * R * a.num_q_heads + h0) * D;  // head h0 of the sequence's first row
    const int64_t rstride = (int64_t)a.num_q_heads * D;
    const T* qrow = reinterpret_cast<const T*>(a.q) + row0;
    const int32_t* tab = tables + (int64_t)s * a.max_blocks_per_seq + j;
    if constexpr (VR)
      seg.run(a, qrow, tab, g, j, jn - j, min(L, jn * kBlock), -1, rstride, L - P0, P0 + 1);
    else
      seg.run(a, qrow, tab, g, j, jn - j, min(L, jn * kBlock),
              (a.init_o != nullptr && j == 0) ? (int64_t)s * a.num_q_heads + h0 : -1);
    seg.merge_groups();
    if (j == 0 && jn == nb) {
      seg.store_out(reinterpret_cast<T*>(a.out) + row0, rstride);
    } else {
      const int64_t slot = (int64_t)w * 2 + (first ? 0 : 1);
      seg.store_partial(a.part_o + slot * kSlotCols * D, D, a.part_ml + slot * kSlotCols * 2, 2);
    }
    first = false;
    u = seg_end;
    if (u >= u1) break;
    if (k + 1 == HH) {  // next sequence that has blocks (one exists: u < U)
      cum += (int64_t)HH * span;
      do {
        ++s;
        L = small ? __builtin_amdgcn_readlane(Llane, s) : lens[s];
        if constexpr (VR) P0 = small ? __builtin_amdgcn_readlane(Plane, s) : starts[s];
        nb = stream_blocks<VR>(L, P0, cap, R);
      } while (nb == 0);
    }
  }
}

// One wave per (sequence, stream, HM heads of the stream's group of GB):
// writes NaN / 0 for sequences with an invalid / empty context, and merges the
// partials of a stream that was cut across wave ranges.  The loads are issued
// together, not one owner after the other: lane j examines candidate wave
// wf + j (the owners of a stream are consecutive waves, except for empty
// ranges when waves outnumber units) and loads its (m, l); the outputs of the
// first kPre owners are loaded at the same time, and the sum over the owners
// has lane k owning dims k, k + 64, ...  HM = 1 (one head per wave) suits
// batches of few, long streams: the long-context batch's 64 streams have 32
// owners each, and its merge takes 14 us against 21 us with the whole group
// per wave; with many streams every wave repeats the cost scan over the
// lengths, and the whole group per wave is faster (the 256-sequence batch,
// 2048 streams: the call took 104 us with one head per wave against 100 us).
//
// VR (the rows that verify draft tokens): one wave per (sequence, stream,
// row, HM heads), the partial columns of row r being r GB .. r GB + GB - 1; a
// partial slot holds SC columns.  A sequence outside its contract gets NaN in
// all its rows; rows past its count are not written.
template <typename T, int D, int GB, int HM, bool VR = false, int SC = GB>
__global__ __launch_bounds__(64) void decode_balanced_merge_kernel(const DecodeArgs a, int W) {
  constexpr int PER = D / kWave;
  constexpr int kPre = HM == 1 ? 16 : 4;
  static_assert(GB % HM == 0, "a wave takes a whole share of the group");
  const int lane = __lane_id();
  const int B = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hsubs = G / GB;
  const int HH = a.num_kv_heads * hsubs;
  const int cap = a.max_blocks_per_seq * kBlock;
  const int R = VR ? a.rows_per_seq : 1;
  const int CW = R * (GB / HM);  // waves per stream
  const int cw = blockIdx.x % CW;
  const int stream = blockIdx.x / CW;       // (sequence, stream)
  const int r = cw / (GB / HM);             // row of the sequence (decode: 0)
  const int hh0 = (cw % (GB / HM)) * HM;    // first head of this wave within the stream's group
  const int pc0 = r * GB + hh0;             // its first column in a partial slot
  const int s = stream / HH;
  const int k = stream - s * HH;
  const int g = k / hsubs, hs = k - g * hsubs;
  const int head0 = g * G + hs * GB + hh0;
  T* outp = reinterpret_cast<T*>(a.out) + (((int64_t)s * R + r) * a.num_q_heads + head0) * D;

  const int L = a.context_lens[s];
  int P0 = 0;
  if constexpr (VR) {
    P0 = a.chunk_start[s];
    const int n = L - P0;
    if (P0 < 0 || n < 0 || n > R || L > cap) {
      for (int i = lane; i < HM * D; i += kWave) outp[i] = (T)__builtin_nanf("");
      return;
    }
    if (r >= n) return;  // no such row (or none at all)
  } else if (L == 0 && a.init_o != nullptr) {  // nothing after the shared prefix: its state alone
    const int64_t split_stride = (int64_t)B * a.num_q_heads;
    const int64_t row0 = (int64_t)s * a.num_q_heads + head0;
    for (int h = 0; h < HM; ++h) {
      float M = -__builtin_inff();
      bool nan = false;
      for (int sp = 0; sp < a.init_splits; ++sp) {
        const float ms = a.init_ml[(sp * split_stride + row0 + h) * 2];
        nan |= ms != ms;
        M = fmaxf(M, ms);
      }
      float lam = 0.0f, o[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = 0.0f;
      for (int sp = 0; sp < a.init_splits; ++sp) {
        const int64_t r = sp * split_stride + row0 + h;
        const float f = fast_exp2(a.init_ml[r * 2] - M);
        lam = fmaf(f, a.init_ml[r * 2 + 1], lam);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = fmaf(f, a.init_o[r * D + lane + e * kWave], o[e]);
      }
      const float inv = nan ? __builtin_nanf("") : 1.0f / lam;
#pragma unroll
      for (int e = 0; e < PER; ++e) outp[h * D + lane + e * kWave] = (T)(o[e] * inv);
    }
    return;
  }
  if (!VR && (L < 0 || L > cap || L == 0)) {
    const float fill = L == 0 ? 0.0f : __builtin_nanf("");
    for (int i = lane; i < HM * D; i += kWave) outp[i] = (T)fill;
    return;
  }
  int64_t U, before;
  cost_counts<VR>(a.context_lens, a.chunk_start, B, s, cap, R, HH, U, before);
  const int nb = stream_blocks<VR>(L, P0, cap, R);
  const int64_t as = before + (int64_t)k * (nb + kSegCost);  // the stream's cost interval starts here
  const int64_t us = as + kSegCost;                           // and its blocks here
  const int64_t ue = us + nb - 1;
  const int wf = wave_of(us, W, U), wl = wave_of(ue, W, U);
  if (wf == wl) return;  // finished inside one wave

  float M[HM], lam[HM], o[HM][PER];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    M[h] = -__builtin_inff();
    lam[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[h][e] = 0.0f;
  }
  for (int c0 = wf; c0 <= wl; c0 += kWave) {
    // pass 1: which candidates own a piece of the stream, and their (m, l)
    const int c = c0 + lane;
    const int64_t rb = range_begin(c, W, U);
    const bool owner = c <= wl && rb < range_begin(c + 1, W, U);  // non-empty range inside [wf, wl]
    // slot 1 if wave c worked on an earlier stream first, i.e. its range starts before this stream's
    const int64_t slot = (int64_t)c * 2 + ((c == wf && rb < as) ? 1 : 0);
    float mc[HM], lc[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      mc[h] = owner ? a.part_ml[(slot * SC + pc0 + h) * 2] : -__builtin_inff();
      lc[h] = owner ? a.part_ml[(slot * SC + pc0 + h) * 2 + 1] : 0.0f;
    }
    // the outputs of the first kPre candidates do not depend on the (m, l)
    // values: their loads go out together with them
    const uint64_t owners = __builtin_amdgcn_ballot_w64(owner);
    float opre[kPre][HM][PER];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const bool oj = (owners >> j) & 1ull;
      // slot 0 for a non-owner: the address stays inside the workspace even if the load is issued
      const int64_t sj = oj ? __builtin_amdgcn_readlane((int)(slot & 0x7fffffff), j) : 0;
#pragma unroll
      for (int h = 0; h < HM; ++h)
#pragma unroll
        for (int e = 0; e < PER; ++e)
          opre[j][h][e] = oj ? a.part_o[(sj * SC + pc0 + h) * D + lane + e * kWave] : 0.0f;
    }
    float f[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      const float Mn = fmaxf(M[h], wave_max(mc[h]));
      const float rescale = fast_exp2(M[h] - Mn);  // earlier chunks of owners
      f[h] = owner ? fast_exp2(mc[h] - Mn) : 0.0f;
      lam[h] = lam[h] * rescale + wave_sum(f[h] * lc[h]);
#pragma unroll
      for (int e = 0; e < PER; ++e) o[h][e] *= rescale;
      M[h] = Mn;
    }
    // pass 2: weighted sum of the owners' outputs
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      if (!((owners >> j) & 1ull)) continue;
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f[h]), j));
#pragma unroll
        for (int e = 0; e < PER; ++e) o[h][e] = fmaf(fj, opre[j][h][e], o[h][e]);
      }
    }
    const int n = 64 - __builtin_clzll(owners | 1ull);
#pragma unroll 4
    for (int j = kPre; j < n; ++j) {
      if (!((owners >> j) & 1ull)) continue;
      const int64_t sj = __builtin_amdgcn_readlane((int)(slot & 0x7fffffff), j);
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f[h]), j));
#pragma unroll
        for (int e = 0; e < PER; ++e)
          o[h][e] = fmaf(fj, a.part_o[(sj * SC + pc0 + h) * D + lane + e * kWave], o[h][e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    const float inv = 1.0f / lam[h];
#pragma unroll
    for (int e = 0; e < PER; ++e) outp[h * D + lane + e * kWave] = (T)(o[h][e] * inv);
  }
}

// ---------------------------------------------------------------- read probe
//
// The bytes a decode call's K/V loads touch, read the way it reads them and
// nothing else: every (sequence, kv head) tile row before the context length,
// 16-byte non-temporal buffer loads sized to the valid rows, four blocks in
// flight per wave, the batch's blocks (in sequence, kv head, block order)
// divided evenly over the grid.  Each wave folds what it read into one word
// (XOR) so that no load can be dropped.  No attention: the duration is what
// the memory system allows for this access pattern.
template <int RB>
__global__ __launch_bounds__(64) void read_probe_kernel(const char* __restrict__ kc, const char* __restrict__ vc,
                                                        const int32_t* __restrict__ tables,
                                                        const int32_t* __restrict__ lens, int B, int Hkv,
                                                        int num_blocks, int max_blocks, uint32_t* __restrict__ out) {
  constexpr int kTile = kBlock * RB;
  constexpr int kLoads = kTile / (kWave * 16);  // 16-byte loads per lane per tile
  static_assert(kLoads >= 1 && kTile % (kWave * 16) == 0, "a tile is whole 1 KiB rows of the wave");
  constexpr int NS = 4;
  const int lane = __lane_id();
  const int W = gridDim.x, w = blockIdx.x;
  const int cap = max_blocks * kBlock;
  int64_t T, unused;
  cost_counts_blocks(lens, B, cap, Hkv, T, unused);
  const int64_t b0 = (int64_t)w * T / W, b1 = (int64_t)(w + 1) * T / W;
  uint32_t acc = 0;
  if (b0 < b1) {
    // locate b0: sequence s, kv head g, block j
    int s = 0;
    int64_t cum = 0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int i = c0 + lane;
      const int64_t c = i < B ? (int64_t)seq_blocks(lens[i], cap) * Hkv : 0;
      const int64_t incl = wave_incl_scan(c);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(i < B && cum + incl > b0);
      if (hit) {
        const int ln = __builtin_ctzll(hit);
        s = c0 + ln;
        cum += readlane64(incl - c, ln);
        break;
      }
      cum += readlane64(incl, kWave - 1);
    }
    s = __builtin_amdgcn_readfirstlane(s);
    cum = uniform64(cum);
    int L = lens[s];
    int nb = seq_blocks(L, cap);
    int g = (int)((b0 - cum) / nb);
    int j = (int)(b0 - cum - (int64_t)g * nb);
    const int64_t head_stride = kTile, blk_stride = (int64_t)kTile * Hkv;
    // the tile of the next block to load, advancing (s, g, j); past b1 a size of 0
    int64_t left = b1 - b0;
    auto next_tile = [&](int64_t& off, int& bytes) {
      if (left <= 0) {
        off = 0;
        bytes = 0;
        return;
      }
      --left;
      int p = tables[(int64_t)s * max_blocks + j];
      p = (p < 0 || p >= num_blocks) ? 0 : p;
      off = (int64_t)p * blk_stride + (int64_t)g * head_stride;
      const int v = L - j * kBlock;
      bytes = (v >= kBlock ? kBlock : v) * RB;
      if (++j == nb) {
        j = 0;
        if (++g == Hkv) {
          g = 0;
          do {  // the next sequence with blocks (one exists while left > 0)
            ++s;
            L = s < B ? lens[s] : 0;
            nb = s < B ? seq_blocks(L, cap) : 1;
          } while (nb == 0 && s < B);
        }
      }
    };
    Chunk kS[NS][kLoads], vS[NS][kLoads];
    auto issue = [&](Chunk (&kk)[kLoads], Chunk (&vv)[kLoads]) {
      int64_t off;
      int bytes;
      next_tile(off, bytes);
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + off, bytes), vr = tile_rsrc(vc + off, bytes);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        kk[i] = as_chunk(__builtin_amdgcn_raw_buffer_load_b128(kr, (i * kWave + lane) * 16, 0, 2));
        vv[i] = as_chunk(__builtin_amdgcn_raw_buffer_load_b128(vr, (i * kWave + lane) * 16, 0, 2));
      }
    };
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(kS[st], vS[st]);
    for (int64_t n = b1 - b0; n > 0; n -= NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc ^= kS[st][i].w[e] ^ vS[st][i].w[e];
        issue(kS[st], vS[st]);
      }
    }
  }
  // one word per wave: the XOR over its lanes
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)acc);
  if (lane == 0) out[w] = acc;
}

hipError_t launch_read_probe(const void* k_cache, const void* v_cache, const int32_t* tables, const int32_t* lens,
                             int num_seqs, int num_kv_heads, int head_dim, int elem_bytes, int num_blocks,
                             int max_blocks, int waves, uint32_t* out, hipStream_t stream) {
  const char* kc = reinterpret_cast<const char*>(k_cache);
  const char* vc = reinterpret_cast<const char*>(v_cache);
  const int rb = head_dim * elem_bytes;
  if (rb == 256)
    hipLaunchKernelGGL(read_probe_kernel<256>, dim3(waves), dim3(64), 0, stream, kc, vc, tables, lens, num_seqs,
                       num_kv_heads, num_blocks, max_blocks, out);
  else if (rb == 128)
    hipLaunchKernelGGL(read_probe_kernel<128>, dim3(waves), dim3(64), 0, stream, kc, vc, tables, lens, num_seqs,
                       num_kv_heads, num_blocks, max_blocks, out);
  else if (rb == 512)
    hipLaunchKernelGGL(read_probe_kernel<512>, dim3(waves), dim3(64), 0, stream, kc, vc, tables, lens, num_seqs,
                       num_kv_heads, num_blocks, max_blocks, out);
  else if (rb == 64)
    hipLaunchKernelGGL(read_probe_kernel<64>, dim3(waves), dim3(64), 0, stream, kc, vc, tables, lens, num_seqs,
                       num_kv_heads, num_blocks, max_blocks, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Shared prefix: merge the `splits` partials of every (sequence, head) row
// into the first one, in place (max M, sum sum_p 2^{m_p - M} l_p, output
// sum_p 2^{m_p - M} o_p), so that a stream starts from one partial.  One wave
// per row; lane k owns dims k, k + 64, ...
template <int D>
__global__ __launch_bounds__(64) void prefix_merge_kernel(float* __restrict__ part_o, float* __restrict__ part_ml,
                                                          int64_t rows, int splits) {
  constexpr int PER = D / kWave;
  const int lane = __lane_id();
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  float M, lam, o[PER];
  bool nan;
  merge_partials<D>(part_o, part_ml, row, rows, splits, o, M, lam, nan);
  // the wave has read every partial (piece 0 included) before it overwrites piece 0
#pragma unroll
  for (int e = 0; e < PER; ++e) part_o[row * D + lane + e * kWave] = o[e];
  if (lane == 0) {
    part_ml[row * 2] = nan ? __builtin_nanf("") : M;
    part_ml[row * 2 + 1] = lam;
  }
}

hipError_t launch_prefix_merge(float* part_o, float* part_ml, int64_t rows, int splits, int head_dim,
                               hipStream_t stream) {
  if (rows <= 0 || splits <= 1) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  if (head_dim == 64)
    hipLaunchKernelGGL(prefix_merge_kernel<64>, dim3((unsigned)rows), dim3(64), 0, stream, part_o, part_ml, rows,
                       splits);
  else if (head_dim == 128)
    hipLaunchKernelGGL(prefix_merge_kernel<128>, dim3((unsigned)rows), dim3(64), 0, stream, part_o, part_ml, rows,
                       splits);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Lanes per token: fewer lanes per token means fewer DPP reduction steps and
// less redundant softmax work per block, at the price of more accumulator
// registers per lane (head_dim / LPT floats per head).  8 for up to four heads
// per wave, 16 for eight (whose accumulators would not fit otherwise).
#ifndef PKV_DECODE_LPT_SMALL_GROUP
#define PKV_DECODE_LPT_SMALL_GROUP 8
#endif
// Register stages of the K/V pipeline (0: by type, see pipeline_stages).
#ifndef PKV_DECODE_STAGES
#define PKV_DECODE_STAGES 0
#endif
// fp8 at head_dim 128 keeps 8 lanes per token: 4 (two blocks per pipeline
// tile, half the replicated softmax work) was measured slower, 72.8 us against
// 60 us on the Llama-3-8B batch -- the accumulators no longer fit the
// architectural registers and the token-group merge doubles.
#ifndef PKV_DECODE_LPT_FP8
#define PKV_DECODE_LPT_FP8 8
#endif
template <typename KV, int D, int GB>
constexpr int lanes_per_token() {
  constexpr int row_chunks = D * KvTraits<KV>::kElemBytes / 16;
  constexpr int want = GB >= 8 ? 16 : (KvTraits<KV>::kScaled ? PKV_DECODE_LPT_FP8 : PKV_DECODE_LPT_SMALL_GROUP);
  return row_chunks < want ? row_chunks : want;
}
// Register stages of the K/V prefetch pipeline.  bf16 with up to four heads
// per wave runs at one wave per SIMD; for long contexts it keeps more blocks in
// flight (cold caches, the Llama-3-8B batch: 95-98 us with four against 102 us
// with two on the vector-ALU segment; on the matrix-core segment three beat
// four, 89.8 against 90.6 us), while short ones keep two, whose pipeline fills
// faster at every segment start (the shared-prefix suffixes of at most 512
// tokens: 101 us against 110 us).  E4M3 on the matrix-core segment takes three
// as well (56.4 against 57.6 us with two, 57.3 with four).  The types and
// groups that run two waves per SIMD, or need the registers (float32), keep two.
template <typename KV, int D, int GB>
constexpr int deep_stages() {
  if (PKV_DECODE_STAGES > 0) return PKV_DECODE_STAGES;
  constexpr bool matrix = D == 128 && (GB == 4 || GB == 8);  // the matrix-core segment
  if (std::is_same<KV, Fp8E4M3>::value) return matrix ? 3 : 2;
  if (std::is_same<KV, __bf16>::value) return matrix ? 3 : (GB <= 4 ? 4 : 2);
  return 2;
}

// Merge grids of at most this many waves take one head per wave.
constexpr int64_t kMergeWavesPerHead = 4096;

template <typename KV, int D, int GB, int NS>
static hipError_t launch_stages(const DecodeArgs& a, hipStream_t stream) {
  using T = typename KvTraits<KV>::Q;
  constexpr int LPT = lanes_per_token<KV, D, GB>();
  if (a.balanced_waves > 0) {
    const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;
    const int64_t streams = (int64_t)a.num_seqs * a.num_kv_heads * hsubs;
    if (streams * GB > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_balanced_kernel<KV, D, GB, LPT, NS>), dim3(a.balanced_waves), dim3(64), 0, stream, a,
                       a.block_tables, a.context_lens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one head per merge wave while that keeps the grid small (few, long streams)
    if (streams * GB <= kMergeWavesPerHead)
      hipLaunchKernelGGL((decode_balanced_merge_kernel<T, D, GB, 1>), dim3((unsigned)(streams * GB)), dim3(64), 0,
                         stream, a, a.balanced_waves);
    else
      hipLaunchKernelGGL((decode_balanced_merge_kernel<T, D, GB, GB>), dim3((unsigned)streams), dim3(64), 0, stream,
                         a, a.balanced_waves);
    return hipGetLastError();
  }
  const int64_t rows = (int64_t)a.num_seqs * a.rows_per_seq;
  const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;
  const int64_t items = rows * a.num_kv_heads * hsubs * a.max_parts;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partition_kernel<KV, D, GB, LPT, NS>), dim3((unsigned)items), dim3(64), 0, stream, a,
                     a.block_tables);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t merges = rows * a.num_q_heads;
  if (merges > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)merges), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename KV, int D, int GB>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NSD = deep_stages<KV, D, GB>();
  if constexpr (NSD != 2) {
    if (a.max_context_tokens >= kDeepPipelineMinTokens) return launch_stages<KV, D, GB, NSD>(a, stream);
  }
  return launch_stages<KV, D, GB, 2>(a, stream);
}

template <typename KV, int D>
static hipError_t launch_gb(const DecodeArgs& a, hipStream_t stream) {
  switch (heads_per_wave(a.num_q_heads / a.num_kv_heads)) {
    case 1: return launch_typed<KV, D, 1>(a, stream);
    case 2: return launch_typed<KV, D, 2>(a, stream);
    case 4: return launch_typed<KV, D, 4>(a, stream);
    case 8: return launch_typed<KV, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

// The rows that verify draft tokens, on the balanced split with the
// matrix-core segment: GB heads x rows_per_seq rows are the columns of CT
// column tiles.
template <int GB, int CT>
static hipError_t launch_verify_cols(const DecodeArgs& a, hipStream_t stream) {
  using KV = __bf16;
  constexpr int D = 128;
  constexpr int NS = deep_stages<KV, D, GB>();
  constexpr int LPT = lanes_per_token<KV, D, GB>();
  static_assert(Segment<KV, D, GB, LPT, NS, CT>::kMfma, "verify rows take the matrix-core segment");
  const int hsubs = (a.num_q_heads / a.num_kv_heads) / GB;
  const int64_t rows = (int64_t)a.num_seqs * a.num_kv_heads * hsubs * a.rows_per_seq;  // (stream, row) pairs
  if (rows * GB > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_balanced_kernel<KV, D, GB, LPT, NS, CT, true>), dim3(a.balanced_waves), dim3(64), 0,
                     stream, a, a.block_tables, a.context_lens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one head per merge wave while that keeps the grid small, as for decode
  // (measured on 16..64 sequences x 5 rows: 37.5 against 40.7 us at 16
  // sequences, 82.3 against 79.3 us at 48)
  if (rows * GB <= kMergeWavesPerHead)
    hipLaunchKernelGGL((decode_balanced_merge_kernel<__bf16, D, GB, 1, true, 16 * CT>), dim3((unsigned)(rows * GB)),
                       dim3(64), 0, stream, a, a.balanced_waves);
  else
    hipLaunchKernelGGL((decode_balanced_merge_kernel<__bf16, D, GB, GB, true, 16 * CT>), dim3((unsigned)rows),
                       dim3(64), 0, stream, a, a.balanced_waves);
  return hipGetLastError();
}

hipError_t launch_verify(const DecodeArgs& a, hipStream_t stream) {
  const int gb = heads_per_wave(a.num_q_heads / a.num_kv_heads);
  if (!verify_balanced(gb, a.dtype, a.head_dim, a.rows_per_seq) || a.chunk_start == nullptr ||
      a.balanced_waves <= 0)
    return hipErrorInvalidValue;
  const bool one = gb * a.rows_per_seq <= 16;
  if (gb == 4) return one ? launch_verify_cols<4, 1>(a, stream) : launch_verify_cols<4, 2>(a, stream);
  return one ? launch_verify_cols<8, 1>(a, stream) : launch_verify_cols<8, 2>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == 0) {
    if (a.head_dim == 64) return launch_gb<float, 64>(a, stream);
    if (a.head_dim == 128) return launch_gb<float, 128>(a, stream);
  } else if (a.dtype == 1) {
    if (a.head_dim == 64) return launch_gb<__bf16, 64>(a, stream);
    if (a.head_dim == 128) return launch_gb<__bf16, 128>(a, stream);
  } else if (a.dtype == 2) {
    if (a.k_scale == nullptr || a.v_scale == nullptr) return hipErrorInvalidValue;
    if (a.head_dim == 64) return launch_gb<Fp8E4M3, 64>(a, stream);
    if (a.head_dim == 128) return launch_gb<Fp8E4M3, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
