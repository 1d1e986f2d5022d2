// Host-side launch interface between the C ABI (api.hip) and the kernels.
// Arguments here are already validated; launchers only pick an instantiation
// and size the grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2eHost = 1.4426950408889634f;

struct WriteArgs {
  const void* k;
  const void* v;
  const int32_t* slots;
  int64_t num_tokens;
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
};

// One "query row" is a decode query (rows_per_seq == 1, chunk_start == nullptr)
// or one row of a prefill chunk (rows_per_seq == chunk_len_max, chunk_start set).
struct DecodeArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* chunk_start;  // nullptr for decode
  float* part_o;               // [rows][Hq][max_parts][D] unnormalised partial outputs
  float* part_ml;              // [rows][Hq][max_parts][2] (running max in log2 units, sum)
  int32_t num_seqs;
  int32_t rows_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t partition_tokens;
  int32_t max_parts;  // partitions the grid covers per query row
  float scale_log2;   // softmax scale * log2(e)
  // > 0: balanced split over this many waves (decode only); part_o / part_ml
  // then hold [waves][2][heads per wave][D] and [waves][2][heads per wave][2]
  int32_t balanced_waves;
  // Shared prefix (balanced split only; init_o == nullptr otherwise): every
  // stream's first segment starts from the attention state of the prefix,
  // given as init_splits partials [split][seq][Hq][D] (unnormalised) and
  // [split][seq][Hq][2] (max in log2 units, sum).
  const float* init_o;
  const float* init_ml;
  int32_t init_splits;
  // fp8 caches (dtype 2): float scales [num_blocks][num_kv_heads][16]
  const float* k_scale;
  const float* v_scale;
  // host-side bound on the keys of any row (picks the pipeline depth)
  int32_t max_context_tokens;
};

struct PrefillArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* chunk_start;
  int32_t num_chunks;
  int32_t chunk_len_max;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  float scale_log2;
  // Shared-prefix mode (prefix_len > 0): the rows are the num_chunks decode
  // queries q [num_chunks][Hq][D]; keys are the prefix_len tokens of
  // block_tables[0 .. prefix_len / 16), split into pieces of split_tokens;
  // each piece writes (m, l, o) partials to part_o [piece][seq][Hq][D] and
  // part_ml [piece][seq][Hq][2].
  int32_t prefix_len;
  int32_t split_tokens;
  int32_t num_splits;
  float* part_o;
  float* part_ml;
};

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
// fp8 caches: quantise bfloat16 (in_dtype 1) or float32 (0) rows to E4M3 codes + per-row scales.
hipError_t launch_kv_write_fp8(const WriteArgs& a, int32_t in_dtype, float* k_scale, float* v_scale,
                               hipStream_t stream);
hipError_t launch_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                                 int64_t num_pairs, int32_t num_blocks, int64_t block_bytes, hipStream_t stream);
// Returns hipErrorInvalidValue if no instantiation covers the shape.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefix_mfma(const PrefillArgs& a, hipStream_t stream);
// The log-sum-exp merge on its own: rows x parts partials ([row][part]) into
// out [rows][head_dim] of out_dtype (0 float32, 1 bfloat16).
hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int64_t rows, int parts, int head_dim,
                            int out_dtype, void* out, hipStream_t stream);
// The read probe: the K/V bytes of a decode call, read with its loads over `waves` waves.
hipError_t launch_read_probe(const void* k_cache, const void* v_cache, const int32_t* tables, const int32_t* lens,
                             int num_seqs, int num_kv_heads, int head_dim, int elem_bytes, int num_blocks,
                             int max_blocks, int waves, uint32_t* out, hipStream_t stream);
// Merges the splits partials of each of `rows` rows into the first split's slot.
hipError_t launch_prefix_merge(float* part_o, float* part_ml, int64_t rows, int splits, int head_dim,
                               hipStream_t stream);

// Heads processed together by one wave for a GQA group of size g.
constexpr int heads_per_wave(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

// Longest context from which the decode keeps more than two blocks in
// flight per wave (and bf16 caches take the matrix-core segment).
constexpr int kDeepPipelineMinTokens = 1024;

// Whether a decode runs the matrix-core segment (scores and value products on
// the matrix cores): D = 128 with four or eight heads per wave, E4M3 caches
// always, bf16 caches with the deep pipeline.
constexpr bool matrix_segment(int gb, int dtype, int head_dim, int max_context_tokens) {
  return head_dim == 128 && (gb == 4 || gb == 8) &&
         (dtype == 2 || (dtype == 1 && max_context_tokens >= kDeepPipelineMinTokens));
}

// Waves of the balanced decode split.  One wave per SIMD (1024 on the
// MI355X's 256 compute units) wherever the matrix-core segment runs, and for
// float32 / bf16 caches with up to four heads per wave on the vector-ALU
// segment; a second wave per SIMD where the vector-ALU segment's work per byte
// is high -- eight heads per wave, or fp8 codes widened and dotted on the
// vector ALU -- so that one wave's arithmetic hides the other's memory waits.
// Measured with cold caches: the Llama-3-8B batch on the E4M3 cache, vector
// ALU 61 us at 2048 waves against 90 us at 1024, matrix cores 56.9 us at 1024
// against 58.3 us at 2048; bf16 on the vector ALU 98 us at 2048 against 95 us
// at 1024; the long-context batch (eight heads per wave) on the matrix cores
// 458.5 us at 1024 against 479.7 us at 2048.
#ifndef PKV_BALANCED_WAVES
#define PKV_BALANCED_WAVES 0
#endif
constexpr int balanced_waves(int gb, int dtype, int head_dim, int max_context_tokens) {
  if (PKV_BALANCED_WAVES > 0) return PKV_BALANCED_WAVES;
  if (matrix_segment(gb, dtype, head_dim, max_context_tokens)) return 1024;
  return (gb >= 8 || dtype == 2) ? 2048 : 1024;
}
// The largest of them over the cache dtypes, head dims and context lengths:
// what a workspace must hold.
constexpr int balanced_waves_max(int gb) {
  int w = 0;
  for (int dtype = 0; dtype <= 2; ++dtype)
    for (int d = 64; d <= 128; d += 64)
      for (int ctx = 0; ctx <= kDeepPipelineMinTokens; ctx += kDeepPipelineMinTokens)
        w = balanced_waves(gb, dtype, d, ctx) > w ? balanced_waves(gb, dtype, d, ctx) : w;
  return w;
}

// The rows that verify draft tokens run on the balanced split with the
// matrix-core segment where its columns (heads per wave x rows) fit two column
// tiles -- bf16 caches, D = 128, four or eight heads per wave -- and the batch
// has at least kVerifyMinStreams (sequence, kv head, head subgroup) streams,
// over kVerifyWaves waves, each leaving at most two partial slots of 16 or 32
// columns.  Fewer streams keep the matrix-core chunk kernel with its key
// split: their keys are cut into so many pieces over the 1024 waves that the
// partials of 20 columns per piece cost as much as the split saves (5 rows x
// 32q / 8kv heads, contexts U{128..4096}, cold caches: 8 sequences 26.1 us
// against 26.0 on the chunk kernel, the same at 256 and 512 waves; 16
// sequences 37.5 against 52.1; 32: 55.9 against 73.0; 64: 99.8 against 107.1;
// 128: 200.3 against 203.2).
constexpr int kVerifyWaves = 1024;
constexpr int64_t kVerifyMinStreams = 128;
constexpr bool verify_balanced(int gb, int dtype, int head_dim, int rows) {
  return dtype == 1 && head_dim == 128 && (gb == 4 || gb == 8) && rows >= 1 && gb * rows <= 32;
}
constexpr bool verify_takes_balanced(int64_t num_seqs, int rows, int num_q_heads, int num_kv_heads, int head_dim,
                                     int dtype) {
  return num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 &&
         verify_balanced(heads_per_wave(num_q_heads / num_kv_heads), dtype, head_dim, rows) &&
         num_seqs * num_q_heads / heads_per_wave(num_q_heads / num_kv_heads) >= kVerifyMinStreams;
}
constexpr size_t verify_workspace(int gb, int head_dim, int rows) {
  return (size_t)kVerifyWaves * 2 * (gb * rows <= 16 ? 16 : 32) * ((size_t)head_dim + 2) * sizeof(float);
}
// a.chunk_start: each sequence's first row position; a.rows_per_seq rows at
// most; a.part_o / a.part_ml: the partial slots (kVerifyWaves of them).
hipError_t launch_verify(const DecodeArgs& a, hipStream_t stream);

}  // namespace pkv
