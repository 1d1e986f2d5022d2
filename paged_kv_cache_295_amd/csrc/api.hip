// C ABI of libpagedkv.so: host-side validation, partition sizing and launches.
// Nothing here reads device memory or synchronises; every launch goes to the
// caller's stream.  See include/pagedkv.h for the contract of each call.
#include <math.h>

#include <mutex>

#include "pagedkv.h"
#include "pkv_internal.hpp"

using namespace pkv;

namespace {

// fp8: the entry points that take scale arrays want an E4M3 cache, the others
// a float32 or bfloat16 one.
int check_cache(const pkv_cache_desc* c, bool fp8 = false) {
  if (c == nullptr) return PKV_ERR_NULL;
  if (fp8 ? c->dtype != PKV_DTYPE_FP8_E4M3 : (c->dtype != PKV_DTYPE_F32 && c->dtype != PKV_DTYPE_BF16))
    return PKV_ERR_DTYPE;
  if (c->block_size != PKV_BLOCK_SIZE) return PKV_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_SHAPE;
  // slots and per-block offsets are int32 on the device
  if ((int64_t)c->num_blocks * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  return PKV_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// A workspace the call needs must be present, large enough and 16-byte
// aligned (the kernels read partial states with 8- and 16-byte loads).
bool workspace_ok(const void* ws, size_t bytes, size_t need) {
  return need == 0 || (ws != nullptr && bytes >= need && (reinterpret_cast<uintptr_t>(ws) & 15) == 0);
}

// Balanced split (partition_tokens == 0): up to balanced_waves_max(gb) waves, each with
// up to two partials of gb = heads_per_wave heads.
size_t balanced_workspace(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  const int gb = heads_per_wave(num_q_heads / num_kv_heads);
  return (size_t)balanced_waves_max(gb) * 2 * gb * ((size_t)head_dim + 2) * sizeof(float);
}

// Fixed partitions of `part` tokens: one partial per (row, head, partition).
size_t partition_workspace(int32_t num_seqs, int32_t hq, int32_t head_dim, int32_t max_len, int32_t part) {
  const int64_t max_parts = ((int64_t)max_len + part - 1) / part;
  if (max_parts <= 1) return 0;
  return (size_t)num_seqs * hq * max_parts * ((size_t)head_dim + 2) * sizeof(float);
}

// Workgroups of the matrix-core kernel the MI355X runs at once: two per
// compute unit on 256 compute units (its LDS ring and registers admit two).
#ifndef PKV_MATRIX_SLOTS
#define PKV_MATRIX_SLOTS 512
#endif
constexpr int64_t kMatrixSlots = PKV_MATRIX_SLOTS;

// Shared prefix: pieces of the prefix for the matrix-core kernel, enough to
// fill every workgroup slot about once (128 rows x 64-key tiles each).
struct PrefixSplit {
  int32_t splits;
  int32_t split_tokens;
};

// Workgroups the prefix pieces aim for: one per compute unit.  The pieces'
// (m, l, o) partials cross HBM twice (written, then merged), so fewer, longer
// pieces pay while every unit still has one: on the 256-sequence batch with a
// 2048-token prefix (64 row tiles) 4 pieces take 99.0 us per call against
// 101.0 us for 8 (one per workgroup slot), 106.7 us for 2 and 114.8 us for 16.
#ifndef PKV_PREFIX_WORKGROUPS
#define PKV_PREFIX_WORKGROUPS 256
#endif
constexpr int64_t kPrefixWorkgroups = PKV_PREFIX_WORKGROUPS;

PrefixSplit prefix_split(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t prefix_len) {
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t row_tiles = (num_seqs * G + 127) / 128;
  const int64_t wgs = row_tiles * num_kv_heads;
  const int64_t tiles = (prefix_len + 63) / 64;
  int64_t want = (kPrefixWorkgroups + wgs - 1) / wgs;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  PrefixSplit r;
  r.split_tokens = (int32_t)(per * 64);
  r.splits = (int32_t)((prefix_len + r.split_tokens - 1) / r.split_tokens);
  return r;
}

size_t prefix_workspace(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t prefix_len) {
  if (prefix_len <= 0) return 0;
  const PrefixSplit ps = prefix_split(num_seqs, num_q_heads, num_kv_heads, prefix_len);
  return (size_t)ps.splits * num_seqs * num_q_heads * ((size_t)head_dim + 2) * sizeof(float);
}

// Chunks with a workspace (prefill chunks, the speculative-verify rows): when
// the batch has fewer (chunk, row tile, kv head) units than workgroup slots,
// cut each row tile's keys into pieces so that the matrix-core kernel gets
// about two workgroups per slot, the second wave of them hiding the first's
// start and end, and no long row tile runs alone at the end.  Measured on the MI355X (5 rows per
// sequence, contexts U{128..4096}, one workgroup per compute unit at the
// time): 4 / 8 / 16 sequences took 23 / 45 / 68 us split against 76 / 84 /
// 101 us unsplit; with every slot already holding a pair, cutting further only
// added per-workgroup cost (64 sequences x 8 kv heads: 183 us unsplit, 217 us
// and 237 us for 1024 and 2048 workgroups).  Pieces are whole 64-key tiles and
// at least 256 keys, so the partials stay a small fraction of the K/V bytes.
constexpr int64_t kChunkWorkgroups = 2 * kMatrixSlots;

struct ChunkSplit {
  int32_t splits;  // 1: no split
  int32_t split_tokens;
};

ChunkSplit chunk_split(int32_t num_seqs, int32_t rows_max, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t max_blocks_per_seq) {
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t QT = (int64_t)rows_max * G <= 128 ? rows_max : 128 / G;  // rows per tile, as the kernel packs them
  const int64_t units = (int64_t)num_seqs * num_kv_heads * ((rows_max + QT - 1) / QT);
  const int64_t max_keys = (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE;
  int64_t split = (units * max_keys + kChunkWorkgroups - 1) / kChunkWorkgroups;
  split = (split + 63) / 64 * 64;
  if (split < 256) split = 256;
  ChunkSplit v;
  // with a unit for every other slot already, pieces cost more than they
  // balance: the mixed-step chunks (2 x 512 rows, 256 units) take 52 us
  // unsplit against 78 us in pieces of 1024 keys plus a 14 us merge, while one
  // 512-row chunk at 3584 keys (128 units) takes 95 us unsplit, 58 + 18 us in
  // pieces of 512
  // Tiles whose rows fit one wave (the packed verify rows) write partials of
  // at most 32 rows, so they split while units are fewer than the slots: 32
  // sequences x 5 rows (256 units) 76 -> 63 us in four pieces; with a unit
  // for every slot (64 sequences) any split was slower (115 -> 129..164 us).
  const bool short_tile = rows_max * G <= 32;
  if ((short_tile ? units >= kMatrixSlots : 2 * units >= kMatrixSlots) || split >= max_keys) {
    v.splits = 1;
    v.split_tokens = 0;
  } else {
    v.splits = (int32_t)((max_keys + split - 1) / split);
    v.split_tokens = (int32_t)split;
  }
  return v;
}

size_t chunk_workspace(int32_t num_seqs, int32_t rows_max, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq) {
  const ChunkSplit v = chunk_split(num_seqs, rows_max, num_q_heads, num_kv_heads, max_blocks_per_seq);
  if (v.splits <= 1) return 0;
  return (size_t)v.splits * num_seqs * rows_max * num_q_heads * ((size_t)head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer argument";
    case PKV_ERR_DTYPE: return "unsupported or mismatched dtype";
    case PKV_ERR_SHAPE: return "invalid shape or size";
    case PKV_ERR_UNSUPPORTED: return "unsupported block size or head dim";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_NO_BLOCKS: return "no free cache block";
    case PKV_ERR_SCRATCH: return "the call needs more scratch than the no-allocation decode holds";
  }
  return "unknown status";
}

int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, int64_t num_tokens, void* k_cache,
                   void* v_cache, const pkv_cache_desc* cache, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
  WriteArgs a{k, v, slot_mapping, num_tokens, k_cache, v_cache, cache->num_blocks, cache->num_kv_heads,
              cache->head_dim, cache->dtype};
  return from_hip(launch_kv_write(a, as_stream(hip_stream)));
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int64_t num_pairs, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks) return PKV_ERR_NULL;
  const int64_t elem = cache->dtype == PKV_DTYPE_BF16 ? 2 : 4;
  const int64_t block_bytes = (int64_t)cache->num_kv_heads * PKV_BLOCK_SIZE * cache->head_dim * elem;
  return from_hip(launch_kv_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, num_pairs, cache->num_blocks,
                                        block_bytes, as_stream(hip_stream)));
}

int32_t paged_attn_decode_split_waves(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  return balanced_waves(heads_per_wave(num_q_heads / num_kv_heads), PKV_DTYPE_BF16, 128, kDeepPipelineMinTokens);
}

int paged_kv_read_probe(const void* k_cache, const void* v_cache, const pkv_cache_desc* cache,
                        const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_waves, uint32_t* out_words, void* hip_stream) {
  if (cache == nullptr) return PKV_ERR_NULL;
  int st = check_cache(cache, cache->dtype == PKV_DTYPE_FP8_E4M3);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_waves <= 0 || num_waves > 65536) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !out_words) return PKV_ERR_NULL;
  const int elem = cache->dtype == PKV_DTYPE_F32 ? 4 : (cache->dtype == PKV_DTYPE_BF16 ? 2 : 1);
  return from_hip(launch_read_probe(k_cache, v_cache, block_tables, context_lens, num_seqs, cache->num_kv_heads,
                                    cache->head_dim, elem, cache->num_blocks, max_blocks_per_seq, num_waves,
                                    out_words, as_stream(hip_stream)));
}

int paged_attn_lse_merge(const float* part_o, const float* part_ml, int64_t num_rows, int32_t num_parts,
                         int32_t head_dim, int32_t out_dtype, void* out, void* hip_stream) {
  if (num_rows < 0) return PKV_ERR_SHAPE;
  if (num_rows == 0) return PKV_OK;
  if (!part_o || !part_ml || !out) return PKV_ERR_NULL;
  if (out_dtype != PKV_DTYPE_F32 && out_dtype != PKV_DTYPE_BF16) return PKV_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_parts <= 0 || num_rows > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (((reinterpret_cast<uintptr_t>(part_o) | reinterpret_cast<uintptr_t>(part_ml)) & 15) != 0) return PKV_ERR_SHAPE;
  return from_hip(launch_lse_merge(part_o, part_ml, num_rows, num_parts, head_dim, out_dtype, out,
                                   as_stream(hip_stream)));
}

size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_tokens < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  if (partition_tokens == 0) return balanced_workspace(num_q_heads, num_kv_heads, head_dim);
  return partition_workspace(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens);
}

}  // extern "C"

namespace {

int decode_common(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache, const void* v_cache,
                  const float* k_scale, const float* v_scale, const pkv_cache_desc* cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                  int32_t max_context_len, float scale, void* out, int32_t partition_tokens, void* workspace,
                  size_t workspace_bytes, void* hip_stream) {
  const bool fp8 = k_scale != nullptr || v_scale != nullptr;
  int st = check_cache(cache, fp8);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (fp8 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (max_blocks_per_seq <= 0 || max_context_len < 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE) return PKV_ERR_SHAPE;
  if (partition_tokens < 0 || partition_tokens % PKV_BLOCK_SIZE != 0) return PKV_ERR_SHAPE;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  const bool balanced = partition_tokens == 0;
  const int32_t part = balanced ? max_blocks_per_seq * PKV_BLOCK_SIZE : partition_tokens;
  const int64_t max_parts64 = balanced || max_context_len == 0 ? 1 : ((int64_t)max_context_len + part - 1) / part;
  if (max_parts64 > 0x7fffffffLL) return PKV_ERR_SHAPE;
  const size_t need = balanced ? balanced_workspace(num_q_heads, cache->num_kv_heads, cache->head_dim)
                               : partition_workspace(num_seqs, num_q_heads, cache->head_dim, max_context_len, part);
  if (!workspace_ok(workspace, workspace_bytes, need)) return PKV_ERR_WORKSPACE;
  // A batch whose every stream fits one wave's share of the balanced split
  // (at most as many blocks in all as the split has waves) runs one wave per
  // (sequence, head group) over its whole context: no partials, no merge
  // kernel.  (The 4-sequence float32 batch: 15.5 us balanced.)
  const int gb = heads_per_wave(num_q_heads / cache->num_kv_heads);
  const int64_t streams = (int64_t)num_seqs * cache->num_kv_heads * ((num_q_heads / cache->num_kv_heads) / gb);
  const bool whole = balanced && streams * (((int64_t)max_context_len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE) <=
                                     balanced_waves(gb, cache->dtype, cache->head_dim, max_context_len);
  DecodeArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.chunk_start = nullptr;
  const size_t o_bytes = need == 0 ? 0 : need / ((size_t)cache->head_dim + 2) * cache->head_dim;
  a.part_o = need ? reinterpret_cast<float*>(workspace) : nullptr;
  a.part_ml = need ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + o_bytes) : nullptr;
  a.num_seqs = num_seqs;
  a.rows_per_seq = 1;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.dtype = cache->dtype;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.partition_tokens = part;
  a.max_parts = (int32_t)max_parts64;
  a.scale_log2 = scale * kLog2eHost;
  a.balanced_waves = balanced && !whole ? balanced_waves(gb, cache->dtype, cache->head_dim, max_context_len) : 0;
  a.max_context_tokens = max_context_len;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return from_hip(launch_decode(a, as_stream(hip_stream)));
}

}  // namespace

extern "C" {

int paged_attn_decode(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache, const void* v_cache,
                      const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                      int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_common(q, num_seqs, num_q_heads, k_cache, v_cache, nullptr, nullptr, cache, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, scale, out, partition_tokens, workspace,
                       workspace_bytes, hip_stream);
}

}  // extern "C"

// ---- decode without allocation ---------------------------------------------
// The split decode's partial states in a buffer inside the library instead of
// a caller workspace: enough for the balanced split at every supported shape
// (the most waves, two partials each, eight heads per wave, head_dim 128), so
// only fixed partitions of large batches can need more.  Each GPU the library
// runs on holds its own copy until the process ends.  The kernels write every
// partial they read later in the same call, so nothing needs clearing.
static constexpr size_t kScratchBytes = (size_t)balanced_waves_max(8) * 2 * 8 * (128 + 2) * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's copy of `scratch`, looked up once
// per device (the array's name in host code is not a device address).
int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t paged_attn_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

int paged_attn_decode_noalloc(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                              const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                              float scale, void* out, int32_t partition_tokens, void* hip_stream) {
  // the checks that size the partial states come first, so an oversized call
  // fails on the host before anything touches the GPU
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (max_context_len < 0 || partition_tokens < 0 || partition_tokens % PKV_BLOCK_SIZE != 0) return PKV_ERR_SHAPE;
  const size_t need = partition_tokens == 0
                          ? balanced_workspace(num_q_heads, cache->num_kv_heads, cache->head_dim)
                          : partition_workspace(num_seqs, num_q_heads, cache->head_dim, max_context_len,
                                                partition_tokens);
  if (need > kScratchBytes) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_common(q, num_seqs, num_q_heads, k_cache, v_cache, nullptr, nullptr, cache, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, scale, out, partition_tokens, ws,
                       need > 0 ? kScratchBytes : 0, hip_stream);
}

int paged_attn_decode_fp8(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                          int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!k_scale || !v_scale) return PKV_ERR_NULL;
  return decode_common(q, num_seqs, num_q_heads, k_cache, v_cache, k_scale, v_scale, cache, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, scale, out, partition_tokens, workspace,
                       workspace_bytes, hip_stream);
}

int paged_kv_write_fp8(const void* k, const void* v, int32_t in_dtype, const int32_t* slot_mapping,
                       int64_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pkv_cache_desc* cache, void* hip_stream) {
  int st = check_cache(cache, true);
  if (st != PKV_OK) return st;
  if (in_dtype != PKV_DTYPE_F32 && in_dtype != PKV_DTYPE_BF16) return PKV_ERR_DTYPE;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale) return PKV_ERR_NULL;
  WriteArgs a{k, v, slot_mapping, num_tokens, k_cache, v_cache, cache->num_blocks, cache->num_kv_heads,
              cache->head_dim, cache->dtype};
  return from_hip(launch_kv_write_fp8(a, in_dtype, k_scale, v_scale, as_stream(hip_stream)));
}

int paged_kv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             const pkv_cache_desc* cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                             int64_t num_pairs, void* hip_stream) {
  int st = check_cache(cache, true);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_scale || !v_scale || !src_blocks || !dst_blocks) return PKV_ERR_NULL;
  const int64_t code_bytes = (int64_t)cache->num_kv_heads * PKV_BLOCK_SIZE * cache->head_dim;
  const int64_t scale_bytes = (int64_t)cache->num_kv_heads * PKV_BLOCK_SIZE * (int64_t)sizeof(float);
  hipStream_t s = as_stream(hip_stream);
  hipError_t e = launch_kv_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, num_pairs, cache->num_blocks,
                                       code_bytes, s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  return from_hip(launch_kv_copy_blocks(k_scale, v_scale, src_blocks, dst_blocks, num_pairs, cache->num_blocks,
                                        scale_bytes, s));
}

size_t paged_attn_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t prefix_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || prefix_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const size_t pre = prefix_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, prefix_len);
  const size_t pre_aligned = (pre + 255) / 256 * 256;
  return pre_aligned + balanced_workspace(num_q_heads, num_kv_heads, head_dim);
}

int paged_attn_decode_shared_prefix(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                                    const void* v_cache, const pkv_cache_desc* cache, const int32_t* prefix_blocks,
                                    int32_t prefix_len, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, float scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (cache->dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;  // the prefix runs on the matrix cores
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if (prefix_len < 0 || prefix_len % PKV_BLOCK_SIZE != 0 || prefix_len >= (1 << 30)) return PKV_ERR_SHAPE;
  if (prefix_len > 0 && !prefix_blocks) return PKV_ERR_NULL;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  const size_t pre = prefix_workspace(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim, prefix_len);
  const size_t pre_aligned = (pre + 255) / 256 * 256;
  const size_t need = pre_aligned + balanced_workspace(num_q_heads, cache->num_kv_heads, cache->head_dim);
  if (!workspace_ok(workspace, workspace_bytes, need)) return PKV_ERR_WORKSPACE;
  const float sl2 = scale * kLog2eHost;
  char* ws = reinterpret_cast<char*>(workspace);
  float* pre_o = reinterpret_cast<float*>(ws);
  PrefixSplit ps{0, 0};
  if (prefix_len > 0) {
    ps = prefix_split(num_seqs, num_q_heads, cache->num_kv_heads, prefix_len);
    float* pre_ml = pre_o + (size_t)ps.splits * num_seqs * num_q_heads * cache->head_dim;
    PrefillArgs pa{};
    pa.q = q;
    pa.k_cache = k_cache;
    pa.v_cache = v_cache;
    pa.block_tables = prefix_blocks;
    pa.num_chunks = num_seqs;
    pa.chunk_len_max = 1;
    pa.num_q_heads = num_q_heads;
    pa.num_kv_heads = cache->num_kv_heads;
    pa.head_dim = cache->head_dim;
    pa.num_blocks = cache->num_blocks;
    pa.max_blocks_per_seq = prefix_len / PKV_BLOCK_SIZE;
    pa.scale_log2 = sl2;
    pa.prefix_len = prefix_len;
    pa.split_tokens = ps.split_tokens;
    pa.num_splits = ps.splits;
    pa.part_o = pre_o;
    pa.part_ml = pre_ml;
    st = from_hip(launch_prefix_mfma(pa, as_stream(hip_stream)));
    if (st != PKV_OK) return st;
    // one partial per (sequence, head): every stream then starts from a single load
    st = from_hip(launch_prefix_merge(pre_o, pre_ml, (int64_t)num_seqs * num_q_heads, ps.splits, cache->head_dim,
                                      as_stream(hip_stream)));
    if (st != PKV_OK) return st;
  }
  DecodeArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.chunk_start = nullptr;
  const size_t dec = balanced_workspace(num_q_heads, cache->num_kv_heads, cache->head_dim);
  a.part_o = reinterpret_cast<float*>(ws + pre_aligned);
  a.part_ml = reinterpret_cast<float*>(ws + pre_aligned + dec / ((size_t)cache->head_dim + 2) * cache->head_dim);
  a.num_seqs = num_seqs;
  a.rows_per_seq = 1;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.dtype = cache->dtype;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.partition_tokens = max_blocks_per_seq * PKV_BLOCK_SIZE;
  a.max_parts = 1;
  a.scale_log2 = sl2;
  a.balanced_waves =
      balanced_waves(heads_per_wave(num_q_heads / cache->num_kv_heads), cache->dtype, cache->head_dim, 0);
  if (prefix_len > 0) {
    a.init_o = pre_o;
    a.init_ml = pre_o + (size_t)ps.splits * num_seqs * num_q_heads * cache->head_dim;
    a.init_splits = 1;  // merged above
  }
  return from_hip(launch_decode(a, as_stream(hip_stream)));
}

int paged_attn_prefill_chunk(const void* q_chunk, int32_t num_chunks, int32_t chunk_len_max, int32_t num_q_heads,
                             const int32_t* chunk_start, const void* k_cache, const void* v_cache,
                             const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, float scale, void* out, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_chunks < 0) return PKV_ERR_SHAPE;
  if (num_chunks == 0) return PKV_OK;
  if (!q_chunk || !chunk_start || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKV_ERR_NULL;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (chunk_len_max <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  const float sl2 = scale * kLog2eHost;
  if (cache->dtype == PKV_DTYPE_BF16) {
    PrefillArgs a{q_chunk, out, k_cache, v_cache, block_tables, context_lens, chunk_start, num_chunks,
                  chunk_len_max, num_q_heads, cache->num_kv_heads, cache->head_dim, cache->num_blocks,
                  max_blocks_per_seq, sl2};
    return from_hip(launch_prefill_mfma(a, as_stream(hip_stream)));
  }
  // float32: every chunk row is a decode query over its causal prefix, one
  // partition covering the whole table (no workspace)
  DecodeArgs a{};
  a.q = q_chunk;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.chunk_start = chunk_start;
  a.num_seqs = num_chunks;
  a.rows_per_seq = chunk_len_max;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.dtype = cache->dtype;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.partition_tokens = max_blocks_per_seq * PKV_BLOCK_SIZE;
  a.max_parts = 1;
  a.scale_log2 = sl2;
  return from_hip(launch_decode(a, as_stream(hip_stream)));
}

size_t paged_attn_prefill_chunk_workspace_bytes(int32_t num_chunks, int32_t chunk_len_max, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq) {
  if (num_chunks <= 0 || chunk_len_max <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 128)
    return 0;
  return chunk_workspace(num_chunks, chunk_len_max, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq);
}

int paged_attn_prefill_chunk_ws(const void* q_chunk, int32_t num_chunks, int32_t chunk_len_max, int32_t num_q_heads,
                                const int32_t* chunk_start, const void* k_cache, const void* v_cache,
                                const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, float scale, void* out, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_chunks < 0) return PKV_ERR_SHAPE;
  if (num_chunks == 0) return PKV_OK;
  if (!q_chunk || !chunk_start || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKV_ERR_NULL;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (chunk_len_max <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  if (cache->dtype != PKV_DTYPE_BF16 || num_q_heads / cache->num_kv_heads > 128)
    return paged_attn_prefill_chunk(q_chunk, num_chunks, chunk_len_max, num_q_heads, chunk_start, k_cache, v_cache,
                                    cache, block_tables, max_blocks_per_seq, context_lens, scale, out, hip_stream);
  const ChunkSplit v = chunk_split(num_chunks, chunk_len_max, num_q_heads, cache->num_kv_heads, max_blocks_per_seq);
  const size_t need = chunk_workspace(num_chunks, chunk_len_max, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                      max_blocks_per_seq);
  if (!workspace_ok(workspace, workspace_bytes, need)) return PKV_ERR_WORKSPACE;
  PrefillArgs a{q_chunk, out, k_cache, v_cache, block_tables, context_lens, chunk_start, num_chunks, chunk_len_max,
                num_q_heads, cache->num_kv_heads, cache->head_dim, cache->num_blocks, max_blocks_per_seq,
                scale * kLog2eHost};
  if (v.splits > 1) {
    a.split_tokens = v.split_tokens;
    a.num_splits = v.splits;
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)v.splits * num_chunks * chunk_len_max * num_q_heads * cache->head_dim;
  }
  return from_hip(launch_prefill_mfma(a, as_stream(hip_stream)));
}

size_t paged_attn_spec_verify_workspace_bytes(int32_t num_seqs, int32_t rows_max, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq) {
  const size_t chunk = paged_attn_prefill_chunk_workspace_bytes(num_seqs, rows_max, num_q_heads, num_kv_heads,
                                                                head_dim, max_blocks_per_seq);
  if (chunk == 0 && (num_seqs <= 0 || rows_max <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
                     max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0))
    return 0;
  // the balanced split's partial slots where a bf16 cache of this shape takes it
  const int gb = heads_per_wave(num_q_heads / num_kv_heads);
  const size_t bal =
      verify_takes_balanced(num_seqs, rows_max, num_q_heads, num_kv_heads, head_dim, PKV_DTYPE_BF16)
          ? verify_workspace(gb, head_dim, rows_max)
          : 0;
  return chunk > bal ? chunk : bal;
}

int paged_attn_spec_verify(const void* q, int32_t num_seqs, int32_t rows_max, int32_t num_q_heads,
                           const int32_t* row_start, const void* k_cache, const void* v_cache,
                           const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, float scale, void* out, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  int st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !row_start || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (rows_max <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE >= (int64_t)1 << 31) return PKV_ERR_SHAPE;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  const int gb = heads_per_wave(num_q_heads / cache->num_kv_heads);
  if (!verify_takes_balanced(num_seqs, rows_max, num_q_heads, cache->num_kv_heads, cache->head_dim, cache->dtype))
    return paged_attn_prefill_chunk_ws(q, num_seqs, rows_max, num_q_heads, row_start, k_cache, v_cache, cache,
                                       block_tables, max_blocks_per_seq, context_lens, scale, out, workspace,
                                       workspace_bytes, hip_stream);
  const size_t need = verify_workspace(gb, cache->head_dim, rows_max);
  if (!workspace_ok(workspace, workspace_bytes, need)) return PKV_ERR_WORKSPACE;
  DecodeArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.chunk_start = row_start;
  a.num_seqs = num_seqs;
  a.rows_per_seq = rows_max;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.dtype = cache->dtype;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = scale * kLog2eHost;
  a.balanced_waves = kVerifyWaves;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)kVerifyWaves * 2 * (gb * rows_max <= 16 ? 16 : 32) * cache->head_dim;
  return from_hip(launch_verify(a, as_stream(hip_stream)));
}

}  // extern "C"
