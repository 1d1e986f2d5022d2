/*
 * pagedkv.h -- C ABI of libpagedkv.so: attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The cache organisation follows the pages this library is built from:
 *   - the ainews.alishangtian.com article on inference engines, section
 *     "PagedAttention": the KV cache is cut into fixed-size blocks (usually 16
 *     tokens), allocated on demand and chained per request by a block table;
 *     requests with a common prefix reference the same physical blocks;
 *   - "Part 47 | Inference basics: KV Cache, batching, sampling"
 *     (chengxuchu.com): section 2.1 (softmax(Q K^T / sqrt(d)) V, the query of
 *     position t reads keys 1..t), section 2.2 (decode appends the new K/V to
 *     the cache, then its query reads the whole cache; production code writes
 *     the new K/V into preallocated pages at a given position), section 2.3
 *     (cache shape and GQA: fewer kv heads than query heads), section 5.2
 *     (the GPU kernel finds each token's K/V through the block table);
 *   - the caffein.top essay on modern LLM inference runtimes, sections on
 *     chunked prefill (a long prompt is processed in chunks interleaved with
 *     decode steps) and on paging (logically contiguous tokens live in
 *     non-contiguous physical blocks).
 *
 * Layouts (all row-major, contiguous, device memory owned by the caller):
 *   k_cache, v_cache  [num_blocks][num_kv_heads][16][head_dim]
 *                     slot s = physical_block * 16 + offset_in_block
 *   block_tables      int32 [rows][max_blocks_per_seq]; entry j is the
 *                     physical block of logical tokens 16j .. 16j+15
 *   q (decode)        [num_seqs][num_q_heads][head_dim]
 *   q_chunk           [num_chunks][chunk_len_max][num_q_heads][head_dim]
 *   out               same shape and dtype as q / q_chunk
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 * Element type: float32 or bfloat16, the same for caches, k, v, q and out.
 * Accumulation is float32; a bf16 output is rounded to nearest even.
 *
 * Every call is asynchronous on `hip_stream` (a hipStream_t; NULL means the
 * default stream).  The library allocates nothing, keeps no pointer after
 * return and holds no state.  Arguments are validated on the host only
 * (nothing is read back from the device); on a non-zero return nothing was
 * launched.  Device-resident values that break the contract below are not
 * reported by a return code; the kernels never read or write outside the
 * buffers described here because of them, and the affected outputs are set
 * to NaN (or, for the write, the row is skipped) as each function states.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK 0
#define PKV_ERR_NULL (-1)        /* a required pointer is NULL */
#define PKV_ERR_DTYPE (-2)       /* dtype is neither PKV_DTYPE_F32 nor PKV_DTYPE_BF16 */
#define PKV_ERR_SHAPE (-3)       /* a size is negative/zero where it must be positive, Hq % Hkv != 0,
                                    max_context_len > 16 * max_blocks_per_seq, or index range overflow */
#define PKV_ERR_UNSUPPORTED (-4) /* block_size != 16, or head_dim not 64 or 128 */
#define PKV_ERR_WORKSPACE (-5)   /* workspace NULL, smaller than the query function requires, or not
                                    16-byte aligned */
#define PKV_ERR_HIP (-6)         /* a kernel launch failed (hipGetLastError after launch) */
#define PKV_ERR_NO_BLOCKS (-7)   /* block bookkeeping: the free pool is empty */
#define PKV_ERR_SCRATCH (-8)     /* paged_attn_decode_noalloc: the call needs more partial-state memory than
                                    the library's buffer holds */

#define PKV_DTYPE_F32 0
#define PKV_DTYPE_BF16 1
#define PKV_DTYPE_FP8_E4M3 2 /* quantised cache: the *_fp8 entry points only */
#define PKV_BLOCK_SIZE 16

/* Description of one layer's paged cache (both K and V use it). */
typedef struct pkv_cache_desc {
  int32_t num_blocks;   /* physical blocks in the pool, >= 1 */
  int32_t block_size;   /* tokens per block; must be 16 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t dtype;        /* PKV_DTYPE_F32, PKV_DTYPE_BF16, or PKV_DTYPE_FP8_E4M3 (*_fp8 calls) */
} pkv_cache_desc;

/*
 * paged_kv_write -- scatter new K/V rows into their cache slots.
 * ("Part 47", section 2.2: the new token's K/V are written at a given
 * position of preallocated pages before the query reads the cache.)
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], cache dtype
 *   slot_mapping  int32 [num_tokens]; row i goes to block slot_mapping[i] / 16,
 *                 offset slot_mapping[i] % 16, for every kv head
 *   k_cache, v_cache   updated in place
 *
 * A raw copy of the bit patterns (bit-exact).  A negative slot skips its row
 * (lets a caller pad); a slot >= 16 * num_blocks is also skipped.  Two rows with
 * the same slot in one call leave either row there (unspecified which).
 * num_tokens == 0 is a no-op that returns PKV_OK.
 */
int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, const pkv_cache_desc* cache, void* hip_stream);

/*
 * paged_kv_copy_blocks -- copy whole cache blocks: for each i,
 * block dst_blocks[i] of k_cache and of v_cache (every kv head, all 16 slots)
 * becomes a copy of block src_blocks[i].  (ainews.alishangtian.com article,
 * section "PagedAttention": a block shared by several sequences is copied to
 * a block of its own before one of them writes into it -- copy-on-write.)
 *
 *   src_blocks, dst_blocks   int32 [num_pairs] (device)
 *
 * A raw copy of the bit patterns (bit-exact).  A pair with an id outside
 * [0, num_blocks) is skipped, src == dst is a no-op; a block that is the
 * destination of one pair and the source or destination of another in the same
 * call gets an unspecified one of the candidate contents.  num_pairs == 0 is a
 * no-op that returns PKV_OK.
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int64_t num_pairs, void* hip_stream);

/*
 * fp8 KV cache.  ("Part 47 | Inference basics", chengxuchu.com, section 2.4:
 * a server short of memory may keep the cache quantised.  The page names no
 * format; this library's is the following.)  Cache elements are OCP E4M3
 * bytes -- sign, 4 exponent bits with bias 7, 3 mantissa bits, largest finite
 * 448, no infinities -- in the same [num_blocks][num_kv_heads][16][head_dim]
 * layout, with one float32 scale per (slot, kv head):
 *
 *   k_scale, v_scale   float32 [num_blocks][num_kv_heads][16] (device)
 *   value of element d of a slot's row = e4m3(code_d) * scale
 *
 * The descriptor's dtype is PKV_DTYPE_FP8_E4M3; queries and outputs are
 * bfloat16.  Quantisation (paged_kv_write_fp8), per new row of one kv head,
 * in float32:  amax = max |x|,  scale = amax / 448,  inv = 448 / amax (0 when
 * amax is 0),  code = the E4M3 value nearest to clamp(x * inv, -448, 448),
 * ties to the even code.  The codes and scales are reproducible bit for bit;
 * each write touches only its own slots.
 *
 * paged_kv_write_fp8: as paged_kv_write, from k, v [num_tokens][num_kv_heads]
 *   [head_dim] of in_dtype (PKV_DTYPE_BF16 or PKV_DTYPE_F32), storing codes
 *   and scales.  Rows must be finite.
 * paged_attn_decode_fp8: as paged_attn_decode over the dequantised cache
 *   (workspace sizes from paged_attn_decode_workspace_bytes).  Each token's K
 *   scale multiplies its scores and its V scale its weights, so the codes are
 *   widened exactly and never rescaled element by element.
 * paged_kv_copy_blocks_fp8: as paged_kv_copy_blocks, copying the blocks'
 *   codes and their scales.
 *
 * The prefill-chunk and shared-prefix calls take float32 / bfloat16 caches
 * only.  Errors as for the unquantised calls; PKV_ERR_DTYPE for a descriptor
 * that is not PKV_DTYPE_FP8_E4M3 or an in_dtype other than bf16 / f32.
 */
int paged_kv_write_fp8(const void* k, const void* v, int32_t in_dtype, const int32_t* slot_mapping,
                       int64_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pkv_cache_desc* cache, void* hip_stream);
int paged_attn_decode_fp8(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                          int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* hip_stream);
int paged_kv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             const pkv_cache_desc* cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                             int64_t num_pairs, void* hip_stream);

/*
 * Host-side block bookkeeping for copy-on-write sharing (same "PagedAttention"
 * section of the inference-engine article on ainews.alishangtian.com).  Plain
 * host memory, no GPU work, not thread-safe; every array is owned by the
 * caller:
 *
 *   ref_counts   int32 [num_blocks]  how many block tables hold each block
 *   free_list    int32 [num_blocks]  a stack of unheld blocks, the first
 *                                    *free_count entries valid; pops take the last
 *   tables       int32 [max_blocks_per_seq] per sequence, as for the attention calls
 *
 * paged_block_fork: child_table[0 .. num_table_blocks) = parent_table[...], and
 *   each of those blocks gains a holder.  Nothing is copied: the child shares
 *   every block, the partially filled last one included.
 * paged_block_append_slot: the slot for a sequence's next token, at position
 *   context_len (the tokens it already has).  A token at offset 0 of a block
 *   takes a block from the free list.  A token inside a block that other
 *   sequences also hold first moves this sequence to a copy: a free block
 *   replaces the shared one in `table`, the shared one loses a holder, and
 *   (*copy_src, *copy_dst) is the pair to pass to paged_kv_copy_blocks before
 *   the token is written (*num_copies = 1; else 0).  *slot = block * 16 + offset.
 * paged_block_release: each of the table's blocks loses a holder; a block left
 *   with none goes back on the free list.  A table must not hold a block twice.
 *
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (a count out of range, a block id outside
 * [0, num_blocks), a held block whose count is below one, a free block whose
 * count is not zero, a position beyond max_blocks_per_seq * 16, a duplicate in
 * a released table), PKV_ERR_NO_BLOCKS (free list empty).  On any error
 * nothing has been changed.
 */
int paged_block_fork(const int32_t* parent_table, int32_t num_table_blocks, int32_t* child_table,
                     int32_t* ref_counts, int32_t num_blocks);
int paged_block_append_slot(int32_t* table, int32_t max_blocks_per_seq, int32_t context_len, int32_t* ref_counts,
                            int32_t num_blocks, int32_t* free_list, int32_t* free_count, int32_t* slot,
                            int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies);
int paged_block_release(const int32_t* table, int32_t num_table_blocks, int32_t* ref_counts, int32_t num_blocks,
                        int32_t* free_list, int32_t* free_count);

/*
 * Split-context decode.  A sequence's context is cut into pieces; each piece
 * yields a running max, a sum of exponentials and an unnormalised output, and
 * a log-sum-exp merge combines the pieces, which equals the one-pass softmax
 * in exact arithmetic.  Two ways of cutting:
 *
 *   partition_tokens == 0 (recommended): balanced split.  The whole batch's
 *     work -- every (sequence, kv head, 16-token block) -- is divided over
 *     wavefronts in runs of consecutive blocks:
 *     paged_attn_decode_split_waves(num_q_heads, num_kv_heads) of them for a
 *     bf16 cache whose longest context (max_context_len) reaches 1024 tokens;
 *     otherwise 1024 or 2048 as the arithmetic per byte needs (2048 where the
 *     vector ALU computes the scores of eight heads per wave or of E4M3
 *     codes).  Each (sequence, kv head) stream is
 *     charged its blocks plus a fixed cost for starting it, and every wavefront
 *     gets the same total charge, so all finish together whatever the mix of
 *     context lengths; a context is cut wherever a run ends.  The workspace
 *     size does not depend on the context lengths or the cache dtype.  A batch
 *     with no more blocks in all than wavefronts runs one wavefront per stream
 *     over its whole context instead.
 *   partition_tokens > 0 (a multiple of 16): fixed partitions of that many
 *     tokens per sequence, one wavefront each.
 *
 * paged_attn_decode_split_waves returns 0 for invalid head counts.
 * paged_attn_decode_workspace_bytes returns the workspace paged_attn_decode
 * needs for these sizes (0 if none).
 */
int32_t paged_attn_decode_split_waves(int32_t num_q_heads, int32_t num_kv_heads);

/*
 * paged_attn_lse_merge -- the log-sum-exp merge of split-context partials on
 * its own: for every row r, with partials p = 0 .. num_parts-1,
 *     M = max_p m_p,   out[r] = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
 * which is softmax(x) V over the union of the parts' keys ("Part 47",
 * section 2.1, for the softmax; splitting a context into parts is this
 * library's, the pages do not describe it).  It is the merge the decode calls
 * run after fixed partitions, exported so that it can be checked alone.
 *
 *   part_o    float32 [num_rows][num_parts][head_dim]: o_p = sum_t 2^(y_t - m_p) v_t,
 *             unnormalised, over part p's keys t (y_t = score * log2(e))
 *   part_ml   float32 [num_rows][num_parts][2]: (m_p, l_p) with m_p >= max_t y_t of
 *             the part, in log2 units, and l_p = sum_t 2^(y_t - m_p)
 *   out       [num_rows][head_dim], out_dtype PKV_DTYPE_F32 or PKV_DTYPE_BF16
 *             (bf16 rounded to nearest even)
 *
 * A part with no keys is (m_p, 0, 0) for any m_p that is not NaN (-inf
 * included, as long as some part of the row has a finite m_p).  A row with a
 * NaN m_p gets NaN; a row whose parts are all empty is undefined.  part_o and
 * part_ml must be 16-byte aligned (PKV_ERR_SHAPE otherwise).  num_rows == 0
 * is a no-op.
 */
int paged_attn_lse_merge(const float* part_o, const float* part_ml, int64_t num_rows, int32_t num_parts,
                         int32_t head_dim, int32_t out_dtype, void* out, void* hip_stream);
size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len, int32_t partition_tokens);

/*
 * paged_attn_decode -- one continuous-batching decode step: for every sequence
 * s and query head h,
 *     out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 * over the first context_lens[s] tokens of sequence s, reached through
 * block_tables[s].  ("Part 47", sections 2.1-2.2; the new token's K/V must
 * already be in the cache, so its query sits at position context_lens[s]-1.)
 *
 *   q, out            [num_seqs][num_q_heads][head_dim]
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]
 *   context_lens      int32 [num_seqs] (device); context_lens[s] == 0 gives out = 0
 *   max_context_len   host-side upper bound of context_lens (sizes the grid
 *                     and the workspace of fixed partitions)
 *   scale             softmax scale, usually 1/sqrt(head_dim)
 *   partition_tokens  0 = balanced split, else fixed partitions of that many
 *                     tokens (a positive multiple of 16)
 *   workspace         device scratch of at least
 *                     paged_attn_decode_workspace_bytes(...) bytes, 16-byte
 *                     aligned (may be NULL when that is 0); contents need no
 *                     initialisation
 *
 * Device-side contract: 0 <= context_lens[s] <= max_context_len and the first
 * ceil(context_lens[s]/16) table entries lie in [0, num_blocks).  A sequence
 * that breaks it gets NaN in every output row of the heads concerned (with
 * fixed partitions a context above max_context_len counts as broken; the
 * balanced split accepts any context up to 16 * max_blocks_per_seq).
 * num_seqs == 0 is a no-op.
 */
int paged_attn_decode(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                      const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                      float scale, void* out, int32_t partition_tokens, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same arguments and result as
 * paged_attn_decode, without the workspace: the partial states of the split
 * live in a buffer inside the library, paged_attn_decode_noalloc_scratch_bytes()
 * bytes (16.25 MiB) on each GPU it runs on, held until the process ends and
 * set up on the first call on that GPU (that GPU must be current).  The call
 * allocates nothing (no hipMalloc, no allocating library routine).  That
 * buffer covers the balanced split (partition_tokens == 0) at every supported
 * shape; fixed partitions whose workspace would exceed it return
 * PKV_ERR_SCRATCH before anything is launched.  Every call on one GPU shares
 * that GPU's buffer: two calls that may run at the same time on one GPU (on
 * different streams without an ordering between them) race and give
 * undefined results.  Nothing in the buffer needs to start at zero.
 */
size_t paged_attn_decode_noalloc_scratch_bytes(void);
int paged_attn_decode_noalloc(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                              const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                              float scale, void* out, int32_t partition_tokens, void* hip_stream);

/*
 * paged_attn_decode_shared_prefix -- a decode step (as paged_attn_decode) for
 * a batch of sequences that all start with the same prompt prefix held once
 * in shared physical blocks.  (ainews.alishangtian.com article, section
 * "PagedAttention": requests with a common prefix reference the same physical
 * blocks; caffein.top essay, section on the prefix tree.)  The prefix is
 * attended once for the whole batch as a dense matrix-core problem (every
 * query of the batch against the prefix keys, read from HBM once); each
 * sequence's own tokens then continue from that state, and the log-sum-exp
 * merge makes the result equal to attention over the concatenated context.
 *
 *   q, out            [num_seqs][num_q_heads][head_dim]
 *   prefix_blocks     int32 [prefix_len / 16]: the shared prefix's blocks, in order
 *   prefix_len        tokens of the prefix, a multiple of 16 (0: plain decode)
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]: each sequence's
 *                     blocks after the prefix (its logical tokens prefix_len ..)
 *   context_lens      int32 [num_seqs] (device): tokens after the prefix,
 *                     including the new one; 0 gives attention over the prefix alone
 *   workspace         device scratch of at least
 *                     paged_attn_decode_shared_prefix_workspace_bytes(...) bytes,
 *                     16-byte aligned
 *
 * Sequence s attends to prefix tokens 0 .. prefix_len-1 followed by its own
 * context_lens[s] tokens.  bfloat16 caches only (PKV_ERR_UNSUPPORTED for
 * float32).  Device-side contract and NaN behaviour as paged_attn_decode (the
 * balanced split; a prefix block id out of range makes every output NaN).
 */
size_t paged_attn_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t prefix_len);
int paged_attn_decode_shared_prefix(const void* q, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                                    const void* v_cache, const pkv_cache_desc* cache, const int32_t* prefix_blocks,
                                    int32_t prefix_len, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, float scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

/*
 * paged_attn_prefill_chunk -- causal attention for chunks of prompts whose
 * K/V (including the chunk's own rows) are already in the cache.
 * (caffein.top essay, section on chunked prefill; "Part 47", section 2.1 for
 * the causal rule.)
 *
 *   q_chunk, out      [num_chunks][chunk_len_max][num_q_heads][head_dim]
 *   chunk_start       int32 [num_chunks] (device): position of the chunk's row 0
 *   context_lens      int32 [num_chunks] (device): tokens in the cache for the
 *                     chunk's sequence, through the chunk's last row
 *   block_tables      int32 [num_chunks][max_blocks_per_seq]
 *
 * Chunk c has n_c = context_lens[c] - chunk_start[c] rows; row i (i < n_c)
 * sits at position chunk_start[c] + i and attends to keys 0 .. chunk_start[c]+i.
 * Rows i >= n_c of out are not written.  Device-side contract:
 * 0 <= chunk_start[c] <= context_lens[c] <= 16 * max_blocks_per_seq,
 * n_c <= chunk_len_max, and table entries in range; a chunk that breaks it gets
 * NaN in its valid rows (rows up to chunk_len_max for n_c too large).
 * bf16 runs on the matrix cores (MFMA); float32 runs on the vector ALUs.
 * num_chunks == 0 is a no-op.
 */
int paged_attn_prefill_chunk(const void* q_chunk, int32_t num_chunks, int32_t chunk_len_max,
                             int32_t num_q_heads, const int32_t* chunk_start, const void* k_cache,
                             const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                             void* out, void* hip_stream);

/*
 * paged_attn_prefill_chunk_ws -- paged_attn_prefill_chunk with a workspace:
 * the same arguments, result and device-side contract, and a caller-owned
 * device workspace of at least paged_attn_prefill_chunk_workspace_bytes(...)
 * bytes, 16-byte aligned (0 means none is needed: the call then behaves as
 * the plain one).
 * When the batch has fewer (chunk, row tile, kv head) units than the GPU runs
 * workgroups at once, the keys of every row tile are cut into pieces spread
 * over the GPU and combined by a log-sum-exp merge, so one long row tile does
 * not run alone at the end.  bfloat16 runs on the matrix cores; float32 takes
 * the plain call's path (no workspace used).
 */
size_t paged_attn_prefill_chunk_workspace_bytes(int32_t num_chunks, int32_t chunk_len_max, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq);
int paged_attn_prefill_chunk_ws(const void* q_chunk, int32_t num_chunks, int32_t chunk_len_max, int32_t num_q_heads,
                                const int32_t* chunk_start, const void* k_cache, const void* v_cache,
                                const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, float scale, void* out, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/*
 * paged_attn_spec_verify -- the target model's attention pass that verifies
 * speculative draft tokens.  (Serving deep-dive page, paragraph on
 * speculative decoding, and the caffein.top essay, section "Speculative
 * Decoding": cheap drafts propose several tokens and the target model checks
 * them all in one pass.)  Each sequence brings a short run of new rows -- its
 * last accepted token and k drafts -- whose K/V are already written, and row
 * i at position row_start[s] + i attends causally to keys 0 .. that position:
 * exactly paged_attn_prefill_chunk's result with chunk_len_max = rows_max
 * (same argument layout and device-side contract, rows past a sequence's
 * count not written).  Two work splits.  With a bf16 cache at head_dim 128,
 * four or eight query heads per wavefront (num_q_heads / num_kv_heads a
 * multiple of 4) whose rows fit 32 matrix-core columns (heads per wavefront x
 * rows_max <= 32), and at least 128 (sequence, kv head, head subgroup)
 * streams: the decode's balanced split, each stream's heads x rows the
 * columns of its score and value products, every row masked at its own
 * position, its blocks cut over 1024 wavefronts by cost and the cut streams
 * merged.  Otherwise as paged_attn_prefill_chunk_ws: the rows of a sequence
 * share one row tile per kv head, and with few sequences each (sequence, kv
 * head)'s keys are cut into pieces spread over the GPU.  Workspace: at least
 * paged_attn_spec_verify_workspace_bytes(...) bytes, 16-byte aligned (0: none
 * needed; the size covers a bf16 cache, which the balanced split needs).
 */
size_t paged_attn_spec_verify_workspace_bytes(int32_t num_seqs, int32_t rows_max, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq);
int paged_attn_spec_verify(const void* q, int32_t num_seqs, int32_t rows_max, int32_t num_q_heads,
                           const int32_t* row_start, const void* k_cache, const void* v_cache,
                           const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, float scale, void* out, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/*
 * paged_kv_read_probe -- a measurement aid: reads the K/V bytes a decode call
 * over the same batch reads, the way its kernel reads them, and computes
 * nothing else.  ("Part 47", section 5.2: the kernel's cost of following the
 * block table; the decode step is bound by memory bandwidth.)  Every row
 * t < context_lens[s] of every (sequence s, kv head) K and V tile reached
 * through block_tables is loaded with the decode's 16-byte non-temporal
 * loads, four blocks in flight per wavefront, the batch's blocks divided
 * evenly over num_waves wavefronts (1 .. 65536); wavefront w folds the 32-bit
 * words it read with XOR into out_words[w] (device, uint32 [num_waves]), so
 * no load can be dropped.  Its duration is what the memory system allows for
 * this access pattern -- a floor under the decode call -- and its hardware
 * byte counters, against the exact bytes it reads, calibrate those counters
 * for these loads.  Any cache dtype; of an E4M3 cache it reads the codes
 * only (the per-row scales a decode also reads are left out).  Device-side
 * contract as paged_attn_decode (a context outside
 * [0, 16 * max_blocks_per_seq] reads nothing; a block id outside the pool
 * reads block 0).
 */
int paged_kv_read_probe(const void* k_cache, const void* v_cache, const pkv_cache_desc* cache,
                        const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_waves, uint32_t* out_words, void* hip_stream);

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int32_t pkv_abi_version(void);
#define PKV_ABI_VERSION ((1 << 16) | 7)

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
