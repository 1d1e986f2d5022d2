// Host-side block bookkeeping for copy-on-write sharing of cache blocks.
//
// ainews.alishangtian.com article on inference engines, section
// "PagedAttention": sequences (parallel samples, beams) may hold the same
// physical blocks; a block held by more than one sequence is copied to a block
// of its own before one of them writes into it.  This file keeps the counts of
// holders and the free pool in caller-owned host arrays and decides, for each
// new token, its slot and whether a copy is needed.  The copies themselves run
// on the device (paged_kv_copy_blocks); nothing here touches the GPU.
//
// Every call validates all it will touch before changing anything, so a call
// that returns an error leaves the tables, counts and free list as they were.
#include <stdint.h>

#include "pagedkv.h"

namespace {

bool in_range(int32_t b, int32_t n) { return b >= 0 && b < n; }

int32_t pop_free(int32_t* free_list, int32_t* free_count) { return free_list[--*free_count]; }

}  // namespace

extern "C" {

int paged_block_fork(const int32_t* parent_table, int32_t num_table_blocks, int32_t* child_table,
                     int32_t* ref_counts, int32_t num_blocks) {
  if (num_table_blocks < 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (num_table_blocks == 0) return PKV_OK;
  if (!parent_table || !child_table || !ref_counts) return PKV_ERR_NULL;
  for (int32_t i = 0; i < num_table_blocks; ++i) {
    const int32_t b = parent_table[i];
    if (!in_range(b, num_blocks) || ref_counts[b] < 1) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_table_blocks; ++i) {
    const int32_t b = parent_table[i];
    child_table[i] = b;
    ++ref_counts[b];
  }
  return PKV_OK;
}

int paged_block_append_slot(int32_t* table, int32_t max_blocks_per_seq, int32_t context_len, int32_t* ref_counts,
                            int32_t num_blocks, int32_t* free_list, int32_t* free_count, int32_t* slot,
                            int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies) {
  if (!table || !ref_counts || !free_list || !free_count || !slot || !copy_src || !copy_dst || !num_copies)
    return PKV_ERR_NULL;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0 || context_len < 0) return PKV_ERR_SHAPE;
  if (*free_count < 0 || *free_count > num_blocks) return PKV_ERR_SHAPE;
  const int32_t idx = context_len / PKV_BLOCK_SIZE;
  const int32_t off = context_len % PKV_BLOCK_SIZE;
  if (idx >= max_blocks_per_seq) return PKV_ERR_SHAPE;
  *num_copies = 0;
  if (off == 0) {  // the token opens a new block
    if (*free_count == 0) return PKV_ERR_NO_BLOCKS;
    const int32_t nb = free_list[*free_count - 1];
    if (!in_range(nb, num_blocks) || ref_counts[nb] != 0) return PKV_ERR_SHAPE;
    pop_free(free_list, free_count);
    ref_counts[nb] = 1;
    table[idx] = nb;
  } else {
    const int32_t b = table[idx];
    if (!in_range(b, num_blocks) || ref_counts[b] < 1) return PKV_ERR_SHAPE;
    if (ref_counts[b] > 1) {  // shared partial block: this sequence takes a copy
      if (*free_count == 0) return PKV_ERR_NO_BLOCKS;
      const int32_t nb = free_list[*free_count - 1];
      if (!in_range(nb, num_blocks) || ref_counts[nb] != 0) return PKV_ERR_SHAPE;
      pop_free(free_list, free_count);
      --ref_counts[b];
      ref_counts[nb] = 1;
      table[idx] = nb;
      *copy_src = b;
      *copy_dst = nb;
      *num_copies = 1;
    }
  }
  *slot = table[idx] * PKV_BLOCK_SIZE + off;
  return PKV_OK;
}

int paged_block_release(const int32_t* table, int32_t num_table_blocks, int32_t* ref_counts, int32_t num_blocks,
                        int32_t* free_list, int32_t* free_count) {
  if (num_table_blocks < 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (num_table_blocks == 0) return PKV_OK;
  if (!table || !ref_counts || !free_list || !free_count) return PKV_ERR_NULL;
  if (*free_count < 0 || *free_count > num_blocks) return PKV_ERR_SHAPE;
  // a table holds each block once, and every block it holds has a holder
  int32_t freed = 0;
  for (int32_t i = 0; i < num_table_blocks; ++i) {
    const int32_t b = table[i];
    if (!in_range(b, num_blocks) || ref_counts[b] < 1) return PKV_ERR_SHAPE;
    for (int32_t j = 0; j < i; ++j)
      if (table[j] == b) return PKV_ERR_SHAPE;
    if (ref_counts[b] == 1) ++freed;
  }
  if (*free_count + freed > num_blocks) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < num_table_blocks; ++i) {
    const int32_t b = table[i];
    if (--ref_counts[b] == 0) free_list[(*free_count)++] = b;
  }
  return PKV_OK;
}

}  // extern "C"
