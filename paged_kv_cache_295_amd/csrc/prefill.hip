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
//  * Key tiles of 64 tokens (4 cache blocks, one per wave) stream through NS
//    LDS stages with direct-to-LDS loads, NS - 1 tiles ahead of the compute;
//    the block-table entry of a wave's block is a scalar load fetched a tile
//    earlier.  K and V land row-major with their 16-byte chunks XOR-swizzled
//    by row (chunk c of key row r at position c ^ (r mod chunks-per-row)), so
//    the operand reads below hit distinct LDS banks.  Blocks past the keys
//    any row may see load block 0, and once the last tile has landed its V
//    rows past those keys are zeroed in LDS: masked keys then carry exact
//    zeros, never the contents of unused cache slots (0 * NaN is NaN).
//  * Transposed formulation so that each lane owns one query row:
//      S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K (LDS), B = Q (registers)
//      O^T += V^T P^T   A = V^T (LDS transpose reads), B = P (registers)
//    In the 32x32 accumulator layout lane l holds column l % 32 (its query
//    row) and 16 of the 32 rows, the other 16 sit in lane l ^ 32; so the row
//    max needs one exchange with lane l ^ 32, and the softmax rescale of O^T
//    is a per-lane multiply.  P feeds the second product straight from the
//    registers of the first: its key order (keys 4h..4h+3 and 8+4h..8+4h+3 of
//    each 16-key step for half h of the wave) is what two ds_read_b64_tr_b16
//    per operand deliver from the row-major V tile: within each 16-lane group,
//    lane i receives element i mod 4 of the 8-byte rows addressed by lanes
//    i/4 + 4k, k = 0..3, so lanes addressing 4 consecutive keys x 4 dims hand
//    every lane 4 consecutive keys of one dim.
//  * LDS reads are issued from asm blocks (with their own wait): the compiler
//    cannot tell which pending direct-to-LDS load a read depends on and would
//    otherwise drain them all before every read.
//  * Online softmax in the log2 domain; causal mask by select (never by
//    multiplying); P is rounded to bf16 for the matrix cores, accumulation
//    stays float32.
#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Keys per tile: 64 (four cache blocks, one per wave) or 32 (two blocks, half
// a block per wave).
#ifndef PKV_PREFILL_TILE_KEYS
#define PKV_PREFILL_TILE_KEYS 64
#endif
constexpr int kKT = PKV_PREFILL_TILE_KEYS;
constexpr int kNB = kKT / 32;  // 32-key blocks of the matrix products per tile
constexpr int kMRows = 128;   // (head, row) pairs per workgroup
constexpr int kThreads = 256;
// Rescale slack of the online softmax, in powers of two (see the tile loop).
constexpr float kPrefillSlack = 8.0f;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = kKT / kWaves;  // key rows each wave loads per tile
static_assert(kKT == 64 || kKT == 32, "tiles of 64 or 32 keys");

// Two LDS stages (64 KiB per workgroup at head_dim 128) and registers kept
// to two waves per SIMD let two workgroups share a compute unit, so one
// workgroup's matrix-core work overlaps the other's softmax and LDS waits.
// Measured on the MI355X against three stages with one workgroup per compute
// unit: 16 chunks x 512 rows at 3584 keys 676 us against 892 us, the
// mixed-step chunks 52 us against 60 us, the 64-sequence verify pass 144 us
// against 198 us.
#ifndef PKV_PREFILL_STAGES
#define PKV_PREFILL_STAGES (PKV_PREFILL_TILE_KEYS == 32 ? 4 : 2)
#endif
// Waves per SIMD the register allocation must allow.
#ifndef PKV_PREFILL_WAVES_PER_SIMD
#define PKV_PREFILL_WAVES_PER_SIMD 2
#endif
// (A loop with K one tile ahead of V in separate rings, the next tile's
// scores issued before this tile's softmax, was measured no faster: 54 us
// against 52.5 us on the mixed-step chunks, 673 us against 658 us for 16 x 512
// rows at 3584 keys.)

// XOR swizzle of the 16-byte chunks of V row `key` (K rows use key mod chunks);
// it must repeat every 16 rows (the reads add whole 16-row steps as immediate
// offsets).  0: key mod chunks; 1: 2 key mod chunks; 2: 4 (key mod 4) +
// (key / 4) mod 4.  A transpose read serves 32 lanes at a time over 64 banks
// on gfx950: each 16-lane group reads 4 consecutive keys x 32 bytes, and only
// option 2 spreads the two groups' 8 key-chunk pairs over distinct banks
// (rocprofv3 SQ_LDS_BANK_CONFLICT: 95.2 M cycles with option 0, 31.7 M with
// option 1, 0 with option 2; 16 x 512 rows at 3584 keys 668 -> 644 us).
#ifndef PKV_PREFILL_VSWZ
#define PKV_PREFILL_VSWZ 2
#endif

template <int D>
struct PrefillShape {
  static constexpr int kRowBytes = D * 2;                // one K or V row (bf16)
  static constexpr int kRC = kRowBytes / 16;             // 16-byte chunks per row
  static constexpr int kTileBytes = kKT * kRowBytes;     // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;     // K then V
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one direct-to-LDS load fills
  static constexpr int kLoadsPerWave = kRowsPerWave / kRowsPerLoad;  // per matrix, for the wave's rows
  static constexpr int kDW = 2 * kLoadsPerWave;          // direct-to-LDS loads per wave and tile
  static constexpr int kNS = PKV_PREFILL_STAGES;         // LDS stages
  static constexpr int kKSteps = D / 16;                 // QK^T steps of 16 head dims
  static constexpr int kND = D / 32;                     // PV output blocks of 32 head dims
  static_assert(kRowsPerLoad * kRC == 64, "one load covers whole rows");
  static_assert(kLoadsPerWave >= 1, "a wave's rows fill whole loads");
  static_assert((kNS - 2) * kDW < 64, "vmcnt is six bits");
  __host__ __device__ static constexpr int vswz(int key) {
    return PKV_PREFILL_VSWZ == 1 ? (2 * key) % kRC
         : PKV_PREFILL_VSWZ == 2 ? (4 * (key % 4) + (key / 4) % 4) % kRC
                                 : key % kRC;
  }
};

// Chunk rows per row tile: a tile holds 128 (head, row) pairs of one kv head.
// When all of a chunk's rows for the G heads fit one tile (short chunks: the
// speculative-verify rows), they are packed densely -- head-major, chunk_len_max
// rows per head -- so the waves past them carry no query and skip the math.
__host__ __device__ __forceinline__ int tile_rows(int chunk_len_max, int G) {
  return chunk_len_max * G <= kMRows ? chunk_len_max : kMRows / G;
}


// LDS reads, read i at base[i] + O.  ASM: in one asm block, completed before
// the block ends.  Otherwise plain loads that the compiler schedules and
// waits for one at a time (it must not see the direct-to-LDS loads as stores
// it has to wait for: those are then issued from asm, see load_lds_x4).
template <bool ASM, int O, int N>
__device__ __forceinline__ void lds_read_b128(const int (&base)[N], u32x4_t (&r)[N]) {
  static_assert(N == 4 || N == 8, "4 or 8 reads");
  static_assert(O >= 0 && O < 65536, "ds offset is 16 bits");
  if constexpr (!ASM) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      r[i] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)(uint32_t)(base[i] + O));
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\tds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\tds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "n"(O));
  } else {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\tds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\tds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\tds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\tds_read_b128 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "v"(base[4]), "v"(base[5]), "v"(base[6]),
          "v"(base[7]), "n"(O));
  }
}

template <bool ASM, int O, int N>
__device__ __forceinline__ void lds_read_tr16(const int (&base)[N], u32x2_t (&r)[N]) {
  static_assert(N == 4 || N == 8, "4 or 8 reads");
  static_assert(O >= 0 && O < 65536, "ds offset is 16 bits");
  if constexpr (!ASM) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < N; ++i)
      r[i] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(
                                                 (uintptr_t)(uint32_t)(base[i] + O))));
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\tds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\tds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "n"(O));
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\tds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\tds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\tds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\tds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "v"(base[4]), "v"(base[5]), "v"(base[6]),
          "v"(base[7]), "n"(O));
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}

// The ring's step boundary when the LDS reads are plain loads: this wave's
// direct-to-LDS loads of the step are done (at most N remain) and so are its
// LDS reads of the previous step, then the workgroup barrier; the asm
// statements also keep the compiler from moving LDS reads across it.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS load of 16 bytes per lane: global address base + voff
// (a scalar base and a per-lane offset fixed for the kernel, so no address is
// computed per tile), LDS address lds + 16 lane.  From asm, so that the
// compiler's wait insertion does not put a wait for it before every LDS read
// (the ring's own waits order the two); the large prefill 552-562 ->
// 541-545 us against the builtin's per-lane 64-bit addresses.
// M0 is clobbered: the kernels that use this set it nowhere else.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void load_lds_x4(const char* base, int voff, int lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds) : "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "m0");
}
#pragma clang diagnostic pop

// MODE kChunk: chunked prefill (rows = chunk rows x G heads of one kv head,
// keys 0 .. row position, causal).  MODE kPrefix: the shared prefix of a
// batch of decode queries (rows = (sequence, head) pairs of one kv head, keys
// = one piece of the prefix, no causal mask), written as (m, l, o) partials.
// MODE kSplit: chunked prefill with each row tile's keys cut into pieces of
// split_tokens, one workgroup per piece; a row tile with one piece writes its
// output, the others write (m, l, o) partials for prefill_split_merge_kernel.
constexpr int kChunk = 0, kPrefix = 1, kSplit = 2;

//
// KH = 2 (key halves): a workgroup of two groups of four waves over the same
// 128 rows, group kh taking key tiles kt0 + kh, kt0 + kh + 2, ... through its
// own LDS ring (128 KiB per workgroup at head_dim 128), the two states of each
// row merged through LDS at the end.  For grids of at most one workgroup per
// compute unit it halves the chain of key tiles a row tile walks, at the same
// waves per SIMD as two four-wave workgroups.
template <int D, int MODE, int KH>
__global__ __launch_bounds__(kThreads * KH) __attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WAVES_PER_SIMD)))
void prefill_mfma_kernel(const PrefillArgs a, const int32_t* __restrict__ tables) {
  constexpr bool PREFIX = MODE == kPrefix;
  using S = PrefillShape<D>;
  constexpr int NS = S::kNS;
  constexpr int RC = S::kRC;
  constexpr int RB = S::kRowBytes;
  constexpr int TB = S::kTileBytes;
  static_assert(KH == 1 || KH == 2, "one or two key halves");
  // How the LDS reads are waited for.  Two key halves (one eight-wave
  // workgroup per compute unit): plain loads, the compiler overlapping each
  // read with the products of the reads before it (the mixed-step chunks
  // 44 -> 42 us).  Four-wave workgroups, two per compute unit: each group of
  // reads waited for at once in asm, the other workgroup's waves filling the
  // wait (plain loads there: the large prefill 553 -> 560 us, the 8-sequence
  // verify 26.7 -> 28.4 us).
  constexpr bool ASMR = KH == 1;
  __shared__ __attribute__((aligned(1024))) char smem[KH * NS * S::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave_all / kWaves;  // key half of this wave
  const int wave = wave_all - kh * kWaves;  // its place among the four waves of the half
  const int htid = tid - kh * kThreads;  // thread index within the half
  char* const hsm = smem + kh * NS * S::kStageBytes;  // the half's LDS ring
  const int smem_base = (int)(uintptr_t)(const __attribute__((address_space(3))) void*)hsm;
  const int half = lane >> 5;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int id = blockIdx.x;
  // this lane's query row (column of S^T and O^T)
  const int mrow = wave * 32 + (lane & 31);
  __bf16* __restrict__ out = reinterpret_cast<__bf16*>(a.out);

  int c, g, kt0, kend, ntiles, nblk, mask_from, qpos, head;
  bool row_ok;
  bool partial = PREFIX;  // write (m, l, o) partials instead of the output
  const __bf16* qrow;
  int64_t part_row = 0;  // PREFIX: (piece, sequence, head) row of the partials
  int64_t out_row = 0;   // prefill: (chunk, row) of q and out
  if constexpr (PREFIX) {
    const int sp = id % a.num_splits;
    const int t = id / a.num_splits;
    g = t % a.num_kv_heads;
    const int mt = t / a.num_kv_heads;
    const int k0 = sp * a.split_tokens;
    kend = min(a.prefix_len, k0 + a.split_tokens);
    kt0 = k0 / kKT;
    ntiles = (kend + kKT - 1) / kKT;
    nblk = (kend + kBlock - 1) / kBlock;
    mask_from = kend;  // keys past the piece (its last tile only) are masked
    qpos = kend - 1;
    const int rr = mt * kMRows + mrow;
    const int seq = rr / G, hl = rr - seq * G;
    row_ok = seq < a.num_chunks;
    head = g * G + hl;
    c = 0;  // the prefix is row 0 of the table
    qrow = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)(row_ok ? seq : 0) * a.num_q_heads + head) * D;
    part_row = ((int64_t)sp * a.num_chunks + seq) * a.num_q_heads + head;
  } else {
    const int QT = tile_rows(a.chunk_len_max, G);
    const int n_mt = (a.chunk_len_max + QT - 1) / QT;
    const int npair = a.num_chunks * a.num_kv_heads;
    int t = id, sp = 0;
    if constexpr (MODE == kSplit) {  // the pieces of a row tile are consecutive workgroups
      sp = t % a.num_splits;
      t /= a.num_splits;
    }
    int pair = t % npair;
    int mt = n_mt - 1 - t / npair;  // the longest row tiles start first
    if (MODE == kChunk && npair % 8 == 0) {
      // Workgroups go to the eight XCDs round-robin by id.  Give each XCD its
      // pairs (pair mod 8) one after the other, all row tiles of a pair at
      // consecutive slots (longest first): they read the same key tiles at
      // about the same time, from that XCD's L2.
      const int x = t % 8, j = t / 8;
      pair = x + 8 * (j / n_mt);
      mt = n_mt - 1 - j % n_mt;
    }
    c = pair / a.num_kv_heads;
    g = pair - c * a.num_kv_heads;

    const int P0 = a.chunk_start[c];
    const int L = a.context_lens[c];
    const int n = L - P0;
    const bool bad_chunk = P0 < 0 || n < 0 || L > a.max_blocks_per_seq * kBlock || n > a.chunk_len_max;
    const int row0 = mt * QT;
    if (bad_chunk) {
      if (sp != 0) return;  // piece 0 writes the NaN rows
      const int rows = min(QT, a.chunk_len_max - row0);
      for (int idx = tid; idx < rows * G * D; idx += kThreads * KH) {
        const int r = idx / (G * D), rem = idx - r * G * D;
        out[((int64_t)(c * a.chunk_len_max + row0 + r) * a.num_q_heads + g * G) * D + rem] =
            (__bf16)__builtin_nanf("");
      }
      return;
    }
    const int rows_here = min(QT, n - row0);
    if (rows_here <= 0) return;
    kend = P0 + row0 + rows_here;  // keys [0, kend) are visible to some row
    kt0 = 0;
    mask_from = P0 + row0 + 1;  // the first key some row may not see
    const int hl = mrow / QT;
    const int qi = row0 + (mrow - hl * QT);
    qpos = P0 + qi;
    if constexpr (MODE == kSplit) {
      const int k0 = sp * a.split_tokens;  // a multiple of the key tile
      if (k0 >= kend) return;             // no keys left for this piece
      partial = kend > a.split_tokens;    // more than one piece: partials
      kt0 = k0 / kKT;
      kend = min(kend, k0 + a.split_tokens);
      // keys of later pieces are masked like keys past the row's position
      mask_from = min(mask_from, kend);
      qpos = min(qpos, kend - 1);
    }
    ntiles = (kend + kKT - 1) / kKT;
    nblk = (kend + kBlock - 1) / kBlock;  // table entries that are read
    row_ok = hl < G && qi < n;
    head = g * G + hl;
    out_row = (int64_t)c * a.chunk_len_max + qi;
    part_row = (((int64_t)sp * a.num_chunks + c) * a.chunk_len_max + qi) * a.num_q_heads + head;
    qrow = reinterpret_cast<const __bf16*>(a.q) + (out_row * a.num_q_heads + head) * D;
  }

  // The softmax works on raw scores and folds the scale into the exponent's
  // FMA, which needs a positive scale: a negative one flips the sign of q
  // (exact in bf16) and of the scale.
  const float sl2 = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  // Every lane loads its query chunks together, rows without a query from a
  // row that exists (the chunk's first row of the group's first head), and
  // zeroes them after: loads under the row test would each be waited for
  // before the next is issued.
  const __bf16* qsrc = row_ok ? qrow
                              : reinterpret_cast<const __bf16*>(a.q) +
                                    (PREFIX ? (int64_t)g * G * D
                                            : ((int64_t)c * a.chunk_len_max * a.num_q_heads + g * G) * D);
  Chunk qch[S::kKSteps];
#pragma unroll
  for (int kk = 0; kk < S::kKSteps; ++kk) qch[kk] = load_chunk(qsrc + kk * 16 + 8 * half);
  const uint32_t qkeep = row_ok ? 0xffffffffu : 0u;
  bf16x8_t qop[S::kKSteps];
#pragma unroll
  for (int kk = 0; kk < S::kKSteps; ++kk)
    qop[kk] = as_bf16x8((qch[kk].w[0] ^ qsign) & qkeep, (qch[kk].w[1] ^ qsign) & qkeep,
                        (qch[kk].w[2] ^ qsign) & qkeep, (qch[kk].w[3] ^ qsign) & qkeep);

  // ---- load side: this wave's block (key rows 16 wave .. 16 wave + 15) of each tile
  const int32_t* __restrict__ table = tables + (int64_t)c * a.max_blocks_per_seq;
  const char* __restrict__ kc = reinterpret_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = reinterpret_cast<const char*>(a.v_cache);
  const int64_t tile_bytes = (int64_t)kBlock * RB;  // one (block, kv head) tile of the cache
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  int local_bad = 0;
  // byte offset in a cache tile of the global chunk that lands at this lane's
  // LDS position in load i (row i * rows-per-load + lane / RC, swizzled chunk)
  int goff[S::kLoadsPerWave], goffv[S::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < S::kLoadsPerWave; ++i) {
    // row within the cache block; the wave's rows sit at the same place modulo
    // 16 in the LDS tile, where the swizzle is taken
    const int r = (wave % (16 / kRowsPerWave)) * kRowsPerWave + i * S::kRowsPerLoad + lane / RC;
    goff[i] = r * RB + (((lane % RC) ^ (r % RC)) * 16);
    goffv[i] = r * RB + (((lane % RC) ^ S::vswz(r)) * 16);
  }
  // Block of this wave in tile kt (uniform).  Blocks past the visible keys
  // read block 0 (their rows are never used: K rows past the keys are masked,
  // and the V rows of the last tile past the keys are zeroed in LDS).
  auto table_entry = [&](int kt) -> int {
    const int jb = kt * (kKT / kBlock) + wave * kRowsPerWave / kBlock;
    int p = jb < nblk ? table[jb] : 0;
    if (p < 0 || p >= a.num_blocks) {
      local_bad = 1;
      p = 0;
    }
    return p;
  };
  // When a chunk's rows fit one row tile (the speculative-verify rows), every
  // K/V tile is read by this workgroup alone: the loads carry the non-temporal
  // hint (verify of 64 x 5 rows 112.9 -> 100.0 us, 157 -> 103 us with cold
  // caches).  Row tiles that share their keys through L2 (prefill chunks, the
  // prefix) keep the default policy: with the hint the large prefill took
  // 570 us against 542.
  const bool stream_kv = !PREFIX && a.chunk_len_max * G <= kMRows;
  auto issue = [&](int stage, int p) {  // direct-to-LDS loads of this wave's rows of a tile (block p)
    char* kdst = hsm + stage * S::kStageBytes + wave * kRowsPerWave * RB;
    const int64_t boff = (int64_t)p * blk_stride + (int64_t)g * tile_bytes;
    const char* kb = kc + boff;
    const char* vb = vc + boff;
    const int kl = __builtin_amdgcn_readfirstlane((int)(uintptr_t)(__attribute__((address_space(3))) char*)kdst);
#pragma unroll
    for (int i = 0; i < S::kLoadsPerWave; ++i) {
      if (stream_kv) {
        load_lds_x4<true>(kb, goff[i], kl + i * 1024);
        load_lds_x4<true>(vb, goffv[i], kl + TB + i * 1024);
      } else {
        load_lds_x4<false>(kb, goff[i], kl + i * 1024);
        load_lds_x4<false>(vb, goffv[i], kl + TB + i * 1024);
      }
    }
  };

  // ---- compute side: per-lane LDS byte offsets of the operands, without the
  // stage and without the key-block part that is the same for every lane
  // (that part goes into the reads' immediate offset).
  // K operand of step kk for key block nb: key row nb*32 + lane%32, dims 16 kk + 8 half.
  const int kr = lane & 31;
  int koff[S::kKSteps];
#pragma unroll
  for (int kk = 0; kk < S::kKSteps; ++kk) koff[kk] = kr * RB + (((2 * kk + half) ^ (kr % RC)) * 16);
  // V^T operand (transpose reads) of step (nb, s), read r, dim block nd: source lane addresses
  // key nb*32 + 16 s + 8 r + vkey, dims 32 nd + vdim + 0..3; the chunk swizzle of that row only
  // depends on 8 r + vkey (nb*32 + 16 s is a multiple of the chunks per row).
  const int grp = lane >> 4;
  const int vkey = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int vdim = 16 * (grp & 1) + 4 * (lane & 3);
  constexpr int NR = 2 * S::kND;  // transpose reads per PV step
  int voff[NR];
#pragma unroll
  for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int key = 8 * r + vkey, dim = 32 * nd + vdim;
      voff[2 * nd + r] = key * RB + (((dim >> 3) ^ S::vswz(key)) * 16) + (dim & 7) * 2;
    }

  float m_run = kMaxInit, l_run = 0.0f;
  f32x16_t oacc[S::kND];
#pragma unroll
  for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[nd][v] = 0.0f;

  // a wave whose 32 rows carry no query only loads and synchronises
  const bool wave_active = __builtin_amdgcn_ballot_w64(row_ok) != 0;

  // S^T = K Q^T for the tile whose K rows sit at LDS byte address kbase.
  auto scores = [&](int kbase, f32x16_t (&st)[kNB]) {
    int kb[S::kKSteps];
#pragma unroll
    for (int kk = 0; kk < S::kKSteps; ++kk) kb[kk] = kbase + koff[kk];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[nb][v] = 0.0f;
      u32x4_t kv[S::kKSteps];
      if (nb == 0) lds_read_b128<ASMR, 0>(kb, kv);
      else lds_read_b128<ASMR, 32 * RB>(kb, kv);
#pragma unroll
      for (int kk = 0; kk < S::kKSteps; ++kk)
        st[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv[kk]), qop[kk], st[nb], 0, 0,
                                                         0);
    }
    if constexpr (!ASMR) {  // every K read of the tile first, then the products as the reads arrive
      __builtin_amdgcn_sched_group_barrier(0x100, kNB * S::kKSteps, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kNB * S::kKSteps, 0);
    }
  };

  // The online softmax of tile kt's scores and O^T += V^T P^T with its V rows
  // at LDS byte address vbase.  MASK: the tile holds keys past some row's
  // position (diagonal tiles).
  auto finish = [&](auto mask_tag, int kt, f32x16_t (&st)[kNB], int vbase) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // causal mask (select, diagonal tiles only) and the row max of the raw
    // scores over this lane and lane ^ 32; the scale (positive) is applied to
    // the max once and to each score inside the exponent's FMA
    // (masked keys are left out of the max and get weight 0 by a select on the
    // weight, so neither their K rows -- possibly NaN -- nor a zero scale can
    // leak into the sums)
    auto masked = [&](int nb, int v) {
      return kt * kKT + nb * 32 + 8 * (v >> 2) + 4 * half + (v & 3) > qpos;
    };
    float mx = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, (MASK && masked(nb, v)) ? -__builtin_inff() : st[nb][v]);
    mx = fmaxf(mx, shfl_xor_f32(mx, 32)) * sl2;
    // Lazy rescale: the running max moves (and O, l are rescaled) only when a
    // score exceeds it by more than 2^8, which bounds every P by 256; the
    // final normalisation makes the stale max exact.
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > m_run + kPrefillSlack) != 0, 0)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[nd][v] *= alpha;
    }
    const float mn = m_run;

    // P in bf16 for the matrix cores; the running sum adds those same rounded
    // weights, two at a time (v_dot2 with (1, 1)), so O and l share their weights
    uint32_t pk[kNB][8];
    float ps = 0.0f;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float p0 = fast_exp2(fmaf(st[nb][2 * u], sl2, -mn));
        float p1 = fast_exp2(fmaf(st[nb][2 * u + 1], sl2, -mn));
        if constexpr (MASK) {
          p0 = masked(nb, 2 * u) ? 0.0f : p0;
          p1 = masked(nb, 2 * u + 1) ? 0.0f : p1;
        }
        pk[nb][u] = pack_bf16x2(p0, p1);
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[nb][u]), ones, ps, false);
      }
    l_run += ps;

#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8_t bop = as_bf16x8(pk[nb][4 * s], pk[nb][4 * s + 1], pk[nb][4 * s + 2], pk[nb][4 * s + 3]);
        int vb[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) vb[i] = vbase + voff[i];
        u32x2_t vv[NR];
        if (nb == 0 && s == 0) lds_read_tr16<ASMR, 0>(vb, vv);
        else if (nb == 0) lds_read_tr16<ASMR, 16 * RB>(vb, vv);
        else if (s == 0) lds_read_tr16<ASMR, 32 * RB>(vb, vv);
        else lds_read_tr16<ASMR, 48 * RB>(vb, vv);
#pragma unroll
        for (int nd = 0; nd < S::kND; ++nd)
          oacc[nd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(vv[2 * nd].x, vv[2 * nd].y, vv[2 * nd + 1].x, vv[2 * nd + 1].y), bop, oacc[nd], 0, 0, 0);
      }
  };

  // tiles with no key past any row's position come before the diagonal ones
  const int nfull = min(ntiles, mask_from / kKT);
  // this half's tiles, kt0 + kh, kt0 + kh + KH, ...; both halves take the same
  // number of steps (a step past the last tile only loads and synchronises)
  const int nsteps = (ntiles - kt0 + KH - 1) / KH;
  auto kt_of = [&](int i) { return kt0 + KH * i + kh; };
  // The last tile also holds keys past every row's (unless kend is a multiple
  // of the tile): its V rows from kend on are zeroed in LDS before they are
  // read (they may hold NaN), at a step every wave of the workgroup takes.
  const int kt_tail = kend % kKT ? ntiles - 1 : -1;
  const int i_tail = kt_tail >= 0 ? (kt_tail - kt0) / KH : -1;

  // prologue: steps 0 .. NS-2 in flight (past the last tile: block 0, whose rows
  // are never used, so every step finds the same number of loads outstanding)
  int pnext = table_entry(kt_of(0));
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    const int p = pnext;
    pnext = table_entry(kt_of(t + 1));
    issue(t, p);
  }
  // Step i: wait for its tile's loads, start the loads of step i + NS - 1,
  // then S^T = K Q^T, the online softmax and O^T += V^T P^T.  Two loops, the
  // steps whose tile has no masked key, then the others: every step has the
  // same barriers, so the halves stay in step whichever loop they are in.
  auto step = [&](auto mask_tag, int i) {
    // this wave's loads of step i are done once at most NS-2 steps' loads remain;
    // the barrier then makes every wave's part visible and frees the stage of i-1
    if constexpr (ASMR) {
      wait_vmcnt_le<(NS - 2) * S::kDW>();
      __builtin_amdgcn_s_barrier();
      const int p = pnext;
      pnext = table_entry(kt_of(i + NS));
      issue((i + NS - 1) % NS, p);
    } else {
      // the table entry of a later step is loaded and waited for before the
      // barrier: a scalar load in flight would make the compiler wait for
      // every LDS read at once (the two share a counter)
      const int p = pnext;
      pnext = table_entry(kt_of(i + NS));
      asm volatile("" ::"s"(pnext));
      ring_barrier<(NS - 2) * S::kDW>();
      issue((i + NS - 1) % NS, p);
    }
    const int kt = kt_of(i);
    if (i == i_tail) {
      if (kt == kt_tail) {
        char* vt = hsm + (i % NS) * S::kStageBytes + TB;
        const int r0 = kend - kt * kKT;
        for (int idx = htid; idx < (kKT - r0) * RC; idx += kThreads)
          *reinterpret_cast<uint4*>(vt + (r0 + idx / RC) * RB + (idx % RC) * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    if (kt >= ntiles || !wave_active) return;
    const int sbase = smem_base + (i % NS) * S::kStageBytes;
    f32x16_t st[kNB];
    scores(sbase, st);
    // Two waves share each SIMD (two four-wave workgroups, or the two key
    // halves): the wave past its score products (softmax, value products)
    // takes issue priority over one starting its scores, so the two drift
    // into alternating phases (the large prefill 551 / 544 -> 533 / 536 us
    // cold on one box; priority for the scores instead: 542 us, for the value
    // products alone: 565 us; the key halves' mixed-step chunks 42.4 -> 40.6 us
    // with their reads waited for one at a time, 43 -> 44 us with the reads
    // of a group waited for at once).
    __builtin_amdgcn_s_setprio(1);
    finish(mask_tag, kt, st, sbase + TB);
    __builtin_amdgcn_s_setprio(0);
  };
  const int i_full = min(nsteps, max(0, (nfull - kt0 - kh + KH - 1) / KH));  // this half's unmasked steps
  int i = 0;
  for (; i < i_full; ++i) step(std::false_type{}, i);
  for (; i < nsteps; ++i) step(std::true_type{}, i);

  // no direct-to-LDS load may still be writing when the workgroup's LDS is released
  wait_vmcnt_le<0>();
  const int any_bad = __syncthreads_or(local_bad);
  if constexpr (KH == 2) {
    // the second half hands its state of each row (m, l and O^T, lane by lane)
    // to the first through the LDS the rings no longer use
    constexpr int kX = 2 + S::kND * 16;  // floats per lane
    static_assert(kWaves * kX * 64 * 4 <= KH * NS * S::kStageBytes, "the states fit the rings' LDS");
    float* x = reinterpret_cast<float*>(smem) + wave * kX * 64 + lane;
    if (kh == 1) {
      x[0] = m_run;
      x[64] = l_run;
#pragma unroll
      for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[(2 + nd * 16 + v) * 64] = oacc[nd][v];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = x[0];
    const float mn = fmaxf(m_run, m1);
    const float f0 = fast_exp2(m_run - mn), f1 = fast_exp2(m1 - mn);
    l_run = l_run * f0 + x[64] * f1;
#pragma unroll
    for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[nd][v] = oacc[nd][v] * f0 + x[(2 + nd * 16 + v) * 64] * f1;
    m_run = mn;
  }
  const float l_tot = l_run + shfl_xor_f32(l_run, 32);
  if (!row_ok) return;
  if (partial) {
    float* po = a.part_o + part_row * D;
#pragma unroll
    for (int nd = 0; nd < S::kND; ++nd)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dim = nd * 32 + 8 * q4 + 4 * half;
        *reinterpret_cast<float4*>(po + dim) =
            make_float4(oacc[nd][4 * q4], oacc[nd][4 * q4 + 1], oacc[nd][4 * q4 + 2], oacc[nd][4 * q4 + 3]);
      }
    if (half == 0) {
      a.part_ml[part_row * 2] = any_bad ? __builtin_nanf("") : m_run;
      a.part_ml[part_row * 2 + 1] = l_tot;
    }
  } else if constexpr (!PREFIX) {
    const float inv = any_bad ? __builtin_nanf("") : 1.0f / l_tot;
    __bf16* orow = out + (out_row * a.num_q_heads + head) * D;
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
}

// Merge of the key pieces of every split row tile: one wave per (chunk, row,
// head) row whose tile was cut into more than one piece; lane k owns dims
// k, k + 64, ...  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with M the
// largest m_p; a NaN m_p (contract broken) makes the row NaN.
template <int D>
__global__ __launch_bounds__(64) void prefill_split_merge_kernel(const PrefillArgs a) {
  constexpr int PER = D / kWave;
  const int lane = __lane_id();
  const int64_t item = blockIdx.x;  // (chunk, row, head)
  const int head = (int)(item % a.num_q_heads);
  const int64_t cr = item / a.num_q_heads;
  const int c = (int)(cr / a.chunk_len_max);
  const int qi = (int)(cr - (int64_t)c * a.chunk_len_max);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int QT = tile_rows(a.chunk_len_max, G);
  const int P0 = a.chunk_start[c];
  const int L = a.context_lens[c];
  const int n = L - P0;
  if (P0 < 0 || n < 0 || L > a.max_blocks_per_seq * kBlock || n > a.chunk_len_max || qi >= n) return;
  const int row0 = qi / QT * QT;
  const int kend = P0 + row0 + min(QT, n - row0);
  if (kend <= a.split_tokens) return;  // one piece: written by the main kernel
  const int np = (kend + a.split_tokens - 1) / a.split_tokens;
  const int64_t stride = (int64_t)a.num_chunks * a.chunk_len_max * a.num_q_heads;  // rows per piece
  float M, lam, o[PER];
  bool nan;
  merge_partials<D>(a.part_o, a.part_ml, item, stride, np, o, M, lam, nan);
  const float inv = nan ? __builtin_nanf("") : 1.0f / lam;
  __bf16* orow = reinterpret_cast<__bf16*>(a.out) + item * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[lane + e * kWave] = (__bf16)(o[e] * inv);
}

// Grids of at most this many workgroups (one per compute unit) take two key
// halves per workgroup.
#ifndef PKV_PREFILL_KEY_HALVES_GRID
#define PKV_PREFILL_KEY_HALVES_GRID 256
#endif

template <int MODE, int KH>
static hipError_t launch_chunk_halves(const PrefillArgs& a, int64_t grid, hipStream_t stream) {
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL((prefill_mfma_kernel<64, MODE, KH>), dim3((unsigned)grid), dim3(kThreads * KH), 0, stream,
                         a, a.block_tables);
      break;
    case 128:
      hipLaunchKernelGGL((prefill_mfma_kernel<128, MODE, KH>), dim3((unsigned)grid), dim3(kThreads * KH), 0, stream,
                         a, a.block_tables);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_chunk_modes(const PrefillArgs& a, int64_t grid, hipStream_t stream) {
  if (grid <= PKV_PREFILL_KEY_HALVES_GRID) return launch_chunk_halves<MODE, 2>(a, grid, stream);
  return launch_chunk_halves<MODE, 1>(a, grid, stream);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G < 1 || G > kMRows) return hipErrorInvalidValue;
  const bool split = a.num_splits > 1;
  if (split && (a.split_tokens <= 0 || a.split_tokens % kKT != 0 || !a.part_o || !a.part_ml))
    return hipErrorInvalidValue;
  const int QT = tile_rows(a.chunk_len_max, G);
  const int64_t n_mt = (a.chunk_len_max + QT - 1) / QT;
  const int64_t grid = n_mt * a.num_chunks * a.num_kv_heads * (split ? a.num_splits : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (!split) return launch_chunk_modes<kChunk>(a, grid, stream);
  hipError_t e = launch_chunk_modes<kSplit>(a, grid, stream);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.num_chunks * a.chunk_len_max * a.num_q_heads;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(prefill_split_merge_kernel<64>, dim3((unsigned)rows), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_split_merge_kernel<128>, dim3((unsigned)rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefix_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G < 1 || a.prefix_len <= 0 || a.split_tokens <= 0 || a.split_tokens % kKT != 0) return hipErrorInvalidValue;
  const int64_t n_mt = ((int64_t)a.num_chunks * G + kMRows - 1) / kMRows;
  const int64_t grid = n_mt * a.num_kv_heads * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  return launch_chunk_modes<kPrefix>(a, grid, stream);
}

}  // namespace pkv
