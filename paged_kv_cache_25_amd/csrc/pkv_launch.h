// Host-side launchers of the libpkv kernels (internal; the public ABI is include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class DType : int { F32 = 0, BF16 = 1, FP8 = 2 };

constexpr int kBlockSizeBuilt = 16;                 // tokens per KV block
constexpr float kLog2eHost = 1.4426950408889634f;

inline int dtype_bytes(DType t) { return t == DType::F32 ? 4 : (t == DType::BF16 ? 2 : 1); }

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_kv_heads, row_bytes, num_blocks, max_blocks_per_seq;
  // Several new tokens per sequence: rows q_start[b] .. q_start[b+1]-1 of
  // k_new/v_new (num_rows rows in all) belong to sequence b.  Null: one row each.
  const int32_t* q_start;
  int num_rows;
};

// Quantise-on-append into an e4m3 cache (pools are codes, scales float32
// [num_blocks, num_kv_heads]); k_new/v_new are bf16 (new_bf16) or float32.
struct QuantAppendArgs {
  void* k_pool;
  void* v_pool;
  float* k_scales;
  float* v_scales;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* q_start;          // null: one new row per sequence
  int num_seqs, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq;
  int new_bf16;
  int mode;                        // 0: fixed scales, 1: running amax
};

// Copy-on-write block copies: pairs int32 [num_pairs][2] = (src, dst).
struct CopyBlocksArgs {
  void* k_pool;
  void* v_pool;
  float* k_scales;                 // null unless the cache is e4m3
  float* v_scales;
  const int32_t* pairs;
  int num_pairs, num_blocks, num_kv_heads;
  size_t block_bytes;              // one physical block of one pool, all KV heads
};

// Absorbed MLA decode over a paged latent cache: pool [num_blocks, 16, 576]
// bf16 rows (512 latent + 64 rotary key), q [B, H, 576], out [B, H, 512].
struct MlaArgs {
  void* out;                       // final latent output (bf16) when write_final
  float* part_o;                   // [B, H, maxP, 512]
  float* part_lse;                 // [B, H, maxP]
  const void* q;
  const void* pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_heads, head_chunks, num_blocks, max_blocks_per_seq;
  int blocks_per_partition, max_partitions;
  float scale_log2;
  int write_final, final_single, mark_empty;
  // Balanced split (null otherwise): sequence b owns the chunk slots
  // chunk_first[b] .. chunk_first[b+1]-1 and splits its pairs of blocks evenly
  // over them; workgroup c takes slot c; partial rows are [slot, H].
  const int32_t* chunk_first;
};

// The balanced split of a batch's work into at most max(budget, num_seqs)
// chunks: each sequence's units (unit_tokens tokens each, the context
// clamped to [0, cap_tokens]) go to n_b = max(1, ceil(units_b / t)) chunks,
// t the smallest size that keeps the total within the budget; chunk_first
// [num_seqs + 1] receives the exclusive prefix sums of n_b.
struct SplitArgs {
  const int32_t* context_lens;
  int num_seqs, cap_tokens, unit_tokens, budget;
  int32_t* chunk_first;
  // Optional (null: not written): per chunk slot s < num_slots, {sequence,
  // first unit, end unit, chunks of that sequence}; slots past the last chunk
  // get sequence -1.  num_slots >= max(budget, num_seqs).
  int4* slot_info;
  int num_slots;
};

struct DecodeArgs {
  void* out;               // final output (q dtype) when write_final
  float* part_o;           // [B, Hq, maxP, D] when !write_final
  float* part_lse;         // [B, Hq, maxP]
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scales;   // [NB, Hkv] (e4m3 only)
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Fused append (null otherwise): the new token's K/V rows [B, Hkv, D] are
  // read from here instead of the pool, and written into the pool slot by the
  // workgroup that reads the sequence's last block.
  const void* k_new;
  const void* v_new;
  void* k_pool_w;
  void* v_pool_w;
  // Several new tokens per sequence (null: one each, row b of q and out).
  // Rows q_start[b] .. q_start[b+1]-1 of q/out are sequence b's newest tokens.
  const int32_t* q_start;
  int max_q;                  // most new tokens of any sequence (1 without q_start)
  int tiles_per_wave;         // matrix-core kernel with q_start: 16-column tiles per wave (1 or 2)
  int num_seqs, num_q_heads, num_kv_heads, group, head_chunks;
  int num_blocks, max_blocks_per_seq;
  int blocks_per_partition;   // partition size / 16
  int max_partitions;         // grid extent over partitions
  float scale_log2;           // softmax_scale * log2(e)
  int write_final;            // every sequence has one partition: write `out`
  int final_single;           // a sequence with one partition writes `out` (the merge skips it)
  int mark_empty;             // partitions past a sequence's end write lse = -inf
  // Balanced split (null: fixed partitions): the plan's slot_info[slot] =
  // {sequence, first block, end block, chunks of the sequence}; the grid runs
  // max_partitions slots; partial rows are [slot, Hq] and an empty chunk
  // writes lse = -inf.  One new token per sequence only.
  const int4* slot_info;
};

// The columns of one (sequence, KV head) work item: column n is new token
// j = n / group of the sequence (of t) and query head i = n % group of the KV
// head's group.  Token j sees the cached tokens up to its own position.
struct Columns {
  int group, t, row0, num_q_heads, kv_head;
  __host__ __device__ bool valid(int n) const { return n < t * group; }
  // row of the [tokens, q heads] arrays (q, out, partials)
  __host__ __device__ size_t row(int n) const {
    return size_t(row0 + n / group) * num_q_heads + size_t(kv_head) * group + n % group;
  }
  // cached tokens column n attends to
  __host__ __device__ int visible(int n, int ctx) const { return ctx - t + n / group + 1; }
};

// Grid order of the decode kernels.  The hardware hands workgroup ids to the
// 8 XCDs round-robin (id % 8), and each XCD has its own L2.  A unit is one
// (KV head, sequence, partition), KV head fastest and partition slowest, so
// consecutive units carry equal work (every sequence has a partition 0, only
// long ones have high partitions).  The column tiles ("chunks") of one unit
// read the same K/V blocks: they take ids 8 apart, i.e. run back to back on
// one XCD, so the blocks come from HBM once and from that L2 after.
constexpr int kXcds = 8;

inline size_t decode_grid(size_t units, int chunks) {
  return (units + kXcds - 1) / kXcds * kXcds * size_t(chunks);
}

// Workgroup id -> (chunk, unit); false for the padding ids past the last unit.
__device__ inline bool decode_unit(int id, int chunks, int units, int& chunk, int& unit) {
  const int xcd = id % kXcds;
  const int r = id / kXcds;
  chunk = r % chunks;
  unit = (r / chunks) * kXcds + xcd;
  return unit < units;
}

// The work of one decode workgroup: column chunk, KV head, sequence and the
// blocks [blk_begin, blk_end) it walks (not yet clipped to the sequence);
// part is the partition (fixed split) or the chunk slot (balanced split), and
// n_parts the sequence's chunk count (balanced only).  False: no work.
struct DecodeItem {
  int chunk, h, b, part, blk_begin, blk_end, n_parts;
};

__device__ inline bool decode_item(const DecodeArgs& a, DecodeItem& it) {
  const int per_head = a.slot_info ? a.max_partitions : a.num_seqs * a.max_partitions;
  int idx;
  if (!decode_unit(blockIdx.x, a.head_chunks, per_head * a.num_kv_heads, it.chunk, idx)) return false;
  it.h = idx % a.num_kv_heads;
  idx /= a.num_kv_heads;
  if (a.slot_info) {
    const int4 si = a.slot_info[idx];
    if (si.x < 0 || si.x >= a.num_seqs) return false;  // slot past the last chunk
    it.b = si.x;
    it.part = idx;
    it.blk_begin = si.y;
    it.blk_end = si.z;
    it.n_parts = si.w;
  } else {
    it.b = idx % a.num_seqs;
    it.part = idx / a.num_seqs;
    it.blk_begin = it.part * a.blocks_per_partition;
    it.blk_end = it.blk_begin + a.blocks_per_partition;
    it.n_parts = 0;
  }
  return true;
}

// Row of the partial arrays for query row qrow: [rows, max_partitions] for a
// fixed split, [slot, Hq] for a balanced one (qrow = b * Hq + head).
__device__ inline size_t partial_row(const DecodeArgs& a, const DecodeItem& it, size_t qrow) {
  return a.slot_info ? qrow + (size_t(it.part) - size_t(it.b)) * a.num_q_heads
                     : qrow * a.max_partitions + it.part;
}

struct MergeArgs {
  void* out;
  const float* part_o;
  const float* part_lse;
  const int32_t* num_partitions;   // may be null
  const int32_t* context_lens;     // may be null: partitions = ceil(ctx / partition_size)
  int partition_size;
  int num_seqs, num_q_heads, max_partitions;
  int skip_single;                 // 1: sequences with one partition were written by the decode kernel
  // Several new tokens per sequence: row r (num_seqs above counts rows) belongs
  // to the sequence s with q_start[s] <= r < q_start[s+1], whose context_lens
  // entry sets its partition count.  Null: row r is sequence r.
  const int32_t* q_start;
  int num_batch;                   // sequences, when q_start is set
  // Balanced split (MLA): partitions of sequence b are the chunk slots
  // chunk_first[b] .. chunk_first[b+1]-1; rows [slot, num_q_heads].
  const int32_t* chunk_first;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_kv_append_quant(const QuantAppendArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
int mla_heads_per_workgroup(int num_heads);
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream);
hipError_t launch_balanced_split(const SplitArgs& a, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeArgs& a, int head_dim, int tile_heads, DType q_dtype,
                               DType kv_dtype, hipStream_t stream);
// Matrix-core variant for bf16 queries over a bf16 cache; heads in tiles of 16.
hipError_t launch_paged_decode_mfma(const DecodeArgs& a, int head_dim, hipStream_t stream);
int mfma_head_tile();
hipError_t launch_merge(const MergeArgs& a, int head_dim, DType out_dtype, hipStream_t stream);

}  // namespace pkv
