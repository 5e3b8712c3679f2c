// Host-side launchers of the libpkv kernels (internal; the public ABI is include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

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
  // Balanced split planned inside the kernel (null: not): wave 0 of every
  // workgroup derives its slot's chunk from context_lens (at most
  // kPlanMaxSeqs sequences) and the first chunk's workgroup writes
  // plan_first[b] (and plan_first[B]) for the merge.
  int32_t* plan_first;
  // Partial rows of part_o stored as bf16 (RNE) instead of float32.
  int part_bf16;
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
  int part_bf16;              // partial rows stored as bf16 (several new tokens, matrix cores)
  // Balanced split (null: fixed partitions): the plan's slot_info[slot] =
  // {sequence, first block, end block, chunks of the sequence}; the grid runs
  // max_partitions slots; partial rows are [slot, Hq] and an empty chunk
  // writes lse = -inf.  One new token per sequence only.
  const int4* slot_info;
  // Balanced split planned inside the decode kernel (null: not): every
  // workgroup derives the schedule from context_lens itself (at most
  // kPlanMaxSeqs sequences) and the workgroup of a sequence's first chunk
  // writes plan_first[b] (and plan_first[B] for the last sequence) for the
  // merge.  The grid runs max_partitions slots.
  int32_t* plan_first;
  // Chunk slots of a balanced split instead of fixed partitions.
  __host__ __device__ bool balanced() const { return slot_info != nullptr || plan_first != nullptr; }
};

// Sequences a decode workgroup plans for itself: four per lane, in registers.
constexpr int kPlanSeqsPerLane = 4;
constexpr int kPlanMaxSeqs = kPlanSeqsPerLane * 64;

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

// The balanced schedule of chunk slot `slot`, computed by the whole wave from
// context_lens (uniform result).  Sequence l + 64 g is held by lane l.  Its
// u_b = ceil(min(max(ctx, 0), capacity) / 16) blocks go to n_b = max(1,
// ceil(u_b / t)) chunks, t the smallest size with sum n_b <= R =
// max_partitions; the bisection for t is bracketed by [total / R,
// total / (R - B)] (the count lies in [total / t, total / t + B]), so no
// count it evaluates exceeds R + B.  The slot's sequence is the one whose
// run of slots [first_b, first_b + n_b) holds it (a prefix sum over the
// lanes, then a ballot), and chunk k of it covers blocks
// [k u / n, (k+1) u / n).  False: the slot is past the last chunk.
// Every decode workgroup runs this at once, so it is written for few VALU
// instructions: groups of 64 sequences past the batch are skipped, and
// quotients by the uniform chunk size come from a float reciprocal, exact
// after one correction each way (u < 2^22 blocks; longer tables take the
// integer division).
__device__ __forceinline__ int ceil_div_uniform(int u, int t, float rt, bool fast) {
  if (!fast) return (u + t - 1) / t;
  int q = int(float(u) * rt);             // within one of floor(u / t)
  q -= q * t > u ? 1 : 0;
  q += (q + 1) * t <= u ? 1 : 0;
  return q + (q * t < u ? 1 : 0);
}

// The chunk of slot `slot`: sequence b, units [u_begin, u_end) of it and its
// chunk count n (unit_tokens tokens per unit; contexts clamped to
// [0, cap_tokens]; R = max(slots, B)).
struct PlanChunk {
  int b, u_begin, u_end, n;
};

__device__ inline bool plan_slot(const int32_t* context_lens, int B, int cap, int unit_tokens,
                                 int slots, int slot, PlanChunk& pc, int& total_chunks) {
  constexpr int G = kPlanSeqsPerLane;
  const int l = threadIdx.x & 63;
  const int groups = (B + 63) >> 6;        // uniform, at most G
  int u[G];
  int mx = 0, lo16 = 0, hi16 = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    u[g] = 0;
    if (g < groups) {
      const int b = l + 64 * g;
      int ctx = b < B ? context_lens[b] : 0;
      ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
      u[g] = (ctx + unit_tokens - 1) / unit_tokens;
      mx = max(mx, u[g]);
      lo16 += u[g] & 0xFFFF;              // total = hi16 * 65536 + lo16, each sum < 2^24
      hi16 += u[g] >> 16;
    }
  }
  mx = wave_max_uniform(mx);
  const int64_t total = int64_t(wave_sum_uniform(hi16)) * 65536 + wave_sum_uniform(lo16);
  const int64_t R = slots > B ? slots : B;
  const int top = mx > 1 ? mx : 1;
  const int64_t lo_l = (total + R - 1) / R;
  const int64_t hi_l = R > B ? (total + (R - B) - 1) / (R - B) : top;
  int lo = int(lo_l < 1 ? 1 : (lo_l > top ? top : lo_l));
  int hi = int(hi_l < lo ? lo : (hi_l > top ? top : hi_l));
  const bool fast = mx < (1 << 22);
  // Chunks of one lane's sequences for chunk size t (0 for sequences past B).
  auto lane_chunks = [&](int g, int t, float rt) {
    const int b = l + 64 * g;
    return b >= B ? 0 : (u[g] <= t ? 1 : ceil_div_uniform(u[g], t, rt, fast));
  };
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    const float rt = 1.0f / float(mid);
    int c = 0;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g < groups) c += lane_chunks(g, mid, rt);
    if (wave_sum_uniform(c) <= R) hi = mid; else lo = mid + 1;
  }
  const float rt = 1.0f / float(lo);
  int carry = 0;
  bool found = false;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < groups) {
      const int n = lane_chunks(g, lo, rt);
      const int incl = wave_incl_scan(n);
      const int first = carry + incl - n;
      const uint64_t owner = __ballot(n > 0 && first <= slot && slot < first + n);
      if (!found && owner != 0) {
        const int lane = __builtin_ctzll(owner);
        const int nb = __builtin_amdgcn_readlane(n, lane);
        const int ub = __builtin_amdgcn_readlane(u[g], lane);
        const int k = slot - __builtin_amdgcn_readlane(first, lane);
        // k u / n = k q + k r / n with u = q n + r; k r < n^2 fits 32 bits
        // (the host keeps R below 46341 slots for this path).
        const int q = ub / nb, r = ub - q * nb;
        pc.b = lane + 64 * g;
        pc.u_begin = k * q + (k * r) / nb;
        pc.u_end = (k + 1) * q + ((k + 1) * r) / nb;
        pc.n = nb;
        found = true;
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  total_chunks = carry;
  return found;
}

__device__ inline bool decode_item(const DecodeArgs& a, DecodeItem& it) {
  const int per_head = a.balanced() ? a.max_partitions : a.num_seqs * a.max_partitions;
  int idx;
  if (!decode_unit(blockIdx.x, a.head_chunks, per_head * a.num_kv_heads, it.chunk, idx)) return false;
  it.h = idx % a.num_kv_heads;
  idx /= a.num_kv_heads;
  if (a.plan_first) {
    int total_chunks;
    PlanChunk pc;
    if (!plan_slot(a.context_lens, a.num_seqs, a.max_blocks_per_seq * kBlockSize, kBlockSize,
                   a.max_partitions, idx, pc, total_chunks))
      return false;
    it.b = pc.b;
    it.part = idx;
    it.blk_begin = pc.u_begin;
    it.blk_end = pc.u_end;
    it.n_parts = pc.n;
    // The first chunk's workgroup publishes the sequence's first slot.
    if (it.chunk == 0 && it.h == 0 && it.blk_begin == 0 && (threadIdx.x & 63) == 0) {
      a.plan_first[it.b] = idx;
      if (it.b == a.num_seqs - 1) a.plan_first[a.num_seqs] = total_chunks;
    }
    return true;
  }
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

// Row of the partial arrays for query row qrow = (row0 + j) * Hq + head (row0
// the sequence's first query row, j its new token): [rows, max_partitions]
// for a fixed split; [slot, Hq] for a balanced one, or [slot, max_q, Hq] with
// several new tokens per sequence.
__device__ inline size_t partial_row(const DecodeArgs& a, const DecodeItem& it, size_t qrow,
                                     int row0) {
  if (!a.balanced()) return qrow * a.max_partitions + it.part;
  if (!a.q_start) return qrow + (size_t(it.part) - size_t(it.b)) * a.num_q_heads;
  const size_t j = qrow / a.num_q_heads - size_t(row0);
  return (size_t(it.part) * a.max_q + j) * a.num_q_heads + qrow % a.num_q_heads;
}
// False for a new token past max_q (a violated contract): a balanced split
// with several tokens has no partial row for it.
__device__ inline bool partial_row_ok(const DecodeArgs& a, size_t qrow, int row0) {
  return !(a.balanced() && a.q_start) || qrow / a.num_q_heads - size_t(row0) < size_t(a.max_q);
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
  // entry sets its partition count.  Null: row r is sequence r.  The grid then
  // runs (sequence, new token j < rows_per_seq, head): row q_start[s] + j,
  // none for j >= q_start[s+1] - q_start[s].
  const int32_t* q_start;
  int num_batch;                   // sequences, when q_start is set
  int rows_per_seq;                // most new tokens of a sequence, when q_start is set
  // Balanced split: partitions of sequence b are the chunk slots
  // chunk_first[b] .. chunk_first[b+1]-1; rows [slot, slot_rows, num_q_heads]
  // (slot_rows: the most new tokens of a sequence; 0 or 1 for one each).
  const int32_t* chunk_first;
  int slot_rows;
  // part_o holds bf16 rows (head_dim 512 only) instead of float32.
  int part_bf16;
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
