// The C ABI of libpkv (declared in include/pkv.h): argument checks, workspace
// layout and launch configuration.  Every check runs on the host before any
// launch, so an invalid call enqueues nothing.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pkv_launch.h"
#include "stream_read.h"

namespace {

using pkv::DType;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(pkv_dtype_t t) { return t == PKV_F32 || t == PKV_BF16 || t == PKV_FP8_E4M3; }
DType to_internal(pkv_dtype_t t) {
  return t == PKV_F32 ? DType::F32 : (t == PKV_BF16 ? DType::BF16 : DType::FP8);
}
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

// The kernels move data in 16-byte vectors.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Partitions per sequence for a grid: ceil(max_ctx / P), or 1 when P == 0.
int64_t max_partitions(int32_t max_context_len, int32_t partition_size) {
  if (max_context_len <= 0) return 1;
  if (partition_size == 0) return 1;
  return (int64_t(max_context_len) + partition_size - 1) / partition_size;
}

// Query columns (heads of a group, times new tokens) handled by one vector
// workgroup: their count rounded up to a power of two, at most 8 for head_dim
// 64 and 4 for head_dim 128 (the per-lane accumulators must stay in
// registers); more columns are split into tiles.
int tile_heads(int group, int head_dim) {
  const int cap = head_dim == 64 ? 8 : 4;
  int t = 1;
  while (t < group && t < cap) t *= 2;
  return t;
}

struct PartLayout {
  size_t o_bytes, lse_offset, lse_bytes, total;
};

PartLayout part_layout(int64_t B, int64_t Hq, int64_t D, int64_t maxp) {
  PartLayout L;
  L.o_bytes = size_t(B * Hq * maxp * D) * sizeof(float);
  L.lse_offset = align_up(L.o_bytes);
  L.lse_bytes = size_t(B * Hq * maxp) * sizeof(float);
  L.total = L.lse_offset + align_up(L.lse_bytes);
  return L;
}

// Balanced MLA split: chunk slots (one 8-wave workgroup per CU at a time, or
// two smaller ones: their LDS halves fit one CU) and the workspace layout
// o [R, H, D] | lse [R, H] | chunk starts [B + 1], each 256-byte aligned.
int64_t mla_balanced_slots(int32_t num_seqs, int32_t num_heads) {
  const int waves = pkv::mla_heads_per_workgroup(num_heads) / 16;
  const int64_t budget = waves >= 8 ? 256 : 512;
  return budget > num_seqs ? budget : num_seqs;
}

struct BalancedLayout {
  PartLayout part;
  int64_t slots;
  size_t first_offset, total;
};

BalancedLayout balanced_layout(int32_t num_seqs, int32_t num_heads, int32_t d) {
  BalancedLayout L;
  L.slots = mla_balanced_slots(num_seqs, num_heads);
  L.part = part_layout(L.slots, num_heads, d, 1);
  L.first_offset = L.part.total;
  L.total = L.first_offset + align_up((size_t(num_seqs) + 1) * sizeof(int32_t));
  return L;
}

// Balanced split of the one-token decode: the grid runs slots x KV heads x
// column chunks one-wave workgroups, and S, the slots of one wave of them, is
// what the GPU holds at once: 256 CUs x 4 SIMDs x 3 waves of the decode
// kernels.  With few sequences (2B <= S) one wave of slots is enough: each
// chunk is about total / S blocks and every workgroup runs at once.  With
// more, short sequences take slots while holding little work, and sequences
// of equal length cannot split into fractions of a chunk, so two waves' worth
// (and at least two slots per sequence) balances better.
constexpr int64_t kDecodeResidentWaves = 3072;

int64_t decode_balanced_slots(int32_t num_seqs, int64_t units_per_slot,
                              int64_t resident = kDecodeResidentWaves) {
  const int64_t per = units_per_slot > 0 ? units_per_slot : 1;
  const int64_t budget = resident / per > 0 ? resident / per : 1;
  const int64_t two_b = 2 * int64_t(num_seqs);
  if (two_b <= budget) return budget;
  return 2 * budget > two_b ? 2 * budget : two_b;
}

// The plan: int32 chunk starts [num_seqs + 1], then, 256-byte aligned, one
// int4 {sequence, first block, end block, chunks of the sequence} per slot.
struct PlanLayout {
  size_t info_offset, total;
};

PlanLayout plan_layout(int64_t num_seqs, int64_t slots) {
  PlanLayout L;
  L.info_offset = align_up(size_t(num_seqs + 1) * sizeof(int32_t));
  L.total = L.info_offset + align_up(size_t(slots) * 4 * sizeof(int32_t));
  return L;
}

// Workspace of a balanced decode call: partials o [R, Hq, D] | lse [R, Hq] |
// the plan.
struct DecodeBalancedLayout {
  PartLayout part;
  PlanLayout plan;
  size_t plan_offset, total;
};

DecodeBalancedLayout decode_balanced_layout(int64_t num_seqs, int64_t Hq, int64_t D,
                                            int64_t slots) {
  DecodeBalancedLayout L;
  L.part = part_layout(slots, Hq, D, 1);
  L.plan = plan_layout(num_seqs, slots);
  L.plan_offset = L.part.total;
  L.total = L.plan_offset + L.plan.total;
  return L;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(pkv_status_t status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    default: return "PKV_UNKNOWN_STATUS";
  }
}

}  // extern "C"

namespace {

// Both appends: q_start == nullptr means one new row per sequence.
pkv_status_t append_impl(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* q_start, int32_t num_seqs, int32_t num_rows,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, pkv_dtype_t kv_dtype,
                         void* stream) {
  if (num_seqs < 0 || num_rows < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || !dtype_ok(kv_dtype))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || block_size != pkv::kBlockSizeBuilt) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_rows == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(q_start))
    return PKV_ERR_INVALID_ARG;
  pkv::AppendArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.row_bytes = head_dim * pkv::dtype_bytes(to_internal(kv_dtype));
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.q_start = q_start;
  a.num_rows = num_rows;
  return pkv::launch_kv_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK
                                                                                  : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

pkv_status_t pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           pkv_dtype_t kv_dtype, void* stream) {
  return append_impl(k_pool, v_pool, k_new, v_new, block_tables, context_lens, nullptr, num_seqs,
                     num_seqs, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, kv_dtype, stream);
}

pkv_status_t pkv_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new,
                                  const void* v_new, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* query_start_loc,
                                  int32_t num_seqs, int32_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, pkv_dtype_t kv_dtype,
                                  void* stream) {
  if (num_seqs > 0 && num_tokens > 0 && !query_start_loc) return PKV_ERR_INVALID_ARG;
  return append_impl(k_pool, v_pool, k_new, v_new, block_tables, context_lens, query_start_loc,
                     num_seqs, num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, kv_dtype, stream);
}

pkv_status_t pkv_kv_append_quant(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                                 const void* k_new, const void* v_new, pkv_dtype_t new_dtype,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start_loc, int32_t num_seqs,
                                 int32_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, pkv_scale_mode_t mode,
                                 void* stream) {
  if (num_seqs < 0 || num_rows < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (new_dtype != PKV_F32 && new_dtype != PKV_BF16) ||
      (mode != PKV_SCALE_FIXED && mode != PKV_SCALE_RUNNING_AMAX))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || block_size != pkv::kBlockSizeBuilt) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_rows == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_scales || !v_scales || !k_new || !v_new || !block_tables ||
      !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned4(k_scales) || !aligned4(v_scales) || !aligned4(block_tables) ||
      !aligned4(context_lens) || !aligned4(query_start_loc))
    return PKV_ERR_INVALID_ARG;
  pkv::QuantAppendArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_start = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.new_bf16 = new_dtype == PKV_BF16;
  a.mode = mode == PKV_SCALE_RUNNING_AMAX ? 1 : 0;
  return pkv::launch_kv_append_quant(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_copy_blocks(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                             const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             pkv_dtype_t kv_dtype, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || !dtype_ok(kv_dtype))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || block_size != pkv::kBlockSizeBuilt) return PKV_ERR_UNSUPPORTED;
  if (num_kv_heads > 256) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !pairs) return PKV_ERR_INVALID_ARG;
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scales || !v_scales)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned4(pairs) || !aligned4(k_scales) ||
      !aligned4(v_scales))
    return PKV_ERR_INVALID_ARG;
  pkv::CopyBlocksArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = kv_dtype == PKV_FP8_E4M3 ? k_scales : nullptr;
  a.v_scales = kv_dtype == PKV_FP8_E4M3 ? v_scales : nullptr;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.num_kv_heads = num_kv_heads;
  a.block_bytes = size_t(num_kv_heads) * size_t(block_size) * size_t(head_dim) *
                  size_t(pkv::dtype_bytes(to_internal(kv_dtype)));
  return pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_stream_read(uint32_t* out, const void* src, size_t bytes,
                             int32_t num_workgroups, void* stream) {
  if (num_workgroups <= 0 || num_workgroups > PKV_STREAM_READ_MAX_WORKGROUPS || bytes % 16 != 0)
    return PKV_ERR_INVALID_ARG;
  if (!out || !aligned4(out) || (bytes > 0 && (!src || !aligned16(src))))
    return PKV_ERR_INVALID_ARG;
  return pkv::launch_stream_read(out, src, bytes, num_workgroups,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_gather_read(uint32_t* out, const void* src, size_t bytes,
                             const int32_t* chunk_ids, int32_t num_chunks,
                             int32_t chunks_per_workgroup, void* stream) {
  if (num_chunks < 0 || chunks_per_workgroup <= 0 || bytes % 4096 != 0 ||
      bytes / 4096 > 0x7fffffff || num_chunks % chunks_per_workgroup != 0 ||
      num_chunks / chunks_per_workgroup > PKV_STREAM_READ_MAX_WORKGROUPS)
    return PKV_ERR_INVALID_ARG;
  if (num_chunks == 0) return PKV_OK;
  if (!out || !aligned4(out) || !chunk_ids || !aligned4(chunk_ids) || !src || !aligned16(src))
    return PKV_ERR_INVALID_ARG;
  return pkv::launch_gather_read(out, src, bytes, chunk_ids, num_chunks, chunks_per_workgroup,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

int32_t pkv_stream_read_out_words(int32_t num_workgroups) {
  if (num_workgroups <= 0 || num_workgroups > PKV_STREAM_READ_MAX_WORKGROUPS) return 0;
  return num_workgroups * pkv::stream_read_waves_per_workgroup();
}

size_t pkv_mla_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank,
                               int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || kv_lora_rank <= 0) return 0;
  if (partition_size == PKV_PARTITION_BALANCED)
    return balanced_layout(num_seqs, num_heads, kv_lora_rank).total;
  if (partition_size < 0) return 0;
  const int64_t maxp = max_partitions(max_context_len, partition_size);
  if (maxp <= 1) return 0;
  return part_layout(num_seqs, num_heads, kv_lora_rank, maxp).total;
}

pkv_status_t pkv_mla_append(void* latent_pool, const void* latent_new,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t row_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq, void* stream) {
  if (num_seqs < 0 || row_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID_ARG;
  if (row_dim != 576 || block_size != pkv::kBlockSizeBuilt) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!latent_pool || !latent_new || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned16(latent_pool) || !aligned16(latent_new) || !aligned4(block_tables) ||
      !aligned4(context_lens))
    return PKV_ERR_INVALID_ARG;
  // The latent pool is a pool with one shared head of 576 bf16 numbers; the
  // same bitwise scatter serves it (row ctx-1, the second pool is the same).
  pkv::AppendArgs a{};
  a.k_pool = latent_pool;
  a.v_pool = latent_pool;
  a.k_new = latent_new;
  a.v_new = latent_new;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = 1;
  a.row_bytes = row_dim * 2;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  return pkv::launch_kv_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK
                                                                                  : PKV_ERR_HIP;
}

pkv_status_t pkv_mla_decode_attention(
    void* out, const void* q, const void* latent_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank,
    int32_t rope_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, void* stream) {
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  if (num_seqs < 0 || num_heads <= 0 || kv_lora_rank <= 0 || rope_dim < 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      (partition_size < 0 && !balanced) || !(softmax_scale == softmax_scale))
    return PKV_ERR_INVALID_ARG;
  if (!balanced && partition_size % block_size != 0) return PKV_ERR_INVALID_ARG;
  if (kv_lora_rank != 512 || rope_dim != 64 || block_size != pkv::kBlockSizeBuilt ||
      num_heads % 16 != 0)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !latent_pool || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(latent_pool) || !aligned4(block_tables) ||
      !aligned4(context_lens) || !aligned16(workspace))
    return PKV_ERR_INVALID_ARG;
  if (balanced) {
    if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
    const BalancedLayout L = balanced_layout(num_seqs, num_heads, kv_lora_rank);
    if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
    const int per_wg = pkv::mla_heads_per_workgroup(num_heads);
    const int head_chunks = (num_heads + per_wg - 1) / per_wg;
    if (L.slots * head_chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
    char* ws = static_cast<char*>(workspace);
    int32_t* first = reinterpret_cast<int32_t*>(ws + L.first_offset);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // Up to kPlanMaxSeqs sequences each workgroup plans its own chunk (and the
    // first chunks publish chunk_first); larger batches run the plan kernel.
    const bool plan_inside = num_seqs <= pkv::kPlanMaxSeqs && L.slots < 46341;
    if (!plan_inside) {
      pkv::SplitArgs sp{};
      sp.context_lens = context_lens;
      sp.num_seqs = num_seqs;
      sp.cap_tokens = max_blocks_per_seq * block_size;
      sp.unit_tokens = 2 * block_size;               // the kernel walks pairs of blocks
      sp.budget = int(L.slots);
      sp.chunk_first = first;
      if (pkv::launch_balanced_split(sp, st) != hipSuccess) return PKV_ERR_HIP;
    }
    pkv::MlaArgs a{};
    a.out = out;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + L.part.lse_offset);
    a.q = q;
    a.pool = latent_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.head_chunks = head_chunks;
    a.num_blocks = num_blocks;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.blocks_per_partition = max_blocks_per_seq;
    a.max_partitions = int(L.slots);
    a.scale_log2 = softmax_scale * pkv::kLog2eHost;
    if (plan_inside) a.plan_first = first; else a.chunk_first = first;
    // The chunks' partial rows go through the workspace as bf16: the merge
    // reads half the bytes (they are as large as a sizeable share of the
    // latent rows read), at the cost of one more rounding of each partial.
    a.part_bf16 = 1;
    if (pkv::launch_mla_decode(a, st) != hipSuccess) return PKV_ERR_HIP;
    pkv::MergeArgs m{};
    m.out = out;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.part_bf16 = 1;
    m.num_seqs = num_seqs;
    m.num_q_heads = num_heads;
    m.max_partitions = int(L.slots);
    m.skip_single = 1;                               // one-chunk sequences are already final
    m.num_batch = num_seqs;
    m.chunk_first = first;
    return pkv::launch_merge(m, kv_lora_rank, DType::BF16, st) == hipSuccess ? PKV_OK
                                                                              : PKV_ERR_HIP;
  }
  const int64_t maxp = max_partitions(max_context_len, partition_size);
  const bool single = maxp <= 1;
  pkv::MlaArgs a{};
  a.out = out;
  a.q = q;
  a.pool = latent_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  const int per_wg = pkv::mla_heads_per_workgroup(num_heads);
  a.head_chunks = (num_heads + per_wg - 1) / per_wg;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = softmax_scale * pkv::kLog2eHost;
  if (!single) {
    const PartLayout L = part_layout(num_seqs, num_heads, kv_lora_rank, maxp);
    if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_offset);
  }
  a.blocks_per_partition =
      single ? max_blocks_per_seq : partition_size / block_size;
  a.max_partitions = int(maxp);
  a.write_final = single ? 1 : 0;
  a.final_single = 1;
  a.mark_empty = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pkv::launch_mla_decode(a, st) != hipSuccess) return PKV_ERR_HIP;
  if (single) return PKV_OK;
  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.num_partitions = nullptr;
  m.context_lens = context_lens;
  m.partition_size = partition_size;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_heads;
  m.max_partitions = int(maxp);
  m.skip_single = 1;
  m.q_start = nullptr;
  m.num_batch = num_seqs;
  return pkv::launch_merge(m, kv_lora_rank, DType::BF16, st) == hipSuccess ? PKV_OK
                                                                            : PKV_ERR_HIP;
}

pkv_status_t pkv_mla_decode_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions_, const void* q,
    const void* latent_pool, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank, int32_t rope_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale,
    int32_t partition_size, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || kv_lora_rank <= 0 || rope_dim < 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || partition_size < 0 || max_partitions_ <= 0 ||
      !(softmax_scale == softmax_scale))
    return PKV_ERR_INVALID_ARG;
  if (partition_size % block_size != 0) return PKV_ERR_INVALID_ARG;
  if (kv_lora_rank != 512 || rope_dim != 64 || block_size != pkv::kBlockSizeBuilt ||
      num_heads % 16 != 0)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!partial_out || !partial_lse || !q || !latent_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(partial_out) || !aligned4(partial_lse) || !aligned16(q) ||
      !aligned16(latent_pool) || !aligned4(block_tables) || !aligned4(context_lens))
    return PKV_ERR_INVALID_ARG;
  pkv::MlaArgs a{};
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.q = q;
  a.pool = latent_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  const int per_wg = pkv::mla_heads_per_workgroup(num_heads);
  a.head_chunks = (num_heads + per_wg - 1) / per_wg;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = softmax_scale * pkv::kLog2eHost;
  a.blocks_per_partition =
      partition_size == 0 ? max_blocks_per_seq : partition_size / block_size;
  a.max_partitions = max_partitions_;
  a.write_final = 0;
  a.final_single = 0;
  a.mark_empty = 1;
  return pkv::launch_mla_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK
                                                                                   : PKV_ERR_HIP;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  if (partition_size == PKV_PARTITION_BALANCED) {
    // KV heads x column chunks >= ceil(Hq / 16) (no workgroup serves more than
    // 16 query heads), so S <= S_max = 3072 / ceil(Hq / 16) and the slots of
    // a call, S or max(2 S, 2 B), are at most max(2 S_max, 2 B).
    const int64_t s_max = kDecodeResidentWaves / ((int64_t(num_q_heads) + 15) / 16);
    const int64_t slots = 2 * s_max > 2 * int64_t(num_seqs) ? 2 * s_max : 2 * int64_t(num_seqs);
    return decode_balanced_layout(num_seqs, num_q_heads, head_dim, slots).total;
  }
  if (partition_size < 0) return 0;
  const int64_t maxp = max_partitions(max_context_len, partition_size);
  if (maxp <= 1) return 0;
  return part_layout(num_seqs, num_q_heads, head_dim, maxp).total;
}

size_t pkv_multi_query_workspace_bytes(int32_t num_tokens, int32_t num_q_heads,
                                       int32_t head_dim, int32_t max_context_len,
                                       int32_t partition_size) {
  // The partial results are laid out per query row, exactly as the
  // one-token workspace is per sequence (no balanced split here).
  if (partition_size < 0) return 0;
  return pkv_decode_workspace_bytes(num_tokens, num_q_heads, head_dim, max_context_len,
                                    partition_size);
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points (everything but the output
// and workspace pointers).
pkv_status_t check_decode(const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, float softmax_scale,
                          int32_t partition_size, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || partition_size < 0 || !dtype_ok(q_dtype) ||
      !dtype_ok(kv_dtype) || !(softmax_scale == softmax_scale))
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (partition_size % block_size != 0) return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || block_size != pkv::kBlockSizeBuilt) return PKV_ERR_UNSUPPORTED;
  if (q_dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scales || !v_scales)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_tables) ||
      !aligned4(context_lens) || !aligned4(k_scales) || !aligned4(v_scales))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

// bf16 queries over a bf16 cache run on the matrix cores when 2 or more
// queries share each KV head (the group's heads times the new tokens); every
// other combination on the vector kernel.  Built with
// -DPKV_DECODE_VECTOR_ONLY (libpkv_vector.so), every decode runs on the
// vector kernel: the build that the matrix-core choice is measured against.
bool uses_mfma(pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, int64_t columns) {
#ifdef PKV_DECODE_VECTOR_ONLY
  (void)q_dtype;
  (void)kv_dtype;
  (void)columns;
  return false;
#else
  return q_dtype == PKV_BF16 && kv_dtype == PKV_BF16 && columns >= 2;
#endif
}

pkv::DecodeArgs decode_args(const void* q, const void* k_pool, const void* v_pool,
                            const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t num_blocks, int32_t max_blocks_per_seq,
                            float softmax_scale, int tile) {
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_chunks = (a.group + tile - 1) / tile;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = softmax_scale * pkv::kLog2eHost;
  (void)head_dim;
  return a;
}

hipError_t launch_decode(const pkv::DecodeArgs& a, int head_dim, int tile, bool mfma,
                         pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, hipStream_t st) {
  return mfma ? pkv::launch_paged_decode_mfma(a, head_dim, st)
              : pkv::launch_paged_decode(a, head_dim, tile, to_internal(q_dtype),
                                         to_internal(kv_dtype), st);
}

// Kernel choice shared by the one-token decode entry points.
struct DecodeKind {
  bool mfma;
  int tile;
};

DecodeKind decode_kind(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  const int group = num_q_heads / num_kv_heads;
  DecodeKind k;
  k.mfma = uses_mfma(q_dtype, kv_dtype, group);
  k.tile = k.mfma ? pkv::mfma_head_tile() : tile_heads(group, head_dim);
  return k;
}

// Chunk slots of a balanced one-token decode (ignoring the cap of the grid).
int64_t decode_slots_for(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  const DecodeKind k = decode_kind(num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  const int64_t chunks = (num_q_heads / num_kv_heads + k.tile - 1) / k.tile;
  return decode_balanced_slots(num_seqs, int64_t(num_kv_heads) * chunks);
}

// Writes the plan of a balanced split of the one-token decode: chunk_first
// and slot_info (see PlanLayout) from the context lengths.
hipError_t launch_plan(void* plan, const int32_t* context_lens, int32_t num_seqs, int64_t slots,
                       int32_t block_size, int32_t max_blocks_per_seq, hipStream_t st) {
  const PlanLayout L = plan_layout(num_seqs, slots);
  pkv::SplitArgs sp{};
  sp.context_lens = context_lens;
  sp.num_seqs = num_seqs;
  sp.cap_tokens = max_blocks_per_seq * block_size;
  sp.unit_tokens = block_size;                     // chunks are runs of whole blocks
  sp.budget = int(slots);
  sp.chunk_first = static_cast<int32_t*>(plan);
  sp.slot_info = reinterpret_cast<int4*>(static_cast<char*>(plan) + L.info_offset);
  sp.num_slots = int(slots);
  return pkv::launch_balanced_split(sp, st);
}

// Sets up the schedule of a balanced decode in `plan` (PlanLayout): batches
// of up to kPlanMaxSeqs sequences are planned inside the decode kernel, which
// writes chunk_first; larger ones by the plan kernel first, whose slot_info the
// decode kernel reads.
bool plan_decode(pkv::DecodeArgs& a, char* plan, int64_t slots, int32_t block_size,
                 hipStream_t st) {
  if (a.num_seqs <= pkv::kPlanMaxSeqs && slots < 46341) {   // chunk bounds in 32 bits
    a.plan_first = reinterpret_cast<int32_t*>(plan);
    a.slot_info = nullptr;
    return true;
  }
  a.plan_first = nullptr;
  a.slot_info = reinterpret_cast<const int4*>(plan + plan_layout(a.num_seqs, slots).info_offset);
  return launch_plan(plan, a.context_lens, a.num_seqs, slots, block_size, a.max_blocks_per_seq,
                     st) == hipSuccess;
}

// The balanced one-token decode: plan, chunks, merge (sequences with one
// chunk are written by the decode kernel and skipped by the merge).
pkv_status_t balanced_impl(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale,
    void* workspace, size_t workspace_bytes, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype,
    hipStream_t st, const void* k_new, const void* v_new, void* k_pool_w, void* v_pool_w);

pkv_status_t attention_impl(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    float softmax_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream, const void* k_new,
    const void* v_new, void* k_pool_w, void* v_pool_w) {
  if (max_context_len < 0) return PKV_ERR_INVALID_ARG;
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  const pkv_status_t st0 = check_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                        context_lens, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, num_blocks, max_blocks_per_seq,
                                        softmax_scale, balanced ? 0 : partition_size, q_dtype,
                                        kv_dtype);
  if (st0 != PKV_OK || num_seqs == 0) return st0;
  if (!out || !aligned16(out) || !aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  if (balanced)
    return balanced_impl(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         max_blocks_per_seq, softmax_scale, workspace, workspace_bytes, q_dtype,
                         kv_dtype, static_cast<hipStream_t>(stream), k_new, v_new, k_pool_w,
                         v_pool_w);

  const int64_t maxp = max_partitions(max_context_len, partition_size);
  const int64_t blocks_per_part =
      partition_size == 0 ? int64_t(max_blocks_per_seq) : int64_t(partition_size / block_size);
  // A single partition per sequence also covers partition sizes past the table's capacity.
  const bool single = maxp <= 1;
  const int group = num_q_heads / num_kv_heads;
  const bool mfma = uses_mfma(q_dtype, kv_dtype, group);
  const int tile = mfma ? pkv::mfma_head_tile() : tile_heads(group, head_dim);

  pkv::DecodeArgs a = decode_args(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  num_blocks, max_blocks_per_seq, softmax_scale, tile);
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool_w = k_pool_w;
  a.v_pool_w = v_pool_w;
  if (!single) {
    const PartLayout L = part_layout(num_seqs, num_q_heads, head_dim, maxp);
    if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_offset);
  }
  a.blocks_per_partition = int(single ? max_blocks_per_seq : blocks_per_part);
  a.max_partitions = int(maxp);
  a.write_final = single ? 1 : 0;
  a.final_single = 1;
  a.mark_empty = 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (launch_decode(a, head_dim, tile, mfma, q_dtype, kv_dtype, st) != hipSuccess)
    return PKV_ERR_HIP;
  if (single) return PKV_OK;

  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.num_partitions = nullptr;
  m.context_lens = context_lens;
  m.partition_size = partition_size;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_q_heads;
  m.max_partitions = int(maxp);
  m.skip_single = 1;
  m.q_start = nullptr;
  m.num_batch = num_seqs;
  return pkv::launch_merge(m, head_dim, to_internal(q_dtype), st) == hipSuccess ? PKV_OK
                                                                                : PKV_ERR_HIP;
}

pkv_status_t balanced_impl(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale,
    void* workspace, size_t workspace_bytes, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype,
    hipStream_t st, const void* k_new, const void* v_new, void* k_pool_w, void* v_pool_w) {
  if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  const DecodeKind k = decode_kind(num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  const int64_t slots =
      decode_slots_for(num_seqs, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  pkv::DecodeArgs a = decode_args(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  num_blocks, max_blocks_per_seq, softmax_scale, k.tile);
  if (slots * num_kv_heads * a.head_chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  const DecodeBalancedLayout L = decode_balanced_layout(num_seqs, num_q_heads, head_dim, slots);
  if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  char* plan = ws + L.plan_offset;
  if (!plan_decode(a, plan, slots, block_size, st)) return PKV_ERR_HIP;
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool_w = k_pool_w;
  a.v_pool_w = v_pool_w;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_lse = reinterpret_cast<float*>(ws + L.part.lse_offset);
  a.blocks_per_partition = max_blocks_per_seq;
  a.max_partitions = int(slots);
  a.write_final = 0;
  a.final_single = 1;
  a.mark_empty = 0;
  if (launch_decode(a, head_dim, k.tile, k.mfma, q_dtype, kv_dtype, st) != hipSuccess)
    return PKV_ERR_HIP;
  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_q_heads;
  m.max_partitions = int(slots);
  m.skip_single = 1;
  m.num_batch = num_seqs;
  m.chunk_first = reinterpret_cast<const int32_t*>(plan);
  return pkv::launch_merge(m, head_dim, to_internal(q_dtype), st) == hipSuccess ? PKV_OK
                                                                                : PKV_ERR_HIP;
}

// Kernel choice for several new tokens per sequence: query columns per KV
// head = max_query_len x group, on the matrix cores in tiles of 16 (two tiles
// per wave past 16 columns) or on the vector kernel.
struct MultiKind {
  bool mfma;
  int tile, tiles_per_wave;
  int64_t chunks;
};

MultiKind multi_kind(int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  MultiKind k;
  const int group = num_q_heads / num_kv_heads;
  const int64_t columns = int64_t(max_query_len) * group;     // queries per KV head
  k.mfma = uses_mfma(q_dtype, kv_dtype, columns);
  k.tiles_per_wave = k.mfma && columns > pkv::mfma_head_tile() ? 2 : 1;
  k.tile = k.mfma ? pkv::mfma_head_tile() * k.tiles_per_wave
                  : tile_heads(columns < (1 << 20) ? int(columns) : (1 << 20), head_dim);
  k.chunks = (columns + k.tile - 1) / k.tile;
  return k;
}

// Resident waves of the decode kernel for several new tokens: two tiles per
// wave take more registers (two waves per SIMD instead of three).
int64_t multi_resident_waves(const MultiKind& k) {
  return k.tiles_per_wave == 2 ? 2048 : kDecodeResidentWaves;
}

// Workspace of a balanced call with several new tokens: partials o
// [R, max_q, Hq, D] | lse [R, max_q, Hq] | the plan.
DecodeBalancedLayout multi_balanced_layout(int64_t num_seqs, int64_t max_q, int64_t Hq, int64_t D,
                                           int64_t slots) {
  DecodeBalancedLayout L;
  L.part = part_layout(slots * max_q, Hq, D, 1);
  L.plan = plan_layout(num_seqs, slots);
  L.plan_offset = L.part.total;
  L.total = L.plan_offset + L.plan.total;
  return L;
}

// Checks and kernel set-up shared by the two multi-token entry points.
struct MultiSetup {
  pkv::DecodeArgs a;
  bool mfma = false, nothing = false;
  int tile = 1;
};

pkv_status_t multi_setup(MultiSetup& ms, const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scales, const float* v_scales,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, float softmax_scale,
                         int32_t partition_size, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  if (num_tokens < 0 || max_query_len < 0) return PKV_ERR_INVALID_ARG;
  // No new token anywhere: sizes are checked, pointers are not needed.
  const pkv_status_t st0 = check_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                        context_lens, num_tokens == 0 ? 0 : num_seqs,
                                        num_q_heads, num_kv_heads, head_dim, block_size,
                                        num_blocks, max_blocks_per_seq, softmax_scale,
                                        partition_size, q_dtype, kv_dtype);
  if (st0 != PKV_OK) return st0;
  if (num_seqs == 0 || num_tokens == 0) {
    ms.nothing = true;
    return PKV_OK;
  }
  if (max_query_len < 1 || !query_start_loc || !aligned4(query_start_loc))
    return PKV_ERR_INVALID_ARG;
  // More than 16 columns on the matrix cores: two 16-column tiles per wave
  // share each block's K/V registers.
  const MultiKind k = multi_kind(max_query_len, num_q_heads, num_kv_heads, head_dim, q_dtype,
                                 kv_dtype);
  ms.mfma = k.mfma;
  ms.tile = k.tile;
  const int tiles_per_wave = k.tiles_per_wave;
  const int64_t chunks = k.chunks;
  if (chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  ms.a = decode_args(q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, softmax_scale, ms.tile);
  ms.a.q_start = query_start_loc;
  ms.a.max_q = max_query_len;
  ms.a.tiles_per_wave = tiles_per_wave;
  ms.a.head_chunks = int(chunks);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status_t pkv_paged_decode_attention(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    float softmax_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream) {
  return attention_impl(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len, softmax_scale, partition_size,
                        workspace, workspace_bytes, q_dtype, kv_dtype, stream, nullptr, nullptr,
                        nullptr, nullptr);
}

pkv_status_t pkv_paged_decode_step(
    void* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const float* k_scales, const float* v_scales, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)))
    return PKV_ERR_INVALID_ARG;
  return attention_impl(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len, softmax_scale, partition_size,
                        workspace, workspace_bytes, q_dtype, kv_dtype, stream, k_new, v_new,
                        k_pool, v_pool);
}

}  // extern "C"

namespace {

// The device memory pkv_paged_decode_step_noalloc uses instead of a caller's
// workspace: one copy per GPU, in the library's code object, alive until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the address that
// hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.  Null on failure.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Workspace bytes one decode step needs with these sizes (the exact layout
// of attention_impl, not pkv_decode_workspace_bytes' upper bound).
size_t step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                            pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  if (partition_size == PKV_PARTITION_BALANCED) {
    const int64_t slots =
        decode_slots_for(num_seqs, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
    return decode_balanced_layout(num_seqs, num_q_heads, head_dim, slots).total;
  }
  const int64_t maxp = max_partitions(max_context_len, partition_size);
  return maxp <= 1 ? 0 : part_layout(num_seqs, num_q_heads, head_dim, maxp).total;
}

}  // namespace

extern "C" {

pkv_status_t pkv_paged_decode_step_noalloc(
    void* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const float* k_scales, const float* v_scales, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream) {
  // The size checks of pkv_paged_decode_step, so the workspace size below is
  // computed from valid sizes only.
  if (max_context_len < 0) return PKV_ERR_INVALID_ARG;
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  const pkv_status_t st0 = check_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                        context_lens, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, num_blocks, max_blocks_per_seq,
                                        softmax_scale, balanced ? 0 : partition_size, q_dtype,
                                        kv_dtype);
  if (st0 != PKV_OK || num_seqs == 0) return st0;
  if (!out || !aligned16(out) || !k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_INVALID_ARG;
  if (step_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                           partition_size, q_dtype, kv_dtype) > PKV_NOALLOC_SCRATCH_BYTES)
    return PKV_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return PKV_ERR_HIP;
  return pkv_paged_decode_step(out, q, k_pool, v_pool, k_new, v_new, k_scales, v_scales,
                               block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                               head_dim, block_size, num_blocks, max_blocks_per_seq,
                               max_context_len, softmax_scale, partition_size, ws,
                               PKV_NOALLOC_SCRATCH_BYTES, q_dtype, kv_dtype, stream);
}

pkv_status_t pkv_paged_decode_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions_, const void* q,
    const void* k_pool, const void* v_pool, const float* k_scales, const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, int32_t partition_size,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream) {
  if (max_partitions_ <= 0) return PKV_ERR_INVALID_ARG;
  const pkv_status_t st0 = check_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                        context_lens, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, num_blocks, max_blocks_per_seq,
                                        softmax_scale, partition_size, q_dtype, kv_dtype);
  if (st0 != PKV_OK || num_seqs == 0) return st0;
  if (!partial_out || !partial_lse || !aligned16(partial_out) || !aligned4(partial_lse))
    return PKV_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  const bool mfma = uses_mfma(q_dtype, kv_dtype, group);
  const int tile = mfma ? pkv::mfma_head_tile() : tile_heads(group, head_dim);
  pkv::DecodeArgs a = decode_args(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  num_blocks, max_blocks_per_seq, softmax_scale, tile);
  a.out = nullptr;
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.blocks_per_partition =
      partition_size == 0 ? max_blocks_per_seq : partition_size / block_size;
  a.max_partitions = max_partitions_;
  a.write_final = 0;
  a.final_single = 0;
  a.mark_empty = 1;
  return launch_decode(a, head_dim, tile, mfma, q_dtype, kv_dtype,
                       static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

int32_t pkv_decode_plan_slots(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      !head_dim_ok(head_dim) || !dtype_ok(q_dtype) || !dtype_ok(kv_dtype))
    return 0;
  const int64_t slots =
      decode_slots_for(num_seqs, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  return slots > 0x7fffffff ? 0 : int32_t(slots);
}

size_t pkv_decode_plan_bytes(int32_t num_seqs, int32_t num_slots) {
  if (num_seqs < 0 || num_slots <= 0 || num_slots < num_seqs) return 0;
  return plan_layout(num_seqs, num_slots).total;
}

pkv_status_t pkv_decode_plan(void* plan, size_t plan_bytes, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_slots, int32_t block_size,
                             int32_t max_blocks_per_seq, void* stream) {
  if (num_seqs < 0 || num_slots <= 0 || num_slots < num_seqs || block_size <= 0 ||
      max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID_ARG;
  if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  if (!plan || !aligned16(plan)) return PKV_ERR_INVALID_ARG;
  if (plan_bytes < plan_layout(num_seqs, num_slots).total) return PKV_ERR_WORKSPACE;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !aligned4(context_lens)) return PKV_ERR_INVALID_ARG;
  return launch_plan(plan, context_lens, num_seqs, num_slots, block_size, max_blocks_per_seq,
                     static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_paged_decode_partials_planned(
    float* partial_out, float* partial_lse, void* plan, size_t plan_bytes, int32_t num_slots,
    const void* q,
    const void* k_pool, const void* v_pool, const float* k_scales, const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream) {
  if (num_slots <= 0 || num_slots < num_seqs) return PKV_ERR_INVALID_ARG;
  const pkv_status_t st0 = check_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                        context_lens, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, num_blocks, max_blocks_per_seq,
                                        softmax_scale, 0, q_dtype, kv_dtype);
  if (st0 != PKV_OK || num_seqs == 0) return st0;
  if (!plan || !aligned16(plan) || !partial_out || !partial_lse || !aligned16(partial_out) ||
      !aligned4(partial_lse))
    return PKV_ERR_INVALID_ARG;
  if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  if (plan_bytes < plan_layout(num_seqs, num_slots).total) return PKV_ERR_WORKSPACE;
  const DecodeKind k = decode_kind(num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  pkv::DecodeArgs a = decode_args(q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  num_blocks, max_blocks_per_seq, softmax_scale, k.tile);
  if (int64_t(num_slots) * num_kv_heads * a.head_chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  a.out = nullptr;
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.blocks_per_partition = max_blocks_per_seq;
  a.max_partitions = num_slots;
  a.write_final = 0;
  a.final_single = 0;
  a.mark_empty = 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!plan_decode(a, static_cast<char*>(plan), num_slots, block_size, st)) return PKV_ERR_HIP;
  return launch_decode(a, head_dim, k.tile, k.mfma, q_dtype, kv_dtype, st) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_merge_partials_planned(void* out, const float* partial_out,
                                        const float* partial_lse, const void* plan,
                                        int32_t num_slots, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t head_dim, pkv_dtype_t out_dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || num_slots <= 0 ||
      num_slots < num_seqs || !dtype_ok(out_dtype))
    return PKV_ERR_INVALID_ARG;
  if ((!head_dim_ok(head_dim) && head_dim != 512) || out_dtype == PKV_FP8_E4M3)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !partial_out || !partial_lse || !plan) return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(partial_out) || !aligned4(partial_lse) || !aligned16(plan))
    return PKV_ERR_INVALID_ARG;
  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = partial_out;
  m.part_lse = partial_lse;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_q_heads;
  m.max_partitions = num_slots;
  m.skip_single = 0;
  m.num_batch = num_seqs;
  m.chunk_first = static_cast<const int32_t*>(plan);
  return pkv::launch_merge(m, head_dim, to_internal(out_dtype), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

size_t pkv_multi_query_balanced_workspace_bytes(int32_t num_seqs, int32_t max_query_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, pkv_dtype_t q_dtype,
                                                pkv_dtype_t kv_dtype) {
  if (num_seqs <= 0 || max_query_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) || !dtype_ok(q_dtype) ||
      !dtype_ok(kv_dtype))
    return 0;
  const MultiKind k =
      multi_kind(max_query_len, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  const int64_t slots = decode_balanced_slots(num_seqs, int64_t(num_kv_heads) * k.chunks,
                                              multi_resident_waves(k));
  return multi_balanced_layout(num_seqs, max_query_len, num_q_heads, head_dim, slots).total;
}

pkv_status_t pkv_paged_multi_query_attention(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    float softmax_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream) {
  if (max_context_len < 0) return PKV_ERR_INVALID_ARG;
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  MultiSetup ms;
  const pkv_status_t st0 = multi_setup(
      ms, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, query_start_loc,
      num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
      num_blocks, max_blocks_per_seq, softmax_scale, balanced ? 0 : partition_size, q_dtype,
      kv_dtype);
  if (st0 != PKV_OK || ms.nothing) return st0;
  if (!out || !aligned16(out) || !aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (balanced) {
    // Chunk slots as for one new token (the units are KV heads x column tiles);
    // partial rows [slot, max_query_len, Hq]; the merge finds each row's
    // sequence and new token from query_start_loc.
    if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
    pkv::DecodeArgs& a = ms.a;
    const MultiKind k =
        multi_kind(max_query_len, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
    const int64_t slots = decode_balanced_slots(num_seqs, int64_t(num_kv_heads) * a.head_chunks,
                                                multi_resident_waves(k));
    if (slots * num_kv_heads * a.head_chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
    const DecodeBalancedLayout L =
        multi_balanced_layout(num_seqs, max_query_len, num_q_heads, head_dim, slots);
    if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    char* plan = ws + L.plan_offset;
    a.out = out;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + L.part.lse_offset);
    a.blocks_per_partition = max_blocks_per_seq;
    a.max_partitions = int(slots);
    a.write_final = 0;
    a.final_single = 1;
    a.mark_empty = 0;
    // On the matrix cores at head dim 128 the chunks' partial rows pass
    // through the workspace as bf16 (one more rounding of each partial; the
    // output is bf16 anyway): half the bytes the decode kernel writes and the
    // merge reads, 2 x 32,768 rows of 512 bytes at 16 new tokens on the
    // batch-64 layer.
    a.part_bf16 = ms.mfma && head_dim == 128 && q_dtype == PKV_BF16 ? 1 : 0;
    if (!plan_decode(a, plan, slots, block_size, st)) return PKV_ERR_HIP;
    if (launch_decode(a, head_dim, ms.tile, ms.mfma, q_dtype, kv_dtype, st) != hipSuccess)
      return PKV_ERR_HIP;
    pkv::MergeArgs m{};
    m.part_bf16 = a.part_bf16;
    m.out = out;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.num_seqs = num_tokens;
    m.num_q_heads = num_q_heads;
    m.max_partitions = int(slots);
    m.skip_single = 1;
    m.q_start = query_start_loc;
    m.num_batch = num_seqs;
    m.rows_per_seq = max_query_len;
    m.chunk_first = reinterpret_cast<const int32_t*>(plan);
    m.slot_rows = max_query_len;
    return pkv::launch_merge(m, head_dim, to_internal(q_dtype), st) == hipSuccess ? PKV_OK
                                                                                  : PKV_ERR_HIP;
  }

  const int64_t maxp = max_partitions(max_context_len, partition_size);
  const bool single = maxp <= 1;
  pkv::DecodeArgs& a = ms.a;
  a.out = out;
  if (!single) {
    const PartLayout L = part_layout(num_tokens, num_q_heads, head_dim, maxp);
    if (!workspace || workspace_bytes < L.total) return PKV_ERR_WORKSPACE;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_offset);
  }
  a.blocks_per_partition =
      single ? max_blocks_per_seq : partition_size / block_size;
  a.max_partitions = int(maxp);
  a.write_final = single ? 1 : 0;
  // Rows of a sequence whose blocks fit one partition are written final by
  // the decode kernel; the merge finds each row's sequence and its partition
  // count from query_start_loc and context_lens, and skips those rows.
  a.final_single = 1;
  a.mark_empty = 0;

  if (launch_decode(a, head_dim, ms.tile, ms.mfma, q_dtype, kv_dtype, st) != hipSuccess)
    return PKV_ERR_HIP;
  if (single) return PKV_OK;

  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.num_partitions = nullptr;
  m.context_lens = context_lens;
  m.partition_size = partition_size;
  m.num_seqs = num_tokens;
  m.num_q_heads = num_q_heads;
  m.max_partitions = int(maxp);
  m.skip_single = 1;
  m.q_start = query_start_loc;
  m.num_batch = num_seqs;
  m.rows_per_seq = max_query_len;
  return pkv::launch_merge(m, head_dim, to_internal(q_dtype), st) == hipSuccess ? PKV_OK
                                                                                : PKV_ERR_HIP;
}

pkv_status_t pkv_paged_multi_query_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions_, const void* q,
    const void* k_pool, const void* v_pool, const float* k_scales, const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
    int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float softmax_scale, int32_t partition_size,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream) {
  if (max_partitions_ <= 0) return PKV_ERR_INVALID_ARG;
  MultiSetup ms;
  const pkv_status_t st0 = multi_setup(
      ms, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, query_start_loc,
      num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
      num_blocks, max_blocks_per_seq, softmax_scale, partition_size, q_dtype, kv_dtype);
  if (st0 != PKV_OK || ms.nothing) return st0;
  if (!partial_out || !partial_lse || !aligned16(partial_out) || !aligned4(partial_lse))
    return PKV_ERR_INVALID_ARG;
  pkv::DecodeArgs& a = ms.a;
  a.out = nullptr;
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.blocks_per_partition =
      partition_size == 0 ? max_blocks_per_seq : partition_size / block_size;
  a.max_partitions = max_partitions_;
  a.write_final = 0;
  a.final_single = 0;
  a.mark_empty = 1;
  return launch_decode(a, head_dim, ms.tile, ms.mfma, q_dtype, kv_dtype,
                       static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

int32_t pkv_multi_query_plan_slots(int32_t num_seqs, int32_t max_query_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype) {
  if (num_seqs <= 0 || max_query_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) || !dtype_ok(q_dtype) ||
      !dtype_ok(kv_dtype) || q_dtype == PKV_FP8_E4M3)
    return 0;
  const MultiKind k =
      multi_kind(max_query_len, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype);
  const int64_t slots =
      decode_balanced_slots(num_seqs, int64_t(num_kv_heads) * k.chunks, multi_resident_waves(k));
  return slots > 0x7fffffff ? 0 : int32_t(slots);
}

pkv_status_t pkv_paged_multi_query_partials_planned(
    float* partial_out, float* partial_lse, void* plan, size_t plan_bytes, int32_t num_slots,
    const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream) {
  if (num_slots <= 0 || num_slots < num_seqs) return PKV_ERR_INVALID_ARG;
  MultiSetup ms;
  const pkv_status_t st0 = multi_setup(
      ms, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, query_start_loc,
      num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
      num_blocks, max_blocks_per_seq, softmax_scale, 0, q_dtype, kv_dtype);
  if (st0 != PKV_OK || ms.nothing) return st0;
  if (!plan || !aligned16(plan) || !partial_out || !partial_lse || !aligned16(partial_out) ||
      !aligned4(partial_lse))
    return PKV_ERR_INVALID_ARG;
  if (int64_t(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  if (plan_bytes < plan_layout(num_seqs, num_slots).total) return PKV_ERR_WORKSPACE;
  pkv::DecodeArgs& a = ms.a;
  if (int64_t(num_slots) * num_kv_heads * a.head_chunks > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  a.out = nullptr;
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.blocks_per_partition = max_blocks_per_seq;
  a.max_partitions = num_slots;
  a.write_final = 0;
  a.final_single = 0;
  a.mark_empty = 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!plan_decode(a, static_cast<char*>(plan), num_slots, block_size, st)) return PKV_ERR_HIP;
  return launch_decode(a, head_dim, ms.tile, ms.mfma, q_dtype, kv_dtype, st) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status_t pkv_merge_partials(void* out, const float* partial_out, const float* partial_lse,
                                const int32_t* num_partitions, int32_t num_seqs,
                                int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
                                pkv_dtype_t out_dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_partitions <= 0 ||
      !dtype_ok(out_dtype))
    return PKV_ERR_INVALID_ARG;
  if ((!head_dim_ok(head_dim) && head_dim != 512) || out_dtype == PKV_FP8_E4M3)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !partial_out || !partial_lse) return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(partial_out) || !aligned4(partial_lse) ||
      !aligned4(num_partitions))
    return PKV_ERR_INVALID_ARG;
  pkv::MergeArgs m{};
  m.out = out;
  m.part_o = partial_out;
  m.part_lse = partial_lse;
  m.num_partitions = num_partitions;
  m.context_lens = nullptr;
  m.partition_size = 0;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_q_heads;
  m.max_partitions = max_partitions;
  m.skip_single = 0;
  m.q_start = nullptr;
  m.num_batch = num_seqs;
  return pkv::launch_merge(m, head_dim, to_internal(out_dtype), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

}  // extern "C"
