// Log-sum-exp merge of split-KV partial results, for gfx950.
//
// For each merged (row, head) item: M = max lse over the partitions that
// count, out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M).  Partitions
// that do not count (past the row's count, or with lse = -inf) are skipped,
// never multiplied by a zero weight, so whatever they hold cannot reach the
// output.  A row group of D/4 threads (D/8 for bf16 partial rows) reads one
// partition row with 16-byte loads, several rows in flight.  Three launch
// shapes:
//   - bf16 rows (the balanced MLA split; several new tokens per sequence):
//     merge_wide_kernel, 32 or 8 threads per item, each two 16-byte pieces
//     of every row;
//   - very many items with few partitions each (several new tokens per
//     sequence): merge_items_kernel, several items per 256-thread workgroup,
//     one row group per item reading all of its partitions;
//   - otherwise merge_kernel, one workgroup per item, its row groups taking
//     every kGroups-th partition, summed in LDS.
//   learn.mohebi.ai serving lesson, "PagedAttention" and "Where it shows up":
//   partial attention results merged with the online-softmax update.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// The merged row of grid item `item` = (row, head) (with several new tokens
// per sequence: (sequence, new token j, head)) and where its partitions lie.
// False: nothing to merge (no such token, or a single partition the decode
// kernel already wrote as the final output).
struct MergeItem {
  size_t row;          // row of out: b * num_q_heads + head
  int np;              // partitions that may count
  size_t base, stride; // partition p of the row: partial row base + p * stride
};

__device__ inline bool merge_item(const MergeArgs& a, int item, MergeItem& it) {
  const int qh = item % a.num_q_heads;
  // The row (b) and, with several new tokens per sequence, its sequence and
  // new token j there: the row is q_start[seq] + j, loaded together with the
  // sequence's partition bounds.
  int b = item / a.num_q_heads, seq = b, j = 0;
  if (a.q_start) {
    const int sj = b;                              // seq * rows_per_seq + j
    seq = sj / a.rows_per_seq;
    j = sj - seq * a.rows_per_seq;
    const int r0 = a.q_start[seq];
    if (j >= a.q_start[seq + 1] - r0) return false;    // no such token
    b = r0 + j;
  }
  const int slot_rows = a.slot_rows > 1 ? a.slot_rows : 1;
  int np = a.max_partitions;
  int first = 0;
  if (a.chunk_first) {                            // kept inside the max_partitions slots
    first = min(max(a.chunk_first[seq], 0), a.max_partitions);
    np = min(max(a.chunk_first[seq + 1], first), a.max_partitions) - first;
    if (j < 0 || j >= slot_rows) np = 0;          // no slot row for this token
  } else if (a.num_partitions) {
    np = a.num_partitions[b];
  } else if (a.context_lens) {
    const int ctx = a.context_lens[seq];
    np = ctx <= 0 ? 0 : (ctx + a.partition_size - 1) / a.partition_size;
  }
  np = np < 0 ? 0 : (np > a.max_partitions ? a.max_partitions : np);
  if (a.skip_single && np == 1) return false;     // already final
  it.row = size_t(b) * a.num_q_heads + qh;
  it.np = np;
  // Partition p of this row: rows [b, H, max_partitions] (stride 1), or, for
  // a balanced split, chunk slot chunk_first[seq] + p of rows [slot,
  // slot_rows, H] (stride slot_rows * H).
  it.base = a.chunk_first ? (size_t(first) * slot_rows + j) * a.num_q_heads + qh
                          : it.row * a.max_partitions;
  it.stride = a.chunk_first ? size_t(slot_rows) * a.num_q_heads : 1;
  return true;
}

template <int N>
struct VecF {
  float v[N];
};

// Partition p's 16 bytes of row data for thread c of a row group: float32
// rows, or bf16 rows widened to float32.
template <int D, bool kBf16Part>
__device__ __forceinline__ VecF<kBf16Part ? 8 : 4> merge_row_at(const MergeArgs& a,
                                                                const MergeItem& it, int c, int p) {
  constexpr int kVec = kBf16Part ? 8 : 4;
  const size_t off = (it.base + size_t(p) * it.stride) * D + size_t(kVec) * c;
  VecF<kVec> r;
  if constexpr (kBf16Part) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.part_o) + off);
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r.v[2 * e] = __uint_as_float(x[e] << 16);
      r.v[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
    }
  } else {
    const float4 f = *reinterpret_cast<const float4*>(a.part_o + off);
    r.v[0] = f.x; r.v[1] = f.y; r.v[2] = f.z; r.v[3] = f.w;
  }
  return r;
}

template <int D, typename OT, bool kBf16Part>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  constexpr int kVec = kBf16Part ? 8 : 4;         // 16 bytes of a row per thread and load
  constexpr int kRowThreads = D / kVec;           // threads covering one partition row
  constexpr int kMaxGroups = kThreads / kRowThreads;
  constexpr int kUnroll = kBf16Part ? 4 : 8;      // rows in flight per row group
  using Vec = VecF<kVec>;
  __shared__ Vec s_acc[kMaxGroups][kRowThreads];
  __shared__ float s_w[kMaxGroups];
  __shared__ float s_max[kThreads / kWave];
  const int kGroups = blockDim.x / kRowThreads;   // row groups in this launch
  const int n_waves = blockDim.x / kWave;
  const int t = threadIdx.x;
  const int g = t / kRowThreads, c = t % kRowThreads;

  MergeItem it;
  if (!merge_item(a, blockIdx.x, it)) return;     // uniform: the whole block
  const int np = it.np;
  const size_t row = it.row;
  auto lse_at = [&](int p) { return a.part_lse[it.base + size_t(p) * it.stride]; };
  auto row_at = [&](int p) { return merge_row_at<D, kBf16Part>(a, it, c, p); };
  const Vec zero = {};

  // First batch of rows and their lse, issued together with the max pass.
  Vec rowv[kUnroll];
  float lp[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int p = g + u * kGroups;
    lp[u] = p < np ? lse_at(p) : -INFINITY;
    rowv[u] = p < np ? row_at(p) : zero;
  }
  float M = -INFINITY;
  for (int p = t; p < np; p += blockDim.x) M = fmaxf(M, lse_at(p));
  M = wave_max(M);
  if ((t & (kWave - 1)) == 0) s_max[t / kWave] = M;
  __syncthreads();
  M = s_max[0];
  for (int w = 1; w < n_waves; ++w) M = fmaxf(M, s_max[w]);

  // Row group g takes partitions g, g + kGroups, ...; -inf partitions never count.
  Vec acc = zero;
  float wsum = 0.0f;
  if (M > -INFINITY) {
    for (int p0 = g;; ) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (lp[u] == -INFINITY) continue;
        const float w = __expf(lp[u] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc.v[e] = fmaf(w, rowv[u].v[e], acc.v[e]);
      }
      p0 += kGroups * kUnroll;
      if (p0 >= np) break;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = p0 + u * kGroups;
        lp[u] = p < np ? lse_at(p) : -INFINITY;
        rowv[u] = p < np ? row_at(p) : zero;
      }
    }
  }
  s_acc[g][c] = acc;
  if (c == 0) s_w[g] = wsum;
  __syncthreads();
  if (g != 0) return;
  float W = 0.0f;
  for (int k = 0; k < kGroups; ++k) {
    const Vec v = s_acc[k][c];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc.v[e] = k == 0 ? v.v[e] : acc.v[e] + v.v[e];
    W += s_w[k];
  }
  const float inv = W > 0.0f ? 1.0f / W : 0.0f;
  char* orow = reinterpret_cast<char*>(a.out) + row * D * sizeof(typename OT::Storage);
#pragma unroll
  for (int e = 0; e < kVec; ++e) OT::store(orow, kVec * c + e, acc.v[e] * inv);
}

struct OutF32 {
  using Storage = float;
  __device__ static void store(char* row, int i, float v) { reinterpret_cast<float*>(row)[i] = v; }
};
struct OutBF16 {
  using Storage = uint16_t;
  __device__ static void store(char* row, int i, float v) {
    reinterpret_cast<uint16_t*>(row)[i] = f32_to_bf16_rne(v);
  }
};

// Rows with few partitions: several (row, head) items per workgroup, one row
// group of D/4 threads (D/8 for bf16 rows) per item, which reads all of the
// item's partitions itself (kUnroll rows in flight) and needs no LDS or
// barrier.  Fewer, fuller workgroups than one per item: at 16 new tokens per
// sequence a step has 32,768 items of two partitions each.
template <int D, typename OT, bool kBf16Part>
__global__ __launch_bounds__(kThreads) void merge_items_kernel(MergeArgs a, int n_items) {
  constexpr int kVec = kBf16Part ? 8 : 4;
  constexpr int kRowThreads = D / kVec;
  constexpr int kItems = kThreads / kRowThreads;  // items per workgroup
  constexpr int kUnroll = kBf16Part ? 4 : 8;
  using Vec = VecF<kVec>;
  const int item = blockIdx.x * kItems + threadIdx.x / kRowThreads;
  const int c = threadIdx.x % kRowThreads;
  if (item >= n_items) return;
  MergeItem it;
  if (!merge_item(a, item, it)) return;           // uniform over the row group
  const int np = it.np;
  auto lse_at = [&](int p) { return a.part_lse[it.base + size_t(p) * it.stride]; };
  const Vec zero = {};

  // First batch of rows with their lse; the maximum over every partition.
  Vec rowv[kUnroll];
  float lp[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    lp[u] = u < np ? lse_at(u) : -INFINITY;
    rowv[u] = u < np ? merge_row_at<D, kBf16Part>(a, it, c, u) : zero;
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) M = fmaxf(M, lp[u]);
  for (int p = kUnroll; p < np; ++p) M = fmaxf(M, lse_at(p));

  // -inf partitions never count.
  Vec acc = zero;
  float wsum = 0.0f;
  if (M > -INFINITY) {
    for (int p0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (lp[u] == -INFINITY) continue;
        const float w = __expf(lp[u] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc.v[e] = fmaf(w, rowv[u].v[e], acc.v[e]);
      }
      p0 += kUnroll;
      if (p0 >= np) break;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = p0 + u;
        lp[u] = p < np ? lse_at(p) : -INFINITY;
        rowv[u] = p < np ? merge_row_at<D, kBf16Part>(a, it, c, p) : zero;
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  char* orow = reinterpret_cast<char*>(a.out) + it.row * D * sizeof(typename OT::Storage);
#pragma unroll
  for (int e = 0; e < kVec; ++e) OT::store(orow, kVec * c + e, acc.v[e] * inv);
}

// bf16 partial rows, wide: a row group of kRowThreads threads per item, each
// thread D / (8 kRowThreads) 16-byte pieces of a row (pieces c + kRowThreads
// i: every load instruction reads contiguous bytes), four rows of an item in
// flight; the arithmetic is the other kernels' element by element (the
// maximum over every partition, then the weighted sum in partition order), so
// the bits are the same.  Fewer, fuller waves, all resident at once: the
// absorbed MLA merge (8,192 items of 1 KB rows, 32 threads each) runs as
// 4,096 waves instead of 8,192 one-wave workgroups, 12.4 -> 10.5 us (16 or 8
// threads per item measured the same within the noise); 16 new tokens per
// sequence (32,768 items of 256-byte rows, 8 threads each) as 4,096 waves
// instead of 8,192, 5.9-6.4 -> 4.4-4.6 us.
template <int D, typename OT, int kRowThreads = 32>
__global__ __launch_bounds__(kThreads) void merge_wide_kernel(MergeArgs a, int n_items) {
  constexpr int kPieces = D / 8 / kRowThreads;    // 16-byte pieces per thread and row
  constexpr int kItems = kThreads / kRowThreads;  // items per workgroup
  constexpr int kUnroll = 4;
  static_assert(D % (8 * kRowThreads) == 0, "whole pieces per thread");
  const int item = blockIdx.x * kItems + threadIdx.x / kRowThreads;
  const int c = threadIdx.x % kRowThreads;
  if (item >= n_items) return;
  MergeItem it;
  if (!merge_item(a, item, it)) return;           // uniform over the row group
  const int np = it.np;
  auto lse_at = [&](int p) { return a.part_lse[it.base + size_t(p) * it.stride]; };
  auto piece_at = [&](int p, int i) {
    const size_t off = (it.base + size_t(p) * it.stride) * D + 8 * size_t(c + kRowThreads * i);
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.part_o) + off);
  };

  uint4 rowv[kUnroll][kPieces];
  float lp[kUnroll];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u;
      lp[u] = p < np ? lse_at(p) : -INFINITY;
#pragma unroll
      for (int i = 0; i < kPieces; ++i) rowv[u][i] = p < np ? piece_at(p, i) : make_uint4(0, 0, 0, 0);
    }
  };
  load_batch(0);
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) M = fmaxf(M, lp[u]);
  for (int p = kUnroll; p < np; ++p) M = fmaxf(M, lse_at(p));

  float acc[kPieces][8];
#pragma unroll
  for (int i = 0; i < kPieces; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
  float wsum = 0.0f;
  if (M > -INFINITY) {
    for (int p0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (lp[u] == -INFINITY) continue;
        const float w = __expf(lp[u] - M);
        wsum += w;
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
          const uint32_t x[4] = {rowv[u][i].x, rowv[u][i].y, rowv[u][i].z, rowv[u][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[i][2 * e] = fmaf(w, __uint_as_float(x[e] << 16), acc[i][2 * e]);
            acc[i][2 * e + 1] = fmaf(w, __uint_as_float(x[e] & 0xffff0000u), acc[i][2 * e + 1]);
          }
        }
      }
      p0 += kUnroll;
      if (p0 >= np) break;
      load_batch(p0);
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  char* orow = reinterpret_cast<char*>(a.out) + it.row * D * sizeof(typename OT::Storage);
#pragma unroll
  for (int i = 0; i < kPieces; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) OT::store(orow, 8 * (c + kRowThreads * i) + e, acc[i][e] * inv);
}

template <int D, bool kBf16Part = false>
hipError_t launch_d(const MergeArgs& a, DType out_dtype, hipStream_t stream) {
  const size_t grid = (a.q_start ? size_t(a.num_batch) * a.rows_per_seq : size_t(a.num_seqs)) *
                      a.num_q_heads;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  // One wave per (sequence, head) when its rows fit one batch (kUnroll rows
  // per row group), or when there are enough (sequence, head) pairs to fill the
  // chip with single waves; four waves for few, long sequences.  Chunk slots
  // of a balanced split are spread over the sequences: judge by their mean.
  const int rows = a.chunk_first ? (a.max_partitions + a.num_batch - 1) / a.num_batch
                                 : a.max_partitions;     // partial rows per merged row
  constexpr int kRowThreads = D / (kBf16Part ? 8 : 4);   // 16 bytes of a row per thread
  constexpr int kUnroll = kBf16Part ? 4 : 8;              // rows in flight per row group
  // Very many items with few partitions each (16 new tokens per sequence:
  // 32,768 items of two partitions): several items per workgroup, a row group
  // each.  Measured at 12.2 us there against 16.2 us one workgroup per item;
  // at 8,192 items (MLA) the two shapes tie, at 2,048 (one new token) the
  // workgroup per item is faster (4.7 against 5.2 us).
  if constexpr (kBf16Part && D == 128) {                 // several new tokens per sequence
    constexpr int kItems = kThreads / 8;
    const size_t blocks = (grid + kItems - 1) / kItems;
    if (out_dtype == DType::F32)
      hipLaunchKernelGGL((merge_wide_kernel<D, OutF32, 8>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                         stream, a, int(grid));
    else
      hipLaunchKernelGGL((merge_wide_kernel<D, OutBF16, 8>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                         stream, a, int(grid));
    return hipGetLastError();
  }
  if constexpr (kBf16Part && D == 512) {                 // MLA latent rows
    constexpr int kItems = kThreads / 32;
    const size_t blocks = (grid + kItems - 1) / kItems;
    if (out_dtype == DType::F32)
      hipLaunchKernelGGL((merge_wide_kernel<D, OutF32>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                         stream, a, int(grid));
    else
      hipLaunchKernelGGL((merge_wide_kernel<D, OutBF16>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                         stream, a, int(grid));
    return hipGetLastError();
  }
  if (kRowThreads <= kWave && rows <= 2 * kUnroll && grid >= 16384) {
    constexpr int kItems = kThreads / kRowThreads;
    const size_t blocks = (grid + kItems - 1) / kItems;
    if (out_dtype == DType::F32)
      hipLaunchKernelGGL((merge_items_kernel<D, OutF32, kBf16Part>), dim3(unsigned(blocks)),
                         dim3(kThreads), 0, stream, a, int(grid));
    else
      hipLaunchKernelGGL((merge_items_kernel<D, OutBF16, kBf16Part>), dim3(unsigned(blocks)),
                         dim3(kThreads), 0, stream, a, int(grid));
    return hipGetLastError();
  }
  const bool one_batch = rows * kRowThreads <= kUnroll * kWave;
  int threads = (one_batch || grid >= 4096) ? kWave : kThreads;
  threads = threads < kRowThreads ? kRowThreads : threads;   // one row group reads a whole row
  if (out_dtype == DType::F32)
    hipLaunchKernelGGL((merge_kernel<D, OutF32, kBf16Part>), dim3(unsigned(grid)), dim3(threads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, OutBF16, kBf16Part>), dim3(unsigned(grid)), dim3(threads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, DType out_dtype, hipStream_t stream) {
  if (a.part_bf16) {      // bf16 partial rows: MLA latent rows, and head dim 128 with several tokens
    if (head_dim == 512) return launch_d<512, true>(a, out_dtype, stream);
    if (head_dim == 128) return launch_d<128, true>(a, out_dtype, stream);
    return hipErrorInvalidValue;
  }
  if (head_dim == 64) return launch_d<64>(a, out_dtype, stream);
  if (head_dim == 512) return launch_d<512>(a, out_dtype, stream);   // MLA latent rows
  return launch_d<128>(a, out_dtype, stream);
}

}  // namespace pkv
