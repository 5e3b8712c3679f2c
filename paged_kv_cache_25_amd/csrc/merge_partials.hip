// Log-sum-exp merge of split-KV partial results, for gfx950.
//
// One workgroup per (sequence, query head): one wave when every sequence's
// partition rows fit in one batch or the batch is large, else 256 threads.  A row group reads one
// partition row with 16-byte loads (D/4 threads for float32 rows, D/8 for
// the bf16 rows of the balanced MLA split) and keeps eight rows in flight
// (four for bf16 rows; 64 rows per 256 threads for D=128); the
// first batch is issued together with the pass that finds M = max lse over the
// partitions that count.  Each group accumulates sum_p exp(lse_p - M) o_p over
// its partitions, and the groups are summed in LDS and divided by the summed
// weights.  Partitions that do not count (past
// the sequence's count, or with lse = -inf) are skipped, never multiplied by a
// zero weight, so whatever they hold cannot reach the output.
//   learn.mohebi.ai serving lesson, "PagedAttention" and "Where it shows up":
//   partial attention results merged with the online-softmax update.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

template <int N>
struct VecF {
  float v[N];
};

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

  const int qh = blockIdx.x % a.num_q_heads;
  const int b = blockIdx.x / a.num_q_heads;
  const int t = threadIdx.x;
  const int g = t / kRowThreads, c = t % kRowThreads;

  // Row b's sequence (several new tokens per sequence: the last s with
  // q_start[s] <= b) and its new token j there.
  int seq = b, j = 0;
  if (a.q_start && (a.chunk_first || a.context_lens)) {
    int lo = 0, hi = a.num_batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.q_start[mid] <= b) lo = mid; else hi = mid - 1;
    }
    seq = lo;
    j = b - a.q_start[seq];
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
  if (a.skip_single && np == 1) return;           // already final (uniform: whole block)

  const size_t row = size_t(b) * a.num_q_heads + qh;
  // Partition p of this row: rows [b, H, max_partitions] (stride 1), or, for
  // a balanced split, chunk slot chunk_first[seq] + p of rows [slot,
  // slot_rows, H] (stride slot_rows * H).
  const size_t base = a.chunk_first ? (size_t(first) * slot_rows + j) * a.num_q_heads + qh
                                    : row * a.max_partitions;
  const size_t stride = a.chunk_first ? size_t(slot_rows) * a.num_q_heads : 1;
  const float* lse_base = a.part_lse + base;
  const size_t o_off = base * D + size_t(kVec) * c;        // elements, float32 or bf16
  auto lse_at = [&](int p) { return lse_base[size_t(p) * stride]; };
  auto row_at = [&](int p) {
    Vec r;
    if constexpr (kBf16Part) {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.part_o) +
                                                      o_off + size_t(p) * stride * D);
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r.v[2 * e] = __uint_as_float(x[e] << 16);
        r.v[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
      }
    } else {
      const float4 f = *reinterpret_cast<const float4*>(a.part_o + o_off + size_t(p) * stride * D);
      r.v[0] = f.x; r.v[1] = f.y; r.v[2] = f.z; r.v[3] = f.w;
    }
    return r;
  };
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

template <int D, bool kBf16Part = false>
hipError_t launch_d(const MergeArgs& a, DType out_dtype, hipStream_t stream) {
  const size_t grid = size_t(a.num_seqs) * a.num_q_heads;
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
  if (a.part_bf16) {                              // bf16 partial rows: MLA latent rows only
    if (head_dim != 512) return hipErrorInvalidValue;
    return launch_d<512, true>(a, out_dtype, stream);
  }
  if (head_dim == 64) return launch_d<64>(a, out_dtype, stream);
  if (head_dim == 512) return launch_d<512>(a, out_dtype, stream);   // MLA latent rows
  return launch_d<128>(a, out_dtype, stream);
}

}  // namespace pkv
