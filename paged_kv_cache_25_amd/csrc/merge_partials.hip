// Log-sum-exp merge of split-KV partial results, for gfx950.
//
// One 64-lane workgroup per (sequence, query head).  The lanes find
// M = max lse over the partitions that count, lane i computes the weight
// exp(lse_i - M) of partition i, and every lane accumulates sum_p w_p o_p over
// its D/64 dims with eight partial rows in flight, then divides by the summed
// weights.  Partitions that do not count (past the sequence's count, or with
// lse = -inf) are skipped, never multiplied by a zero weight, so whatever they
// hold cannot reach the output.
//   learn.mohebi.ai serving lesson, "PagedAttention" and "Where it shows up":
//   partial attention results merged with the online-softmax update.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

template <int D, typename OT>
__global__ __launch_bounds__(kWave) void merge_kernel(MergeArgs a) {
  constexpr int kPer = D / kWave;                 // dims per lane: 1 or 2
  constexpr int kUnroll = 8;                      // partial rows in flight per lane
  const int qh = blockIdx.x % a.num_q_heads;
  const int b = blockIdx.x / a.num_q_heads;
  const int lane = threadIdx.x;

  int np = a.max_partitions;
  if (a.num_partitions) {
    np = a.num_partitions[b];
  } else if (a.context_lens) {
    const int ctx = a.context_lens[b];
    np = ctx <= 0 ? 0 : (ctx + a.partition_size - 1) / a.partition_size;
  }
  np = np < 0 ? 0 : (np > a.max_partitions ? a.max_partitions : np);
  if (a.skip_single && np == 1) return;           // already final

  const size_t row = size_t(b) * a.num_q_heads + qh;
  const float* lse = a.part_lse + row * a.max_partitions;
  const float* o = a.part_o + row * a.max_partitions * D + lane * kPer;

  float M = -INFINITY;
  for (int p = lane; p < np; p += kWave) M = fmaxf(M, lse[p]);
  M = wave_max(M);

  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  float wsum = 0.0f;
  if (M > -INFINITY) {
    for (int p0 = 0; p0 < np; p0 += kWave) {
      // Lane i holds the weight of partition p0 + i; -inf partitions never count.
      const float lp = p0 + lane < np ? lse[p0 + lane] : -INFINITY;
      const uint64_t counts = __ballot(lp != -INFINITY);
      const float w_lane = lp != -INFINITY ? __expf(lp - M) : 0.0f;
      wsum += w_lane;
      const int cnt = np - p0 < kWave ? np - p0 : kWave;
      for (int k0 = 0; k0 < cnt; k0 += kUnroll) {
        float part[kUnroll][kPer];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int k = k0 + u;
          const bool use = k < cnt && ((counts >> k) & 1);
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            part[u][e] = use ? o[size_t(p0 + k) * D + e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int k = k0 + u;
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane),
                                                                   k < kWave ? k : 0));
          const bool use = k < cnt && ((counts >> k) & 1);
#pragma unroll
          for (int e = 0; e < kPer; ++e) acc[e] = use ? fmaf(w, part[u][e], acc[e]) : acc[e];
        }
      }
    }
  }
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  char* orow = reinterpret_cast<char*>(a.out) + row * D * sizeof(typename OT::Storage);
#pragma unroll
  for (int k = 0; k < kPer; ++k) OT::store(orow, lane * kPer + k, acc[k] * inv);
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

template <int D>
hipError_t launch_d(const MergeArgs& a, DType out_dtype, hipStream_t stream) {
  const size_t grid = size_t(a.num_seqs) * a.num_q_heads;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (out_dtype == DType::F32)
    hipLaunchKernelGGL((merge_kernel<D, OutF32>), dim3(unsigned(grid)), dim3(kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, OutBF16>), dim3(unsigned(grid)), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, DType out_dtype, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, out_dtype, stream);
  return launch_d<128>(a, out_dtype, stream);
}

}  // namespace pkv
