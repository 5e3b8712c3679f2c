// Log-sum-exp merge of split-KV partial results, for gfx950.
//
// One 64-lane workgroup per (sequence, query head).  The lanes first find
// M = max lse over the partitions that count, then each lane accumulates
// sum_p exp(lse_p - M) * o_p over its D/64 dims and divides by the summed
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

  const size_t row = size_t(b) * a.num_q_heads + qh;
  const float* lse = a.part_lse + row * a.max_partitions;
  const float* o = a.part_o + row * a.max_partitions * D;

  float M = -INFINITY;
  for (int p = lane; p < np; p += kWave) M = fmaxf(M, lse[p]);
  M = wave_max(M);

  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  float wsum = 0.0f;
  if (M > -INFINITY) {
    for (int p = 0; p < np; ++p) {
      const float lp = lse[p];
      if (lp == -INFINITY) continue;              // empty partition: skipped
      const float w = __expf(lp - M);
      wsum += w;
      const float* op = o + size_t(p) * D + lane * kPer;
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[k] = fmaf(w, op[k], acc[k]);
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  char* orow = reinterpret_cast<char*>(a.out) + row * D * sizeof(typename OT::Storage);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const float v = acc[k] * inv;
    OT::store(orow, lane * kPer + k, v);
  }
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
