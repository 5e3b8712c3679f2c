// Attainable HBM read rate, for measurement.  A decode step sits left of the
// ridge point, where the only roof is memory bandwidth (brunomaga inference
// post, "Roofline model"), and the bandwidth a kernel can reach in practice
// is below the 8 TB/s data-sheet figure: a kernel that does nothing but read
// one large buffer measures it, so a decode kernel can be judged against
// what reading alone achieves.
//
// Each workgroup of 256 threads reads 32 KiB contiguous per pass (eight
// 16-byte nontemporal loads per thread, the loads the decode kernels use for
// K/V) and the grid strides over the buffer; workgroup 0 also reads the
// last, partial pass.  Every word read is folded with
// XOR, so no load can be dropped, and each wave writes its fold to out: the
// XOR of all out words equals the XOR of the buffer's 32-bit words.
//
// A second kernel reads a list of scattered 4 KiB chunks the same way: the
// read rate of the decode kernels' own access pattern (one block's slice of
// one KV head, anywhere in the pool), without any attention arithmetic.
#include "stream_read.h"

#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(uint32_t* out, const char* src,
                                                               size_t n_vec) {
  constexpr size_t kPass = size_t(kThreads) * kUnroll;   // 16-byte vectors per workgroup pass
  const size_t stride = size_t(gridDim.x) * kPass;
  const size_t n_whole = n_vec / kPass * kPass;          // vectors in whole passes
  uint32_t acc = 0;
  for (size_t blk = size_t(blockIdx.x) * kPass; blk < n_whole; blk += stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      r[u] = load_streamed<uint4>(src + (blk + threadIdx.x + size_t(u) * kThreads) * 16);
    __builtin_amdgcn_sched_barrier(0);                   // all eight loads before any use
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  if (blockIdx.x == 0) {                                 // the partial pass at the end
    for (size_t i = n_whole + threadIdx.x; i < n_vec; i += kThreads) {
      const uint4 v = load_streamed<uint4>(src + i * 16);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), o));
  if ((threadIdx.x & (kWave - 1)) == 0)
    out[size_t(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave] = acc;
}

// The same folded read over scattered 4 KiB chunks, the unit the decode
// kernels read (16 tokens x 128 dims x 2 bytes of one block and KV head):
// one wave per workgroup, chunks ids[wg * per_wg ...] in order, two chunks in
// registers (one in flight while the other is folded), 16 bytes per lane and
// load.  An id outside [0, n_chunks) reads nothing.
__global__ __launch_bounds__(kWave) void gather_read_kernel(uint32_t* out, const char* src,
                                                            const int32_t* ids, int per_wg,
                                                            int n_chunks) {
  constexpr int kChunk = 4096;
  const int lane = threadIdx.x;
  const int32_t* my = ids + size_t(blockIdx.x) * per_wg;
  uint32_t acc = 0;
  uint4 r[2][4];
  auto fetch = [&](int k, uint4* d) {
    const int id = my[k];
    const bool ok = unsigned(id) < unsigned(n_chunks);
    const char* c = src + size_t(ok ? id : 0) * kChunk + 16 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = ok ? load_streamed<uint4>(c + 1024 * j) : make_uint4(0, 0, 0, 0);
  };
  if (per_wg > 0) fetch(0, r[0]);
  for (int k = 0; k < per_wg; k += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (k + d + 1 < per_wg) fetch(k + d + 1, r[d ^ 1]);
      if (k + d < per_wg)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= r[d][j].x ^ r[d][j].y ^ r[d][j].z ^ r[d][j].w;
    }
  }
  out[size_t(blockIdx.x) * kWave + lane] = acc;
}

}  // namespace

hipError_t launch_gather_read(uint32_t* out, const void* src, size_t bytes, const int32_t* ids,
                              int num_ids, int per_workgroup, hipStream_t stream) {
  const int workgroups = num_ids / per_workgroup;
  hipLaunchKernelGGL(gather_read_kernel, dim3(unsigned(workgroups)), dim3(kWave), 0, stream, out,
                     static_cast<const char*>(src), ids, per_workgroup, int(bytes / 4096));
  return hipGetLastError();
}

int stream_read_waves_per_workgroup() { return kThreads / kWave; }

hipError_t launch_stream_read(uint32_t* out, const void* src, size_t bytes, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(workgroups)), dim3(kThreads), 0, stream,
                     out, static_cast<const char*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace pkv
