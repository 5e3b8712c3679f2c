// Copy-on-write block copies for gfx950: for each (src, dst) pair, physical
// block dst of the K pool and of the V pool (every KV head and slot) becomes
// a bitwise copy of block src, and so do the per-(block, head) scales of an
// e4m3 cache.  The allocator asks for these when a sequence is about to
// write into a block another sequence still holds (KV-cache post,
// "PagedAttention: the KV cache in blocks": a shared block is copied only
// when the sequences diverge; serving lesson, "Sharing (section 4.4)").
//
// One 256-thread workgroup per (pair, 4 KiB chunk of a block); each thread
// moves 16 bytes of K and 16 of V.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkBytes = kThreads * 16;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksArgs a, int chunks) {
  const int pair = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int src = a.pairs[2 * size_t(pair)];
  const int dst = a.pairs[2 * size_t(pair) + 1];
  if (unsigned(src) >= unsigned(a.num_blocks) || unsigned(dst) >= unsigned(a.num_blocks)) return;
  const size_t off = size_t(chunk) * kChunkBytes + size_t(threadIdx.x) * 16;
  if (off < a.block_bytes) {
    const char* ks = static_cast<const char*>(a.k_pool) + size_t(src) * a.block_bytes + off;
    const char* vs = static_cast<const char*>(a.v_pool) + size_t(src) * a.block_bytes + off;
    char* kd = static_cast<char*>(a.k_pool) + size_t(dst) * a.block_bytes + off;
    char* vd = static_cast<char*>(a.v_pool) + size_t(dst) * a.block_bytes + off;
    const uint4 k = *reinterpret_cast<const uint4*>(ks);
    const uint4 v = *reinterpret_cast<const uint4*>(vs);
    *reinterpret_cast<uint4*>(kd) = k;
    *reinterpret_cast<uint4*>(vd) = v;
  }
  if (chunk == 0 && a.k_scales && int(threadIdx.x) < a.num_kv_heads) {
    const size_t h = threadIdx.x;
    a.k_scales[size_t(dst) * a.num_kv_heads + h] = a.k_scales[size_t(src) * a.num_kv_heads + h];
    a.v_scales[size_t(dst) * a.num_kv_heads + h] = a.v_scales[size_t(src) * a.num_kv_heads + h];
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  const size_t chunks = (a.block_bytes + kChunkBytes - 1) / kChunkBytes;
  const size_t grid = size_t(a.num_pairs) * chunks;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a,
                     int(chunks));
  return hipGetLastError();
}

}  // namespace pkv
