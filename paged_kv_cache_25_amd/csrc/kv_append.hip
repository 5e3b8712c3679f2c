// KV append for gfx950: scatter each sequence's new K and V rows into slot
// ctx - 1 of its paged cache.  A bitwise copy, 16 bytes per thread, so the
// result is exact for every storage format.
//   KV-cache post (xuewyang.github.io/posts/kv), "A toy vLLM" (write_kv: the
//   block-table lookup pos // BLOCK and the slot pos % BLOCK);
//   brunomaga inference post, "PagedAttention..." (PagedKVCache.append).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// Thread t copies chunk c of row (b, h) of K and of V; chunks are 16 bytes.
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a, int chunks_per_row,
                                                             int total) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int c = t % chunks_per_row;
  const int bh = t / chunks_per_row;
  const int h = bh % a.num_kv_heads;
  const int b = bh / a.num_kv_heads;
  const int ctx = a.context_lens[b];
  if (ctx <= 0 || ctx > a.max_blocks_per_seq * kBlockSize) return;
  const int pos = ctx - 1;
  const int phys = a.block_tables[size_t(b) * a.max_blocks_per_seq + pos / kBlockSize];
  if (unsigned(phys) >= unsigned(a.num_blocks)) return;
  const size_t dst = ((size_t(phys) * a.num_kv_heads + h) * kBlockSize + pos % kBlockSize) *
                         size_t(a.row_bytes) + size_t(c) * 16;
  const size_t src = (size_t(b) * a.num_kv_heads + h) * size_t(a.row_bytes) + size_t(c) * 16;
  const uint4 kv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.k_new) + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.v_new) + src);
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_pool) + dst) = kv;
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_pool) + dst) = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int chunks_per_row = a.row_bytes / 16;
  const long long total = 1LL * a.num_seqs * a.num_kv_heads * chunks_per_row;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = unsigned((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(kThreads), 0, stream, a, chunks_per_row,
                     int(total));
  return hipGetLastError();
}

}  // namespace pkv
