// KV append for gfx950: scatter each sequence's new K and V rows into their
// slots of the paged cache.  With one new token per sequence the row goes to
// position ctx - 1; with t new tokens, row j goes to position ctx - t + j.  A
// bitwise copy, 16 bytes per thread, so the result is exact for every storage
// format.
//   KV-cache post (xuewyang.github.io/posts/kv), "A toy vLLM" (write_kv: the
//   block-table lookup pos // BLOCK and the slot pos % BLOCK);
//   brunomaga inference post, "PagedAttention..." (PagedKVCache.append);
//   4yush post, "Adding the cache to GPT-2" (several new tokens take the
//   positions after the cached ones, in order).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// Thread t copies chunk c of row (r, h) of K and of V; chunks are 16 bytes.
// Row r is new token r - q_start[b] of the sequence b that holds it (r = b
// when every sequence has one new token).
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a, int chunks_per_row,
                                                             int total) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int c = t % chunks_per_row;
  const int rh = t / chunks_per_row;
  const int h = rh % a.num_kv_heads;
  const int r = rh / a.num_kv_heads;
  int b = r, j = 0, n_new = 1;
  if (a.q_start) {
    // last b with q_start[b] <= r (q_start is non-decreasing, q_start[0] = 0)
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.q_start[mid] <= r) lo = mid; else hi = mid - 1;
    }
    b = lo;
    j = r - a.q_start[b];
    n_new = a.q_start[b + 1] - a.q_start[b];
    if (j >= n_new) return;                 // r past the last row (q_start[B] < rows)
  }
  const int ctx = a.context_lens[b];
  if (ctx <= 0 || ctx > a.max_blocks_per_seq * kBlockSize) return;
  const int pos = ctx - n_new + j;
  if (pos < 0) return;
  const int phys = a.block_tables[size_t(b) * a.max_blocks_per_seq + pos / kBlockSize];
  if (unsigned(phys) >= unsigned(a.num_blocks)) return;
  const size_t dst = ((size_t(phys) * a.num_kv_heads + h) * kBlockSize + pos % kBlockSize) *
                         size_t(a.row_bytes) + size_t(c) * 16;
  const size_t src = (size_t(r) * a.num_kv_heads + h) * size_t(a.row_bytes) + size_t(c) * 16;
  const uint4 kv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.k_new) + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.v_new) + src);
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_pool) + dst) = kv;
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_pool) + dst) = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int chunks_per_row = a.row_bytes / 16;
  const long long rows = a.q_start ? a.num_rows : a.num_seqs;
  if (a.q_start && a.num_seqs == 0) return hipSuccess;
  const long long total = rows * a.num_kv_heads * chunks_per_row;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = unsigned((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(kThreads), 0, stream, a, chunks_per_row,
                     int(total));
  return hipGetLastError();
}

}  // namespace pkv
