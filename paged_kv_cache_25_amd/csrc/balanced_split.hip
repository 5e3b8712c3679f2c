// Balanced split of a batch's split-KV work, for gfx950.
//
// A fixed partition size gives long sequences many full partitions and short
// ones a single partial one, and the kernel waits for its longest workgroup.
// Here each sequence b with u_b units of work (pairs of blocks for the MLA
// kernel) gets n_b = max(1, ceil(u_b / t)) chunks, t being the smallest chunk
// size for which the batch needs at most R = max(budget, num_seqs) chunks
// (the budget is the number of workgroups that run at once); the kernel that
// follows splits u_b evenly over the n_b chunks.  The output is the exclusive
// prefix sum chunk_first[0..num_seqs] of n_b: sequence b owns chunk slots
// chunk_first[b] .. chunk_first[b+1]-1 (and, when asked, slot_info gives each
// slot its sequence and units directly).  This is scheduling only: the split
// does not change what is computed, only how partial results are grouped
// (the log-sum-exp merge combines any split of the tokens).
//
// One wave: the bisection over t needs a sum over the batch per step, and
// wave reductions need no barriers (the chunk count is non-increasing in t
// and equals num_seqs <= R at t = max u_b).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kCached = 8192;          // units kept in LDS (longer batches re-read them)

__device__ __forceinline__ int units_of(const SplitArgs& a, int b) {
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.cap_tokens ? a.cap_tokens : ctx);
  return (ctx + a.unit_tokens - 1) / a.unit_tokens;
}

__global__ __launch_bounds__(kWave) void balanced_split_kernel(SplitArgs a) {
  __shared__ int s_units[kCached];
  const int l = threadIdx.x;
  const bool cached = a.num_seqs <= kCached;
  auto units = [&](int b) { return cached ? s_units[b] : units_of(a, b); };

  int mx = 0;
  long long total = 0;
  for (int b = l; b < a.num_seqs; b += kWave) {
    const int u = units_of(a, b);
    if (cached) s_units[b] = u;
    mx = max(mx, u);
    total += u;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    total += __shfl_xor(total, o);
  }

  // count(t) = sum over b of max(1, ceil(u_b / t)) lies in [total / t,
  // total / t + B]: t < total / R needs too many chunks, and
  // t >= total / (R - B) never does, which brackets the bisection.  Each
  // lane's share is capped at 2^24, so the 32-bit wave sum cannot overflow
  // (the budget is far below the cap).
  const long long budget = a.budget > a.num_seqs ? a.budget : a.num_seqs;
  auto chunks = [&](int size) {
    long long c = 0;
    for (int b = l; b < a.num_seqs; b += kWave) {
      const int u = units(b);
      c += u <= size ? 1 : (u + size - 1) / size;
    }
    int ci = c < (1 << 24) ? int(c) : (1 << 24);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) ci += __shfl_xor(ci, o);
    return ci;
  };
  const int top = mx > 1 ? mx : 1;                       // count(top) = num_seqs <= budget
  long long lo_l = (total + budget - 1) / budget;
  long long hi_l = budget > a.num_seqs ? (total + (budget - a.num_seqs) - 1) / (budget - a.num_seqs)
                                       : top;
  int lo = int(lo_l < 1 ? 1 : (lo_l > top ? top : lo_l));
  int hi = int(hi_l < lo ? lo : (hi_l > top ? top : hi_l));
  while (lo < hi) {                                      // uniform: every lane sees the same sum
    const int mid = lo + (hi - lo) / 2;
    if (chunks(mid) <= budget) hi = mid; else lo = mid + 1;
  }
  const int size = lo;

  // Exclusive prefix sums of n_b, 64 sequences at a time.
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kWave) {
    const int b = base + l;
    const int u = b < a.num_seqs ? units(b) : 0;
    const int n = b < a.num_seqs ? (u <= size ? 1 : (u + size - 1) / size) : 0;
    int x = n;                                           // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (l >= o) x += y;
    }
    if (b < a.num_seqs) {
      const int first = carry + x - n;
      a.chunk_first[b] = first;
      if (a.slot_info) {
        // Chunk k covers units [floor(k u / n), floor((k+1) u / n)).  With
        // u = q n + r that bound is k q + floor(k r / n); k r mod n grows by
        // r < n per chunk, so one compare keeps the floor exact (no division
        // per chunk).
        const int q = u / n, r = u - q * n;
        int lo = 0, frac = 0;
        for (int k = 0; k < n; ++k) {
          frac += r;
          const int carry_unit = frac >= n ? 1 : 0;
          frac -= carry_unit * n;
          const int hi = lo + q + carry_unit;
          a.slot_info[first + k] = make_int4(b, lo, hi, n);
          lo = hi;
        }
      }
    }
    carry += __shfl(x, kWave - 1);
  }
  if (l == 0) a.chunk_first[a.num_seqs] = carry;
  if (a.slot_info)
    for (int slot = carry + l; slot < a.num_slots; slot += kWave) a.slot_info[slot] = make_int4(-1, 0, 0, 0);
}

}  // namespace

hipError_t launch_balanced_split(const SplitArgs& a, hipStream_t stream) {
  if (a.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(balanced_split_kernel, dim3(1), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
