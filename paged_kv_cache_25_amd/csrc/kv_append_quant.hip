// Append with quantisation into an fp8 (OCP e4m3fn) paged cache, for gfx950.
//
// The new K/V rows arrive in bf16 or float32 and are stored as e4m3 codes of
// their (block, KV head) slice, whose float32 scale s gives the real value
// code * s.  An fp8 cache halves the bytes of a bf16 one (KV-cache post, "The
// KV cache is big": fewer bytes per number; serving lesson, "Smaller caches:
// GQA, MQA, MLA and quantized caches").  Two scale policies:
//   fixed        - the slice keeps the scale it was given at allocation;
//   running amax - the scale grows to max(old, amax(new rows) / 448); when it
//                  grows, the slice's earlier rows are requantised to it.  A
//                  block whose first new row is at slot 0 has no earlier rows
//                  and its stale scale is ignored.
// A value x becomes encode(f32(x / s)), encode rounding to nearest with ties
// to even and saturating at 448 (written from the format below).
//
// One workgroup per (sequence, KV head); wave 0 does K, wave 1 V.  Each wave
// walks the blocks its sequence's new rows land in, in order.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr float kE4m3Max = 448.0f;

// float -> e4m3fn code: round to nearest, ties to even, saturate at +-448,
// NaN -> 0x7F.  e4m3fn: exponent bias 7, 3 mantissa bits, subnormals m/8 *
// 2^-6, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7Fu;                   // NaN
  if (a >= 0x43e00000u) return sign | 0x7Eu;           // |x| >= 448 (and inf)
  const int e = int(a >> 23) - 127;                    // float32 exponent
  if (e < -6) {
    // below the smallest normal 2^-6: multiples of 2^-9; 8 of them is 2^-6,
    // whose code is 0x08, so the count is the code.  x * 512 is exact.
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);   // ties to even
    return sign | uint32_t(q);
  }
  uint32_t m = (a >> 20) & 7u;                         // top 3 mantissa bits
  const uint32_t rest = a & 0xfffffu;                  // the 20 bits rounded away
  uint32_t ef = uint32_t(e + 7);                       // 1 .. 15
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) {
    if (++m == 8u) { m = 0; ++ef; }
  }
  const uint32_t code = (ef << 3) | m;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  return f32_to_e4m3_sat(a) | (f32_to_e4m3_sat(b) << 8) | (f32_to_e4m3_sat(c) << 16) |
         (f32_to_e4m3_sat(d) << 24);
}

// Four consecutive new-row values of row r, KV head h, starting at dim 4w.
template <bool kBf16>
__device__ __forceinline__ void load4(const void* base, size_t elem, float (&x)[4]) {
  if constexpr (kBf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + elem);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(2 * kWave) void kv_append_quant_kernel(QuantAppendArgs a) {
  const int b = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x % a.num_kv_heads;
  const int which = threadIdx.x / kWave;               // 0: K, 1: V
  const int lane = threadIdx.x % kWave;
  uint8_t* pool = static_cast<uint8_t*>(which ? a.v_pool : a.k_pool);
  float* scales = which ? a.v_scales : a.k_scales;
  const void* fresh = which ? a.v_new : a.k_new;

  const int ctx = a.context_lens[b];
  if (ctx <= 0 || ctx > a.max_blocks_per_seq * kBlockSize) return;
  int row0 = b, t = 1;
  if (a.q_start) {
    row0 = a.q_start[b];
    t = a.q_start[b + 1] - row0;
  }
  if (t <= 0) return;
  // Row row0 + j goes to position ctx - t + j; negative positions are skipped.
  const int first_pos = ctx - t > 0 ? ctx - t : 0;
  const int last_pos = ctx - 1;
  const int D = a.head_dim;
  const int W = D / 4;                                 // 4-code words per row
  const size_t slice_bytes = size_t(kBlockSize) * D;

  for (int blk = first_pos / kBlockSize; blk <= last_pos / kBlockSize; ++blk) {
    const int lo = blk == first_pos / kBlockSize ? first_pos % kBlockSize : 0;
    const int hi = blk == last_pos / kBlockSize ? last_pos % kBlockSize : kBlockSize - 1;
    const int phys = a.block_tables[size_t(b) * a.max_blocks_per_seq + blk];
    if (unsigned(phys) >= unsigned(a.num_blocks)) continue;
    uint8_t* slice = pool + (size_t(phys) * a.num_kv_heads + h) * slice_bytes;
    float* sp = scales + size_t(phys) * a.num_kv_heads + h;
    const int n_new = hi - lo + 1;
    // new row of slot s: row0 + (blk * 16 + s) - (ctx - t)
    const int row_of_lo = row0 + blk * kBlockSize + lo - (ctx - t);

    float s = *sp;
    if (a.mode == 1) {
      float amax = 0.0f;
      for (int i = lane; i < n_new * W; i += kWave) {
        float x[4];
        load4<kBf16>(fresh, (size_t(row_of_lo + i / W) * a.num_kv_heads + h) * D + 4 * (i % W), x);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
      }
      amax = wave_max(amax);
      const float cand = amax / kE4m3Max;
      const float old = lo > 0 ? s : 0.0f;
      s = fmaxf(old, cand);
      if (s > old && lo > 0) {
        // requantise the slice's earlier rows (slots 0 .. lo-1) to the new scale
        uint32_t* words = reinterpret_cast<uint32_t*>(slice);
        for (int i = lane; i < lo * W; i += kWave) {
          float c0, c1, c2, c3;
          fp8x4_to_f32(words[i], c0, c1, c2, c3);
          words[i] = pack4((c0 * old) / s, (c1 * old) / s, (c2 * old) / s, (c3 * old) / s);
        }
      }
      if (lane == 0) *sp = s;
    }
    uint32_t* out = reinterpret_cast<uint32_t*>(slice + size_t(lo) * D);
    const bool zero = a.mode == 1 && s == 0.0f;        // every value so far is 0
    for (int i = lane; i < n_new * W; i += kWave) {
      float x[4];
      load4<kBf16>(fresh, (size_t(row_of_lo + i / W) * a.num_kv_heads + h) * D + 4 * (i % W), x);
      out[i] = zero ? 0u : pack4(x[0] / s, x[1] / s, x[2] / s, x[3] / s);
    }
  }
}

}  // namespace

hipError_t launch_kv_append_quant(const QuantAppendArgs& a, hipStream_t stream) {
  const size_t grid = size_t(a.num_seqs) * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (a.new_bf16)
    hipLaunchKernelGGL(kv_append_quant_kernel<true>, dim3(unsigned(grid)), dim3(2 * kWave), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(kv_append_quant_kernel<false>, dim3(unsigned(grid)), dim3(2 * kWave), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace pkv
