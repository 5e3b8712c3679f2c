// Split-KV paged decode attention on the matrix cores (gfx950), for bf16
// queries over a bf16 cache with query-head groups of 2..16 sharing a KV head.
//
// Same work split as the vector kernel: one 64-lane workgroup per (sequence,
// KV head, tile of up to 16 query heads, partition) walks the partition's
// block-table entries and reads each physical (block, KV head) slice
// [16 tokens x D] once from HBM for every query head of its group.  The
// quantity is the one the brunomaga inference post's paged_decode_attention
// defines; blocks are merged with the online-softmax update (learn.mohebi.ai
// serving lesson, "PagedAttention").
//
// Per 16-token block:
//   S^T[16 tok x 16 heads] = K[16 x D] . Q^T      D/32 x mfma_f32_16x16x32_bf16
//   online softmax on S^T in fp32 (log2 units; lazily raised maxima)
//   O[16 heads x D] += P[16 x 16 tok] . V[16 x D]  D/16 x mfma_f32_16x16x16_bf16
// The accumulator layout of the first product (lane l holds tokens 4*(l/16)+i
// of head l%16) is exactly the A-operand layout the second needs, so P never
// moves between lanes.  Unused head rows (group < 16) compute on zero queries
// and are not written.  P is rounded to bf16 for the second product; scores,
// weights, sums and O stay fp32.
//
// Loads (16 bytes per lane, straight into registers):
//   K: lane l reads token l%16, bytes 64j + 16*(l/16) of its row for slab j:
//      64 contiguous bytes per token per load.
//   V: lane l reads rows 4*(l/16)+i, bytes 16*(l%16): each load covers four
//      whole rows.  The B operand of tile e (dims 8c + e, c = l%16) is two
//      v_perm_b32 of the four rows' words.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kRescaleThreshold = 8.0f;   // log2 units: weights <= 2^8
constexpr int kHeadTile = 16;

// Build-time tuning: blocks held in registers per wave (DEPTH-1 in flight
// while one is computed) and the waves per SIMD the register budget targets.
// Measured on the batch-64 Llama-3-8B layer: depth 2 at 3 waves/SIMD beats
// depth 3 or 4 at 2 waves/SIMD, and 4 waves/SIMD spills.
#ifndef PKV_MFMA_DEPTH
#define PKV_MFMA_DEPTH 2
#endif
#ifndef PKV_MFMA_WAVES_PER_EU
#define PKV_MFMA_WAVES_PER_EU 3
#endif
constexpr int kDepth = PKV_MFMA_DEPTH;

template <int D>
struct MfmaTile {
  static constexpr int kSlabs = D / 32;          // QK products per block
  static constexpr int kTiles = D / 16;          // PV products per block
  static constexpr int kRowBytes = D * 2;
  static constexpr int kSliceBytes = 16 * kRowBytes;
  static constexpr int kVChunkBytes = D / 8;     // bytes of one row a lane reads for V (16 or 8)
  static constexpr int kVWords = kVChunkBytes / 4;
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {   // (a.lo, b.lo)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {   // (a.hi, b.hi)
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D>
struct BlockRegs {
  uint4 k[MfmaTile<D>::kSlabs];                       // A operands of QK
  uint32_t v[4][MfmaTile<D>::kVWords];                // rows 4r+i, this lane's bytes
};

template <int D, bool kNT>
__device__ __forceinline__ void load_block(BlockRegs<D>& br, const char* kslice,
                                           const char* vslice, int lane) {
  using T = MfmaTile<D>;
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int j = 0; j < T::kSlabs; ++j)
    br.k[j] = load_streamed<uint4, kNT>(kslice + c * T::kRowBytes + 64 * j + 16 * r);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* p = vslice + (4 * r + i) * T::kRowBytes + T::kVChunkBytes * c;
    if constexpr (T::kVWords == 4) {
      const uint4 w = load_streamed<uint4, kNT>(p);
      br.v[i][0] = w.x; br.v[i][1] = w.y; br.v[i][2] = w.z; br.v[i][3] = w.w;
    } else {
      const uint2 w = load_streamed<uint2, kNT>(p);
      br.v[i][0] = w.x; br.v[i][1] = w.y;
    }
  }
}

// The fused append, for the block holding a sequence's new token (row t_new):
// the lanes that own that row replace it with the new K/V row, then store it
// into its pool slot.  Static register indexes only.
template <int D>
__device__ __forceinline__ void take_new_row(BlockRegs<D>& br, const char* knew, const char* vnew,
                                             int t_new, int lane) {
  using T = MfmaTile<D>;
  const int r = lane >> 4, c = lane & 15;
  if (c == t_new) {
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j) br.k[j] = *reinterpret_cast<const uint4*>(knew + 64 * j + 16 * r);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * r + i != t_new) continue;
    const char* p = vnew + T::kVChunkBytes * c;
    if constexpr (T::kVWords == 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(p);
      br.v[i][0] = w.x; br.v[i][1] = w.y; br.v[i][2] = w.z; br.v[i][3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      br.v[i][0] = w.x; br.v[i][1] = w.y;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_new_row(const BlockRegs<D>& br, char* kslice, char* vslice,
                                              int t_new, int lane) {
  using T = MfmaTile<D>;
  const int r = lane >> 4, c = lane & 15;
  if (c == t_new) {
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j)
      *reinterpret_cast<uint4*>(kslice + c * T::kRowBytes + 64 * j + 16 * r) = br.k[j];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {                  // static register index: no scratch copy
    if (4 * r + i != t_new) continue;
    char* p = vslice + t_new * T::kRowBytes + T::kVChunkBytes * c;
    if constexpr (T::kVWords == 4)
      *reinterpret_cast<uint4*>(p) = make_uint4(br.v[i][0], br.v[i][1], br.v[i][2], br.v[i][3]);
    else
      *reinterpret_cast<uint2*>(p) = make_uint2(br.v[i][0], br.v[i][1]);
  }
}

// V rows past `valid` hold poison: zero them (their weights are 0, and 0 * NaN
// would not be).
template <int D>
__device__ __forceinline__ void zero_v_tail(BlockRegs<D>& br, int valid, int lane) {
  const int r = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = 4 * r + i < valid;
#pragma unroll
    for (int w = 0; w < MfmaTile<D>::kVWords; ++w) br.v[i][w] = ok ? br.v[i][w] : 0u;
  }
}

template <int D>
struct MfmaDecode {
  using T = MfmaTile<D>;
  bf16x8 q[T::kSlabs];          // B operands of QK (head l%16)
  f32x4 o[T::kTiles];           // O rows 4r+i, dims 8c+e (D=128) / 4c+e (D=64)
  float m, l;                   // per head l%16 (log2 units)

  // valid: tokens of the block inside the context (rows past it hold poison and
  // are zeroed in V); vis: tokens of the block this lane's column may see
  // (uniform need_mask says whether any column sees fewer than 16).
  // With one new token vis == valid and need_mask == (valid < 16): one branch.
  // kZeroV: zero V past `valid` here (off when several tiles share the block
  // and it was zeroed once before them).
  template <bool kMulti, bool kZeroV = true>
  __device__ __forceinline__ void block(BlockRegs<D>& br, int valid, int vis, bool need_mask,
                                        float k_mul, int lane) {
    const int r = lane >> 4;
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, br.k[j]), q[j], s,
                                                  0, 0, 0);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s[i] * k_mul;
    if constexpr (kMulti) {
      if (need_mask) {                      // wave-uniform: the sequence's last block(s)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = 4 * r + i < vis ? sc[i] : -INFINITY;
      }
    }
    if (kZeroV && valid < 16) {             // wave-uniform: the sequence's last block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * r + i < valid;
        if constexpr (!kMulti) sc[i] = ok ? sc[i] : -INFINITY;
#pragma unroll
        for (int w = 0; w < T::kVWords; ++w) br.v[i][w] = ok ? br.v[i][w] : 0u;
      }
    }
    const float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__any(bm > m + kRescaleThreshold)) {     // rare: raise the reference maxima
      float hm = fmaxf(bm, __shfl_xor(bm, 16));
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      const float mn = fmaxf(m, hm);
      // a column with nothing visible yet keeps m = -inf (and alpha = 1)
      const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      m = mn;
      float a_row[4];                        // alpha of head 4r+i, held by lane 4r+i
#pragma unroll
      for (int i = 0; i < 4; ++i) a_row[i] = __shfl(alpha, 4 * r + i);
#pragma unroll
      for (int t = 0; t < T::kTiles; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] *= a_row[i];
    }
    float p[4];
    const float m_eff = m == -INFINITY ? 0.0f : m;     // all scores -inf: weights 0, not NaN
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_eff);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    const bf16x4 pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
#pragma unroll
    for (int w = 0; w < T::kVWords; ++w) {
      // tile 2w: low halves (dim 2w of this lane's chunk), tile 2w+1: high halves
      const uint32_t b0lo = lo_pair(br.v[0][w], br.v[1][w]), b1lo = lo_pair(br.v[2][w], br.v[3][w]);
      const uint32_t b0hi = hi_pair(br.v[0][w], br.v[1][w]), b1hi = hi_pair(br.v[2][w], br.v[3][w]);
      const uint2 blo = {b0lo, b1lo}, bhi = {b0hi, b1hi};
      o[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(bf16x4, blo),
                                                           o[2 * w], 0, 0, 0);
      o[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          pa, __builtin_bit_cast(bf16x4, bhi), o[2 * w + 1], 0, 0, 0);
    }
  }
};

// Partial row of column 4r+i (this lane's dims) as bf16, round to nearest
// even: the balanced split with several new tokens keeps its partial rows in
// bf16, half the bytes the decode kernel writes and the merge reads.
template <int D>
__device__ __forceinline__ void store_bf16_partial(float* part_o, size_t prow, int c,
                                                   const MfmaDecode<D>& dt, int i, float inv) {
  constexpr int kDimsPerLane = D / 16;
  uint16_t* op = reinterpret_cast<uint16_t*>(part_o) + prow * D + kDimsPerLane * c;
  uint32_t packed[kDimsPerLane / 2];
#pragma unroll
  for (int e = 0; e < kDimsPerLane; e += 2)
    packed[e / 2] = uint32_t(f32_to_bf16_rne(dt.o[e][i] * inv)) |
                    (uint32_t(f32_to_bf16_rne(dt.o[e + 1][i] * inv)) << 16);
  if constexpr (kDimsPerLane == 8)
    *reinterpret_cast<uint4*>(op) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  else
    *reinterpret_cast<uint2*>(op) = make_uint2(packed[0], packed[1]);
}

// Three waves per SIMD: about 150 VGPRs for head dim 128 with two blocks in registers.
// kMulti: several new tokens per sequence (per-column visibility); otherwise
// one new token, whose column sees the whole context.  kNT: K/V loads carry the
// nontemporal hint; off when several workgroups read the same blocks, so the
// later ones find them in L2.  NT: column tiles of 16 per wave, sharing each
// block's K/V registers (2 for more than 16 columns: two waves per SIMD).
template <int D, bool kMulti, bool kNT, int NT>
__global__ __launch_bounds__(kWave)
__attribute__((amdgpu_waves_per_eu(NT == 1 ? PKV_MFMA_WAVES_PER_EU : 2)))
void paged_decode_mfma_kernel(DecodeArgs a) {
  using T = MfmaTile<D>;
  // blockIdx.x -> (column chunk, unit = (kv head, sequence, partition)), or
  // (column chunk, kv head, chunk slot) for a balanced split.
  DecodeItem it;
  if (!decode_item(a, it)) return;
  const int chunk = it.chunk, h = it.h, b = it.b, part = it.part;

  const int lane = threadIdx.x;
  const int r = lane >> 4, c = lane & 15;

  const int32_t* table = a.block_tables + size_t(b) * a.max_blocks_per_seq;
  const int blk_begin = it.blk_begin;
  // The first 64 table entries of the partition are fetched together with the
  // context length (both in bounds of the table row), so the first K/V loads
  // wait for one memory round trip, not two.
  const int first_n = a.max_blocks_per_seq - blk_begin;
  int id0 = (lane < first_n && lane < it.blk_end - blk_begin) ? table[blk_begin + lane] : -1;

  const int raw_ctx = a.context_lens[b];
  int ctx = raw_ctx < 0 ? 0 : raw_ctx;
  const int cap = a.max_blocks_per_seq * kBlockSize;
  ctx = ctx > cap ? cap : ctx;
  const int n_blk_seq = (ctx + kBlockSize - 1) / kBlockSize;
  int blk_end = it.blk_end < n_blk_seq ? it.blk_end : n_blk_seq;
  // Fused append: the block of position ctx-1 takes its new row from k_new/v_new
  // (a sequence outside 1 <= ctx <= capacity appends nothing, as pkv_kv_append).
  const int append_blk = (a.k_new && raw_ctx >= 1 && raw_ctx <= cap) ? (raw_ctx - 1) / kBlockSize : -1;
  const int t_new = (raw_ctx - 1) % kBlockSize;
  // Column c of this tile: new token n / group, head n % group, n = chunk*16 + c.
  Columns cols;
  cols.group = a.group;
  cols.num_q_heads = a.num_q_heads;
  cols.kv_head = h;
  if constexpr (kMulti) {
    cols.row0 = a.q_start[b];
    cols.t = a.q_start[b + 1] - cols.row0;
  } else {
    cols.row0 = b;
    cols.t = 1;
  }
  // Row of column n in q/out/partials; one new token needs no division.
  auto row_of = [&](int n) -> size_t {
    if constexpr (kMulti) return cols.row(n);
    return size_t(b) * a.num_q_heads + size_t(h) * a.group + n;
  };
  const int n0 = chunk * kHeadTile * NT;
  if (!cols.valid(n0)) return;                        // no column of this workgroup exists

  // A sequence whose blocks fit one partition (or chunk) is finished here:
  // write the final output instead of a partial (the merge skips it).
  const bool final_out =
      a.write_final ||
      (a.final_single && (a.balanced() ? it.n_parts == 1 : n_blk_seq <= a.blocks_per_partition));
  if (blk_begin >= blk_end && !(a.write_final && part == 0) &&
      !(a.balanced() && final_out)) {                  // partition past the end, or an empty chunk
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if ((a.mark_empty || a.balanced()) && lane < kHeadTile && cols.valid(n0 + 16 * nt + c) &&
          partial_row_ok(a, row_of(n0 + 16 * nt + c), cols.row0))
        a.part_lse[partial_row(a, it, row_of(n0 + 16 * nt + c), cols.row0)] = -INFINITY;
    return;
  }
  int my_vis[NT];                                     // tokens my column of tile nt attends to
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + c;
    my_vis[nt] = kMulti && cols.valid(n) ? cols.visible(n, ctx) : ctx;
  }
  const int min_vis = kMulti ? cols.visible(n0, ctx) : ctx;     // fewest: the first column

  MfmaDecode<D> dec[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + c;
    const bool ok = cols.valid(n);
    const char* qrow = reinterpret_cast<const char*>(a.q) + (ok ? row_of(n) : 0) * T::kRowBytes;
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(qrow + 64 * j + 16 * r) : make_uint4(0, 0, 0, 0);
      dec[nt].q[j] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int t = 0; t < T::kTiles; ++t) dec[nt].o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    dec[nt].m = -INFINITY;
    dec[nt].l = 0.0f;
  }

  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const size_t head_off = size_t(h) * T::kSliceBytes;
  const size_t block_stride = size_t(a.num_kv_heads) * T::kSliceBytes;
  const float k_mul = a.scale_log2;

  BlockRegs<D> buf[kDepth];
  for (int seg = blk_begin; seg < blk_end; seg += kWave) {
    const int n = (blk_end - seg) < kWave ? (blk_end - seg) : kWave;
    int my_id = seg == blk_begin ? id0 : (lane < n ? table[seg + lane] : -1);
    my_id = lane < n ? my_id : -1;
    const bool my_ok = unsigned(my_id) < unsigned(a.num_blocks);
    my_id = my_ok ? my_id : 0;
    const uint64_t ok_mask = __ballot(my_ok);

    auto fetch = [&](BlockRegs<D>& br, int k) {
      const int phys = __builtin_amdgcn_readlane(my_id, k);
      const size_t off = size_t(phys) * block_stride + head_off;
      load_block<D, kNT>(br, kbase + off, vbase + off, lane);
    };
    auto consume = [&](BlockRegs<D>& br, int k) {
      const int first = (seg + k) * kBlockSize;
      int valid = ctx - first;
      valid = valid < kBlockSize ? valid : kBlockSize;
      const bool ok = (ok_mask >> k) & 1;
      valid = ok ? valid : 0;
      bool need_mask = valid < kBlockSize;
      if constexpr (kMulti) need_mask = !ok || first + kBlockSize > min_vis;
      if (seg + k == append_blk && ok) {
        const size_t nrow = (size_t(b) * a.num_kv_heads + h) * T::kRowBytes;
        take_new_row<D>(br, reinterpret_cast<const char*>(a.k_new) + nrow,
                        reinterpret_cast<const char*>(a.v_new) + nrow, t_new, lane);
        if (chunk == 0) {                                // one writer per (sequence, KV head)
          const int phys = __builtin_amdgcn_readlane(my_id, k);
          const size_t off = size_t(phys) * block_stride + head_off;
          store_new_row<D>(br, reinterpret_cast<char*>(a.k_pool_w) + off,
                           reinterpret_cast<char*>(a.v_pool_w) + off, t_new, lane);
        }
      }
      if constexpr (NT == 1) {
        const int vis = kMulti ? (ok ? my_vis[0] - first : 0) : valid;
        dec[0].template block<kMulti>(br, valid, vis, need_mask, k_mul, lane);
      } else {
        if (valid < kBlockSize) zero_v_tail<D>(br, valid, lane);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dec[nt].template block<kMulti, false>(br, valid, ok ? my_vis[nt] - first : 0, need_mask,
                                                k_mul, lane);
      }
    };

    // Ring of kDepth register buffers: block k+kDepth-1 is requested before
    // block k is consumed.
#pragma unroll
    for (int d = 0; d + 1 < kDepth; ++d)
      if (d < n) fetch(buf[d], d);
    for (int k = 0; k < n; k += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int kk = k + d;
        if (kk + kDepth - 1 < n) fetch(buf[(d + kDepth - 1) % kDepth], kk + kDepth - 1);
        if (kk < n) consume(buf[d], kk);
      }
    }
  }

  constexpr int kDimsPerLane = D / 16;       // dims dpl*c .. dpl*c + dpl-1 of each head row
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const MfmaDecode<D>& dt = dec[nt];
    // Denominator of column l%16 over the 4 lane rows; then that of column 4r+i.
    float lt = dt.l + __shfl_xor(dt.l, 16);
    lt += __shfl_xor(lt, 32);
    float l_row[4], m_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l_row[i] = __shfl(lt, 4 * r + i);
      m_row[i] = __shfl(dt.m, 4 * r + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 16 * nt + 4 * r + i;          // output row 4r+i of tile nt is column n
      if (!cols.valid(n)) continue;
      const size_t qrow = row_of(n);
      const bool empty = l_row[i] == 0.0f;
      const float inv = empty ? 0.0f : 1.0f / l_row[i];
      if (final_out) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + qrow * D + kDimsPerLane * c;
        uint32_t packed[kDimsPerLane / 2];
#pragma unroll
        for (int e = 0; e < kDimsPerLane; e += 2)
          packed[e / 2] = uint32_t(f32_to_bf16_rne(dt.o[e][i] * inv)) |
                          (uint32_t(f32_to_bf16_rne(dt.o[e + 1][i] * inv)) << 16);
        if constexpr (kDimsPerLane == 8)
          *reinterpret_cast<uint4*>(orow) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        else
          *reinterpret_cast<uint2*>(orow) = make_uint2(packed[0], packed[1]);
      } else {
        if (!partial_row_ok(a, qrow, cols.row0)) continue;
        const size_t prow = partial_row(a, it, qrow, cols.row0);
        if (kMulti && a.part_bf16) {                       // uniform
          store_bf16_partial<D>(a.part_o, prow, c, dt, i, inv);
        } else {
          float* op = a.part_o + prow * D + kDimsPerLane * c;
#pragma unroll
          for (int e = 0; e < kDimsPerLane; e += 4)
            *reinterpret_cast<float4*>(op + e) = make_float4(dt.o[e][i] * inv, dt.o[e + 1][i] * inv,
                                                             dt.o[e + 2][i] * inv, dt.o[e + 3][i] * inv);
        }
        if (c == 0)
          a.part_lse[prow] = empty ? -INFINITY : (m_row[i] + __builtin_amdgcn_logf(l_row[i])) * kLn2;
      }
    }
  }
}

// Several new tokens per sequence, head dim 128, four or more column tiles
// per KV head: one workgroup of W waves per unit (KV head, chunk slot or
// partition) covers W x NT column tiles, and the unit's blocks are read from
// HBM once, into LDS, for all of them (the kernel above gives each two-tile
// chunk its own workgroup, so every chunk loads every block).  Each wave
// loads its share of a block's K and V slices (8 KiB; 8 / W pieces of 1 KiB)
// into registers two blocks ahead of the one computed, writes it into one of
// two LDS stages, and after a barrier every wave reads the whole block's
// operands from LDS in the register layout of BlockRegs and runs
// MfmaDecode::block on its NT tiles.  Rows are stored with their 16-byte
// chunks rotated (chunk q of row r at position q ^ (r & 15)), so the K reads
// of 16 rows and the V reads of one row hit 16 distinct bank groups.  The
// block table of the unit goes to LDS first, up to kIdWindow entries at a
// time.  Measured at 16 new tokens on the batch-64 layer: 131 us against 166
// us for the kernel above; copying the blocks with direct-to-LDS loads
// instead, 145 us (the copies alone took 142 us at any ring depth), and
// three or four blocks in registers instead of two, 133 and 135 us.
constexpr int kIdWindow = 512;
#ifndef PKV_MULTI_LDS
#define PKV_MULTI_LDS 1
#endif

template <int NT, int W>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_lds_kernel(DecodeArgs a) {
  constexpr int D = 128;
  using T = MfmaTile<D>;
  constexpr int kStage = 2 * T::kSliceBytes;           // K slice then V slice: 8 KiB
  constexpr int kPieces = kStage / (16 * kWave);       // 1 KiB pieces of a block (8)
  constexpr int P = kPieces / W;                       // per wave
  static_assert(kPieces % W == 0, "pieces per wave");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[2 * kStage];
  __shared__ int32_t s_ids[kIdWindow];

  DecodeItem it;
  if (!decode_item(a, it)) return;                     // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r = lane >> 4, c = lane & 15;
  const int h = it.h, b = it.b, part = it.part;

  const int32_t* table = a.block_tables + size_t(b) * a.max_blocks_per_seq;
  const int blk_begin = it.blk_begin;
  const int raw_ctx = a.context_lens[b];
  int ctx = raw_ctx < 0 ? 0 : raw_ctx;
  const int cap = a.max_blocks_per_seq * kBlockSize;
  ctx = ctx > cap ? cap : ctx;
  const int n_blk_seq = (ctx + kBlockSize - 1) / kBlockSize;
  const int blk_end = it.blk_end < n_blk_seq ? it.blk_end : n_blk_seq;
  Columns cols;
  cols.group = a.group;
  cols.num_q_heads = a.num_q_heads;
  cols.kv_head = h;
  cols.row0 = a.q_start[b];
  cols.t = a.q_start[b + 1] - cols.row0;
  auto row_of = [&](int n) -> size_t { return cols.row(n); };
  const int n0 = (it.chunk * W + wave) * kHeadTile * NT;   // this wave's first column
  const bool has_cols = cols.valid(n0);                // uniform per wave

  const bool final_out =
      a.write_final ||
      (a.final_single && (a.balanced() ? it.n_parts == 1 : n_blk_seq <= a.blocks_per_partition));
  if (blk_begin >= blk_end && !(a.write_final && part == 0) &&
      !(a.balanced() && final_out)) {                  // uniform: nothing to attend
    if (has_cols) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if ((a.mark_empty || a.balanced()) && lane < kHeadTile && cols.valid(n0 + 16 * nt + c) &&
            partial_row_ok(a, row_of(n0 + 16 * nt + c), cols.row0))
          a.part_lse[partial_row(a, it, row_of(n0 + 16 * nt + c), cols.row0)] = -INFINITY;
    }
    return;
  }
  int my_vis[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + c;
    my_vis[nt] = cols.valid(n) ? cols.visible(n, ctx) : ctx;
  }
  const int min_vis = cols.visible(n0, ctx);

  MfmaDecode<D> dec[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + c;
    const bool ok = cols.valid(n);
    const char* qrow = reinterpret_cast<const char*>(a.q) + (ok ? row_of(n) : 0) * T::kRowBytes;
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(qrow + 64 * j + 16 * r) : make_uint4(0, 0, 0, 0);
      dec[nt].q[j] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int t = 0; t < T::kTiles; ++t) dec[nt].o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    dec[nt].m = -INFINITY;
    dec[nt].l = 0.0f;
  }
  // The queries are waited for here, before any copy is in flight: a wait
  // for them inside the block loop would also wait for every copy.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j) asm volatile("" ::"v"(dec[nt].q[j]));

  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const size_t head_off = size_t(h) * T::kSliceBytes;
  const size_t block_stride = size_t(a.num_kv_heads) * T::kSliceBytes;
  const float k_mul = a.scale_log2;
  // Operands of the block in stage st, in BlockRegs' layout.
  auto read_block = [&](BlockRegs<D>& br, int st) {
    const uint8_t* kb = s_ring + st * kStage;
    const uint8_t* vb = kb + T::kSliceBytes;
#pragma unroll
    for (int j = 0; j < T::kSlabs; ++j)
      br.k[j] = *reinterpret_cast<const uint4*>(kb + c * T::kRowBytes + (((4 * j + r) ^ c) << 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * r + i;
      const uint4 w = *reinterpret_cast<const uint4*>(vb + row * T::kRowBytes + ((c ^ row) << 4));
      br.v[i][0] = w.x; br.v[i][1] = w.y; br.v[i][2] = w.z; br.v[i][3] = w.w;
    }
  };

  // Attends block k of the window from ring stage st.
  auto compute = [&](int win, int k, int st) {
    const int id = s_ids[k];
    const bool ok = unsigned(id) < unsigned(a.num_blocks);
    BlockRegs<D> br;
    read_block(br, st);
    const int first = (win + k) * kBlockSize;
    int valid = ctx - first;
    valid = valid < kBlockSize ? valid : kBlockSize;
    valid = ok ? valid : 0;
    const bool need_mask = !ok || first + kBlockSize > min_vis;
    if (valid < kBlockSize) zero_v_tail<D>(br, valid, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      dec[nt].template block<true, false>(br, valid, ok ? my_vis[nt] - first : 0, need_mask,
                                          k_mul, lane);
  };
  // The wave's pieces of block kb of the window: piece m (m = wave,
  // wave + W, ...) holds K rows 4m..4m+3 (m < 4) or V rows 4(m-4).. (m >= 4),
  // lane i the 16 bytes that go to position i & 15 of row 4m + (i >> 4),
  // i.e. chunk (i & 15) ^ row.  A bad table entry loads block 0 (its tokens
  // are masked).  Scheduling fences keep each block's loads together and in
  // program order, so the compiler counts the loads in flight exactly and
  // waits for one block, not both, before a store.
  auto load_regs = [&](uint4 (&rb)[P], int kb) {
    int phys = __builtin_amdgcn_readfirstlane(s_ids[kb]);
    phys = unsigned(phys) < unsigned(a.num_blocks) ? phys : 0;
    const size_t off = size_t(phys) * block_stride + head_off;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int m = wave + i * W;
      const int row = 4 * (m & 3) + r;
      rb[i] = load_streamed<uint4, true>((m < 4 ? kbase : vbase) + off + row * T::kRowBytes +
                                         ((c ^ row) << 4));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store_regs = [&](const uint4 (&rb)[P], int st) {
#pragma unroll
    for (int i = 0; i < P; ++i)
      *reinterpret_cast<uint4*>(s_ring + st * kStage + (wave + i * W) * 1024 + 16 * lane) = rb[i];
  };

  for (int win = blk_begin; win < blk_end; win += kIdWindow) {   // uniform
    const int wn = (blk_end - win) < kIdWindow ? (blk_end - win) : kIdWindow;
    for (int i = threadIdx.x; i < wn; i += W * kWave) s_ids[i] = table[win + i];
    __syncthreads();                                   // ids written; no copy in flight
    // Stages 0 and 1 take even and odd blocks; R = 2 blocks ahead of the one
    // computed are in flight in registers (rb[(k + 1) % R] holds block
    // k + 1 until it is stored, then loads block k + 1 + R).  The loads and
    // stores run unconditionally, past the window's end on its last block
    // again (an L2 hit, never computed), and the loop has one exit at the
    // bottom: with a conditional load or an early exit, the compiler could
    // not count the loads in flight on every path and would wait for all
    // of them before a store.
    constexpr int R = 2;
    const int last = wn - 1;
    uint4 rb[R][P];
#pragma unroll
    for (int u = 0; u < R; ++u) load_regs(rb[u], u < last ? u : last);
    store_regs(rb[0], 0);
    load_regs(rb[0], R < last ? R : last);
    for (int k0 = 0; k0 < wn; k0 += 2 * R) {
#pragma unroll
      for (int u = 0; u < 2 * R; ++u) {
        const int k = k0 + u;
        // Stage u % 2 holds block k for every wave; every read of the
        // other stage (block k - 1) is done.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        store_regs(rb[(u + 1) % R], (u + 1) % 2);
        load_regs(rb[(u + 1) % R], k + 1 + R < last ? k + 1 + R : last);
        if (has_cols && k < wn) compute(win, k, u % 2);
      }
    }
    __syncthreads();                                   // ring and ids free for the next window
  }
  if (!has_cols) return;

  constexpr int kDimsPerLane = D / 16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const MfmaDecode<D>& dt = dec[nt];
    float lt = dt.l + __shfl_xor(dt.l, 16);
    lt += __shfl_xor(lt, 32);
    float l_row[4], m_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l_row[i] = __shfl(lt, 4 * r + i);
      m_row[i] = __shfl(dt.m, 4 * r + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 16 * nt + 4 * r + i;
      if (!cols.valid(n)) continue;
      const size_t qrow = row_of(n);
      const bool empty = l_row[i] == 0.0f;
      const float inv = empty ? 0.0f : 1.0f / l_row[i];
      if (final_out) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + qrow * D + kDimsPerLane * c;
        uint32_t packed[kDimsPerLane / 2];
#pragma unroll
        for (int e = 0; e < kDimsPerLane; e += 2)
          packed[e / 2] = uint32_t(f32_to_bf16_rne(dt.o[e][i] * inv)) |
                          (uint32_t(f32_to_bf16_rne(dt.o[e + 1][i] * inv)) << 16);
        *reinterpret_cast<uint4*>(orow) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      } else {
        if (!partial_row_ok(a, qrow, cols.row0)) continue;
        const size_t prow = partial_row(a, it, qrow, cols.row0);
        if (a.part_bf16) {                       // uniform
          store_bf16_partial<D>(a.part_o, prow, c, dt, i, inv);
        } else {
          float* op = a.part_o + prow * D + kDimsPerLane * c;
#pragma unroll
          for (int e = 0; e < kDimsPerLane; e += 4)
            *reinterpret_cast<float4*>(op + e) = make_float4(dt.o[e][i] * inv, dt.o[e + 1][i] * inv,
                                                             dt.o[e + 2][i] * inv, dt.o[e + 3][i] * inv);
        }
        if (c == 0)
          a.part_lse[prow] = empty ? -INFINITY : (m_row[i] + __builtin_amdgcn_logf(l_row[i])) * kLn2;
      }
    }
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const size_t units = (a.balanced() ? size_t(1) : size_t(a.num_seqs)) * a.num_kv_heads * a.max_partitions;
  if (units == 0 || a.head_chunks == 0) return hipSuccess;
  if (units > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const size_t grid = decode_grid(units, a.head_chunks);
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const bool nt = a.head_chunks == 1 && PKV_NT_LOADS;
  const dim3 g{unsigned(grid)}, blk{unsigned(kWave)};
  if (a.q_start) {
    // Two or more two-tile chunks per unit at head dim 128: the LDS ring, one
    // workgroup of two waves per pair of chunks.
    if constexpr (D == 128) {
      if (PKV_MULTI_LDS && a.tiles_per_wave == 2 && a.head_chunks >= 2 && !a.k_new) {
        DecodeArgs b = a;
        b.head_chunks = (a.head_chunks + 1) / 2;
        const size_t g2 = decode_grid(units, b.head_chunks);
        if (g2 > 0x7fffffffu) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((paged_decode_lds_kernel<2, 2>), dim3(unsigned(g2)), dim3(2 * kWave), 0,
                           stream, b);
        return hipGetLastError();
      }
    }
    if (a.tiles_per_wave == 2) {
      if (nt) hipLaunchKernelGGL((paged_decode_mfma_kernel<D, true, true, 2>), g, blk, 0, stream, a);
      else hipLaunchKernelGGL((paged_decode_mfma_kernel<D, true, false, 2>), g, blk, 0, stream, a);
    } else {
      if (nt) hipLaunchKernelGGL((paged_decode_mfma_kernel<D, true, true, 1>), g, blk, 0, stream, a);
      else hipLaunchKernelGGL((paged_decode_mfma_kernel<D, true, false, 1>), g, blk, 0, stream, a);
    }
  } else {
    if (nt) hipLaunchKernelGGL((paged_decode_mfma_kernel<D, false, true, 1>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((paged_decode_mfma_kernel<D, false, false, 1>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int mfma_head_tile() { return kHeadTile; }

hipError_t launch_paged_decode_mfma(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace pkv
