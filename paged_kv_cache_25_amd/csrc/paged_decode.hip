// Split-KV paged decode attention for gfx950.
//
// One 64-lane workgroup per (sequence, KV head, head tile, partition).  It
// walks the partition's entries of the sequence's block table, streams each
// physical (block, KV head) slice [16 tokens x D] straight from HBM into
// registers with 16-byte loads (8 lanes read one token row: 128 contiguous
// bytes per lane group per load), and serves every query head of its GQA
// group from that one read.  Scores are 8-lane sums (DPP), the softmax is an
// fp32 online softmax in log2 units, and P.V accumulates in fp32.  It writes
// a normalised partial output and its natural-log LSE, or the final output
// when a sequence has a single partition.
//   brunomaga inference post, "PagedAttention: memory management for the KV
//   cache" (paged_decode_attention: the quantity computed);
//   learn.mohebi.ai serving lesson, "PagedAttention" (blocks read one at a
//   time, merged with the online-softmax update) and "Where it shows up"
//   (split-KV decoding).
//
// Lane layout inside a 16-token block: lane l belongs to token group
// tg = l / 8 and owns D/8 dims of tokens tg and tg + 8 (sub-lane s = l % 8
// owns 16-byte chunks s, s+8, ... of the row).  The D/8 dims of every lane are
// the same for K, V, q and the output, so no data moves between lanes except
// the 8-lane score sums and one cross-group reduction at the end.
//
// Online softmax: each wave keeps a per-head reference maximum m (log2 units)
// that is only raised when a score exceeds it by more than 8, so the
// accumulators are rescaled rarely; every weight is exp2(s - m) <= 256 and
// the final o = acc / l is exact up to rounding whatever m is.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kLanesPerToken = 8;
constexpr int kGroups = kWave / kLanesPerToken;        // 8 token groups per wave
constexpr int kTokPerLane = kBlockSize / kGroups;      // 2 tokens per lane per block
constexpr float kRescaleThreshold = 8.0f;              // log2 units: weights <= 2^8

template <int D, typename KV>
struct Tile {
  static constexpr int kDims = D / kLanesPerToken;            // dims per lane
  static constexpr int kBytes = kDims * KV::kBytes;           // bytes per lane per token
  static constexpr int kWords = kBytes / 4;
  static constexpr int kChunkBytes = kBytes < 16 ? kBytes : 16;
  static constexpr int kChunks = kBytes / kChunkBytes;
  static constexpr int kChunkWords = kChunkBytes / 4;
  static constexpr int kChunkDims = kChunkBytes / KV::kBytes;
  static constexpr int kRowBytes = D * KV::kBytes;
  static constexpr int kSliceBytes = kBlockSize * kRowBytes;  // one (block, head) slice
  static_assert(kBytes % 4 == 0 && kChunkBytes >= 8, "lane slice must be whole 8-byte chunks");
  // byte offset, within a row, of chunk c of sub-lane s
  __device__ static constexpr int chunk_off(int s, int c) {
    return (c * kLanesPerToken + s) * kChunkBytes;
  }
  // element index, within a row, of the k-th dim owned by sub-lane s
  __device__ static constexpr int dim(int s, int k) {
    return (k / kChunkDims * kLanesPerToken + s) * kChunkDims + k % kChunkDims;
  }
};

template <typename T> struct IsBF16 { static constexpr bool value = false; };
template <> struct IsBF16<BF16> { static constexpr bool value = true; };

// Load one lane's chunks of a row (kWords 32-bit words).
template <int D, typename KV, int NW>
__device__ __forceinline__ void load_row(uint32_t (&w)[NW], const char* row, int s) {
  using TL = Tile<D, KV>;
  static_assert(NW == TL::kWords, "word count");
#pragma unroll
  for (int c = 0; c < TL::kChunks; ++c) {
    const char* p = row + TL::chunk_off(s, c);
    if constexpr (TL::kChunkBytes == 16) {
      uint4 v = load_streamed<uint4>(p);
      w[c * 4 + 0] = v.x; w[c * 4 + 1] = v.y; w[c * 4 + 2] = v.z; w[c * 4 + 3] = v.w;
    } else {
      uint2 v = load_streamed<uint2>(p);
      w[c * 2 + 0] = v.x; w[c * 2 + 1] = v.y;
    }
  }
}

// Store one lane's chunks of a row (the inverse of load_row).
template <int D, typename KV, int NW>
__device__ __forceinline__ void store_row(const uint32_t (&w)[NW], char* row, int s) {
  using TL = Tile<D, KV>;
#pragma unroll
  for (int c = 0; c < TL::kChunks; ++c) {
    char* p = row + TL::chunk_off(s, c);
    if constexpr (TL::kChunkBytes == 16)
      *reinterpret_cast<uint4*>(p) = make_uint4(w[c * 4 + 0], w[c * 4 + 1], w[c * 4 + 2], w[c * 4 + 3]);
    else
      *reinterpret_cast<uint2*>(p) = make_uint2(w[c * 2 + 0], w[c * 2 + 1]);
  }
}

// Storage words of one lane's slice of a row -> kDims floats (in dim order k).
template <int D, typename KV, int NW, int ND>
__device__ __forceinline__ void to_float(const uint32_t (&w)[NW], float (&f)[ND]) {
  using TL = Tile<D, KV>;
  static_assert(NW == TL::kWords && ND == TL::kDims, "lane slice shape");
  if constexpr (KV::kBytes == 4) {
#pragma unroll
    for (int k = 0; k < ND; ++k) f[k] = __uint_as_float(w[k]);
  } else if constexpr (KV::kBytes == 2) {
#pragma unroll
    for (int k = 0; k < NW; ++k) { f[2 * k] = bf16_lo(w[k]); f[2 * k + 1] = bf16_hi(w[k]); }
  } else {
#pragma unroll
    for (int k = 0; k < NW; ++k) fp8x4_to_f32(w[k], f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
  }
}

template <typename QT>
__device__ __forceinline__ float load_q_elem(const char* row, int idx) {
  if constexpr (QT::kBytes == 4) {
    return reinterpret_cast<const float*>(row)[idx];
  } else {
    uint32_t h = reinterpret_cast<const uint16_t*>(row)[idx];
    return __uint_as_float(h << 16);
  }
}

template <int D, int G, typename QT, typename KV>
struct Decode {
  using TL = Tile<D, KV>;
  static constexpr int W = TL::kWords;
  static constexpr int KD = TL::kDims;
  static constexpr bool kDot2 = IsBF16<QT>::value && IsBF16<KV>::value;

  // Query registers: packed bf16 words for the dot2 path, floats otherwise.
  uint32_t qw[kDot2 ? G : 1][kDot2 ? W : 1];
  float qf[kDot2 ? 1 : G][kDot2 ? 1 : KD];
  float m[G], l[G], acc[G][KD];

  // Columns n0 .. n0+G-1 of the tile; a missing column gets a zero query.
  __device__ __forceinline__ void load_q(const char* q, const Columns& cols, int n0, int s) {
    constexpr size_t kQRowBytes = size_t(D) * QT::kBytes;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool ok = cols.valid(n0 + i);
      const char* row = q + (ok ? cols.row(n0 + i) : 0) * kQRowBytes;
      if constexpr (kDot2) {
        uint32_t tmp[W];
        if (ok) load_row<D, QT>(tmp, row, s);
#pragma unroll
        for (int w = 0; w < W; ++w) qw[i][w] = ok ? tmp[w] : 0u;
      } else {
#pragma unroll
        for (int k = 0; k < KD; ++k) qf[i][k] = ok ? load_q_elem<QT>(row, TL::dim(s, k)) : 0.0f;
      }
      m[i] = -INFINITY;
      l[i] = 0.0f;
#pragma unroll
      for (int k = 0; k < KD; ++k) acc[i][k] = 0.0f;
    }
  }

  // One 16-token block: kw/vw hold this lane's two tokens (tg, tg+8).
  // valid_toks: tokens of the block inside the context (V past it is zeroed);
  // vis[i]: tokens of the block column i may see (uniform; used when need_mask).
  __device__ __forceinline__ void block(const uint32_t (&kw)[kTokPerLane][W],
                                        uint32_t (&vw)[kTokPerLane][W], int valid_toks,
                                        const int (&vis)[G], bool need_mask,
                                        float k_mul, float v_mul, int tg) {
    float sc[kTokPerLane][G];
#pragma unroll
    for (int j = 0; j < kTokPerLane; ++j) {
      float part[G];
      if constexpr (kDot2) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          float a = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) a = dot2_bf16(qw[i][w], kw[j][w], a);
          part[i] = a;
        }
      } else {
        float kf[KD];
        to_float<D, KV>(kw[j], kf);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          float a = 0.0f;
#pragma unroll
          for (int k = 0; k < KD; ++k) a = fmaf(qf[i][k], kf[k], a);
          part[i] = a;
        }
      }
#pragma unroll
      for (int i = 0; i < G; ++i) sc[j][i] = sum8(part[i]) * k_mul;
    }
    if (need_mask) {                          // wave-uniform: the sequence's last block(s)
#pragma unroll
      for (int j = 0; j < kTokPerLane; ++j)
#pragma unroll
        for (int i = 0; i < G; ++i) sc[j][i] = tg + kGroups * j < vis[i] ? sc[j][i] : -INFINITY;
    }
    if (valid_toks < kBlockSize) {            // wave-uniform: rows past the context hold poison
#pragma unroll
      for (int j = 0; j < kTokPerLane; ++j) {
        const bool ok = tg + kGroups * j < valid_toks;
#pragma unroll
        for (int w = 0; w < W; ++w) vw[j][w] = ok ? vw[j][w] : 0u;
      }
    }
    bool need = false;
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int j = 0; j < kTokPerLane; ++j) need |= sc[j][i] > m[i] + kRescaleThreshold;
    if (__any(need)) {                          // rare: raise the reference maxima
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float bm = sc[0][i];
#pragma unroll
        for (int j = 1; j < kTokPerLane; ++j) bm = fmaxf(bm, sc[j][i]);
        bm = max_over_groups8(bm);
        const float mn = fmaxf(m[i], bm);
        // a column with nothing visible yet keeps m = -inf (and alpha = 1)
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[i] - mn);
        l[i] *= alpha;
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[i][k] *= alpha;
        m[i] = mn;
      }
    }
#pragma unroll
    for (int j = 0; j < kTokPerLane; ++j) {
      float vf[KD];
      to_float<D, KV>(vw[j], vf);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        // all scores -inf so far: weight 0, not exp2(NaN)
        const float p = __builtin_amdgcn_exp2f(sc[j][i] - (m[i] == -INFINITY ? 0.0f : m[i]));
        l[i] += p;
        const float pv = p * v_mul;
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[i][k] = fmaf(pv, vf[k], acc[i][k]);
      }
    }
  }
};

template <int D, int G, typename QT, typename KV>
__global__ __launch_bounds__(kWave) void paged_decode_kernel(DecodeArgs a) {
  using TL = Tile<D, KV>;
  using Dec = Decode<D, G, QT, KV>;
  constexpr int W = TL::kWords;
  constexpr int KD = TL::kDims;

  // blockIdx.x -> (column chunk, unit = (kv head, sequence, partition)), or
  // (column chunk, kv head, chunk slot) for a balanced split.
  DecodeItem it;
  if (!decode_item(a, it)) return;
  const int chunk = it.chunk, h = it.h, b = it.b, part = it.part;

  const int lane = threadIdx.x;
  const int tg = lane / kLanesPerToken;
  const int s = lane % kLanesPerToken;

  const int raw_ctx = a.context_lens[b];
  int ctx = raw_ctx < 0 ? 0 : raw_ctx;
  const int cap = a.max_blocks_per_seq * kBlockSize;
  ctx = ctx > cap ? cap : ctx;
  const int n_blk_seq = (ctx + kBlockSize - 1) / kBlockSize;
  const int blk_begin = it.blk_begin;
  int blk_end = it.blk_end < n_blk_seq ? it.blk_end : n_blk_seq;
  // Fused append: the block of position ctx-1 takes its new row from k_new/v_new
  // (a sequence outside 1 <= ctx <= capacity appends nothing, as pkv_kv_append).
  const int append_blk = (a.k_new && raw_ctx >= 1 && raw_ctx <= cap) ? (raw_ctx - 1) / kBlockSize : -1;
  const int t_new = (raw_ctx - 1) % kBlockSize;

  // Column n of the tile is new token n / group, head n % group (one new token:
  // the group's heads), n = chunk*G + i.
  Columns cols;
  cols.group = a.group;
  cols.num_q_heads = a.num_q_heads;
  cols.kv_head = h;
  if (a.q_start) {
    cols.row0 = a.q_start[b];
    cols.t = a.q_start[b + 1] - cols.row0;
  } else {
    cols.row0 = b;
    cols.t = 1;
  }
  const int n0 = chunk * G;
  if (!cols.valid(n0)) return;                          // no column of this tile exists

  // A sequence whose blocks fit one partition (or chunk) is finished here:
  // write the final output instead of a partial (the merge skips it).
  const bool final_out =
      a.write_final ||
      (a.final_single && (a.balanced() ? it.n_parts == 1 : n_blk_seq <= a.blocks_per_partition));
  if (blk_begin >= blk_end && !(a.write_final && part == 0) &&
      !(a.balanced() && final_out)) {                  // partition past the end, or an empty chunk
    if ((a.mark_empty || a.balanced()) && lane < G && cols.valid(n0 + lane) &&
        partial_row_ok(a, cols.row(n0 + lane), cols.row0))
      a.part_lse[partial_row(a, it, cols.row(n0 + lane), cols.row0)] = -INFINITY;
    return;
  }
  // Tokens each column attends to (all ctx for a single new token); the
  // tile's first column sees the fewest.
  int vis_all[G];
#pragma unroll
  for (int i = 0; i < G; ++i) vis_all[i] = cols.valid(n0 + i) ? cols.visible(n0 + i, ctx) : ctx;
  const int min_vis = vis_all[0];

  Dec dec;
  dec.load_q(reinterpret_cast<const char*>(a.q), cols, n0, s);

  const int32_t* table = a.block_tables + size_t(b) * a.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const size_t slice_stride = size_t(TL::kSliceBytes);
  const size_t head_off = size_t(h) * slice_stride;
  const size_t block_stride = size_t(a.num_kv_heads) * slice_stride;
  constexpr bool kFp8 = KV::kBytes == 1;

  uint32_t kA[kTokPerLane][W], vA[kTokPerLane][W], kB[kTokPerLane][W], vB[kTokPerLane][W];

  // Walk the partition in segments of up to 64 blocks: lane i holds the i-th
  // physical id of the segment; ids are broadcast with readlane.
  for (int seg = blk_begin; seg < blk_end; seg += kWave) {
    const int n = (blk_end - seg) < kWave ? (blk_end - seg) : kWave;
    int my_id = lane < n ? table[seg + lane] : -1;
    const bool my_ok = unsigned(my_id) < unsigned(a.num_blocks);
    my_id = my_ok ? my_id : 0;
    float my_ks = 1.0f, my_vs = 1.0f;
    if (kFp8 && lane < n) {
      my_ks = a.k_scales[size_t(my_id) * a.num_kv_heads + h];
      my_vs = a.v_scales[size_t(my_id) * a.num_kv_heads + h];
    }
    const uint64_t ok_mask = __ballot(my_ok);

    auto fetch = [&](uint32_t (&kw)[kTokPerLane][W], uint32_t (&vw)[kTokPerLane][W], int k) {
      const int phys = __builtin_amdgcn_readlane(my_id, k);
      const char* kslice = kbase + size_t(phys) * block_stride + head_off;
      const char* vslice = vbase + size_t(phys) * block_stride + head_off;
#pragma unroll
      for (int j = 0; j < kTokPerLane; ++j) {
        const int t = tg + kGroups * j;
        load_row<D, KV>(kw[j], kslice + t * TL::kRowBytes, s);
        load_row<D, KV>(vw[j], vslice + t * TL::kRowBytes, s);
      }
    };
    auto consume = [&](uint32_t (&kw)[kTokPerLane][W], uint32_t (&vw)[kTokPerLane][W], int k) {
      const int blk = seg + k;
      const int first = blk * kBlockSize;
      int valid = ctx - first;
      valid = valid < kBlockSize ? valid : kBlockSize;
      const bool ok = (ok_mask >> k) & 1;
      valid = ok ? valid : 0;
      const bool need_mask = valid < kBlockSize || first + kBlockSize > min_vis;
      int vis[G];
#pragma unroll
      for (int i = 0; i < G; ++i) vis[i] = vis_all[i] - first < valid ? vis_all[i] - first : valid;
      if (blk == append_blk && ok) {
        // Fused append: the lanes owning the new token's row take it from
        // k_new/v_new and (one writer per sequence and KV head) store it.
        const size_t nrow = (size_t(b) * a.num_kv_heads + h) * TL::kRowBytes;
        const int phys = __builtin_amdgcn_readlane(my_id, k);
        const size_t off = size_t(phys) * block_stride + head_off + size_t(t_new) * TL::kRowBytes;
#pragma unroll
        for (int j = 0; j < kTokPerLane; ++j) {
          if (tg + kGroups * j != t_new) continue;
          load_row<D, KV>(kw[j], reinterpret_cast<const char*>(a.k_new) + nrow, s);
          load_row<D, KV>(vw[j], reinterpret_cast<const char*>(a.v_new) + nrow, s);
          if (chunk == 0) {
            store_row<D, KV>(kw[j], reinterpret_cast<char*>(a.k_pool_w) + off, s);
            store_row<D, KV>(vw[j], reinterpret_cast<char*>(a.v_pool_w) + off, s);
          }
        }
      }
      float km = a.scale_log2, vm = 1.0f;
      if constexpr (kFp8) {
        km *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_ks), k));
        vm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_vs), k));
      }
      dec.block(kw, vw, valid, vis, need_mask, km, vm, tg);
    };

    fetch(kA, vA, 0);
    int k = 0;
    for (; k + 2 <= n; k += 2) {
      fetch(kB, vB, k + 1);
      consume(kA, vA, k);
      if (k + 2 < n) fetch(kA, vA, k + 2);
      consume(kB, vB, k + 1);
    }
    if (k < n) consume(kA, vA, k);
  }

  // Combine the 8 token groups; every lane then holds its dims' totals.
  float lt[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    lt[i] = sum_over_groups8(dec.l[i]);
#pragma unroll
    for (int k = 0; k < KD; ++k) dec.acc[i][k] = sum_over_groups8(dec.acc[i][k]);
  }

  // Token group i writes column i of the tile.
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (tg != i || !cols.valid(n0 + i)) continue;
    const size_t qrow = cols.row(n0 + i);
    const bool empty = lt[i] == 0.0f;        // no valid token (a NaN sum is not empty)
    const float inv = empty ? 0.0f : 1.0f / lt[i];
    if (final_out) {
      char* orow = reinterpret_cast<char*>(a.out) + qrow * size_t(D) * QT::kBytes;
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        const float v = dec.acc[i][k] * inv;
        if constexpr (QT::kBytes == 4) reinterpret_cast<float*>(orow)[TL::dim(s, k)] = v;
        else reinterpret_cast<uint16_t*>(orow)[TL::dim(s, k)] = f32_to_bf16_rne(v);
      }
    } else {
      if (!partial_row_ok(a, qrow, cols.row0)) continue;
      const size_t prow = partial_row(a, it, qrow, cols.row0);
      float* o = a.part_o + prow * D;
#pragma unroll
      for (int k = 0; k < KD; ++k) o[TL::dim(s, k)] = dec.acc[i][k] * inv;
      if (s == 0)
        a.part_lse[prow] = empty ? -INFINITY : (dec.m[i] + __builtin_amdgcn_logf(lt[i])) * kLn2;
    }
  }
}

template <int D, int G, typename QT, typename KV>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const size_t units = (a.balanced() ? size_t(1) : size_t(a.num_seqs)) * a.num_kv_heads * a.max_partitions;
  if (units == 0 || a.head_chunks == 0) return hipSuccess;
  if (units > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const size_t grid = decode_grid(units, a.head_chunks);
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((paged_decode_kernel<D, G, QT, KV>), dim3(unsigned(grid)), dim3(kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dispatch_types(const DecodeArgs& a, DType qt, DType kt, hipStream_t st) {
  if (qt == DType::F32) {
    if (kt == DType::F32) return launch_typed<D, G, F32, F32>(a, st);
    if (kt == DType::BF16) return launch_typed<D, G, F32, BF16>(a, st);
    return launch_typed<D, G, F32, FP8>(a, st);
  }
  if (kt == DType::F32) return launch_typed<D, G, BF16, F32>(a, st);
  if (kt == DType::BF16) return launch_typed<D, G, BF16, BF16>(a, st);
  return launch_typed<D, G, BF16, FP8>(a, st);
}

template <int D>
hipError_t dispatch_tile(const DecodeArgs& a, int tile, DType qt, DType kt, hipStream_t st) {
  switch (tile) {
    case 1: return dispatch_types<D, 1>(a, qt, kt, st);
    case 2: return dispatch_types<D, 2>(a, qt, kt, st);
    case 4: return dispatch_types<D, 4>(a, qt, kt, st);
    case 8:
      if constexpr (D == 64) return dispatch_types<D, 8>(a, qt, kt, st);
      [[fallthrough]];
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, int head_dim, int tile_heads, DType q_dtype,
                               DType kv_dtype, hipStream_t stream) {
  if (head_dim == 64) return dispatch_tile<64>(a, tile_heads, q_dtype, kv_dtype, stream);
  return dispatch_tile<128>(a, tile_heads, q_dtype, kv_dtype, stream);
}

}  // namespace pkv
