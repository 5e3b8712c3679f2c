// Absorbed multi-head latent attention (MLA) decode over a paged latent
// cache, on the matrix cores of gfx950.
//
// Every token caches one row of d_c + d_r = 512 + 64 bf16 numbers (the latent
// and the shared rotary key); in the absorbed form every head attends over
// that row directly: the key is the whole row, the value its first 512
// numbers (KV-cache post, "MLA: how does decode get full-size keys and values
// back?": fold W_UK into the query and W_UV into the output).  The queries
// arrive absorbed ([B, H, 576]); the kernel returns the latent outputs
// [B, H, 512] (the caller applies W_UV).  All heads share one K/V row, so the
// product is dense: per token and head 2 * (576 + 512) FLOP for 1,152 bytes.
//
// One workgroup of WAVES waves per (head chunk of 16*WAVES heads, sequence,
// partition); wave w owns 16 heads.  128 heads are one workgroup of 8 waves,
// so the copy of a pair of blocks into LDS (about 1,000 cycles of the CU's
// direct-to-LDS path for 38 KB, the cost that splitting the heads over two
// workgroups doubles) serves every head.  The 16 heads' absorbed queries (72
// registers) and fp32 accumulators (128) stay in registers; two waves per
// SIMD.
//
// The partition's blocks are walked in pairs (32 tokens).  Each pair is
// copied once into LDS, straight from HBM with 16-byte direct-to-LDS loads:
// block j of the pair occupies 19 whole 64-slot slices (16 rows of 74 slots,
// then 32 unused), so that one load instruction never spans two blocks and
// addresses a single block base plus a per-lane offset.  A row is 576 numbers
// + 16 of padding: a stride of 296 dwords, 40 mod 64, puts both the 16-row
// column reads of the score product and the transposed reads of the value
// product on distinct LDS banks (a stride of 292 dwords measured half the
// read rate).  Rows past the context, past the partition or of a block with a
// bad table entry are not loaded: their slots keep zeros (both buffers are
// cleared once) or a row of an earlier pair of this workgroup, and their
// scores are masked, so their values get weight 0.  Two buffers: the next
// pair is in flight while this one is computed.
//
// Per pair and wave:
//   S^T[16 tok x 16 heads] = K . Q^T    2 x 18 mfma_f32_16x16x32_bf16
//   online softmax in fp32 (log2 units, lazily raised maxima)
//   O[16 heads x 512] += P[16 x 32 tok] . V[32 tok x 512]   32 mfma_f32_16x16x32_bf16
// Lane l holds tokens 4*(l/16)+i of head l%16 after the score product; the
// 32-token k index of the value product is ordered (block 0: 4g+i, block 1:
// 16+4g+i) so that P is used in place as the A operand.  The B operand
// (4 tokens x 1 latent column per lane and block) comes from the row-major
// rows through gfx950's transposing LDS read: within a group of 16 lanes, lane
// i receives element (i & 3) of the 8 bytes that lane 4k + (i >> 2) addresses,
// for k = 0..3; lane (g, c) addresses row 4g + (c >> 2), columns 16t + 4(c & 3).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kDc = 512;                        // latent (value) width
constexpr int kDk = 576;                        // row width: latent + rotary key
constexpr int kRowBytes = kDk * 2;
constexpr int kBlockBytes = kBlockSize * kRowBytes;
constexpr int kChunksPerRow = kRowBytes / 16;   // 72
constexpr int kKStride = kDk + 16;              // bf16 elements per staged row
constexpr int kSlotsPerRow = kKStride * 2 / 16; // 74 16-byte slots, the last two padding
constexpr int kBlockSlices = (kBlockSize * kSlotsPerRow + kWave - 1) / kWave;   // 19
constexpr int kSlices = 2 * kBlockSlices;       // 38 direct loads of 64 slots per pair
constexpr int kBlockElems = kBlockSlices * kWave * 8;   // block 1 starts here (9,728)
constexpr int kBufElems = 2 * kBlockElems;
constexpr int kSlabs = kDk / 32;              // 18 score products per block and wave
constexpr int kTiles = kDc / 16;              // 32 value products per pair and wave
constexpr float kRescaleThreshold = 8.0f;
// LDS operand reads in flight ahead of their MFMAs (more spills at 8 waves).
constexpr int kKAhead = 4;                    // K slabs of the score product
constexpr int kVAhead = 3;                    // V tiles of the latent sum
static_assert(kBlockSlices * kWave >= kBlockSize * kSlotsPerRow, "a block's rows fit its slices");

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four token groups of a
// head): each lane swap returns the two halves it exchanged, whose larger
// element is the pairwise maximum in every lane.  (The swap's two results are
// copied to scalars before the float casts: hipcc's __builtin_bit_cast of an
// element of the returned vector reads element 0 whatever the index.)
__device__ __forceinline__ float max_of_swap(int lo, int hi) {
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}
__device__ __forceinline__ float max_over_groups(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const int a0 = a[0], a1 = a[1];
  const int y = __builtin_bit_cast(int, max_of_swap(a0, a1));
  const auto b = __builtin_amdgcn_permlane16_swap(y, y, false, false);
  const int b0 = b[0], b1 = b[1];
  return max_of_swap(b0, b1);
}

// Two floats to bf16 (round to nearest even), low one first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, __bf16(lo))) |
         (uint32_t(__builtin_bit_cast(uint16_t, __bf16(hi))) << 16);
}

// Chunk slot cs and head chunk of this workgroup in a balanced grid of
// slots x head_chunks workgroups.  Workgroups are dealt to the eight XCDs in
// turn (workgroup i to XCD (i + o) mod 8, the offset o carried over from
// earlier launches); the workgroups i = x mod 8 take a run of consecutive
// slots, so the chunks of one sequence, which take consecutive slots, mostly
// share one L2 and read the sequence's absorbed queries from HBM once.
__device__ __forceinline__ void slot_of(int head_chunks, int slots, int& chunk, int& cs) {
  const int bid = blockIdx.x;
  const int total = slots * head_chunks;
  int lin = bid;
  if (total % 8 == 0) lin = (bid & 7) * (total >> 3) + (bid >> 3);
  chunk = lin % head_chunks;
  cs = lin / head_chunks;
}

// The work of one workgroup: its head chunk, sequence b, context ctx and
// blocks [blk_begin, blk_end); its partial rows are slot_row + head *
// slot_stride with slot = the partition of the sequence (fixed partitions:
// rows [b, H, max_partitions]) or the chunk slot (balanced split: rows
// [slot, H]); final_out: the sequence has one chunk or partition, so the
// output is written directly.
struct MlaWork {
  int chunk, b, blk_begin, blk_end, ctx;
  size_t slot_row, slot_stride;
  bool final_out;
};

// Derives the workgroup's work (the balanced split planned by wave 0 and
// shared through LDS, or read from chunk_first, or a fixed partition).
// False: nothing to do (uniform over the workgroup); a fixed partition past
// its sequence's end then marks its partial rows empty when asked to
// (kHeadsPerWave heads per wave).
template <int WAVES, int kHeadsPerWave>
__device__ __forceinline__ bool mla_work(const MlaArgs& a, int wave, int lane, MlaWork& w) {
  constexpr int kThreads = WAVES * kWave;
  const int cap = a.max_blocks_per_seq * kBlockSize;
  int n_blk_seq;
  if (a.plan_first) {
    // Wave 0 plans the workgroup's chunk (pairs of blocks) and shares it.
    int cs;                                              // chunk slot
    slot_of(a.head_chunks, a.max_partitions, w.chunk, cs);
    __shared__ int s_plan[4];                            // sequence (-1: none), first pair, end pair, chunks
    if (wave == 0) {
      PlanChunk pc;
      int total_chunks;
      const bool any = plan_slot(a.context_lens, a.num_seqs, cap, 2 * kBlockSize,
                                 a.max_partitions, cs, pc, total_chunks);
      if (lane == 0) {
        s_plan[0] = any ? pc.b : -1;
        s_plan[1] = pc.u_begin;
        s_plan[2] = pc.u_end;
        s_plan[3] = pc.n;
        if (any && pc.u_begin == 0 && w.chunk == 0) {    // the sequence's first chunk
          a.plan_first[pc.b] = cs;
          if (pc.b == a.num_seqs - 1) a.plan_first[a.num_seqs] = total_chunks;
        }
      }
    }
    __syncthreads();
    // (read back through readfirstlane: uniform values in scalar registers)
    w.b = __builtin_amdgcn_readfirstlane(s_plan[0]);
    if (w.b < 0) return false;                           // a slot past the last chunk
    const int raw_ctx = a.context_lens[w.b];
    w.ctx = raw_ctx < 0 ? 0 : (raw_ctx > cap ? cap : raw_ctx);
    n_blk_seq = (w.ctx + kBlockSize - 1) / kBlockSize;
    w.blk_begin = 2 * __builtin_amdgcn_readfirstlane(s_plan[1]);
    w.blk_end = 2 * __builtin_amdgcn_readfirstlane(s_plan[2]);
    // (one chunk: also a sequence with nothing to attend)
    w.final_out = __builtin_amdgcn_readfirstlane(s_plan[3]) == 1;
    w.slot_row = size_t(cs) * a.num_heads;
    w.slot_stride = 1;
  } else if (a.chunk_first) {
    int cs;                                              // chunk slot (grid: every slot exists)
    slot_of(a.head_chunks, a.max_partitions, w.chunk, cs);
    __shared__ int s_seq;
    if (threadIdx.x == 0) s_seq = -1;
    __syncthreads();
    for (int s = threadIdx.x; s < a.num_seqs; s += kThreads)
      if (a.chunk_first[s] <= cs && cs < a.chunk_first[s + 1]) s_seq = s;
    __syncthreads();
    w.b = __builtin_amdgcn_readfirstlane(s_seq);
    if (w.b < 0) return false;                           // a slot past the last chunk
    const int n_b = a.chunk_first[w.b + 1] - a.chunk_first[w.b];
    const int k = cs - a.chunk_first[w.b];
    const int raw_ctx = a.context_lens[w.b];
    w.ctx = raw_ctx < 0 ? 0 : (raw_ctx > cap ? cap : raw_ctx);
    n_blk_seq = (w.ctx + kBlockSize - 1) / kBlockSize;
    const int pairs = (n_blk_seq + 1) / 2;                // chunk k: pairs [k u / n, (k+1) u / n)
    w.blk_begin = 2 * int(int64_t(k) * pairs / n_b);
    w.blk_end = 2 * int(int64_t(k + 1) * pairs / n_b);
    w.final_out = n_b == 1;                              // (also a sequence with nothing to attend)
    w.slot_row = size_t(cs) * a.num_heads;
    w.slot_stride = 1;
  } else {
    int unit;
    if (!decode_unit(blockIdx.x, a.head_chunks, a.num_seqs * a.max_partitions, w.chunk, unit))
      return false;
    w.b = unit % a.num_seqs;
    const int part = unit / a.num_seqs;
    const int raw_ctx = a.context_lens[w.b];
    w.ctx = raw_ctx < 0 ? 0 : (raw_ctx > cap ? cap : raw_ctx);
    n_blk_seq = (w.ctx + kBlockSize - 1) / kBlockSize;
    w.blk_begin = part * a.blocks_per_partition;
    w.blk_end = w.blk_begin + a.blocks_per_partition;
    w.final_out = a.write_final || (a.final_single && n_blk_seq <= a.blocks_per_partition);
    w.slot_row = size_t(w.b) * a.num_heads * a.max_partitions + part;
    w.slot_stride = a.max_partitions;
    // (b, part) is uniform over the workgroup: every wave returns here or none.
    const int end = w.blk_end < n_blk_seq ? w.blk_end : n_blk_seq;
    if (w.blk_begin >= end && !(a.write_final && part == 0)) {    // partition past the end
      const int h = (w.chunk * WAVES + wave) * kHeadsPerWave + lane;
      if (a.mark_empty && lane < kHeadsPerWave && h < a.num_heads)
        a.part_lse[w.slot_row + size_t(h) * w.slot_stride] = -INFINITY;
      return false;
    }
  }
  w.blk_end = w.blk_end < n_blk_seq ? w.blk_end : n_blk_seq;
  return true;
}

// Copies pairs of blocks into LDS.  Block ids of the workgroup's run, 64 at a
// time in lane registers (lane i holds entry seg + i); a pair's two ids are
// broadcast with readlane, so addresses and validity flags are wave-uniform.
// Pair p goes to dst as 38 slices, one direct-to-LDS load of 64 16-byte
// slots each, slice sl of block sl / 19, taken by wave sl % WAVES; lanes
// whose slot is row padding, past the attended tokens (limit) or in a block
// with a bad table entry load nothing.
template <int WAVES>
struct PairStage {
  const int32_t* table;
  const char* pool;
  int blk_begin, blk_end, limit, num_blocks, wave, lane;
  int seg = -kWave, my_id = 0;
  uint64_t ok_mask = 0;

  __device__ __forceinline__ void ids(int p, int& phys0, int& phys1, bool& ok0, bool& ok1) {
    const int rel = 2 * p;                               // first block of the pair, from blk_begin
    if (rel >= seg + kWave) {
      seg = rel - rel % kWave;
      const int blk = blk_begin + seg + lane;
      my_id = blk < blk_end ? table[blk] : -1;
      ok_mask = __ballot(unsigned(my_id) < unsigned(num_blocks));
    }
    const int k = rel - seg;
    phys0 = __builtin_amdgcn_readlane(my_id, k);
    phys1 = __builtin_amdgcn_readlane(my_id, k + 1);
    ok0 = (ok_mask >> k) & 1;
    ok1 = k + 1 < kWave && ((ok_mask >> (k + 1)) & 1);
  }

  __device__ __forceinline__ void stage(int p, uint16_t* dst, bool& ok0, bool& ok1) {
    constexpr int kSlicesPerWave = (kSlices + WAVES - 1) / WAVES;
    int phys0, phys1;
    ids(p, phys0, phys1, ok0, ok1);
    const int rem0 = limit - (blk_begin + 2 * p) * kBlockSize;   // rows of block 0 attended
    const char* base0 = pool + size_t(unsigned(phys0)) * kBlockBytes;
    const char* base1 = pool + size_t(unsigned(phys1)) * kBlockBytes;
#pragma unroll
    for (int r = 0; r < kSlicesPerWave; ++r) {
      const int sl = wave + r * WAVES;
      if (sl >= kSlices) break;
      const bool blk1 = sl >= kBlockSlices;
      if (!(blk1 ? ok1 : ok0)) continue;
      const int rem = blk1 ? rem0 - kBlockSize : rem0;
      const int local = (sl - (blk1 ? kBlockSlices : 0)) * kWave + lane;
      const int row = local / kSlotsPerRow, ch = local - row * kSlotsPerRow;
      if (row < rem && row < kBlockSize && ch < kChunksPerRow) {
        // (a named pointer: as a direct argument of the builtin this sum
        // makes the host pass drop the kernel's launch stub)
        const char* src = (blk1 ? base1 : base0) + (row * kRowBytes + ch * 16);
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + sl * kWave * 8), 16, 0, 0);
      }
    }
  }
};

template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void mla_decode_kernel(MlaArgs a) {
  constexpr int kThreads = WAVES * kWave;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * kBufElems];
  uint16_t* const s_k0 = s_k;                            // the two pair buffers, one after the other
  uint16_t* const s_k1 = s_k + kBufElems;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform
  const int lane = threadIdx.x % kWave;
  const int g = lane >> 4, c = lane & 15;

  // Clear both buffers, so that slots never loaded read as zeros (while wave
  // 0 plans the chunk).
  for (int i = threadIdx.x; i < kBufElems / 8; i += kThreads) {
    reinterpret_cast<uint4*>(s_k0)[i] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(s_k1)[i] = make_uint4(0, 0, 0, 0);
  }

  MlaWork w;
  if (!mla_work<WAVES, 16>(a, wave, lane, w)) return;
  const int chunk = w.chunk, b = w.b, blk_begin = w.blk_begin, blk_end = w.blk_end, ctx = w.ctx;
  const size_t slot_row = w.slot_row, slot_stride = w.slot_stride;
  const bool final_out = w.final_out;
  const int h0 = (chunk * WAVES + wave) * 16;            // first head of this wave

  const int limit = ctx < blk_end * kBlockSize ? ctx : blk_end * kBlockSize;   // tokens attended

  bf16x8 q[kSlabs];                                   // loaded after the first pair's copy is issued
  f32x4 o[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  const int n_pairs = (blk_end - blk_begin + 1) / 2;

  PairStage<WAVES> st{a.block_tables + size_t(b) * a.max_blocks_per_seq,
                      static_cast<const char*>(a.pool), blk_begin, blk_end, limit, a.num_blocks,
                      wave, lane};

  // Pair p, staged in kb, with its blocks' validity flags.
  auto compute = [&](const uint16_t* kb, int p, bool ok0, bool ok1) {
    // Scores of the pair's two blocks: lane holds tokens 16j + 4g + i of head
    // h0 + c.
    // The 36 products alternate between the blocks (two independent
    // accumulation chains) and read their K slab kKAhead products ahead from
    // a rotating set of registers; the scheduling fences keep that order (left
    // alone, the compiler waits on every LDS read before its MFMA, short of
    // registers).
    f32x4 s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) s[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    {
      constexpr int kN = 2 * kSlabs;                 // product i: slab i / 2 of block i % 2
      const uint16_t* krow = kb + c * kKStride + 8 * g;
      auto kload = [&](int i) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                              krow + (i & 1) * kBlockElems + 32 * (i >> 1)));
      };
      bf16x8 kbuf[kKAhead];
#pragma unroll
      for (int i = 0; i < kKAhead; ++i) kbuf[i] = kload(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[i % kKAhead], q[i >> 1], s[i & 1],
                                                          0, 0, 0);
        if (i + kKAhead < kN) kbuf[i % kKAhead] = kload(i + kKAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    const int rem = limit - (blk_begin + 2 * p) * kBlockSize;      // tokens of the pair attended
    float x[8];
    if (ok0 && ok1 && rem >= 2 * kBlockSize) {           // uniform: the whole pair counts
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * j + i] = s[j][i] * a.scale_log2;
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (j ? ok1 : ok0) && 16 * j + 4 * g + i < rem;
          x[4 * j + i] = ok ? s[j][i] * a.scale_log2 : -INFINITY;
        }
    }
    const float bm = max_over_groups(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
    if (__any(bm > m + kRescaleThreshold)) {              // rare: raise the reference maxima
      const float mn = fmaxf(m, bm);
      const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      m = mn;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] *= ar[i];
    }
    const float m_eff = m == -INFINITY ? 0.0f : m;
    float pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pv[k] = __builtin_amdgcn_exp2f(x[k] - m_eff);
      l += pv[k];
    }
    const bf16x8 pa = __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])));
    // V operand of tile t: rows 4g + (c >> 2) of block 0 and of block 1,
    // columns 16t + 4(c & 3), read transposed.
    // Read kVAhead tiles ahead, as for the scores.
    const uint16_t* vrow = kb + (4 * g + (c >> 2)) * kKStride + 4 * (c & 3);
    auto vload = [&](int t) {
      const v4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vrow + 16 * t));
      const v4i16 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vrow + kBlockElems + 16 * t));
      const uint2 w0 = __builtin_bit_cast(uint2, v0);
      const uint2 w1 = __builtin_bit_cast(uint2, v1);
      return __builtin_bit_cast(bf16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
    };
    bf16x8 vbuf[kVAhead];
#pragma unroll
    for (int t = 0; t < kVAhead; ++t) vbuf[t] = vload(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vbuf[t % kVAhead], o[t], 0, 0, 0);
      if (t + kVAhead < kTiles) vbuf[t % kVAhead] = vload(t + kVAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Even pairs live in s_k0, odd pairs in s_k1.  Every wave runs the same
  // number of iterations, so the barriers match.  (Unrolling the loop by two
  // to name each buffer statically would let the compiler tell the copy of
  // the next pair from the reads of this one, but the second copy of the
  // body does not fit in the registers.)
  // The first pair's copy, then the queries, both in flight together.
  __syncthreads();                                    // buffers cleared
  bool ok0 = false, ok1 = false;
  if (n_pairs > 0) st.stage(0, s_k0, ok0, ok1);
  // The absorbed query of head h0 + c, as the B operand of the score product.
  {
    const bool ok = h0 + c < a.num_heads;
    const char* qrow = static_cast<const char*>(a.q) +
                       (size_t(b) * a.num_heads + (ok ? h0 + c : 0)) * kRowBytes;
#pragma unroll
    for (int j = 0; j < kSlabs; ++j) {
      const uint4 w = ok ? *reinterpret_cast<const uint4*>(qrow + 64 * j + 16 * g) : make_uint4(0, 0, 0, 0);
      q[j] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                      // this wave's copies have landed
  __syncthreads();                                    // and everyone's
  for (int p = 0; p < n_pairs; ++p) {
    bool nk0 = false, nk1 = false;
    uint16_t* cur = (p & 1) ? s_k1 : s_k0;
    uint16_t* nxt = (p & 1) ? s_k0 : s_k1;
    if (p + 1 < n_pairs) st.stage(p + 1, nxt, nk0, nk1);
    compute(cur, p, ok0, ok1);
    ok0 = nk0;
    ok1 = nk1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Denominator of head h0 + c over the four token groups; then of rows 4g+i.
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  float l_row[4], m_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l_row[i] = __shfl(lt, 4 * g + i);
    m_row[i] = __shfl(m, 4 * g + i);
  }
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv[i] = l_row[i] == 0.0f ? 0.0f : 1.0f / l_row[i];
  if (!final_out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g + i;
      if (c == 0 && head < a.num_heads)
        a.part_lse[slot_row + size_t(head) * slot_stride] =
            l_row[i] == 0.0f ? -INFINITY : (m_row[i] + __builtin_amdgcn_logf(l_row[i])) * kLn2;
    }
  }
  if (final_out || a.part_bf16) {                        // uniform
    // bf16 rows, through LDS (free once the last pair's barrier has passed):
    // a wave writes its 16 rows' half of the columns to its own region (rows
    // 528 bytes apart, so the four row groups of a write fall on distinct
    // banks) and stores them back 16 bytes per lane, eight stores per half
    // instead of 64 two-byte ones.
    constexpr int kRowPitch = 264;                       // bf16 elements per staged row
    static_assert(WAVES * 16 * kRowPitch <= 2 * kBufElems, "the staged rows fit the pair buffers");
    uint16_t* region = s_k + wave * 16 * kRowPitch;
    uint16_t* rows_base = final_out ? static_cast<uint16_t*>(a.out) + (size_t(b) * a.num_heads) * kDc
                                    : reinterpret_cast<uint16_t*>(a.part_o) + slot_row * kDc;
    const size_t head_pitch = final_out ? kDc : slot_stride * kDc;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int tt = 0; tt < kTiles / 2; ++tt)
          region[(4 * g + i) * kRowPitch + 16 * tt + c] =
              f32_to_bf16_rne(o[half * kTiles / 2 + tt][i] * inv[i]);
      __builtin_amdgcn_s_waitcnt(0xc07f);                // lgkmcnt(0): this wave's writes are in LDS
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = lane + kWave * j;                  // 16-byte piece: row k / 32, piece k % 32
        const int r = k >> 5, piece = k & 31;
        const uint4 v = *reinterpret_cast<const uint4*>(region + r * kRowPitch + 8 * piece);
        if (h0 + r < a.num_heads)
          *reinterpret_cast<uint4*>(rows_base + size_t(h0 + r) * head_pitch + half * (kDc / 2) +
                                    8 * piece) = v;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);                // the reads are done before the next half's writes
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = h0 + 4 * g + i;
      if (head >= a.num_heads) continue;
      float* op = a.part_o + (slot_row + size_t(head) * slot_stride) * kDc + c;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) op[16 * t] = o[t][i] * inv[i];
    }
  }
}

}  // namespace

int mla_heads_per_workgroup(int num_heads) {
  int w = 1;
  while (w < 8 && 16 * w < num_heads) w *= 2;
  return 16 * w;
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream) {
  const size_t units = size_t(a.num_seqs) * a.max_partitions;
  if (units == 0) return hipSuccess;
  if (units > 0x7fffffffu) return hipErrorInvalidConfiguration;
  // Balanced split (planned before or inside): one workgroup per (chunk slot,
  // head chunk), max_partitions slots; fixed partitions: XCD-ordered
  // (partition, sequence) units.
  const size_t grid = (a.chunk_first || a.plan_first) ? size_t(a.max_partitions) * a.head_chunks
                                                      : decode_grid(units, a.head_chunks);
  if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 g{unsigned(grid)};
  switch (mla_heads_per_workgroup(a.num_heads) / 16) {
    case 1: hipLaunchKernelGGL(mla_decode_kernel<1>, g, dim3(1 * kWave), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(mla_decode_kernel<2>, g, dim3(2 * kWave), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(mla_decode_kernel<4>, g, dim3(4 * kWave), 0, stream, a); break;
    default: hipLaunchKernelGGL(mla_decode_kernel<8>, g, dim3(8 * kWave), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
