// Device code of libpagedattn: GQA-grouped paged-attention decode for gfx950 (CDNA4).
//
// Phase 1 works on "pieces": a contiguous run of 16-token tiles of one
// (sequence, KV head) segment.  One workgroup serves every query head of the
// KV head's group, so each K/V page is fetched from HBM once (page of commit
// 8d26e23, "Key design change": grid on KV heads instead of query heads).  Its W
// waves split the piece's tiles; each wave
//   1. gathers the tile through the block table with coalesced 16-byte global
//      loads (one tile = one contiguous 16 x head_dim run of a page),
//   2. stages it in its own XOR-swizzled LDS slot,
//   3. computes S^T = K_tile Q_group^T with v_mfma_f32_16x16x32 (tokens are the
//      16 rows, the group's query heads the 16 columns, zero-padded),
//   4. runs the online softmax in fp32 registers in base 2,
//   5. accumulates O^T += V_tile^T P^T with v_mfma_f32_16x16x16; the S^T
//      accumulator layout is already the B-operand layout of this product, so P
//      never leaves registers.
// The waves then merge their (max, sum, acc) states through LDS with the
// flash-attention rescale, and the workgroup writes either the final output
// (the piece is the whole segment: single pass) or the piece's compound
// partial (page of commit 8d26e23: max_score, exp_sum, weighted_v).
//
// Two ways of cutting the work into pieces:
//  - pa_phase1_kernel: the pages' grid (sequence, KV head, partition) with a
//    fixed partition size; a sequence no longer than the single-pass bound is
//    one piece (page of commit b80fd2b, three-tier decode dispatch).
//  - pa_phase1_balanced_kernel: the step's tiles, sequences laid end to end, are
//    cut into shares computed on the device from seq_lens, one workgroup per
//    (share, KV head).  A sequence inside one share is one pass; a sequence
//    crossing shares is partitioned at the share boundaries.  Each sequence
//    counts a few virtual tiles for the cost of starting a piece, so every
//    workgroup has about the same work whatever the length mix.
// With automatic splits, partitions and shares come in pairs whose members run
// on XCDs of opposite parity, the even one taking a few percent more (see
// share_cut): the workgroups of MI355X's odd XCDs stream more slowly.
//
// Phase 2 (pa_reduce_kernel) merges the partials of each partitioned segment
// with the rescale of the online-softmax fix (page of commit 87a19d2): with M
// the largest max, partial p weighs l_p 2^(m_p - M) and the output is
// sum_p weight_p acc_p / sum_p weight_p, evaluated as an associative fold.
//
// Fused combine (the cross-partition "Level 3" of the pages' three-level
// decomposition, done inside phase 1): every workgroup that writes a partial
// takes a device-scope ticket for its segment after releasing the record; the
// one that draws the last ticket merges the segment's records with the same fold
// and writes the output, then resets the ticket to zero.  No second launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;          // tokens per tile (MFMA M dimension)
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// Element types.  Q, K, V and the output share one 16-bit type; all math that
// is not an MFMA runs in fp32.
// ---------------------------------------------------------------------------
struct F16 {
  static constexpr bool kSplitP = false;   // P in one f16 (11 significant bits) is exact enough
  static constexpr uint32_t kOnePair = 0x3C003C00u;   // two f16 ones
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  // 32 keys per instruction (the double-rate gfx950 form): A = V^T, B = P^T
  static __device__ __forceinline__ f32x4 mfma_pv32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // round-to-nearest-even fp32 -> f16 bits
  static __device__ __forceinline__ uint32_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float value(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
};

struct BF16 {
  // P in one bf16 (8 significant bits) perturbs each weight by up to 2^-9: with a
  // handful of keys that reaches the output almost undiluted, so P is carried as
  // the sum of two bf16 values and multiplied into V by two MFMAs.
  static constexpr bool kSplitP = true;
  static constexpr uint32_t kOnePair = 0x3F803F80u;   // two bf16 ones
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float value(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
  }
};

// ---------------------------------------------------------------------------
// Kernel arguments (passed by value).
// ---------------------------------------------------------------------------
// Partial records.  A record holds, for each of the G query heads of one KV
// head, the normalised output of a piece (fp32) and (max in base 2, exp sum).
// ws_acc is [D/16][R][G][16] floats (slice-major: phase 2 reads the records of
// one 16-wide slice back to back) and ws_ml is [R][G] float2.
//  - grid mode:     record (s*units + unit)*max_parts + partition,
//                   R = S*units*max_parts (units = Hkv, or Hq in the per-query-head
//                   ablation)
//  - balanced mode: record 2*w + slot of workgroup w (slot 0: the piece that
//                   ends a sequence begun in an earlier share, slot 1: the piece
//                   that begins a sequence continued in a later share), R = 2*num_wg
struct DecodeArgs {
  void* out;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  float* ws_acc;
  float2* ws_ml;
  int2* jobs;               // balanced mode: [num_wg] (segment, partial count) or (-1, 0)
  unsigned* tickets;        // fused combine: one counter per segment, zero between calls; else null
  long long records;        // R
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;                // query heads one workgroup serves (a "head unit")
  int units;                // head units per sequence (num_heads / group)
  int kv_group;             // query heads per KV head (num_heads / num_kv_heads)
  int block_size;
  int max_blocks_per_seq;
  int max_seq_len;          // lengths are clamped to this bound
  int partition_size;       // grid mode
  int single_pass_max_len;  // grid mode
  int max_parts;            // grid mode
  int num_wg;               // balanced mode: workgroups of phase 1
  int xcd_skew;             // XCD-paired shares: permille the even-XCD member of a pair
                            // takes above the mean (0: equal shares), see share_cut
  int piece_cost;           // balanced mode: tiles a piece's start is worth in the cut
  float scale_log2;         // scale * log2(e)
};

struct GatherArgs {
  uint16_t* k_out;
  uint16_t* v_out;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  int num_seqs;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  int max_seq_len;
};

#ifndef PA_MAX_BALANCED_SEQS
#define PA_MAX_BALANCED_SEQS 1024
#endif
constexpr int kMaxBalancedSeqs = PA_MAX_BALANCED_SEQS;   // balanced mode keeps a prefix of seq_lens in LDS

// XCD-paired shares.  The hardware hands out workgroup i to XCD i mod 8, and on
// MI355X the workgroups of the odd XCDs stream K/V ~8-10% slower than those of
// the even ones (measured per workgroup with the 100 MHz wall clock: same
// bytes, same pages, any assignment of KV heads to XCDs), so with equal shares
// the odd XCDs finish last.  Shares therefore come in pairs whose members run
// on workgroups of opposite parity, and the even one takes (1000 + skew)/1000 of
// the pair's mean.  share_cut(T, j, NS, skew) is the first item of share j of NS
// shares of T items in that scheme (pairs (2i, 2i+1), an odd last share alone);
// skew 0 gives T*j/NS.  Exact integer arithmetic, used by the planner too.
__host__ __device__ __forceinline__ long long share_cut(long long T, long long j, long long NS,
                                                        int skew) {
  if (j >= NS) return T;
  return T * (1000 * j + skew * (j & 1)) / (1000 * NS);
}

// Share holding item t < T: the largest j with share_cut(j) <= t.
__host__ __device__ __forceinline__ long long share_holding(long long T, long long t,
                                                            long long NS, int skew) {
  long long j = (t * NS) / T;              // exact without skew; off by at most one with it
  while (j > 0 && share_cut(T, j, NS, skew) > t) --j;
  while (j + 1 < NS && share_cut(T, j + 1, NS, skew) <= t) ++j;
  return j;
}

__device__ __forceinline__ size_t rec_acc_index(int slice, long long rec, int h, int G,
                                                long long R) {
  return ((static_cast<size_t>(slice) * R + rec) * G + h) * 16;
}

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s) {
  return min(a.seq_lens[s], a.max_seq_len);
}

// Element offset of the 16-token tile starting at token t0 (a multiple of 16) of KV
// head kvh, given the page that holds it.  64-bit: pools above 4 G elements are legal.
__device__ __forceinline__ size_t tile_offset_in(int page, int t0, int kvh, int Hkv, int bs,
                                                 int D) {
  const unsigned slot = static_cast<unsigned>(t0) % static_cast<unsigned>(bs);
  return ((static_cast<size_t>(page) * Hkv + kvh) * bs + slot) * static_cast<size_t>(D);
}

// Page holding token t0 of sequence s (wave-uniform).  The table is read through
// the constant address space: no kernel writes it, and a uniform index then
// always becomes a scalar load, whose wait does not drain the vector loads (K/V
// prefetches) issued before it.
__device__ __forceinline__ int page_at(const int32_t* bt, int s, int blk, int mbps) {
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  return __builtin_amdgcn_readfirstlane(((const_i32*)bt)[(size_t)s * mbps + blk]);
}
__device__ __forceinline__ int page_of(const int32_t* bt, int s, int t0, int bs, int mbps) {
  return page_at(bt, s, static_cast<unsigned>(t0) / static_cast<unsigned>(bs), mbps);
}

// A tile is read as two 8-token halves.  Pages holding the halves of the tile
// starting at t0 (wave-uniform): with block_size >= 16 both lie in one page; with
// block_size 8 the second half has its own page, looked up only if it holds a
// token before t_end (later block-table entries may be invalid), else the first
// half is read again and masked like any slot past the end.
__device__ __forceinline__ int2 tile_pages(const int32_t* bt, int s, int t0, int t_end, int bs,
                                           int mbps) {
  const int p0 = page_of(bt, s, t0, bs, mbps);
  int p1 = p0;
  if (bs < kTile && t0 + kTile / 2 < t_end) p1 = page_of(bt, s, t0 + kTile / 2, bs, mbps);
  return make_int2(p0, p1);
}

// Element offsets of the two halves of the tile at t0 (see tile_pages); with one
// page they are 8*D apart.
__device__ __forceinline__ void tile_offsets(int2 pages, int t0, int kvh, int Hkv, int bs, int D,
                                             size_t& lo, size_t& hi) {
  lo = tile_offset_in(pages.x, t0, kvh, Hkv, bs, D);
  hi = bs < kTile ? tile_offset_in(pages.y, t0 + kTile / 2, kvh, Hkv, bs, D) : lo + 8 * D;
}

// One 16-token tile is two 8-row halves of 8*D*2 bytes, each contiguous.  Lane
// `lane` fetches the 16-byte chunks lane, lane+64, ... of each half, so every
// load instruction covers 1 KiB contiguously.  K and V are read exactly once per
// step, so the loads are nontemporal: they do not displace reusable lines from
// the caches (worth ~10% of gather bandwidth).
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ lo,
                                          const uint16_t* __restrict__ hi, int lane,
                                          u32x4 (&r)[D / 32]) {
  constexpr int H = D / 64;                // loads per half
  const u32x4* a = reinterpret_cast<const u32x4*>(lo);
  const u32x4* b = reinterpret_cast<const u32x4*>(hi);
#pragma unroll
  for (int j = 0; j < H; ++j) r[j] = __builtin_nontemporal_load(a + j * 64 + lane);
#pragma unroll
  for (int j = 0; j < H; ++j) r[H + j] = __builtin_nontemporal_load(b + j * 64 + lane);
}

// LDS slot of one tile: 16 rows of D halves; 16-byte chunk c of row t is stored at
// chunk position c ^ f(t & 15).  The masks were picked by measuring
// SQ_LDS_BANK_CONFLICT for each access pattern on gfx950:
//  - K and Q tiles (read as MFMA operands: 16 lanes take one chunk of rows
//    0..15): f(t) = t, conflict-free;
//  - V tiles (read transposed by ds_read_b64_tr_b16: chunks 2c, 2c+1 of rows
//    4q..4q+3 per 16 lanes): f(t) = t ^ 8*(t & 1), conflict-free, where f(t) = t
//    costs two extra cycles per read.
// Staging writes (16 consecutive chunks of a row) are conflict-free either way.
// With head_dim 64 a row has 8 chunks and the mask is cut to 3 bits.
template <int D, bool kIsV = false>
struct Swz {
  static constexpr int kChunks = D / 8;
  static_assert(kChunks >= 8 && (kChunks & (kChunks - 1)) == 0, "8, 16 or 32 chunks per row");
  static __device__ __forceinline__ int f(int row) {
    return kIsV ? (row ^ ((row & 1) << 3)) : row;
  }
  static __device__ __forceinline__ int chunk(int row, int c) {
    return c ^ (f(row & 15) & (kChunks - 1));
  }
  static __device__ __forceinline__ int byte_off(int row, int c) {
    return row * (D * 2) + chunk(row, c) * 16;
  }
};

// Orders a wave's own LDS writes and reads of its private slot: the compiler may
// not move LDS accesses across it, and the hardware executes one wave's LDS
// instructions in order.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Probabilities as P.V MFMA operands: p_e = 2^(x_e - m) for the lane's 4 keys,
// rounded to the element type (to hi + lo, two values of it, with kSplitP; the
// remainder p - hi is exact in fp32).  Returns the sum of the values the MFMAs use,
// so the exp sum and the weighted sum share the same weights.
template <class DT>
__device__ __forceinline__ float prob_operands(const float (&x)[4], float m, u32x2& hi,
                                               u32x2& lo) {
  uint32_t h[4], l[4] = {0, 0, 0, 0};
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = __builtin_amdgcn_exp2f(x[e] - m);
    h[e] = DT::bits(p);
    sum += DT::value(h[e]);
    if constexpr (DT::kSplitP) {
      l[e] = DT::bits(p - DT::value(h[e]));
      sum += DT::value(l[e]);
    }
  }
  hi = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  lo = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  return sum;
}

// acc + V^T P^T for the probabilities of prob_operands.
template <class DT>
__device__ __forceinline__ f32x4 pv_mfma(u32x2 v, u32x2 hi, u32x2 lo, f32x4 acc) {
  acc = DT::mfma_pv(v, hi, acc);
  if constexpr (DT::kSplitP) acc = DT::mfma_pv(v, lo, acc);
  return acc;
}

// pv_mfma over 32 keys with one double-rate MFMA per probability operand.
template <class DT>
__device__ __forceinline__ f32x4 pv_mfma32(u32x4 v, u32x4 hi, u32x4 lo, f32x4 acc) {
  acc = DT::mfma_pv32(v, hi, acc);
  if constexpr (DT::kSplitP) acc = DT::mfma_pv32(v, lo, acc);
  return acc;
}

// A value every lane of the wave holds (read from LDS, say), moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The pair {x[l], x[l ^ M]} in lane l (M = 16 or 32), without LDS: v_permlane16_swap
// (v_permlane32_swap) with x in both operands leaves x[l] in one result and x[l ^ M]
// in the other; which is which differs between the two lanes of a pair, which
// neither max nor + can see.
template <int M>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  static_assert(M == 16 || M == 32, "rows of 16 lanes or halves of the wave");
  const unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned r0, r1;
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0], r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0], r1 = r[1];
  }
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
template <int M>
__device__ __forceinline__ float xor_max(float x) {
  float a, b;
  lane_pair<M>(x, a, b);
  return fmaxf(a, b);
}
template <int M>
__device__ __forceinline__ float xor_add(float x) {
  float a, b;
  lane_pair<M>(x, a, b);
  return a + b;
}

// Merge of two compound partials (m, w, a): m is a base-2 max, w the weight sum
// and a the weighted sum, both relative to m.  (-inf, 0, 0) is the identity.
struct Partial {
  float m, w;
  f32x4 a;
};

__device__ __forceinline__ void combine_into(Partial& x, float om, float ow, f32x4 oa) {
  const float nm = fmaxf(x.m, om);
  const float fx = nm == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x.m - nm);
  const float fo = nm == kNegInf ? 0.f : __builtin_amdgcn_exp2f(om - nm);
  x.w = x.w * fx + ow * fo;
  x.a = x.a * fx + oa * fo;
  x.m = nm;
}

// Device-scope accesses for the fused combine.  Records cross XCDs, each with its
// own L2: they are written with device-scope stores (write-through to the
// device's point of coherence) and read back with device-scope loads, so no
// L2 write-back or invalidate (which would serialise every finishing workgroup
// of an XCD) is needed.  64-bit accesses, two per float4.
typedef unsigned long long u64;

__device__ __forceinline__ void store_dev(float* p, f32x4 v) {
  const u32x4 b = __builtin_bit_cast(u32x4, v);
  u64* q = reinterpret_cast<u64*>(p);
  __hip_atomic_store(q, (u64)b.x | ((u64)b.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (u64)b.z | ((u64)b.w << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_dev(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<u64*>(p), __builtin_bit_cast(u64, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 load_dev(const float* p) {
  const u64* q = reinterpret_cast<const u64*>(p);
  const u64 lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u64 hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(f32x4, u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi,
                                         (unsigned)(hi >> 32)});
}

__device__ __forceinline__ float2 load_dev(const float2* p) {
  return __builtin_bit_cast(
      float2, __hip_atomic_load(reinterpret_cast<const u64*>(p), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT));
}

// ---------------------------------------------------------------------------
// Phase 1: one piece = tokens [t_begin, t_end) of segment (s, kvh).
// ---------------------------------------------------------------------------
template <int D, int W>
struct Phase1Lds {
  static constexpr int kTileBytes = kTile * D * 2;
  unsigned char tiles[W * 2 * kTileBytes];   // per wave: K tile, V tile; merge area at the end
  unsigned char q[kTileBytes];               // the group's Q rows (16 rows, zero-padded)
  int last;                                  // fused combine: this workgroup drew the last ticket
};

// The records a segment's partials went to, for the fused combine: partial p
// (0 <= p < np) is record rec0 + step*p, plus `first` for p = 0.  seg < 0: the
// piece is not a partial.
struct SegMerge {
  int seg;
  int np;
  long long rec0, step, first;
};

// Fused combine, run by the workgroup that drew a segment's last ticket: merges
// the np records of segment (s, unit) into its G output rows.  Wave w takes the
// heads w, w + W, ...; within a wave, lane covers head_dim values 4*(lane % QL)
// .. +3 (QL = D/4) and, when a head row is narrower than the wave, the LPW lane
// groups fold alternate partials and are combined by shuffles.  Each round keeps
// U partials of every head of the wave in flight.  Same arithmetic as
// pa_reduce_kernel.
template <int D, class DT, int G, int W>
__device__ __forceinline__ void merge_records(const DecodeArgs& a, int s, int unit,
                                              const SegMerge& mg) {
  constexpr int QL = D / 4;                 // float4 lanes per head row
  constexpr int LPW = 64 / QL;              // lane groups per wave
  constexpr int HPW = (G + W - 1) / W;      // heads per wave (at most)
  constexpr int U = 16 / HPW;               // partials per round and lane group
  static_assert(QL <= 64 && 64 % QL == 0, "a head row must tile a wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane % QL;
  const int lg = lane / QL;
  const int slice = ql / 4, q4 = ql % 4;
  const long long R = a.records;
  const int np = mg.np;

  Partial st[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k) st[k] = Partial{kNegInf, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int p0 = lg; p0 < np; p0 += LPW * U) {
    f32x4 v[HPW][U];
    float2 m[HPW][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pc = min(p0 + u * LPW, np - 1);          // always a written record
      const long long rec = mg.rec0 + mg.step * pc + (pc == 0 ? mg.first : 0);
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const int h = min(wave + k * W, G - 1);
        m[k][u] = load_dev(a.ws_ml + rec * G + h);
        v[k][u] = load_dev(a.ws_acc + rec_acc_index(slice, rec, h, G, R) + 4 * q4);
      }
    }
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = p0 + u * LPW < np && m[k][u].x != kNegInf;
        combine_into(st[k], ok ? m[k][u].x : kNegInf, ok ? m[k][u].y : 0.f,
                     ok ? m[k][u].y * v[k][u] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  }
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = wave + k * W;
    if (h >= G) break;
#pragma unroll
    for (int x = QL; x < 64; x <<= 1) {
      const float om = __shfl_xor(st[k].m, x, 64);
      const float ow = __shfl_xor(st[k].w, x, 64);
      f32x4 oa;
#pragma unroll
      for (int e = 0; e < 4; ++e) oa[e] = __shfl_xor(st[k].a[e], x, 64);
      combine_into(st[k], om, ow, oa);
    }
    if (lane < QL) {
      const f32x4 y = st[k].a * (1.f / st[k].w);
      uint16_t* o = static_cast<uint16_t*>(a.out) +
                    ((size_t)s * a.num_heads + unit * G + h) * D + 4 * ql;
      const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                            DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
      *reinterpret_cast<u32x2*>(o) = packed;
    }
  }
}

// Fused combine: called by the whole workgroup right after wave 0 has written a
// partial record of segment mg.seg with device-scope stores (wave 0 wrote every
// word of it).  Wave 0 waits until those stores are acknowledged, i.e. visible
// at device scope, then draws a ticket; the workgroup that draws np - 1 reads
// the records back with device-scope loads, merges them and resets the
// counter, so the ticket area is zero again when the kernel ends.
template <int D, class DT, int W>
__device__ __forceinline__ void finish_partial(const DecodeArgs& a, Phase1Lds<D, W>& sm, int s,
                                               int unit, const SegMerge& mg) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    unsigned t = 0;
    if (lane == 0)
      t = __hip_atomic_fetch_add(a.tickets + mg.seg, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    t = __shfl(t, 0, 64);
    if (lane == 0) sm.last = t == static_cast<unsigned>(mg.np - 1) ? 1 : 0;
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sm.last)) {
    switch (a.group) {
#define PA_MERGE_CASE(g) \
      case g: merge_records<D, DT, g, W>(a, s, unit, mg); break;
      PA_MERGE_CASE(1) PA_MERGE_CASE(2) PA_MERGE_CASE(3) PA_MERGE_CASE(4)
      PA_MERGE_CASE(5) PA_MERGE_CASE(6) PA_MERGE_CASE(7) PA_MERGE_CASE(8)
      PA_MERGE_CASE(9) PA_MERGE_CASE(10) PA_MERGE_CASE(11) PA_MERGE_CASE(12)
      PA_MERGE_CASE(13) PA_MERGE_CASE(14) PA_MERGE_CASE(15) PA_MERGE_CASE(16)
#undef PA_MERGE_CASE
      default: break;
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(a.tickets + mg.seg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Runs one piece with the whole workgroup.  `final` writes the output rows of
// the group; otherwise the piece's partial goes to record `rec`, and with the
// fused combine the segment described by `mg` is merged by whichever workgroup
// finishes its last partial.  Starts with a barrier, so LDS from a previous piece
// may be reused.
//
// HS (the head-sequential ablation, page of commit 8d26e23, phase-1 kernel: the
// group's query heads processed one after another): each staged tile is taken G
// times, pass h computing QK^T, the softmax update and P.V for query head h alone
// and re-reading K and V^T from LDS.  The MFMA tile still carries all 16 head
// columns, so pass h zeroes the Q operand of the other columns, gives them P = 0 and
// a rescale of 1, and leaves their state as it was: the accumulators are the same
// registers as in the grouped pass, and every column's arithmetic is the grouped
// one, so the result is bitwise the same, at G times the LDS reads and MFMAs.
template <int D, class DT, int W, bool HS = false>
__device__ __forceinline__ void run_piece(const DecodeArgs& a, Phase1Lds<D, W>& sm, int s,
                                          int unit, int t_begin, int t_end, bool final,
                                          long long rec, const SegMerge& mg) {
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA (32 dims each)
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int LOADS = D / 32;            // 16-byte loads per lane per tile (K or V)
  constexpr int TILE_BYTES = Phase1Lds<D, W>::kTileBytes;
  using Z = Swz<D>;          // K and Q tiles
  using ZV = Swz<D, true>;   // V tiles
  static_assert((W - 1) * DB * 64 * 16 + 2 * (W - 1) * 64 * 4 <= W * 2 * TILE_BYTES,
                "merge area must fit in the tile slots");

  // The lane index is made opaque to the optimiser here, so the per-lane LDS
  // addresses derived from it are computed per piece instead of being hoisted
  // across the balanced kernel's walk, where they would all stay live.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_heads;
  const int kvh = unit * G / a.kv_group;   // KV head read by the unit's query heads
  const int col = lane & 15;     // query head (QK^T/PV columns) or row index within a tile
  const int grp = lane >> 4;     // 4-lane-group index: k-slot block / 4-row block

  // Loads are issued in the order they are needed, because vector-memory counters
  // retire in order: the group's Q rows, the page ids of the wave's first two tiles,
  // then the first tile.  Page ids then run one tile ahead of the K/V loads, so a
  // block-table round trip never sits between two tiles.
  constexpr int QLOADS = (kTile * D / 8 + W * 64 - 1) / (W * 64);
  u32x4 qv[QLOADS];
  {
    const uint16_t* qg = a.q + ((size_t)s * Hq + (size_t)unit * G) * D;
#pragma unroll
    for (int j = 0; j < QLOADS; ++j) {
      const int i = threadIdx.x + j * W * 64;
      const int row = i / Z::kChunks, c = i % Z::kChunks;
      qv[j] = u32x4{0, 0, 0, 0};
      if (i < kTile * Z::kChunks && row < G)
        qv[j] = *reinterpret_cast<const u32x4*>(qg + row * D + 8 * c);
    }
  }
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int bs = a.block_size, mbps = a.max_blocks_per_seq;
  int it = wave;
  const int2 page_cur = it < n_tiles ? tile_pages(a.bt, s, t_begin + kTile * it, t_end, bs, mbps)
                                     : make_int2(0, 0);
  int2 page_next = it + W < n_tiles
                       ? tile_pages(a.bt, s, t_begin + kTile * (it + W), t_end, bs, mbps)
                       : make_int2(0, 0);
  u32x4 rk[LOADS], rv[LOADS];
  if (it < n_tiles) {
    size_t lo, hi;
    tile_offsets(page_cur, t_begin + kTile * it, kvh, Hkv, bs, D, lo, hi);
    load_tile<D>(a.kc + lo, a.kc + hi, lane, rk);
    load_tile<D>(a.vc + lo, a.vc + hi, lane, rv);
  }

  // Q of the group in LDS as the B operand of S^T = K Q^T: row h is query head
  // unit*G + h (rows G..15 are zero), swizzled like a K tile.
  __syncthreads();                 // LDS of a previous piece may still be read
#pragma unroll
  for (int j = 0; j < QLOADS; ++j) {
    const int i = threadIdx.x + j * W * 64;
    if (i < kTile * Z::kChunks)
      *reinterpret_cast<u32x4*>(sm.q + Z::byte_off(i / Z::kChunks, i % Z::kChunks)) = qv[j];
  }
  __syncthreads();

  float m_run = kNegInf;          // running max of the head `col` (base-2 logits)
  float l_run = 0.f;              // this lane's share of the running exp sum
  f32x4 acc[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  unsigned char* ldsK = sm.tiles + wave * 2 * TILE_BYTES;
  unsigned char* ldsV = ldsK + TILE_BYTES;

  for (; it < n_tiles; it += W) {
    const int t0 = t_begin + kTile * it;
    // stage the tile in this wave's LDS slot
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = j * 64 + lane;
      const int row = c / Z::kChunks;
      *reinterpret_cast<u32x4*>(ldsK + Z::byte_off(row, c % Z::kChunks)) = rk[j];
      *reinterpret_cast<u32x4*>(ldsV + ZV::byte_off(row, c % Z::kChunks)) = rv[j];
    }
    wave_lds_fence();
    // prefetch the wave's next tile while this one is consumed, and the page id of
    // the one after
    if (it + W < n_tiles) {
      size_t lo, hi;
      tile_offsets(page_next, t0 + kTile * W, kvh, Hkv, bs, D, lo, hi);
      load_tile<D>(a.kc + lo, a.kc + hi, lane, rk);
      load_tile<D>(a.vc + lo, a.vc + hi, lane, rv);
      if (it + 2 * W < n_tiles)
        page_next = tile_pages(a.bt, s, t0 + 2 * kTile * W, t_end, bs, mbps);
    }

    if constexpr (!HS) {
      // S^T[token, head] = sum_d K[token, d] Q[head, d]
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = Z::byte_off(col, 4 * ks + grp);
        const u32x4 kop = *reinterpret_cast<const u32x4*>(ldsK + off);
        const u32x4 qop = *reinterpret_cast<const u32x4*>(sm.q + off);
        st = DT::mfma_qk(kop, qop, st);
      }

      // online softmax in base 2; this lane holds head `col`, tokens t0 + 4*grp + e
      const int tk = t0 + 4 * grp;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (tk + e < t_end) ? st[e] * a.scale_log2 : kNegInf;
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = xor_max<16>(mx);
      mx = xor_max<32>(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      u32x2 p_hi, p_lo;
      l_run = l_run * alpha + prob_operands<DT>(x, m_new, p_hi, p_lo);

      // O^T[d, head] += sum_t V[t, d] P[head, t].  The A operand (lane: dim 16c + col,
      // tokens 4*grp .. +3) is V^T; ds_read_b64_tr_b16 transposes it out of the
      // row-major tile: within each 16-lane group, result lane i, element j comes
      // from source lane i/4 + 4j, element i%4, so source lane r addresses row
      // 4*grp + r/4, columns 16c + 4*(r%4) .. +3.
      const bool tail = t0 + kTile > t_end;
      uint32_t keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;   // masks slots past the end
      if (tail) {
        const int n = t_end - tk;                                 // valid tokens of this lane
        keep_lo = (n > 0 ? 0x0000ffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
        keep_hi = (n > 2 ? 0x0000ffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
      }
      const int vrow = 4 * grp + (col >> 2);
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        const int vcol = 16 * c + 4 * (col & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(ldsV + ZV::byte_off(vrow, vcol >> 3) + (vcol & 7) * 2));
        u32x2 vop = __builtin_bit_cast(u32x2, raw);
        vop.x &= keep_lo;
        vop.y &= keep_hi;
        acc[c] = pv_mfma<DT>(vop, p_hi, p_lo, acc[c] * alpha);
      }
    } else {
      // head-sequential: pass h updates query head h (column h) alone; the other
      // columns get a zero Q operand, P = 0 and a rescale of 1
      const int tk = t0 + 4 * grp;
      const bool tail = t0 + kTile > t_end;
      uint32_t keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;
      if (tail) {
        const int n = t_end - tk;
        keep_lo = (n > 0 ? 0x0000ffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
        keep_hi = (n > 2 ? 0x0000ffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
      }
      const int vrow = 4 * grp + (col >> 2);
      for (int h = 0; h < G; ++h) {
        const bool live = col == h;
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = Z::byte_off(col, 4 * ks + grp);
          const u32x4 kop = *reinterpret_cast<const u32x4*>(ldsK + off);
          const u32x4 q = *reinterpret_cast<const u32x4*>(sm.q + off);
          st = DT::mfma_qk(kop, live ? q : u32x4{0, 0, 0, 0}, st);
        }
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (tk + e < t_end) ? st[e] * a.scale_log2 : kNegInf;
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = xor_max<16>(mx);
        mx = xor_max<32>(mx);
        const float m_new = live ? fmaxf(m_run, mx) : m_run;
        const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        m_run = m_new;
        u32x2 p_hi, p_lo;
        const float psum = prob_operands<DT>(x, m_new, p_hi, p_lo);
        if (!live) p_hi = p_lo = u32x2{0u, 0u};
        l_run = live ? l_run * alpha + psum : l_run;
#pragma unroll
        for (int c = 0; c < DB; ++c) {
          const int vcol = 16 * c + 4 * (col & 3);
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(ldsV + ZV::byte_off(vrow, vcol >> 3) + (vcol & 7) * 2));
          u32x2 vop = __builtin_bit_cast(u32x2, raw);
          vop.x &= keep_lo;
          vop.y &= keep_hi;
          acc[c] = pv_mfma<DT>(vop, p_hi, p_lo, acc[c] * alpha);
        }
      }
    }
  }

  // full exp sum of head `col` for this wave
  l_run = xor_add<16>(l_run);
  l_run = xor_add<32>(l_run);

  // merge the W wave states: waves 1..W-1 park (acc, m, l) in LDS, wave 0 combines
  __syncthreads();
  f32x4* park = reinterpret_cast<f32x4*>(sm.tiles);                    // [W-1][DB][64]
  float* park_m = reinterpret_cast<float*>(park + (W - 1) * DB * 64);  // [W-1][64]
  float* park_l = park_m + (W - 1) * 64;                               // [W-1][64]
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < DB; ++c) park[((wave - 1) * DB + c) * 64 + lane] = acc[c];
    park_m[(wave - 1) * 64 + lane] = m_run;
    park_l[(wave - 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (wave == 0) {
    float M = m_run;
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, park_m[(w - 1) * 64 + lane]);
    const bool empty = M == kNegInf;   // no token at all (seq_len <= 0)
    const float f = empty ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    float Lsum = f * l_run;
#pragma unroll
    for (int c = 0; c < DB; ++c) acc[c] *= f;
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const float mw = park_m[(w - 1) * 64 + lane];
      const float fw = empty ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      Lsum += fw * park_l[(w - 1) * 64 + lane];
#pragma unroll
      for (int c = 0; c < DB; ++c) acc[c] += fw * park[((w - 1) * DB + c) * 64 + lane];
    }
    if (col < G) {
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
      if (final) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + ((size_t)s * Hq + unit * G + col) * D +
                      4 * grp;
#pragma unroll
        for (int c = 0; c < DB; ++c) {
          const f32x4 y = acc[c] * inv;
          const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                                DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
          *reinterpret_cast<u32x2*>(o + 16 * c) = packed;
        }
      } else if (a.tickets != nullptr) {
#pragma unroll
        for (int c = 0; c < DB; ++c)
          store_dev(a.ws_acc + rec_acc_index(c, rec, col, G, a.records) + 4 * grp, acc[c] * inv);
        if (grp == 0) store_dev(a.ws_ml + rec * G + col, make_float2(M, Lsum));
      } else {
#pragma unroll
        for (int c = 0; c < DB; ++c)
          *reinterpret_cast<f32x4*>(a.ws_acc + rec_acc_index(c, rec, col, G, a.records) +
                                    4 * grp) = acc[c] * inv;
        if (grp == 0) a.ws_ml[rec * G + col] = make_float2(M, Lsum);
      }
    }
  }
  if (!final && a.tickets != nullptr && mg.seg >= 0) finish_partial<D, DT, W>(a, sm, s, unit, mg);
}

// Grid mode: workgroup (partition, sequence, KV head), partition slowest.  HS: the
// head-sequential ablation (see run_piece).
template <int D, class DT, int W, bool HS = false>
__global__ __launch_bounds__(W * 64, HS ? 1 : 8 / W) void pa_phase1_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) Phase1Lds<D, W> sm;
  int wg = blockIdx.x;
  int unit, s, part;
  if (a.xcd_skew > 0) {
    // partition fastest, so the two partitions of a pair run on XCDs of opposite
    // parity
    part = wg % a.max_parts;
    wg /= a.max_parts;
    unit = wg % a.units;
    s = wg / a.units;
  } else {
    unit = wg % a.units;
    wg /= a.units;
    s = wg % a.num_seqs;
    part = wg / a.num_seqs;
  }
  const int L = clamp_len(a, s);
  const bool single = L <= a.single_pass_max_len;
  int t_begin, t_end;
  if (single) {
    if (part != 0) return;
    t_begin = 0;
    t_end = L > 0 ? L : 0;
  } else {
    const int P = a.partition_size;
    const int np = (L + P - 1) / P;
    if (part >= np) return;
    t_begin = part * P;
    t_end = min(L, t_begin + P);
    if (a.xcd_skew > 0 && (part | 1) < np) {
      // partitions 2i and 2i+1 split [2iP, 2iP + 2P) at a 16-token cut that gives
      // the member with the even block index (even XCD) the larger part
      const int base = (part & ~1) * P;
      const int big = min(2 * P, (P + P / 1000 * a.xcd_skew + P % 1000 * a.xcd_skew / 1000 +
                                  kTile - 1) / kTile * kTile);
      const bool first_big = ((blockIdx.x - (part & 1)) & 1) == 0;
      const int cut = base + (first_big ? big : 2 * P - big);
      t_begin = (part & 1) ? min(L, cut) : base;
      t_end = (part & 1) ? min(L, base + 2 * P) : min(L, cut);
    }
  }
  const long long seg = (long long)s * a.units + unit;
  const long long rec = seg * a.max_parts + part;
  SegMerge mg{-1, 0, 0, 0, 0};
  if (!single) {
    mg.seg = static_cast<int>(seg);
    mg.np = (L + a.partition_size - 1) / a.partition_size;
    mg.rec0 = seg * a.max_parts;
    mg.step = 1;
  }
  run_piece<D, DT, W, HS>(a, sm, s, unit, t_begin, t_end, single, rec, mg);
}

// Balanced mode.  Sequence s has n(s) = ceil(L_s/16) tiles per KV head; laid end
// to end they make T tiles, cut into NS = num_wg/Hkv shares.  Workgroup w takes
// share j = w / Hkv of KV head kvh = w % Hkv, so the Hkv workgroups of a share
// run side by side and read the Hkv contiguous chunks of the same pages; with
// XCD-paired shares (xcd_skew > 0, NS even) workgroup w takes share
// j = 2*(w / (2*Hkv)) + w % 2 of KV head (w / 2) % Hkv instead, so the two shares
// of a pair run on XCDs of opposite parity and the even one is the larger.  Its
// partial records are indexed by r = j*Hkv + kvh either way.  Each workgroup
// rebuilds the per-sequence prefix of tiles in LDS from seq_lens
// (S <= kMaxBalancedSeqs), then walks its share.  Starting a piece costs about
// as much as streaming piece_cost tiles (its Q, block-table and first K/V round
// trips, the wave merge and the record), so every sequence with tokens counts
// piece_cost virtual tiles before its real ones, and the shares are cut in
// these virtual tiles: a share that starts more pieces gets fewer real tiles.
template <int D, class DT, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void pa_phase1_balanced_kernel(DecodeArgs a) {
  constexpr int NT = W * 64;
  constexpr int PER = kMaxBalancedSeqs / NT;
  __shared__ __attribute__((aligned(16))) Phase1Lds<D, W> sm;
  __shared__ int pre[kMaxBalancedSeqs + 1];     // pre[s] = virtual tiles of sequences < s
  __shared__ unsigned char last_len[kMaxBalancedSeqs];   // tokens in a sequence's last tile
  __shared__ int wave_tot[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.num_seqs, Hkv = a.num_kv_heads;
  const int w = blockIdx.x;
  const int NS = a.num_wg / Hkv;
  const int skew = a.xcd_skew;
  const int j = skew > 0 ? 2 * (w / (2 * Hkv)) + (w & 1) : w / Hkv;
  const int kvh = skew > 0 ? (w >> 1) % Hkv : w % Hkv;
  const int r = j * Hkv + kvh;      // record slot pair and job of this share
  const int c = a.piece_cost;       // virtual tiles ahead of each sequence with tokens

  // ---- inclusive scan of tiles per sequence: thread tid owns sequences tid*PER ..
  int local[PER];
  int tsum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = tid * PER + i;
    int n = 0;
    if (s < S) {
      const int L = clamp_len(a, s);
      n = L > 0 ? (L + kTile - 1) / kTile : 0;
      last_len[s] = static_cast<unsigned char>(L > 0 ? L - kTile * (n - 1) : 0);
      if (n > 0) n += c;
    }
    tsum += n;
    local[i] = tsum;
  }
  int incl = tsum;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int v = __shfl_up(incl, k, 64);
    if (lane >= k) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - tsum;
  for (int v = 0; v < wave; ++v) base += wave_tot[v];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = tid * PER + i;
    if (s < S) pre[s + 1] = base + local[i];
  }
  if (tid == 0) pre[0] = 0;
  __syncthreads();

  // everything below is the same for all lanes: keep it in scalar registers
  const int T = uniform(pre[S]);
  const long long lo = share_cut(T, j, NS, skew), hi = share_cut(T, j + 1, NS, skew);

  // sequences of length <= 0 get zero rows; spread over the workgroups
  for (int s = w; s < S; s += a.num_wg) {
    if (uniform(pre[s + 1]) == uniform(pre[s])) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + (size_t)s * a.num_heads * D;
      for (int i = tid; i < a.num_heads * D / 8; i += NT)
        reinterpret_cast<u32x4*>(o)[i] = u32x4{0, 0, 0, 0};
    }
  }

  // share holding tile t
  auto share_of = [&](long long t) { return share_holding(T, t, NS, skew); };
  // the records of sequence s's partials: slot 1 of the share that holds its first
  // real tile, then slot 0 of each following share up to the one holding its last
  auto seg_merge = [&](int s) {
    const long long j0 = share_of(uniform(pre[s]) + c);
    const long long j1 = share_of(uniform(pre[s + 1]) - 1);
    return SegMerge{s * Hkv + kvh, static_cast<int>(j1 - j0 + 1), 2 * (j0 * Hkv + kvh),
                    2LL * Hkv, 1};
  };
  // the sequence holding tile t < T: largest s with pre[s] <= t (it has tiles)
  auto seq_of = [&](long long t) {
    int s = 0, top = S - 1;
    while (s < top) {
      const int mid = (s + top + 1) >> 1;
      if (uniform(pre[mid]) <= t) s = mid; else top = mid - 1;
    }
    return s;
  };

  int job_q = -1, job_n = 0;
  if (lo == hi) {
    // an empty share (fewer tiles than shares) may lie inside a sequence that
    // neighbouring shares split: leave the identity (-inf, 0) in slot 0
    for (int h = tid; h < a.group; h += NT) {
      if (a.tickets != nullptr)
        store_dev(a.ws_ml + 2LL * r * a.group + h, make_float2(kNegInf, 0.f));
      else
        a.ws_ml[2LL * r * a.group + h] = make_float2(kNegInf, 0.f);
    }
    if (a.tickets != nullptr && lo > 0 && lo < T) {
      // inside sequence s iff tiles lo - 1 and lo are both real tiles of it; the
      // identity then counts among its partials
      const int s = seq_of(lo);
      if (uniform(pre[s]) + c < lo) finish_partial<D, DT, W>(a, sm, s, kvh, seg_merge(s));
    }
  } else {
    int s = seq_of(lo);
    int x = static_cast<int>(lo);
    const int x_end = static_cast<int>(hi);
    while (x < x_end) {
      // real tiles of s: virtual [seg0, seg1); the share's part of them, if any
      const int seg0 = uniform(pre[s]) + c, seg1 = uniform(pre[s + 1]);
      const int n = seg1 - seg0;
      const int xs = max(x, seg0), xe = min(x_end, seg1);
      if (xs < xe) {
        const int ta = xs - seg0;
        const int tb = xe - seg0;
        const bool final = ta == 0 && tb == n;
        const long long rec = 2LL * r + (ta > 0 ? 0 : 1);
        if (ta == 0 && !final) {
          // this share starts a sequence that later shares continue: it owns the merge
          job_q = s * Hkv + kvh;
          job_n = static_cast<int>(share_of(seg1 - 1) - j + 1);
        }
        // the piece ends at its last tile, or at the sequence's last token
        const int t_end = tb == n ? kTile * (n - 1) + uniform(last_len[s]) : kTile * tb;
        run_piece<D, DT, W>(a, sm, s, kvh, kTile * ta, t_end, final, rec,
                            final ? SegMerge{-1, 0, 0, 0, 0} : seg_merge(s));
      }
      x = min(seg1, x_end);
      do { ++s; } while (s < S && uniform(pre[s + 1]) == uniform(pre[s]) && x < x_end);
    }
  }
  if (tid == 0) a.jobs[r] = make_int2(job_q, job_n);
}

// ---------------------------------------------------------------------------
// Phase 2: merge the partials of every partitioned segment.
// ---------------------------------------------------------------------------
constexpr int kRedThreads = 256;
constexpr int kRedWaves = kRedThreads / 64;
// partials of every head a thread of pa_reduce_kernel loads per round
__host__ __device__ constexpr int reduce_unroll(int G) {
  return G >= 16 ? 1 : (G >= 6 ? 2 : (G >= 3 ? 4 : 8));
}

// Workgroup = (segment, SPW consecutive 16-wide head_dim slices).  Thread
// (pg, ql) covers head_dim values 4*ql .. +3 of the workgroup's slices and folds
// partials p = pg, pg + PG, ... of every head into a running partial, issuing all
// loads of a round (G heads x U partials) before consuming any; the PG groups are
// then combined with the same rule by lane shuffles and through LDS.  SPW = 1
// spreads a segment over D/16 workgroups of up to PG*U = 64*U partials a round, for
// many partials per segment; a larger SPW takes fewer, wider workgroups.
//   fixed partitions (a.jobs == nullptr): workgroup (segment q, slice group),
//     partials q*max_parts + p for p < ceil(L/P); segments in one pass are skipped.
//   balanced split: workgroup (w, slice group) merges the segment begun by phase-1
//     workgroup w, if any: record 2w+1, then 2(w+p*Hkv) for p >= 1 (the same KV
//     head in the following shares).
template <int D, class DT, int G, int SPW>
__global__ __launch_bounds__(kRedThreads) void pa_reduce_kernel(DecodeArgs a) {
  constexpr int NSG = D / 16 / SPW;        // slice groups per segment
  constexpr int QL = 4 * SPW;              // float4 lanes per partial group
  constexpr int PG = kRedThreads / QL;     // partial groups
  constexpr int U = reduce_unroll(G);
  static_assert(QL <= 64, "a partial group must fit in a wave");
  __shared__ float red_m[kRedWaves][G][QL], red_w[kRedWaves][G][QL];
  __shared__ f32x4 red_a[kRedWaves][G][QL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads, Hq = a.num_heads;
  const int sg = blockIdx.x % NSG;
  const int slot = blockIdx.x / NSG;       // segment (grid mode) or phase-1 workgroup

  int q, np;
  long long rec0, step, first;
  if (a.jobs != nullptr) {
    const int2 job = a.jobs[slot];
    if (job.x < 0) return;
    q = job.x;
    np = job.y;
    rec0 = 2LL * slot;
    step = 2LL * Hkv;
    first = 1;
  } else {
    q = slot;
    const int L = clamp_len(a, q / a.units);
    if (L <= a.single_pass_max_len) return;     // served in one pass by phase 1
    np = (L + a.partition_size - 1) / a.partition_size;
    rec0 = (long long)q * a.max_parts;
    step = 1;
    first = 0;
  }
  const int s = q / a.units, unit = q % a.units;   // balanced mode: units == Hkv
  const long long R = a.records;

  const int ql = tid % QL;
  const int pg = tid / QL;
  const int slice = sg * SPW + ql / 4;
  const int q4 = ql % 4;
  Partial st[G];
#pragma unroll
  for (int h = 0; h < G; ++h) st[h] = Partial{kNegInf, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int p0 = pg; p0 < np; p0 += PG * U) {
    f32x4 v[G][U];
    float2 m[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pc = min(p0 + u * PG, np - 1);           // always a written record
      const long long rec = rec0 + step * pc + (pc == 0 ? first : 0);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h][u] = a.ws_ml[rec * G + h];
        v[h][u] = *reinterpret_cast<const f32x4*>(a.ws_acc + rec_acc_index(slice, rec, h, G, R) +
                                                  4 * q4);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // a record holds the piece's normalised output: weight sum l, weighted sum l*acc;
        // a max of -inf marks the identity (an empty share in balanced mode)
        const bool ok = p0 + u * PG < np && m[h][u].x != kNegInf;
        combine_into(st[h], ok ? m[h][u].x : kNegInf, ok ? m[h][u].y : 0.f,
                     ok ? m[h][u].y * v[h][u] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // combine the partial groups of this wave (lane bits log2(QL) .. 5)
#pragma unroll
    for (int k = QL; k < 64; k <<= 1) {
      const float om = __shfl_xor(st[h].m, k, 64);
      const float ow = __shfl_xor(st[h].w, k, 64);
      f32x4 oa;
#pragma unroll
      for (int e = 0; e < 4; ++e) oa[e] = __shfl_xor(st[h].a[e], k, 64);
      combine_into(st[h], om, ow, oa);
    }
    if (lane < QL) {
      red_m[wave][h][lane] = st[h].m;
      red_w[wave][h][lane] = st[h].w;
      red_a[wave][h][lane] = st[h].a;
    }
  }
  __syncthreads();
  for (int i = tid; i < G * QL; i += kRedThreads) {
    const int h = i / QL, qq = i % QL;
    Partial t{red_m[0][h][qq], red_w[0][h][qq], red_a[0][h][qq]};
#pragma unroll
    for (int w = 1; w < kRedWaves; ++w) combine_into(t, red_m[w][h][qq], red_w[w][h][qq], red_a[w][h][qq]);
    const f32x4 y = t.a * (1.f / t.w);
    uint16_t* o = static_cast<uint16_t*>(a.out) + ((size_t)s * Hq + unit * G + h) * D +
                  sg * SPW * 16 + 4 * qq;
    const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                          DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
    *reinterpret_cast<u32x2*>(o) = packed;
  }
}

// Clears n 16-byte words (the fused combine's ticket area).
__global__ __launch_bounds__(256) void pa_zero_kernel(u32x4* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// Gather probe: the phase-1 addressing and tile loads, stored to a contiguous copy.
// One workgroup of 4 waves per (sequence, KV head).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pa_gather_kernel(GatherArgs a) {
  constexpr int LOADS = D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int s = blockIdx.x / a.num_kv_heads;
  const int L = min(a.seq_lens[s], a.max_seq_len);
  const int n_tiles = L > 0 ? (L + kTile - 1) / kTile : 0;
  for (int it = wave; it < n_tiles; it += 4) {
    const int t0 = kTile * it;
    size_t lo, hi;
    tile_offsets(tile_pages(a.bt, s, t0, L, a.block_size, a.max_blocks_per_seq), t0, kvh,
                 a.num_kv_heads, a.block_size, D, lo, hi);
    u32x4 rk[LOADS], rv[LOADS];
    load_tile<D>(a.kc + lo, a.kc + hi, lane, rk);
    load_tile<D>(a.vc + lo, a.vc + hi, lane, rv);
    const size_t dst = (((size_t)s * a.num_kv_heads + kvh) * a.max_seq_len + t0) * D;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = j * 64 + lane;           // 16-byte chunk within the tile
      const int row = c / (D / 8);
      if (t0 + row < L) {
        reinterpret_cast<u32x4*>(a.k_out + dst)[c] = rk[j];
        reinterpret_cast<u32x4*>(a.v_out + dst)[c] = rv[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Read probe: what the box delivers to the decode's access pattern.  The pages'
// case for the KV-head grid is the K/V bytes read (page of commit 8d26e23, "Key
// design change"), so the decode is bounded by read bandwidth; this kernel reads
// n chunks of CB bytes (one (page, KV head) block of the caches: 8 KiB at 16
// tokens x head_dim 256) with the phase-1 load form (nontemporal 16-byte loads,
// 1 KiB contiguous per instruction), in order or in the order of a permutation,
// two chunks in flight per wave, folds them with XOR and writes one word per
// workgroup.  Workgroup b takes chunks [n*b/grid, n*(b+1)/grid), wave w every
// fourth of them starting at w.
// ---------------------------------------------------------------------------
template <int CB>
__global__ __launch_bounds__(256) void pa_read_probe_kernel(const u32x4* __restrict__ src,
                                                            const long long* order, long long n,
                                                            unsigned* sink) {
  constexpr int NL = CB / 1024;             // loads per lane per chunk
  typedef const __attribute__((address_space(4))) long long const_i64;
  __shared__ unsigned fold[256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long c0 = n * blockIdx.x / gridDim.x, c1 = n * (blockIdx.x + 1) / gridDim.x;
  u32x4 acc = {0, 0, 0, 0};
  auto load = [&](long long c, u32x4 (&d)[NL]) {
    const long long id = order ? ((const_i64*)order)[c] : c;
    const u32x4* p = src + id * (CB / 16);
#pragma unroll
    for (int j = 0; j < NL; ++j) d[j] = __builtin_nontemporal_load(p + j * 64 + lane);
  };
  auto consume = [&](const u32x4 (&d)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) acc ^= d[j];
  };
  u32x4 ra[NL], rb[NL];
  long long c = c0 + wave;
  if (c < c1) load(c, ra);
  if (c + 4 < c1) load(c + 4, rb);
  for (; c < c1; c += 8) {
    consume(ra);
    if (c + 8 < c1) load(c + 8, ra);
    if (c + 4 < c1) {
      consume(rb);
      if (c + 12 < c1) load(c + 12, rb);
    }
  }
  fold[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned x = 0;
    for (int i = 0; i < 256; ++i) x ^= fold[i];
    sink[blockIdx.x] = x;
  }
}

}  // namespace pa
