// Device code of libpagedattn: GQA-grouped paged-attention decode for gfx950 (CDNA4).
//
// Phase 1 (pa_phase1_kernel): one workgroup per (sequence, KV head, partition).
// The workgroup serves every query head of the KV head's group, so each K/V
// page is fetched from HBM once (page of commit 8d26e23, "Key design change":
// grid on KV heads instead of query heads).  Its W waves split the partition's
// 16-token tiles; each wave
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
// (single-pass tier) or the partition's compound partial (page of commit
// 8d26e23: max_score, exp_sum, weighted_v).
//
// Phase 2 (pa_reduce_kernel): one workgroup per (sequence, KV head, 16-wide
// slice of head_dim) merges the partials of all partitions for the group's
// query heads with the rescale of the online-softmax fix (page of commit
// 87a19d2): with M the largest max, each partition weighs l_p 2^(m_p - M) and
// out = sum_p weight_p acc_p / sum_p weight_p, evaluated as an associative fold.
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
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
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
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
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
struct DecodeArgs {
  void* out;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  float* ws_acc;            // [S][Hq][max_parts][D]
  float2* ws_ml;            // [S][Hq][max_parts] (max in base 2, exp sum)
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int block_size;
  int max_blocks_per_seq;
  int max_seq_len;          // lengths are clamped to this bound
  int partition_size;
  int single_pass_max_len;
  int max_parts;
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

// Tokens [t_begin, t_end) one phase-1 workgroup covers; false if it has nothing to do.
struct Span {
  int t_begin, t_end;
  bool single;
};

__device__ __forceinline__ bool workgroup_span(int L, int part, int P, int T1, Span& sp) {
  sp.single = L <= T1;
  if (sp.single) {
    if (part != 0) return false;
    sp.t_begin = 0;
    sp.t_end = L > 0 ? L : 0;
    return true;
  }
  const int np = (L + P - 1) / P;
  if (part >= np) return false;
  sp.t_begin = part * P;
  sp.t_end = min(L, sp.t_begin + P);
  return true;
}

// Workspace layout of the normalised partition outputs: [S*Hq][D/16][max_parts][16]
// floats, so the partitions of one 16-wide slice are contiguous (phase 2 reads
// 1 KiB runs) and phase 1 writes 64-byte runs.
__device__ __forceinline__ size_t ws_acc_index(size_t row, int c, int max_parts, int part,
                                               int D) {
  return ((row * (D / 16) + c) * max_parts + part) * 16;
}

// Element offset of token t0 (a multiple of 16) of KV head kvh of sequence s.
// 64-bit: pools above 4 G elements are legal.  The page id is wave-uniform.
__device__ __forceinline__ size_t tile_offset(const int32_t* bt, int s, int t0, int kvh,
                                              int Hkv, int bs, int mbps, int D) {
  const int page = __builtin_amdgcn_readfirstlane(bt[(size_t)s * mbps + t0 / bs]);
  return ((static_cast<size_t>(page) * Hkv + kvh) * bs + (t0 % bs)) * static_cast<size_t>(D);
}

// One 16-token tile is 16*D*2 bytes, contiguous.  Lane `lane` fetches the 16-byte
// chunks lane, lane+64, ... so every load instruction covers 1 KiB contiguously.
// K and V are read exactly once per step, so the loads are nontemporal: they do
// not displace reusable lines from the caches (worth ~10% of gather bandwidth).
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ src, int lane,
                                          u32x4 (&r)[D / 32]) {
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) r[j] = __builtin_nontemporal_load(s4 + j * 64 + lane);
}

// LDS slot of one tile: 16 rows of D halves, with 16-byte chunk c of row t stored
// at chunk position c ^ (t & (SW-1)).  The swizzle makes the row-strided MFMA
// operand reads and the column (transposed) reads of V bank-conflict free.
template <int D>
struct Swz {
  static constexpr int kChunks = D / 8;
  static constexpr int kSw = kChunks < 16 ? kChunks : 16;
  static __device__ __forceinline__ int chunk(int row, int c) { return c ^ (row & (kSw - 1)); }
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

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m, 64)); }
__device__ __forceinline__ float xor_add(float x, int m) { return x + __shfl_xor(x, m, 64); }

// ---------------------------------------------------------------------------
// Phase 1 (and the single-pass tier).
// ---------------------------------------------------------------------------
template <int D, class DT, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void pa_phase1_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA (32 dims each)
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int LOADS = D / 32;            // 16-byte loads per lane per tile (K or V)
  constexpr int TILE_BYTES = kTile * D * 2;
  using Z = Swz<D>;
  static_assert((W - 1) * DB * 64 * 16 + 2 * (W - 1) * 64 * 4 <= W * 2 * TILE_BYTES,
                "merge area must fit in the tile slots");
  __shared__ __attribute__((aligned(16))) unsigned char lds[W * 2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_q[TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_heads;

  int wg = blockIdx.x;
  const int kvh = wg % Hkv;
  wg /= Hkv;
  const int s = wg % a.num_seqs;
  const int part = wg / a.num_seqs;

  const int L = min(a.seq_lens[s], a.max_seq_len);
  Span sp;
  if (!workgroup_span(L, part, a.partition_size, a.single_pass_max_len, sp)) return;

  const int col = lane & 15;     // query head (QK^T/PV columns) or row index within a tile
  const int grp = lane >> 4;     // 4-lane-group index: k-slot block / 4-row block

  // the wave's first tile is requested before Q is staged, so the two latencies overlap
  const int n_tiles = (sp.t_end - sp.t_begin + kTile - 1) / kTile;
  u32x4 rk[LOADS], rv[LOADS];
  int it = wave;
  if (it < n_tiles) {
    const size_t off = tile_offset(a.bt, s, sp.t_begin + kTile * it, kvh, Hkv, a.block_size,
                                   a.max_blocks_per_seq, D);
    load_tile<D>(a.kc + off, lane, rk);
    load_tile<D>(a.vc + off, lane, rv);
  }

  // Q of the group, staged once in LDS as the B operand of S^T = K Q^T: row h is
  // query head kvh*G + h (rows G..15 are zero), swizzled like a K tile.
  {
    const uint16_t* qg = a.q + ((size_t)s * Hq + (size_t)kvh * G) * D;
    for (int i = threadIdx.x; i < kTile * Z::kChunks; i += W * 64) {
      const int row = i / Z::kChunks, c = i % Z::kChunks;
      u32x4 v = {0, 0, 0, 0};
      if (row < G) v = *reinterpret_cast<const u32x4*>(qg + row * D + 8 * c);
      *reinterpret_cast<u32x4*>(lds_q + Z::byte_off(row, c)) = v;
    }
    __syncthreads();
  }

  float m_run = kNegInf;          // running max of the head `col` (base-2 logits)
  float l_run = 0.f;              // this lane's share of the running exp sum
  f32x4 acc[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  unsigned char* ldsK = lds + wave * 2 * TILE_BYTES;
  unsigned char* ldsV = ldsK + TILE_BYTES;

  for (; it < n_tiles; it += W) {
    const int t0 = sp.t_begin + kTile * it;
    // stage the tile in this wave's LDS slot
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = j * 64 + lane;
      const int row = c / Z::kChunks;
      const int off = Z::byte_off(row, c % Z::kChunks);
      *reinterpret_cast<u32x4*>(ldsK + off) = rk[j];
      *reinterpret_cast<u32x4*>(ldsV + off) = rv[j];
    }
    wave_lds_fence();
    // prefetch the wave's next tile while this one is consumed
    if (it + W < n_tiles) {
      const size_t off = tile_offset(a.bt, s, t0 + kTile * W, kvh, Hkv, a.block_size,
                                     a.max_blocks_per_seq, D);
      load_tile<D>(a.kc + off, lane, rk);
      load_tile<D>(a.vc + off, lane, rv);
    }

    // S^T[token, head] = sum_d K[token, d] Q[head, d]
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = Z::byte_off(col, 4 * ks + grp);
      const u32x4 kop = *reinterpret_cast<const u32x4*>(ldsK + off);
      const u32x4 qop = *reinterpret_cast<const u32x4*>(lds_q + off);
      st = DT::mfma_qk(kop, qop, st);
    }

    // online softmax in base 2; this lane holds head `col`, tokens t0 + 4*grp + e
    const int tk = t0 + 4 * grp;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (tk + e < sp.t_end) ? st[e] * a.scale_log2 : kNegInf;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pb[e] = DT::bits(__builtin_amdgcn_exp2f(x[e] - m_new));
      psum += DT::value(pb[e]);          // sum the weights the MFMA actually uses
    }
    l_run = l_run * alpha + psum;
    const u32x2 pop = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};

    // O^T[d, head] += sum_t V[t, d] P[head, t].  The A operand (lane: dim 16c + col,
    // tokens 4*grp .. +3) is V^T; ds_read_b64_tr_b16 transposes it out of the
    // row-major tile: within each 16-lane group, result lane i, element j comes
    // from source lane i/4 + 4j, element i%4, so source lane r addresses row
    // 4*grp + r/4, columns 16c + 4*(r%4) .. +3.
    const bool tail = t0 + kTile > sp.t_end;
    uint32_t keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;   // masks slots past the end
    if (tail) {
      const int n = sp.t_end - tk;                              // valid tokens of this lane
      keep_lo = (n > 0 ? 0x0000ffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
      keep_hi = (n > 2 ? 0x0000ffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
    }
    const int vrow = 4 * grp + (col >> 2);
#pragma unroll
    for (int c = 0; c < DB; ++c) {
      const int vcol = 16 * c + 4 * (col & 3);
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(ldsV + Z::byte_off(vrow, vcol >> 3) + (vcol & 7) * 2));
      u32x2 vop = __builtin_bit_cast(u32x2, raw);
      vop.x &= keep_lo;
      vop.y &= keep_hi;
      acc[c] = DT::mfma_pv(vop, pop, acc[c] * alpha);
    }
  }

  // full exp sum of head `col` for this wave
  l_run = xor_add(l_run, 16);
  l_run = xor_add(l_run, 32);

  // merge the W wave states: waves 1..W-1 park (acc, m, l) in LDS, wave 0 combines
  __syncthreads();
  f32x4* park = reinterpret_cast<f32x4*>(lds);                     // [W-1][DB][64]
  float* park_m = reinterpret_cast<float*>(park + (W - 1) * DB * 64);  // [W-1][64]
  float* park_l = park_m + (W - 1) * 64;                           // [W-1][64]
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < DB; ++c) park[((wave - 1) * DB + c) * 64 + lane] = acc[c];
    park_m[(wave - 1) * 64 + lane] = m_run;
    park_l[(wave - 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (wave != 0) return;

  float M = m_run;
#pragma unroll
  for (int w = 1; w < W; ++w) M = fmaxf(M, park_m[(w - 1) * 64 + lane]);
  const bool empty = M == kNegInf;   // no token at all (seq_len <= 0)
  float f = empty ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
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
  if (col >= G) return;
  const int hq = kvh * G + col;
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  if (sp.single) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + ((size_t)s * Hq + hq) * D + 4 * grp;
#pragma unroll
    for (int c = 0; c < DB; ++c) {
      const f32x4 y = acc[c] * inv;
      const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                            DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
      *reinterpret_cast<u32x2*>(o + 16 * c) = packed;
    }
  } else {
    const size_t row = (size_t)s * Hq + hq;
#pragma unroll
    for (int c = 0; c < DB; ++c)
      *reinterpret_cast<f32x4*>(a.ws_acc + ws_acc_index(row, c, a.max_parts, part, D) +
                                4 * grp) = acc[c] * inv;
    if (grp == 0) a.ws_ml[row * a.max_parts + part] = make_float2(M, Lsum);
  }
}

// ---------------------------------------------------------------------------
// Phase 2: merge the partitions of every partitioned sequence.
// ---------------------------------------------------------------------------
constexpr int kRedSlice = 16;                 // head_dim values per workgroup (one d-block)
constexpr int kRedQuads = kRedSlice / 4;      // float4 lanes per slice (fastest in a wave)
constexpr int kRedThreads = 256;
constexpr int kRedWaves = kRedThreads / 64;
constexpr int kRedGroups = kRedThreads / kRedQuads;   // partition groups (64)

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

// Workgroup (s, kvh, slice) merges the partitions of the G query heads of KV head
// kvh for head_dim values [16*slice, +16).  Thread (pg, q4) folds partitions
// p = pg + 64k of every head into a running partial (the rescale rule of the
// online-softmax fix), issuing all loads of a round (G heads x U partitions)
// before consuming any; the 64 partition groups are then combined with the same
// rule by lane shuffles (16 groups per wave) and through LDS (4 waves).  G is a
// template parameter so the per-head state lives in registers.
template <int D, class DT, int G>
__global__ __launch_bounds__(kRedThreads) void pa_reduce_kernel(DecodeArgs a) {
  constexpr int NSL = D / kRedSlice;
  constexpr int U = G >= 16 ? 1 : (G >= 6 ? 2 : (G >= 3 ? 4 : 8));
  __shared__ float red_m[kRedWaves][G][kRedQuads], red_w[kRedWaves][G][kRedQuads];
  __shared__ f32x4 red_a[kRedWaves][G][kRedQuads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, MP = a.max_parts;
  int wg = blockIdx.x;
  const int sl = wg % NSL;
  wg /= NSL;
  const int kvh = wg % Hkv;
  const int s = wg / Hkv;

  const int L = min(a.seq_lens[s], a.max_seq_len);
  if (L <= a.single_pass_max_len) return;       // served in one pass by phase 1
  const int np = (L + a.partition_size - 1) / a.partition_size;
  const size_t row0 = (size_t)s * Hq + (size_t)kvh * G;   // first query head of the group
  const float2* ml0 = a.ws_ml + row0 * MP;

  const int q4 = tid % kRedQuads;
  const int pg = tid / kRedQuads;
  Partial st[G];
#pragma unroll
  for (int h = 0; h < G; ++h) st[h] = Partial{kNegInf, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int p0 = pg; p0 < np; p0 += kRedGroups * U) {
    f32x4 v[G][U];
    float2 m[G][U];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* base = a.ws_acc + ws_acc_index(row0 + h, sl, MP, 0, D) + 4 * q4;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pc = min(p0 + u * kRedGroups, np - 1);   // always a written record
        m[h][u] = ml0[h * MP + pc];
        v[h][u] = *reinterpret_cast<const f32x4*>(base + (size_t)pc * 16);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // a record holds the partition's normalised output: weight sum l, weighted sum l*acc
        const bool ok = p0 + u * kRedGroups < np;
        combine_into(st[h], ok ? m[h][u].x : kNegInf, ok ? m[h][u].y : 0.f,
                     ok ? m[h][u].y * v[h][u] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // combine the 16 partition groups of this wave (lane bits 2..5)
#pragma unroll
    for (int k = kRedQuads; k < 64; k <<= 1) {
      const float om = __shfl_xor(st[h].m, k, 64);
      const float ow = __shfl_xor(st[h].w, k, 64);
      f32x4 oa;
#pragma unroll
      for (int e = 0; e < 4; ++e) oa[e] = __shfl_xor(st[h].a[e], k, 64);
      combine_into(st[h], om, ow, oa);
    }
    if (lane < kRedQuads) {
      red_m[wave][h][lane] = st[h].m;
      red_w[wave][h][lane] = st[h].w;
      red_a[wave][h][lane] = st[h].a;
    }
  }
  __syncthreads();
  if (tid < G * kRedQuads) {
    const int h = tid / kRedQuads, qq = tid % kRedQuads;
    Partial t{red_m[0][h][qq], red_w[0][h][qq], red_a[0][h][qq]};
#pragma unroll
    for (int w = 1; w < kRedWaves; ++w) combine_into(t, red_m[w][h][qq], red_w[w][h][qq], red_a[w][h][qq]);
    const f32x4 y = t.a * (1.f / t.w);
    uint16_t* o = static_cast<uint16_t*>(a.out) + (row0 + h) * D + sl * kRedSlice + 4 * qq;
    const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                          DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
    *reinterpret_cast<u32x2*>(o) = packed;
  }
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
    const size_t off = tile_offset(a.bt, s, t0, kvh, a.num_kv_heads, a.block_size,
                                   a.max_blocks_per_seq, D);
    u32x4 rk[LOADS], rv[LOADS];
    load_tile<D>(a.kc + off, lane, rk);
    load_tile<D>(a.vc + off, lane, rv);
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

}  // namespace pa
