// Prefill over a paged context on gfx950: the prefix path of the page of commit
// b80fd2b (paged_attn.py: _forward_prefix_pytorch, one online softmax over the
// context gathered from the caches by block id, then over the current chunk
// under the causal mask; rewrite item 1: the context is gathered once).
//
// New token n of sequence s (row r = query_start[s] + n of q, k_new, v_new)
// attends, for every query head of a KV head's group, to the C = ctx_lens[s]
// cached tokens and to the new tokens j <= n.  With many query rows per KV head
// the product is a real GEMM.  A "column" is one (new token, query head of the
// group) pair (column m = n*G + g); a workgroup of 4 waves takes 128 columns, each
// wave two blocks of 16, and streams the keys through them once:
//   - keys go in steps of 32 (two 16-token tiles: context tiles through the block
//     table, then tiles of the chunk's own rows).  Each wave moves one of the step's
//     four tiles (K or V of keys 0..15 or 16..31) from global memory straight into
//     LDS (global_load_lds_dwordx4: 64 lanes x 16 bytes, one KiB of contiguous LDS
//     per instruction, one page lookup per tile), double-buffered with one step of
//     look-ahead and one barrier per step;
//   - tiles are unpadded rows XOR-swizzled as the decode tiles are (Swz), so the
//     MFMA operand reads are conflict-free and each is a lane base XORed with a
//     loop constant;
//   - each wave computes S^T = K Q^T for its two column blocks and the step's two
//     tiles with v_mfma_f32_16x16x32 (Q^T stays in registers; every K operand read
//     feeds both blocks), one online softmax update per column over the 32 keys in
//     base 2, and O^T += V^T P^T with one double-rate v_mfma_f32_16x16x32 per 16
//     head dims and block (every V^T operand, read by ds_read_b64_tr_b16, feeds both
//     blocks).  The accumulators are rescaled only when a column's max grows by
//     more than 2^8; the exp sums are taken from the same rounded probabilities
//     with v_dot2 into one register per lane;
//   - the causal mask keeps key j for column (n, g) iff j <= n; steps past a
//     wave's last token are skipped, steps past the workgroup's last token are
//     not loaded.
// Holding two column blocks per wave halves the LDS bytes read per MFMA against one
// block, which bounds the kernel otherwise; the direct loads free the registers the
// second block needs (no staging registers) at two workgroups per CU.
// The grid is XCD-aware: every column block of one (sequence, KV head) runs on
// the same XCD, so their repeated reads of its K/V hit that XCD's L2.
#pragma once

#include "pa_kernels.h"

namespace pa {

struct PrefillArgs {
  void* out;                 // [T][Hq][D]
  const uint16_t* q;         // [T][Hq][D]
  const uint16_t* k_new;     // [T][Hkv][D]
  const uint16_t* v_new;     // [T][Hkv][D]
  const uint16_t* kc;        // [NB][Hkv][bs][D]
  const uint16_t* vc;
  const int32_t* bt;         // [S][mbps]
  const int32_t* ctx_lens;   // [S]
  const int32_t* qstart;     // [S+1]
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int block_size;
  unsigned bs_magic;         // t / block_size == umulhi(t, bs_magic) >> bs_shift, t < 2^31
  int bs_shift;
  int max_blocks_per_seq;
  int max_query_len;         // lengths are clamped to these bounds
  int max_ctx_len;
  int col_blocks;            // column blocks per (sequence, KV head)
  float scale_log2;
};

constexpr int kPrefillWaves = 4;                    // one wave per tile of a step
constexpr int kPfBlocks = 2;                        // 16-column blocks per wave
constexpr int kPrefillCols = 16 * kPfBlocks * kPrefillWaves;   // columns per workgroup
constexpr int kXcds = 8;                            // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kPfKsGroup = 2;   // K operand reads in flight: two k-steps, between scheduling barriers
constexpr int kPfCGroup = 4;    // V^T operand reads in flight: four head_dim blocks

// The two phases of a workgroup's key loop: the cached context, then the chunk.
template <bool kCtx>
struct PrefillPhase { static constexpr bool ctx = kCtx; };

constexpr int kPrefillHalves = 2;                      // 16-token tiles per step
constexpr int kPrefillStep = kTile * kPrefillHalves;   // keys per softmax step

// The running max of a column moves only when a step's max exceeds it by more than
// this (base 2): otherwise the step's probabilities are taken against the old max,
// each at most 2^8 (well inside f16 and bf16), and the accumulators are not rescaled.
constexpr float kRescaleLog2 = 8.f;

template <int D>
struct PfStep {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = kTile * kRowBytes;         // one 16-row tile
  static constexpr int kBytes = 4 * kTileBytes;                // K0, K1, V0, V1
};


// acc + the two 16-bit values packed in w (an f16 or bf16 pair of P), summed in fp32
template <class DT>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  if constexpr (DT::kSplitP)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           bf16x2{(__bf16)1.f, (__bf16)1.f}, acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
}

// Two probabilities rounded (to nearest even) to the element type and packed, in one
// conversion instruction (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950).
template <class DT>
__device__ __forceinline__ uint32_t pack_pair(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (DT::kSplitP) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
}

// P.V MFMA operands p_e = 2^arg_e rounded to the element type (hi + lo with
// kSplitP), with packed conversions; the exp sum is taken separately.
template <class DT>
__device__ __forceinline__ void prefill_probs(const float (&arg)[4], u32x2& hi, u32x2& lo) {
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(arg[e]);
  hi = u32x2{pack_pair<DT>(p[0], p[1]), pack_pair<DT>(p[2], p[3])};
  if constexpr (DT::kSplitP) {
    // the remainders p - hi are exact in fp32; a bf16 value is its bits << 16
    const float h0 = __builtin_bit_cast(float, hi.x << 16);
    const float h1 = __builtin_bit_cast(float, hi.x & 0xffff0000u);
    const float h2 = __builtin_bit_cast(float, hi.y << 16);
    const float h3 = __builtin_bit_cast(float, hi.y & 0xffff0000u);
    lo = u32x2{pack_pair<DT>(p[0] - h0, p[1] - h1), pack_pair<DT>(p[2] - h2, p[3] - h3)};
  } else {
    lo = u32x2{0u, 0u};
  }
}

// LDS address of 16-byte chunk c of row `row` in a swizzled tile is
// row * 2D + 16 * (c ^ f(row)).  For the MFMA operand reads the lane-dependent part
// and the loop index separate under XOR: with c = 4*ks + grp (K) or 2*c' + h (V),
// 16 * (c ^ f) = lane_part ^ (64*ks) or lane_part ^ (32*c'), since the loop bits sit
// above the lane bits and below the row bits.
// GPP: 8-token groups per page lookup, 1 for 8-token pages, else 2 (a 16-token tile
// always lies in one page when the page size is a multiple of 16)
template <int D, class DT, int GPP>
__global__ __launch_bounds__(kPrefillWaves * 64, 2) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int RPI = 64 / CH;             // rows per load instruction (1 KiB)
  constexpr int NI = kTile / RPI;          // load instructions per tile
  using Z = Swz<D, false>;
  using ZV = Swz<D, true>;
  using L = PfStep<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[L::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[L::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;

  // XCD-aware decode of the workgroup index: workgroup i runs on XCD i % 8; the
  // k-th workgroup of XCD x takes column block k % col_blocks of unit
  // x + 8 * (k / col_blocks), units being (sequence, KV head) pairs.
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int unit = xcd + kXcds * (k / a.col_blocks);
  const int cb = k % a.col_blocks;
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  if (unit >= a.num_seqs * Hkv) return;
  const int s = unit / Hkv, kvh = unit % Hkv;
  const int r0 = a.qstart[s];
  const int Qn = min(max(a.qstart[s + 1] - r0, 0), a.max_query_len);
  const int C = min(max(a.ctx_lens[s], 0), a.max_ctx_len);
  const int m0 = cb * kPrefillCols;
  if (m0 >= Qn * G) return;
  const int n_hi = min(Qn - 1, (m0 + kPrefillCols - 1) / G);          // last token of the workgroup
  const int wave_m0 = m0 + 16 * kPfBlocks * wave;
  const int wave_n_hi = min(Qn - 1, (wave_m0 + 16 * kPfBlocks - 1) / G);
  const bool wave_active = wave_m0 < Qn * G;

  // this lane's column in block b: token n_col[b], query head kvh*G + g.  With a
  // negative scale Q is negated here (sign bits: exact, and K.(-q) = -(K.q) exactly)
  // and |scale| is used, so the scale in the exponent is positive.
  const float sc = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  int n_col[kPfBlocks];
  bool col_valid[kPfBlocks];
  u32x4 qop[kPfBlocks][KS];
#pragma unroll
  for (int b = 0; b < kPfBlocks; ++b) {
    const int m = wave_m0 + 16 * b + col;
    col_valid[b] = m < Qn * G;
    n_col[b] = m / G;
    const uint16_t* qrow = a.q + ((size_t)(r0 + n_col[b]) * Hq + kvh * G + m % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[b][ks] = (col_valid[b] ? *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * ks + grp))
                                 : u32x4{0, 0, 0, 0}) ^ qsign;
  }

  const int bs = a.block_size, mbps = a.max_blocks_per_seq;
  const int n_ctx_steps = (C + kPrefillStep - 1) / kPrefillStep;
  const int n_steps = n_ctx_steps + n_hi / kPrefillStep + 1;

  // The tile this wave loads: K (waves 0, 1) or V (2, 3) of keys 16*h .. 16*h + 15.
  const bool ld_v = wave >= 2;
  const int ld_h = wave & 1;
  const int ld_dst = (ld_v ? 2 : 0) * L::kTileBytes + ld_h * L::kTileBytes;
  // Lane l of load instruction j fills LDS bytes 1024*j + 16*l of the tile: row
  // RPI*j + l/CH, chunk position l%CH, which holds chunk (l%CH) ^ f(row).  With
  // f(RPI*j + q) = f(q) ^ (RPI*j mod CH), the source offset within the tile is
  // 1024*j + (lane_src ^ 16*(RPI*j mod CH)).
  const int q_row = lane / CH, p_pos = lane % CH;
  const int f_q = (ld_v ? ZV::f(q_row) : Z::f(q_row)) & (CH - 1);
  const unsigned lane_pos0 = static_cast<unsigned>(16 * (p_pos ^ f_q));   // within the row
  const unsigned lane_src0 = static_cast<unsigned>(q_row * L::kRowBytes) + lane_pos0;

  const unsigned row_bytes = 2u * D;
  const unsigned kvh_bytes = static_cast<unsigned>(kvh) * static_cast<unsigned>(bs) * row_bytes;
  const unsigned page_bytes = static_cast<unsigned>(Hkv) * static_cast<unsigned>(bs) * row_bytes;
  // Context token of the first row of each 8*GPP-row group of this wave's tile in
  // step `it`, clamped to the group holding the last context token (rows past C are
  // loaded from that page again, in bounds, and masked; V rows past C are zeroed).
  const int t_last = (C - 1) & ~(8 * GPP - 1);
  struct TilePages { int page[2 / GPP]; int slot[2 / GPP]; };
  auto pages_of = [&](int it) __attribute__((always_inline)) {
    TilePages tp{};
    if (C <= 0) return tp;
#pragma unroll
    for (int g = 0; g < 2 / GPP; ++g) {
      const int t = min(kPrefillStep * it + kTile * ld_h + 8 * GPP * g, t_last);
      const int blk = static_cast<int>(__umulhi(static_cast<unsigned>(t), a.bs_magic) >> a.bs_shift);
      tp.page[g] = page_at(a.bt, s, blk, mbps);
      tp.slot[g] = t - blk * bs;
    }
    return tp;
  };
  typedef const __attribute__((address_space(1))) void* gvoid;
  typedef __attribute__((address_space(3))) void* lvoid;
  // context step it into LDS buffer `dst`
  auto load_ctx = [&](unsigned char* dst, TilePages tp) __attribute__((always_inline)) {
    const unsigned char* cache = reinterpret_cast<const unsigned char*>(ld_v ? a.vc : a.kc);
    unsigned lane_src = lane_src0;
    asm volatile("" : "+v"(lane_src));
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int g = (RPI * j) / (8 * GPP);                // page group of the instruction's rows
      // rows 8*GPP*g .. of the tile start at slot tp.slot[g] of page tp.page[g]
      const size_t base = static_cast<size_t>(static_cast<unsigned>(tp.page[g])) * page_bytes +
                          (kvh_bytes + static_cast<unsigned>(tp.slot[g]) * row_bytes);
      const unsigned rel = static_cast<unsigned>(1024 * j - 8 * GPP * g * static_cast<int>(row_bytes));
      const unsigned off = rel + (lane_src ^ static_cast<unsigned>(16 * ((RPI * j) & (CH - 1))));
      __builtin_amdgcn_global_load_lds((gvoid)(cache + base + off), (lvoid)(dst + ld_dst + 1024 * j),
                                       16, 0, 0);
    }
  };
  // chunk step it (this wave's tile: new tokens j0 .. j0 + 15) into `dst`; rows past
  // Qn - 1 load row Qn - 1 (in bounds; the causal mask drops them)
  auto load_new = [&](unsigned char* dst, int it) __attribute__((always_inline)) {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(ld_v ? a.v_new : a.k_new);
    const int j0 = kPrefillStep * (it - n_ctx_steps) + kTile * ld_h;
    const int jb = min(j0, Qn - 1);                    // first row actually read
    const size_t base = ((size_t)(r0 + jb) * Hkv + kvh) * (size_t)(2 * D);
    const unsigned pitch = static_cast<unsigned>(Hkv) * row_bytes;
    unsigned lane_pos = lane_pos0;
    asm volatile("" : "+v"(lane_pos));
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      // row (within the tile) RPI*j + q_row, read from row min(j0 + that, Qn - 1) of
      // the chunk; fewer than 16 rows past jb, so the offset fits 32 bits (the host
      // bounds Hkv * 32 * D * 2 below 2^32)
      const unsigned rel = static_cast<unsigned>(min(j0 + RPI * j + q_row, Qn - 1) - jb);
      const unsigned pos = lane_pos ^ static_cast<unsigned>(16 * ((RPI * j) & (CH - 1)));
      __builtin_amdgcn_global_load_lds((gvoid)(src + base + (rel * pitch + pos)),
                                       (lvoid)(dst + ld_dst + 1024 * j), 16, 0, 0);
    }
  };
  // After this wave's loads of context step `it` have landed: zero its V rows past C
  // (their slots may hold anything, and P = 0 times NaN would not vanish).
  auto zero_tail = [&](unsigned char* dst, int it) __attribute__((always_inline)) {
    if (!ld_v) return;
    const int t0 = kPrefillStep * it + kTile * ld_h;
    if (t0 + kTile <= C) return;
    int ln = lane;                                      // formed here, not kept live
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < kTile * CH / 64; ++i) {
      const int idx = ln + 64 * i;
      if (t0 + idx / CH >= C)
        *reinterpret_cast<u32x4*>(dst + ld_dst + 16 * idx) = u32x4{0, 0, 0, 0};
    }
  };

  // per block: running max of the lane's column, the lane's share of its exp sum
  // (the column's 4 lanes together hold every key), and O^T
  float m_run[kPfBlocks], l_part[kPfBlocks];
  f32x4 acc[kPfBlocks][DB];
#pragma unroll
  for (int b = 0; b < kPfBlocks; ++b) {
    m_run[b] = kNegInf;
    l_part[b] = 0.f;
#pragma unroll
    for (int c = 0; c < DB; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // lane parts of the operand reads (see the XOR note above the kernel)
  const unsigned k_lane = static_cast<unsigned>(col * L::kRowBytes + 16 * (grp ^ (Z::f(col) & 3)) +
                                                64 * ((Z::f(col) & (CH - 1)) >> 2));
  const int vrow = 4 * grp + (col >> 2);
  const int vf = ZV::f(vrow) & (CH - 1);
  const unsigned v_lane = static_cast<unsigned>(2 * L::kTileBytes + vrow * L::kRowBytes +
                                                8 * (col & 1) + 16 * (((col >> 1) & 1) ^ (vf & 1)) +
                                                32 * (vf >> 1));

  auto compute = [&](auto phase, int it, const unsigned char* lds) __attribute__((always_inline)) {
    constexpr bool ctx_step = decltype(phase)::ctx;
    const int u0 = kPrefillStep * (ctx_step ? it : it - n_ctx_steps);
    if (!wave_active || (!ctx_step && u0 > wave_n_hi)) return;
    // opaque per step, so the per-read XORed addresses are formed here instead of
    // being hoisted out of the key loop (24 registers live across it otherwise)
    unsigned kl = k_lane, vl = v_lane;
    asm volatile("" : "+v"(kl), "+v"(vl));
    f32x4 st[kPfBlocks][2];
#pragma unroll
    for (int b = 0; b < kPfBlocks; ++b) st[b][0] = st[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const unsigned char* kp = lds + (kl ^ static_cast<unsigned>(64 * ks));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(kp + h * L::kTileBytes);
#pragma unroll
        for (int b = 0; b < kPfBlocks; ++b) st[b][h] = DT::mfma_qk(kop, qop[b][ks], st[b][h]);
      }
      if ((ks % kPfKsGroup) == kPfKsGroup - 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
    }
    u32x4 p_hi[kPfBlocks], p_lo[kPfBlocks];
#pragma unroll
    for (int b = 0; b < kPfBlocks; ++b) {
      // The scale is folded into the exponent's argument: sc > 0 (a negative scale
      // has negated Q instead; a zero one arrives as 2^-100), so the column max of
      // sc * s is sc times the max of the raw scores s, and the probabilities are
      // 2^(fma(s, sc, -m)).  Keys a step does not keep (past the context, after the
      // column's token) get s = -inf, hence probability 0.
      float x[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[h][e] = st[b][h][e];
      if (!ctx_step || u0 + kPrefillStep > C) {
        const int lim = ctx_step ? C - 1 : n_col[b];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (u0 + kTile * h + 4 * grp + e > lim) x[h][e] = kNegInf;
      }
      float mr = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) mr = fmaxf(mr, x[h][e]);
      mr = xor_max<16>(mr);
      mr = xor_max<32>(mr);
      const float mx = mr * sc;
      // The first step a column sees always holds one of its keys (context token 0,
      // or new token 0 when there is no context), so it moves the max to a finite
      // value; later a wave rescales only when one of its columns' max grows by
      // more than 2^kRescaleLog2, and a column with no key in a step (mx = -inf)
      // never triggers it.
      if (__builtin_amdgcn_ballot_w64(mx > m_run[b] + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run[b], mx);
        const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
        m_run[b] = m_new;
#pragma unroll
        for (int c = 0; c < DB; ++c) acc[b][c] *= alpha;
        l_part[b] *= alpha;
      }
      float arg[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) arg[h][e] = __builtin_fmaf(x[h][e], sc, -m_run[b]);
      u32x2 ph[2], pl[2];
      prefill_probs<DT>(arg[0], ph[0], pl[0]);
      prefill_probs<DT>(arg[1], ph[1], pl[1]);
      p_hi[b] = u32x4{ph[0].x, ph[0].y, ph[1].x, ph[1].y};
      p_lo[b] = u32x4{pl[0].x, pl[0].y, pl[1].x, pl[1].y};
      // the exp sum from the same rounded values the PV MFMAs take
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        l_part[b] = add_pair<DT>(p_hi[b][e], l_part[b]);
        if constexpr (DT::kSplitP) l_part[b] = add_pair<DT>(p_lo[b][e], l_part[b]);
      }
    }
#pragma unroll
    for (int c = 0; c < DB; ++c) {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const unsigned char* vp = lds + (vl ^ static_cast<unsigned>(32 * c));
      const i16x4 raw0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
      const i16x4 raw1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + L::kTileBytes));
      const u32x2 v0 = __builtin_bit_cast(u32x2, raw0);
      const u32x2 v1 = __builtin_bit_cast(u32x2, raw1);
      const u32x4 vop = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
      for (int b = 0; b < kPfBlocks; ++b) acc[b][c] = pv_mfma32<DT>(vop, p_hi[b], p_lo[b], acc[b][c]);
      if ((c % kPfCGroup) == kPfCGroup - 1) __builtin_amdgcn_sched_barrier(0);    // bound the reads in flight
    }
  };

  // One phase of the key loop, unrolled by two so that each LDS buffer is a fixed
  // object at each point (the compiler then sees that reads of one buffer do not
  // alias the loads in flight into the other).
  auto run = [&](auto phase, int first, int end) __attribute__((always_inline)) {
    constexpr bool kCtx = decltype(phase)::ctx;
    auto issue = [&](unsigned char* dst, int it, TilePages tp) __attribute__((always_inline)) {
      if constexpr (kCtx) load_ctx(dst, tp);
      else load_new(dst, it);
    };
    auto land = [&](unsigned char* dst, int it) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x3f70);               // vmcnt(0): this wave's loads are in LDS
      if constexpr (kCtx) zero_tail(dst, it);
      __syncthreads();
    };
    auto pages = [&](int it) __attribute__((always_inline)) {
      if constexpr (kCtx) return pages_of(it);
      else return TilePages{};
    };
    TilePages pg = pages(first);
    issue(buf0, first, pg);
    pg = pages(min(first + 1, end - 1));
    land(buf0, first);
    // Every path that goes round again has waited for all of its loads (the waits'
    // placement is decided without knowing which branches are taken, so a wait
    // behind a branch before the back edge would put a full wait in front of every
    // read of buffer 0).
    // Loads are issued without a branch: past the phase's last step they load that
    // step again (in bounds) into the free buffer, which is then not read.
    for (int it = first;; it += 2) {
      // buffer 0 holds step it; buffer 1 is free
      issue(buf1, min(it + 1, end - 1), pg);
      pg = pages(min(it + 2, end - 1));
      compute(phase, it, buf0);
      if (it + 1 >= end) break;
      land(buf1, it + 1);
      issue(buf0, min(it + 2, end - 1), pg);
      pg = pages(min(it + 3, end - 1));
      compute(phase, it + 1, buf1);
      if (it + 2 >= end) break;
      land(buf0, it + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);                 // the last, unread loads
    __syncthreads();                                    // both buffers free
  };
  if (n_ctx_steps > 0) run(PrefillPhase<true>{}, 0, n_ctx_steps);
  run(PrefillPhase<false>{}, n_ctx_steps, n_steps);

#pragma unroll
  for (int b = 0; b < kPfBlocks; ++b) {
    const float l_run = xor_add<32>(xor_add<16>(l_part[b]));
    if (col_valid[b]) {
      const float inv = 1.f / l_run;
      // formed here (opaque column index), not kept live across the key loop
      int m = wave_m0 + 16 * b + col;
      asm volatile("" : "+v"(m));
      uint16_t* o = static_cast<uint16_t*>(a.out) +
                    ((size_t)(r0 + m / G) * Hq + kvh * G + m % G) * D + 4 * grp;
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        const f32x4 y = acc[b][c] * inv;
        const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                              DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
        *reinterpret_cast<u32x2*>(o + 16 * c) = packed;
      }
    }
  }
}

}  // namespace pa
