// Prefill over a paged context on gfx950: the prefix path of the page of commit
// b80fd2b (paged_attn.py: _forward_prefix_pytorch, one online softmax over the
// context gathered from the caches by block id, then over the current chunk
// under the causal mask; rewrite item 1: the context is gathered once).
//
// New token n of sequence s (row r = query_start[s] + n of q, k_new, v_new)
// attends, for every query head of a KV head's group, to the C = ctx_lens[s]
// cached tokens and to the new tokens j <= n.  With many query rows per KV head
// the product is a real GEMM: a workgroup takes 64 "columns", a column being one
// (new token, query head of the group) pair (column m = n*G + g), 16 per wave,
// and streams the keys through them once:
//   - keys go in steps of 32 (two 16-token tiles: context tiles through the block
//     table, then tiles of the chunk's own rows), loaded cooperatively by the
//     workgroup two steps ahead into registers and staged into double-buffered
//     LDS, one barrier per step;
//   - each wave computes S^T = K Q^T for its 16 columns and the step's two tiles
//     with v_mfma_f32_16x16x32 (its Q^T operand stays in registers), one online
//     softmax update per column over the 32 keys in base 2, and O^T += V^T P^T
//     with one double-rate v_mfma_f32_16x16x32 per 16 head dims (V^T of both
//     tiles read by ds_read_b64_tr_b16), plus one for the exp sums: the decode
//     tile step with query columns in place of query heads, the accumulator
//     rescaled only when a column's max grows by more than 2^8;
//   - the causal mask keeps key j for column (n, g) iff j <= n; steps past a
//     wave's last token are skipped, steps past the workgroup's last token are
//     not loaded.
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

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
constexpr int kPrefillCols = 16 * kPrefillWaves;   // columns per workgroup
constexpr int kXcds = 8;                           // MI355X: 8 XCDs, workgroups dealt round-robin

// The two phases of a workgroup's key loop: the cached context, then the chunk.
template <bool kCtx>
struct PrefillPhase { static constexpr bool ctx = kCtx; };

// global-memory views (address space 1) for loads from a base held in SGPRs
typedef const __attribute__((address_space(1))) unsigned char* gbytes;
typedef const __attribute__((address_space(1))) u32x4 gu32x4;

constexpr int kPrefillHalves = 2;                      // 16-token tiles per step
constexpr int kPrefillStep = kTile * kPrefillHalves;   // keys per softmax step

// The running max of a column moves only when a step's max exceeds it by more than
// this (base 2): otherwise the step's probabilities are taken against the old max,
// each at most 2^8 (well inside f16 and bf16), and the accumulators are not rescaled.
constexpr float kRescaleLog2 = 8.f;

// LDS of one step: 32 K rows, then 32 V rows, each row padded by 32 bytes so that
// consecutive rows start 32 bytes apart modulo 256.  Measured with
// SQ_LDS_BANK_CONFLICT on gfx950 (head_dim 256), that makes both MFMA operand
// reads conflict-free without a swizzle: the 16-byte K reads of 16 rows, and the
// transposed V reads (32 bytes of each of 4 rows per 16 lanes); a 16-byte pad
// makes the K reads two-way conflicted.  With no swizzle, every read of a step is
// one lane base plus an immediate offset.
template <int D>
struct PrefillLds {
  static constexpr int kKPitch = 2 * D + 32;
  static constexpr int kVPitch = 2 * D + 32;
  static constexpr int kKBytes = kPrefillStep * kKPitch;
  static constexpr int kBufBytes = kKBytes + kPrefillStep * kVPitch;
  unsigned char buf[2][kBufBytes];
};

// GPP: 8-token groups per page lookup, 1 for 8-token pages, else 2 (a 16-token tile
// always lies in one page when the page size is a multiple of 16)
template <int D, class DT, int GPP>
__global__ __launch_bounds__(kPrefillWaves * 64, 8 / kPrefillWaves) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int NT = kPrefillWaves * 64;
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int CPT = (kPrefillStep * CH + NT - 1) / NT;   // chunks per thread per step (K or V)
  using L = PrefillLds<D>;
  __shared__ __attribute__((aligned(16))) L sm;

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
  const int m0 = cb * kPrefillCols;                 // first column of the workgroup
  if (m0 >= Qn * G) return;
  const int n_hi = min(Qn - 1, (m0 + kPrefillCols - 1) / G);   // last token of the workgroup
  const int wave_m0 = m0 + 16 * wave;
  const int wave_n_hi = min(Qn - 1, (wave_m0 + 15) / G);        // last token of the wave
  const bool wave_active = wave_m0 < Qn * G;

  // this lane's column: token n_col, query head kvh*G + g_col
  const int m_col = wave_m0 + col;
  const bool col_valid = m_col < Qn * G;
  const int n_col = m_col / G, g_col = m_col % G;

  // Q^T operand of the QK^T MFMA: lane (col, grp) holds chunk 4*ks + grp of its
  // column's query row (zero for padding columns, whose scores are then 0)
  u32x4 qop[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)(r0 + n_col) * Hq + kvh * G + g_col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = col_valid ? *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * ks + grp))
                          : u32x4{0, 0, 0, 0};
  }

  const int bs = a.block_size, mbps = a.max_blocks_per_seq;
  const int n_ctx_steps = (C + kPrefillStep - 1) / kPrefillStep;
  const int n_steps = n_ctx_steps + n_hi / kPrefillStep + 1;

  // Cooperative step load: thread tid owns chunks c = tid + NT*i of the K and V
  // rows (row = c / CH: rows 0..15 are the first tile, 16..31 the second), so load
  // i of every thread of a wave falls in one 8-row group (8*CH chunks), whose
  // rows are contiguous in the cache; the address is that group's (wave-uniform)
  // base plus a per-thread offset that does not change from step to step.
  static_assert(CPT * NT == kPrefillStep * CH, "a step is a whole number of loads");
  const unsigned lane_bytes = 16u * static_cast<unsigned>(tid % (8 * CH));
  auto group_of = [&](int i) {
    if constexpr (8 * CH == NT) return i;              // head_dim 256: load i is group i
    else return i * (NT / (8 * CH)) + wave / (CH / 8);
  };
  // a (page, KV head) block of the cache is page_bytes long; the rows of KV head
  // kvh start kvh_bytes into it (paged_attn_prefill rejects shapes where
  // num_kv_heads * max(block_size, 32) * head_dim * 2 reaches 2^32, so both fit)
  const unsigned row_bytes = 2u * D;
  const unsigned kvh_bytes = static_cast<unsigned>(kvh) * static_cast<unsigned>(bs) * row_bytes;
  const unsigned page_bytes = static_cast<unsigned>(Hkv) * static_cast<unsigned>(bs) * row_bytes;
  // Pages and in-page slots of context step `it` (wave-uniform): one lookup per
  // GPP 8-token groups, with no branch.  Token indices are clamped to the group
  // (or tile) holding the last context token, so a step past the context, or a
  // part of one, reads rows of that page again, in bounds, and masks them; the
  // lookup for step it + 2 is issued a step ahead of its use.
  constexpr int NL = 4 / GPP;
  struct StepPages { int page[NL]; int slot[NL]; };
  const int t_last = (C - 1) & ~(8 * GPP - 1);
  auto pages_of = [&](int it) {
    StepPages sp{};
    if (C <= 0) return sp;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int t = min(kPrefillStep * it + 8 * GPP * j, t_last);
      const int blk = static_cast<int>(__umulhi(static_cast<unsigned>(t), a.bs_magic) >> a.bs_shift);
      sp.page[j] = page_at(a.bt, s, blk, mbps);
      sp.slot[j] = t - blk * bs;
    }
    return sp;
  };
  struct Regs { u32x4 k[CPT], v[CPT]; };
  auto load = [&](auto phase, int it, StepPages sp, Regs& r) {
    if constexpr (decltype(phase)::ctx) {
      size_t off[4];                                   // byte offsets of the groups
#pragma unroll
      for (int g = 0; g < 4; ++g)
        off[g] = static_cast<size_t>(static_cast<unsigned>(sp.page[g / GPP])) * page_bytes +
                 (kvh_bytes + static_cast<unsigned>(sp.slot[g / GPP] + 8 * (g % GPP)) * row_bytes);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int g = group_of(i);
        const size_t o = g == 0 ? off[0] : g == 1 ? off[1] : g == 2 ? off[2] : off[3];
        // the group's base stays a scalar pair and the lane offset a 32-bit value
        // inside the loop, so each load takes the base + 32-bit offset form
        gbytes kb = (gbytes)(a.kc) + o;
        gbytes vb = (gbytes)(a.vc) + o;
        unsigned lb = lane_bytes;
        asm volatile("" : "+s"(kb), "+s"(vb), "+v"(lb));
        r.k[i] = *reinterpret_cast<const gu32x4*>(kb + lb);
        r.v[i] = *reinterpret_cast<const gu32x4*>(vb + lb);
      }
    } else {
      const int j0 = kPrefillStep * (it - n_ctx_steps);
      const size_t base = ((size_t)(r0 + j0) * Hkv + kvh) * (size_t)(2 * D);
      const int last = Qn - 1 - j0;                    // rows past it read row `last`
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + NT * i;
        const int row = c / CH, cc = c % CH;
        const unsigned lb = static_cast<unsigned>((min(row, last) * Hkv * D + 8 * cc) * 2);
        r.k[i] = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const unsigned char*>(a.k_new) + base + lb);
        r.v[i] = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const unsigned char*>(a.v_new) + base + lb);
      }
    }
  };
  // Staging into LDS.  V rows of context slots past C may hold anything (NaN) and
  // are staged as zeros; their keys are masked out of the softmax as well.
  auto stage = [&](auto phase, unsigned char* dst, int it, Regs& r) {
    if constexpr (decltype(phase)::ctx) {
      const int valid = C - kPrefillStep * it;
      if (valid < kPrefillStep) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          if ((tid + NT * i) / CH >= valid) r.v[i] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      const int row = c / CH, cc = c % CH;
      *reinterpret_cast<u32x4*>(dst + row * L::kKPitch + 16 * cc) = r.k[i];
      *reinterpret_cast<u32x4*>(dst + L::kKBytes + row * L::kVPitch + 16 * cc) = r.v[i];
    }
  };

  float m_run = kNegInf;
  f32x4 acc[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // exp sums ride on the PV MFMA: a 17th A operand whose row 0 is all ones gives
  // sum_k P[col][k] in row 0 of lsum (lanes with grp 0), from the same rounded
  // probabilities as the weighted sum
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = col == 0 ? DT::kOnePair : 0u;
  const u32x4 ones = {one2, one2, one2, one2};

  // lane bases of the LDS reads; everything else is an immediate offset
  const int k_lane = col * L::kKPitch + 16 * grp;
  const int v_lane = L::kKBytes + (4 * grp + (col >> 2)) * L::kVPitch + 8 * (col & 3);

  // one step of every wave: S^T, the online softmax and O^T += V^T P^T over the
  // 32 keys of step `it`, read from the LDS buffer at `lds`
  auto compute = [&](auto phase, int it, const unsigned char* lds) {
    constexpr bool ctx_step = decltype(phase)::ctx;
    const int u0 = kPrefillStep * (ctx_step ? it : it - n_ctx_steps);   // first key of the step
    if (wave_active && (ctx_step || u0 <= wave_n_hi)) {
      const unsigned char* ldsK = lds + k_lane;
      const unsigned char* ldsV = lds + v_lane;
      // S^T of the two tiles as two independent MFMA chains
      f32x4 st[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 kop = *reinterpret_cast<const u32x4*>(
              ldsK + h * kTile * L::kKPitch + 64 * ks);
          st[h] = DT::mfma_qk(kop, qop[ks], st[h]);
        }
      }
      // this lane holds column `col`, keys u0 + 16*h + 4*grp + e; key u is kept iff
      // u <= lim (u < C in the context, the causal rule in the chunk); a context
      // step wholly inside the context needs no mask
      float x[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[h][e] = st[h][e] * a.scale_log2;
      if (!ctx_step || u0 + kPrefillStep > C) {
        const int lim = ctx_step ? C - 1 : n_col;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (u0 + kTile * h + 4 * grp + e > lim) x[h][e] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, x[h][e]);
      mx = xor_max<16>(mx);
      mx = xor_max<32>(mx);
      // The first step a column sees always holds one of its keys (context token 0,
      // or new token 0 when there is no context), so the first step of every lane
      // moves the max to a finite value.  Later a wave rescales only when one of its
      // columns' max grows by more than 2^kRescaleLog2.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
#pragma unroll
        for (int c = 0; c < DB; ++c) acc[c] *= alpha;
        lsum *= alpha;
      }
      u32x2 ph[2], pl[2];
      prob_operands<DT>(x[0], m_run, ph[0], pl[0]);
      prob_operands<DT>(x[1], m_run, ph[1], pl[1]);
      // B operand of the 16x16x32 MFMA: k = 8*grp + j is key 4*grp + j of the first
      // tile for j < 4 and key 4*grp + j - 4 of the second for j >= 4; the V^T
      // operand below takes its keys in the same order
      const u32x4 p_hi = {ph[0].x, ph[0].y, ph[1].x, ph[1].y};
      const u32x4 p_lo = {pl[0].x, pl[0].y, pl[1].x, pl[1].y};
      // V^T of both tiles: lane (col, grp) of the transposed read supplies row
      // 4*grp + col/4, columns 16c + 4*(col&3) .. +3
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const unsigned char* vp = ldsV + 32 * c;
        const i16x4 raw0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
        const i16x4 raw1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + kTile * L::kVPitch));
        const u32x2 v0 = __builtin_bit_cast(u32x2, raw0);
        const u32x2 v1 = __builtin_bit_cast(u32x2, raw1);
        const u32x4 vop = {v0.x, v0.y, v1.x, v1.y};
        acc[c] = pv_mfma32<DT>(vop, p_hi, p_lo, acc[c]);
      }
      lsum = pv_mfma32<DT>(ones, p_hi, p_lo, lsum);
    }
  };

  // Software pipeline, two steps deep, run once over the context steps and once
  // over the chunk steps (each phase with a single load path, so the compiler's
  // waits before a staging cover exactly the older register set).  The loads of
  // step it + 2 are issued at the top of step it into the register set freed when
  // step it was staged, and land while steps it and it + 1 are computed; step
  // it + 1 is staged from the other set at the end of step it.  Unrolled by two so
  // that register sets and LDS buffers are fixed at each point.  Every prefetch is
  // issued, one past the phase's end reading its last step again (in bounds, never
  // staged); block-table lookups run a step ahead of the loads that use them.
  auto run = [&](auto phase, int first, int end) {
    constexpr bool kCtx = decltype(phase)::ctx;
    auto pages = [&](int it) {
      if constexpr (kCtx) return pages_of(it);
      else return StepPages{};
    };
    auto prefetch = [&](int it, StepPages sp, Regs& r) {
      load(phase, min(it, end - 1), sp, r);
    };
    Regs ra, rb;
    prefetch(first, pages(first), ra);
    prefetch(first + 1, pages(first + 1), rb);
    StepPages pg_next = pages(first + 2);
    stage(phase, sm.buf[0], first, ra);
    for (int it = first; it < end; it += 2) {
      __syncthreads();                     // step it staged in buffer 0; buffer 1 free
      prefetch(it + 2, pg_next, ra);
      pg_next = pages(it + 3);
      compute(phase, it, sm.buf[0]);
      if (it + 1 < end) {
        stage(phase, sm.buf[1], it + 1, rb);
        __syncthreads();                   // step it + 1 staged in buffer 1; buffer 0 free
        prefetch(it + 3, pg_next, rb);
        pg_next = pages(it + 4);
        compute(phase, it + 1, sm.buf[1]);
        if (it + 2 < end) stage(phase, sm.buf[0], it + 2, ra);
      }
    }
  };
  if (n_ctx_steps > 0) run(PrefillPhase<true>{}, 0, n_ctx_steps);
  __syncthreads();                         // both buffers free before the chunk phase
  run(PrefillPhase<false>{}, n_ctx_steps, n_steps);

  // the column's exp sum from the lane of grp 0, then out = acc / l
  const float l_run = __shfl(lsum[0], col, 64);
  if (col_valid) {
    const float inv = 1.f / l_run;
    uint16_t* o = static_cast<uint16_t*>(a.out) +
                  ((size_t)(r0 + n_col) * Hq + kvh * G + g_col) * D + 4 * grp;
#pragma unroll
    for (int c = 0; c < DB; ++c) {
      const f32x4 y = acc[c] * inv;
      const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                            DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
      *reinterpret_cast<u32x2*>(o + 16 * c) = packed;
    }
  }
}

}  // namespace pa
