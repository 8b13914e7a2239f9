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
//     table, or tiles of the chunk's own rows), loaded cooperatively by the
//     workgroup into double-buffered LDS, one barrier per step;
//   - each wave computes S^T = K Q^T for its 16 columns and the step's two tiles
//     with v_mfma_f32_16x16x32 (its Q^T operand stays in registers), one online
//     softmax update per column over the 32 keys in base 2, and O^T += V^T P^T
//     with one double-rate v_mfma_f32_16x16x32 per 16 head dims (V^T of both
//     tiles read by ds_read_b64_tr_b16): the decode tile step with query columns
//     in place of query heads, its rescale spread over twice the keys;
//   - the causal mask keeps key j for column (n, g) iff j <= n; tiles past a
//     wave's last token are skipped, tiles past the workgroup's last token are
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
  int max_blocks_per_seq;
  int max_query_len;         // lengths are clamped to these bounds
  int max_ctx_len;
  int col_blocks;            // column blocks per (sequence, KV head)
  int units_per_xcd;         // (sequence, KV head) units per XCD
  float scale_log2;
};

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
constexpr int kPrefillCols = 16 * kPrefillWaves;   // columns per workgroup
constexpr int kXcds = 8;                           // MI355X: 8 XCDs, workgroups dealt round-robin

constexpr int kPrefillHalves = 2;                      // 16-token tiles per step
constexpr int kPrefillStep = kTile * kPrefillHalves;   // keys per softmax step

template <int D>
struct PrefillLds {
  static constexpr int kStepBytes = kPrefillStep * D * 2;
  unsigned char k[2][kStepBytes];
  unsigned char v[2][kStepBytes];
};

template <int D, class DT>
__global__ __launch_bounds__(kPrefillWaves * 64, 8 / kPrefillWaves) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int NT = kPrefillWaves * 64;
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int CPT = (kPrefillStep * CH + NT - 1) / NT;   // chunks per thread per step (K or V)
  constexpr int HALF_BYTES = kTile * D * 2;                // one 16-token tile in LDS
  using Z = Swz<D>;
  using ZV = Swz<D, true>;
  __shared__ __attribute__((aligned(16))) PrefillLds<D> sm;

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

  // cooperative step load: thread tid owns chunks tid + NT*i of the K and V rows
  // (row = chunk / CH: rows 0..15 are the first tile, 16..31 the second).  The
  // index is clamped rather than guarded (spare threads, if any, fetch and store
  // the last chunk again, the same bytes to the same place), so the loads are
  // unconditional and the registers they fill are not merged across branches,
  // which would wait for them at once.
  auto chunk = [&](int i) { return min(tid + NT * i, kPrefillStep * CH - 1); };
  u32x4 rk[CPT], rv[CPT];
  auto load = [&](int it, int4 pages) {
    if (it < n_ctx_steps) {
      const int t0 = kPrefillStep * it;
      size_t lo[2], hi[2];
      tile_offsets(make_int2(pages.x, pages.y), t0, kvh, Hkv, bs, D, lo[0], hi[0]);
      tile_offsets(make_int2(pages.z, pages.w), t0 + kTile, kvh, Hkv, bs, D, lo[1], hi[1]);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = chunk(i);
        const int row = c / CH, cc = c % CH;
        const int h = row / kTile, r = row % kTile;
        const size_t base = r < 8 ? (h ? lo[1] : lo[0]) : (h ? hi[1] : hi[0]);
        const size_t off = base + (size_t)(r % 8) * D + 8 * cc;
        rk[i] = *reinterpret_cast<const u32x4*>(a.kc + off);
        rv[i] = *reinterpret_cast<const u32x4*>(a.vc + off);
      }
    } else {
      const int j0 = kPrefillStep * (it - n_ctx_steps);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = chunk(i);
        const int row = c / CH, cc = c % CH;
        // rows past the chunk read its last row: finite, and masked by the causal rule
        const int j = min(j0 + row, Qn - 1);
        const size_t off = ((size_t)(r0 + j) * Hkv + kvh) * D + 8 * cc;
        rk[i] = *reinterpret_cast<const u32x4*>(a.k_new + off);
        rv[i] = *reinterpret_cast<const u32x4*>(a.v_new + off);
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = chunk(i);
      const int row = c / CH, cc = c % CH;
      *reinterpret_cast<u32x4*>(sm.k[buf] + Z::byte_off(row, cc)) = rk[i];
      *reinterpret_cast<u32x4*>(sm.v[buf] + ZV::byte_off(row, cc)) = rv[i];
    }
  };
  // pages of the two tiles of a context step; a second tile wholly past the
  // context (C not a multiple of 32) reads the first tile's pages again, at
  // in-page slots, and every key of it is masked
  auto pages_of = [&](int it) {
    if (it >= n_ctx_steps) return make_int4(0, 0, 0, 0);
    const int t0 = kPrefillStep * it;
    const int2 p0 = tile_pages(a.bt, s, t0, C, bs, mbps);
    const int2 p1 = t0 + kTile < C ? tile_pages(a.bt, s, t0 + kTile, C, bs, mbps) : p0;
    return make_int4(p0.x, p0.y, p1.x, p1.y);
  };

  int4 pg_next = pages_of(1);
  load(0, pages_of(0));
  stage(0);

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < n_steps; ++it) {
    const int buf = it & 1;
    __syncthreads();                       // step `it` staged; the other buffer is free
    if (it + 1 < n_steps) {
      load(it + 1, pg_next);
      pg_next = pages_of(it + 2);
    }
    const bool ctx_step = it < n_ctx_steps;
    const int u0 = kPrefillStep * (ctx_step ? it : it - n_ctx_steps);   // first key of the step
    if (wave_active && (ctx_step || u0 <= wave_n_hi)) {
      const unsigned char* ldsK = sm.k[buf];
      const unsigned char* ldsV = sm.v[buf];
      // S^T of the two tiles as two independent MFMA chains
      f32x4 st[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 kop = *reinterpret_cast<const u32x4*>(
              ldsK + h * HALF_BYTES + Z::byte_off(col, 4 * ks + grp));
          st[h] = DT::mfma_qk(kop, qop[ks], st[h]);
        }
      }
      // this lane holds column `col`, keys u0 + 16*h + 4*grp + e
      float x[2][4];
      float mx = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int uk = u0 + kTile * h + 4 * grp;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = ctx_step ? uk + e < C : uk + e <= n_col;
          x[h][e] = keep ? st[h][e] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, x[h][e]);
        }
      }
      mx = xor_max<16>(mx);
      mx = xor_max<32>(mx);
      // the first step a column sees always holds one of its keys (context token
      // 0, or new token 0 when there is no context), so m_new is finite from then on
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      u32x2 ph[2], pl[2];
      const float sum0 = prob_operands<DT>(x[0], m_new, ph[0], pl[0]);
      const float sum1 = prob_operands<DT>(x[1], m_new, ph[1], pl[1]);
      l_run = l_run * alpha + (sum0 + sum1);
      // B operand of the 16x16x32 MFMA: k = 8*grp + j is key 4*grp + j of the first
      // tile for j < 4 and key 4*grp + j - 4 of the second for j >= 4; the V^T
      // operand below takes its keys in the same order
      const u32x4 p_hi = {ph[0].x, ph[0].y, ph[1].x, ph[1].y};
      const u32x4 p_lo = {pl[0].x, pl[0].y, pl[1].x, pl[1].y};
      // context slots past C may hold anything (NaN): zero those V rows; chunk rows
      // past the causal limit are finite and weigh 0
      uint32_t keep[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (ctx_step && u0 + kPrefillStep > C) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int n = C - (u0 + kTile * h + 4 * grp);
          keep[2 * h] = (n > 0 ? 0x0000ffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
          keep[2 * h + 1] = (n > 2 ? 0x0000ffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
        }
      }
      const int vrow = 4 * grp + (col >> 2);
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        const int vcol = 16 * c + 4 * (col & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const unsigned char* vp = ldsV + ZV::byte_off(vrow, vcol >> 3) + (vcol & 7) * 2;
        const i16x4 raw0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
        const i16x4 raw1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + HALF_BYTES));
        const u32x2 v0 = __builtin_bit_cast(u32x2, raw0);
        const u32x2 v1 = __builtin_bit_cast(u32x2, raw1);
        const u32x4 vop = {v0.x & keep[0], v0.y & keep[1], v1.x & keep[2], v1.y & keep[3]};
        acc[c] = pv_mfma32<DT>(vop, p_hi, p_lo, acc[c] * alpha);
      }
    }
    if (it + 1 < n_steps) stage(buf ^ 1);
  }

  // exp sum of the column over the 4 lane groups, then out = acc / l
  l_run = xor_add<16>(l_run);
  l_run = xor_add<32>(l_run);
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
