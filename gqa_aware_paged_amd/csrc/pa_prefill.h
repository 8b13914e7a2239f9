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
//   - each 16-token K/V tile (a context tile through the block table, or a tile of
//     the chunk's own rows) is loaded cooperatively by the workgroup into
//     double-buffered LDS, one barrier per tile;
//   - each wave computes S^T = K_tile Q^T for its 16 columns with
//     v_mfma_f32_16x16x32 (its Q^T operand stays in registers), the online
//     softmax per column in base 2, and O^T += V^T P^T with v_mfma_f32_16x16x16
//     (V^T read by ds_read_b64_tr_b16), exactly the decode tile step with query
//     columns in place of query heads;
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

template <int D>
struct PrefillLds {
  static constexpr int kTileBytes = kTile * D * 2;
  unsigned char k[2][kTileBytes];
  unsigned char v[2][kTileBytes];
};

template <int D, class DT>
__global__ __launch_bounds__(kPrefillWaves * 64, 8 / kPrefillWaves) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int NT = kPrefillWaves * 64;
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int CPT = (kTile * CH + NT - 1) / NT;   // chunks per thread per tile (K or V)
  constexpr int TILE_BYTES = PrefillLds<D>::kTileBytes;
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
  const int n_ctx_tiles = (C + kTile - 1) / kTile;
  const int n_tiles = n_ctx_tiles + n_hi / kTile + 1;

  // cooperative tile load: thread tid owns chunks tid + NT*i of the K and V tiles.
  // The index is clamped rather than guarded (head_dim 64 has fewer chunks than
  // threads: the spare threads fetch and store the last chunk again, the same
  // bytes to the same place), so the loads are unconditional and the registers
  // they fill are not merged across branches, which would wait for them at once.
  auto chunk = [&](int i) { return min(tid + NT * i, kTile * CH - 1); };
  u32x4 rk[CPT], rv[CPT];
  auto load = [&](int it, int2 pages) {
    if (it < n_ctx_tiles) {
      const int t0 = kTile * it;
      size_t lo, hi;
      tile_offsets(pages, t0, kvh, Hkv, bs, D, lo, hi);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = chunk(i);
        const int row = c / CH, cc = c % CH;
        const size_t off = (row < 8 ? lo : hi) + (size_t)(row % 8) * D + 8 * cc;
        rk[i] = *reinterpret_cast<const u32x4*>(a.kc + off);
        rv[i] = *reinterpret_cast<const u32x4*>(a.vc + off);
      }
    } else {
      const int j0 = kTile * (it - n_ctx_tiles);
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
  auto pages_of = [&](int it) {
    return it < n_ctx_tiles ? tile_pages(a.bt, s, kTile * it, C, bs, mbps) : make_int2(0, 0);
  };

  int2 pg_next = pages_of(1);
  load(0, pages_of(0));
  stage(0);

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    __syncthreads();                       // tile `it` staged; the other buffer is free
    if (it + 1 < n_tiles) {
      load(it + 1, pg_next);
      pg_next = pages_of(it + 2);
    }
    const bool ctx_tile = it < n_ctx_tiles;
    const int u0 = ctx_tile ? kTile * it : kTile * (it - n_ctx_tiles);   // first key of the tile
    if (wave_active && (ctx_tile || u0 <= wave_n_hi)) {
      const unsigned char* ldsK = sm.k[buf];
      const unsigned char* ldsV = sm.v[buf];
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(ldsK + Z::byte_off(col, 4 * ks + grp));
        st = DT::mfma_qk(kop, qop[ks], st);
      }
      // this lane holds column `col`, keys u0 + 4*grp + e
      const int uk = u0 + 4 * grp;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = ctx_tile ? uk + e < C : uk + e <= n_col;
        x[e] = keep ? st[e] * a.scale_log2 : kNegInf;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      // the first tile a column sees always holds one of its keys (context token 0,
      // or new token 0 when there is no context), so m_new is finite from then on
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      u32x2 p_hi, p_lo;
      l_run = l_run * alpha + prob_operands<DT>(x, m_new, p_hi, p_lo);
      // context slots past C may hold anything (NaN): zero those V rows; chunk rows
      // past the causal limit are finite and weigh 0
      uint32_t keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;
      if (ctx_tile && u0 + kTile > C) {
        const int n = C - uk;
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
    }
    if (it + 1 < n_tiles) stage(buf ^ 1);
  }

  // exp sum of the column over the 4 lane groups, then out = acc / l
  l_run = xor_add(l_run, 16);
  l_run = xor_add(l_run, 32);
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
