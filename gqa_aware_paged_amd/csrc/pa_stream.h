// Phase 1 as per-wave streams (gfx950): the length-balanced split and the pages'
// explicit partition sizes without a workgroup barrier per piece.
//
// The step's work for one KV head is the sequences' 16-token tiles laid end to
// end (the "real" tiles).  As in pa_phase1_balanced_kernel, every workgroup
// rebuilds the per-sequence prefix in LDS and takes one share of them, cut in
// virtual tiles (each piece counts piece_cost tiles of start-up ahead of its real
// ones).  With an explicit partition size (PARTS) the pieces are the pages'
// partitions (page of commit 8d26e23: one attention_partial per (sequence, KV
// head, partition)) and a share boundary is moved to the nearest partition
// boundary, so no partition is split between workgroups and each still produces
// exactly one partial; otherwise a piece is the part of a sequence inside the
// share, as in the balanced kernel.
//
// Inside the workgroup the share's real tiles are cut into W contiguous ranges,
// one per wave, and each wave streams its range on its own: K/V and page ids one
// tile ahead, the query rows of the next sequence loaded as soon as the last QK^T
// product of the current one has been issued, the online-softmax state (max, exp
// sum, accumulator) in registers.  No barrier and no merge stand between the
// pieces of a range: a piece that lies inside one range is finished from
// registers (its output rows), or, for a partial record, parked in a free slot of
// an LDS pool that the whole workgroup writes out after the walk, then (head_dim
// 256) in the wave's spare accumulator registers, written when its walk ends, and
// stored directly only when both are full: stores mixed into the saturated read
// stream cost about ten times their bytes.  Only a piece cut by a range boundary
// is shared: each later wave holding part of it parks its state in a reserved pool
// slot (at most one per wave, its first piece), and after the walk the first wave
// holding it merges the parked parts with the flash-attention rescale and writes
// the result.
// Records, phase 2 and the job list are those of the other kernels: PARTS uses the
// fixed-partition record of (sequence, KV head, partition) and the fixed-partition
// phase 2; the balanced split the two records per workgroup.
#pragma once

#include <utility>

#include "pa_kernels.h"

namespace pa {

constexpr int kStreamMaxGroup = 16;       // query heads per KV head (the largest group served)
constexpr float kLazyRescaleLog2 = 8.f;   // slack of the running max before a rescale (base 2)

// Record hold (head_dim 256 with explicit partitions, groups of up to 6 heads): the
// accumulator registers the kernel leaves free (it allocates 68 of the 256 AGPRs,
// one wave per SIMD) hold up to kHoldRecs records per wave once the LDS pool is full,
// so that they too are written after the walk.  A held record is 25 registers per
// lane: its packed state (24: lane l, register 4i + e holds f32x4 l + 64i of the
// pool layout, element e), then (max, exp sum) of head h in lanes 2h, 2h+1 and the
// record index in lanes 2G, 2G+1 (low, high word).  Hold slot k is AGPRs
// kHoldBase + 25k .. + 24, addressed by number in inline asm: the compiler neither
// sees nor allocates them (a clobber of a255 at kernel entry makes the kernel
// allocate the whole AGPR file, and the walk's own accumulators stay in a0 .. a67).
constexpr int kHoldRecs = 7;
constexpr int kHoldStride = 25;
constexpr int kHoldMaxGroup = 6;
constexpr int kHoldBase = 256 - kHoldRecs * kHoldStride;

template <int R>
__device__ __forceinline__ void agpr_put(float x) {
  asm volatile("v_accvgpr_write_b32 a[%1], %0" ::"v"(x), "n"(R));
}
template <int R>
__device__ __forceinline__ float agpr_get() {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, a[%1]" : "=v"(x) : "n"(R));
  return x;
}
template <int Base, int... J>
__device__ __forceinline__ void agpr_put_all(const float (&v)[kHoldStride],
                                             std::integer_sequence<int, J...>) {
  (agpr_put<Base + J>(v[J]), ...);
}
template <int Base, int... J>
__device__ __forceinline__ void agpr_get_all(float (&v)[kHoldStride],
                                             std::integer_sequence<int, J...>) {
  ((v[J] = agpr_get<Base + J>()), ...);
}
template <int K = 0>
__device__ __forceinline__ void hold_put(int k, const float (&v)[kHoldStride]) {
  if constexpr (K < kHoldRecs) {
    if (k == K)
      agpr_put_all<kHoldBase + K * kHoldStride>(v, std::make_integer_sequence<int, kHoldStride>{});
    else
      hold_put<K + 1>(k, v);
  }
}
template <int K = 0>
__device__ __forceinline__ void hold_get(int k, float (&v)[kHoldStride]) {
  if constexpr (K < kHoldRecs) {
    if (k == K)
      agpr_get_all<kHoldBase + K * kHoldStride>(v, std::make_integer_sequence<int, kHoldStride>{});
    else
      hold_get<K + 1>(k, v);
  }
}

template <int D, int W>
struct StreamLdsCore {
  static constexpr int kTileBytes = kTile * D * 2;
  // a state of G <= kStreamMaxGroup heads, packed: f32x4 (cc*G + h)*4 + q4 holds head
  // h, dims 16*cc + 4*q4 .. +3
  static constexpr int kPack = (D / 16) * kStreamMaxGroup * 4;
  unsigned char tiles[W * 2 * kTileBytes];   // per wave: K tile, V tile
  int park_start[W - 1];                     // first real tile of wave v+1's parked piece, or -1
  int pre[kMaxBalancedSeqs + 1];             // virtual tiles of the sequences before s
  int preR[kMaxBalancedSeqs + 1];            // real tiles of the sequences before s
  int len[kMaxBalancedSeqs];                 // lengths clamped to [0, max_seq_len]
  int wave_tot[2][W];
};

// LDS a stream workgroup may take: one workgroup per CU at head_dim 256, two below
// (160 KiB per CU).
template <int D>
constexpr int stream_lds_budget() { return (D >= 256 ? 160 : 80) * 1024; }

// The rest of that budget is a pool of slots, each a piece's state packed: the
// accumulator (f32x4 (cc*G + h)*4 + q4), then (max, exp sum) of each head (8 f32x4
// hold 16 heads), then a record index.  Slots 0..W-2 hold the first piece of waves
// 1..W-1 when an earlier wave began it (parked for the merge after the walk).  The
// others hold partial records (PARTS): a record stored while the wave's K/V reads
// stream costs about ten times its bytes (stores mixed into the saturated read
// stream), the same store after the walk about its bytes, so a record that a wave
// finishes before the end of its run takes a free slot if there is one and the
// whole workgroup writes the pool out after the walk.
template <int D, int W>
struct StreamLds : StreamLdsCore<D, W> {
  static constexpr int kPoolF4 =
      (stream_lds_budget<D>() - static_cast<int>(sizeof(StreamLdsCore<D, W>)) - 64) / 16;
  static_assert(kPoolF4 >= (W - 1) * (StreamLdsCore<D, W>::kPack + 9),
                "the parked pieces of the largest group must fit the pool");
  int pool_next;                             // slots taken (may pass the slot count)
  int pool_pad[3];
  f32x4 pool[kPoolF4 > 0 ? kPoolF4 : 1];
};

template <int D, class DT, int W, bool PARTS>
__global__ __launch_bounds__(W * 64, 1) void pa_phase1_stream_kernel(DecodeArgs a) {
  constexpr int NT = W * 64;
  constexpr int PER = kMaxBalancedSeqs / NT;
  constexpr int KS = D / 32;               // k-steps of the QK^T MFMA (32 dims each)
  constexpr int DB = D / 16;               // 16-wide head_dim blocks of the PV MFMA
  constexpr int LOADS = D / 32;            // 16-byte loads per lane per tile (K or V)
  constexpr int TILE_BYTES = StreamLds<D, W>::kTileBytes;
  using Z = Swz<D>;          // K tiles
  using ZV = Swz<D, true>;   // V tiles
  __shared__ __attribute__((aligned(16))) StreamLds<D, W> sm;
  constexpr bool HOLD = PARTS && D == 256;
  if constexpr (HOLD) asm volatile("" ::: "a255");   // the kernel allocates every AGPR

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  const int w = blockIdx.x;
  const int NS = a.num_wg / Hkv;
  const int skew = a.xcd_skew;
  const int j = skew > 0 ? 2 * (w / (2 * Hkv)) + (w & 1) : w / Hkv;
  const int kvh = skew > 0 ? (w >> 1) % Hkv : w % Hkv;
  const int r = j * Hkv + kvh;           // record pair and job of this share (balanced)
  const int c = a.piece_cost;            // virtual tiles ahead of each piece
  const int P16 = PARTS ? a.partition_size / kTile : 1;
  const int T1 = a.single_pass_max_len;  // PARTS: sequences up to T1 tokens are one piece
  const int unit_v = c + P16;            // PARTS: virtual tiles of a whole partition

  // ---- prefixes of virtual and real tiles: thread tid owns sequences tid*PER ..
  {
    int lc[PER], lr[PER];
    int csum = 0, rsum = 0;
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = tid * PER + i;
      int n = 0, cost = 0;
      if (s < S) {
        const int L = max(clamp_len(a, s), 0);
        n = (L + kTile - 1) / kTile;
        sm.len[s] = L;
        if (n > 0) {
          if constexpr (PARTS) cost = (L <= T1 ? 1 : (n + P16 - 1) / P16) * c + n;
          else cost = c + n;
        }
      }
      csum += cost;
      rsum += n;
      lc[i] = csum;
      lr[i] = rsum;
    }
    int ic = csum, ir = rsum;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int vc = __shfl_up(ic, k, 64);
      const int vr = __shfl_up(ir, k, 64);
      if (lane >= k) {
        ic += vc;
        ir += vr;
      }
    }
    if (lane == 63) {
      sm.wave_tot[0][wave] = ic;
      sm.wave_tot[1][wave] = ir;
    }
    if (tid < W - 1) sm.park_start[tid] = -1;
    if (tid == 0) sm.pool_next = W - 1;      // slots 0..W-2: parked pieces
    __syncthreads();
    int bc = ic - csum, br = ir - rsum;
    for (int v = 0; v < wave; ++v) {
      bc += sm.wave_tot[0][v];
      br += sm.wave_tot[1][v];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = tid * PER + i;
      if (s < S) {
        sm.pre[s + 1] = bc + lc[i];
        sm.preR[s + 1] = br + lr[i];
      }
    }
    if (tid == 0) {
      sm.pre[0] = 0;
      sm.preR[0] = 0;
    }
    __syncthreads();
  }

  // everything below that is not per lane is the same for the whole wave: scalar
  const int T = uniform(sm.pre[S]);
  const int TR = uniform(sm.preR[S]);

  // sequences of length <= 0 get zero rows; spread over the workgroups
  for (int s = w; s < S; s += a.num_wg) {
    if (uniform(sm.preR[s + 1]) == uniform(sm.preR[s])) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + (size_t)s * Hq * D;
      for (int i = tid; i < Hq * D / 8; i += NT) reinterpret_cast<u32x4*>(o)[i] = u32x4{0, 0, 0, 0};
    }
  }

  // largest s < S with pfx[s] <= x (x below the total): the sequence holding x
  auto seq_at = [&](const int* pfx, long long x) {
    int s = 0, top = S - 1;
    while (s < top) {
      const int mid = (s + top + 1) >> 1;
      if (uniform(pfx[mid]) <= x) s = mid; else top = mid - 1;
    }
    return s;
  };
  auto tiles_of = [&](int s) { return uniform(sm.preR[s + 1]) - uniform(sm.preR[s]); };
  auto single_seq = [&](int s) { return uniform(sm.len[s]) <= T1; };
  // PARTS: the partition boundary nearest to virtual tile x (a one-pass sequence is
  // one piece); otherwise x itself
  auto snap = [&](long long x) -> long long {
    if (x >= T) return T;
    if constexpr (!PARTS) return x;
    const int s = seq_at(sm.pre, x);
    const long long p0 = uniform(sm.pre[s]);
    const long long cs = uniform(sm.pre[s + 1]) - p0;
    const long long off = x - p0;
    if (single_seq(s)) return p0 + (2 * off >= cs ? cs : 0);
    const long long np = (tiles_of(s) + P16 - 1) / P16;
    long long p = (2 * off + unit_v) / (2 * unit_v);
    if (p > np) p = np;
    return p0 + (p * unit_v < cs ? p * unit_v : cs);
  };
  // first real tile at or after virtual tile x (x a share boundary)
  auto real = [&](long long x) -> int {
    if (x >= T) return TR;
    const int s = seq_at(sm.pre, x);
    const int off = static_cast<int>(x - uniform(sm.pre[s]));
    const int n = tiles_of(s), R0 = uniform(sm.preR[s]);
    if constexpr (PARTS) {
      if (single_seq(s)) return R0 + (off > 0 ? n : 0);
      return R0 + min(off / unit_v * P16, n);
    } else {
      return R0 + min(max(off - c, 0), n);
    }
  };
  const long long lo = snap(share_cut(T, j, NS, skew));
  const long long hi = snap(share_cut(T, j + 1, NS, skew));
  const int ra = real(lo), rb = real(hi);

  if (!PARTS && lo == hi) {
    // an empty share may lie inside a sequence that neighbouring shares split: the
    // identity (-inf, 0) in slot 0
    for (int h = tid; h < G; h += NT) a.ws_ml[2LL * r * G + h] = make_float2(kNegInf, 0.f);
  }

  // where the result of piece [ps, pe) of sequence s goes: a record index, or -1 - s
  // for the output rows of s (the piece is the whole sequence)
  auto dest_of = [&](int s, int ps, int pe) -> long long {
    const int R0 = uniform(sm.preR[s]), R1 = uniform(sm.preR[s + 1]);
    if constexpr (PARTS) {
      if (single_seq(s)) return -1LL - s;
      return (static_cast<long long>(s) * Hkv + kvh) * a.max_parts + (ps - R0) / P16;
    } else {
      if (ps == R0 && pe == R1) return -1LL - s;
      return 2LL * r + (ps == R0 ? 1 : 0);
    }
  };

  int lane = tid & 63;
  int col = lane & 15;     // query head of the group (MFMA column), or tile row
  int grp = lane >> 4;     // 4-lane-group index: k-slot block / 4-row block
  // Online-softmax state of the wave's current piece (lane: head `col`, tokens of row
  // block `grp`): running max in base 2, the lane's share of the exp sum, O^T.
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int cc = 0; cc < DB; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the result of a piece, written directly: output rows (dest < 0: -1 - sequence) or
  // its partial record; max M, exp sum Lsum, accumulator acc
  auto write_piece = [&](long long dest, float M, float Lsum) {
    if (col < G) {
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
      if (dest < 0) {
        const int s = static_cast<int>(-1 - dest);
        uint16_t* o = static_cast<uint16_t*>(a.out) + ((size_t)s * Hq + kvh * G + col) * D + 4 * grp;
#pragma unroll
        for (int cc = 0; cc < DB; ++cc) {
          const f32x4 y = acc[cc] * inv;
          const u32x2 packed = {DT::bits(y[0]) | (DT::bits(y[1]) << 16),
                                DT::bits(y[2]) | (DT::bits(y[3]) << 16)};
          *reinterpret_cast<u32x2*>(o + 16 * cc) = packed;
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < DB; ++cc)
          *reinterpret_cast<f32x4*>(a.ws_acc + rec_acc_index(cc, dest, col, G, a.records) +
                                    4 * grp) = acc[cc] * inv;
        if (grp == 0) a.ws_ml[dest * G + col] = make_float2(M, Lsum);
      }
    }
  };
  // a record finished inside the walk: into a pool slot if one is free (the whole
  // workgroup writes the pool out after the walk); false if the pool is full
  const int kp4 = DB * G * 4;                        // packed f32x4 of one record
  const int slot_f4 = kp4 + 9;
  const int n_slots = PARTS ? StreamLds<D, W>::kPoolF4 / slot_f4 : 0;
  auto pool_piece = [&](long long dest, float M, float Lsum) -> bool {
    if (n_slots <= W - 1) return false;
    int slot = 0;
    if (lane == 0)
      slot = __hip_atomic_fetch_add(&sm.pool_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    slot = __builtin_amdgcn_readfirstlane(slot);
    if (slot >= n_slots) return false;
    f32x4* base = sm.pool + slot * slot_f4;
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    if (col < G) {
#pragma unroll
      for (int cc = 0; cc < DB; ++cc) base[(cc * G + col) * 4 + grp] = acc[cc] * inv;
      if (grp == 0) reinterpret_cast<float2*>(base + kp4)[col] = make_float2(M, Lsum);
    }
    if (lane == 0) *reinterpret_cast<long long*>(base + kp4 + 8) = dest;
    return true;
  };
  // a record finished inside the walk once the pool is full: into the wave's next
  // hold slot, packed through the wave's tile slot (idle between the tile's last
  // P.V read and the next tile's staging); false when the slots are used up
  int n_held = 0;
  auto hold_piece = [&](long long dest, float M, float Lsum) -> bool {
    if constexpr (!HOLD) {
      return false;
    } else {
      if (G > kHoldMaxGroup || n_held >= kHoldRecs) return false;
      f32x4* scratch = reinterpret_cast<f32x4*>(sm.tiles + wave * 2 * TILE_BYTES);
      float* meta = reinterpret_cast<float*>(scratch + kp4);
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
      wave_lds_fence();
      if (col < G) {
#pragma unroll
        for (int cc = 0; cc < DB; ++cc) scratch[(cc * G + col) * 4 + grp] = acc[cc] * inv;
        if (grp == 0) {
          meta[2 * col] = M;
          meta[2 * col + 1] = Lsum;
        }
      }
      if (lane == 0) *reinterpret_cast<long long*>(meta + 2 * G) = dest;
      wave_lds_fence();
      float v[kHoldStride];
#pragma unroll
      for (int i = 0; i < kHoldMaxGroup; ++i) {
        const f32x4 t = scratch[lane + 64 * i];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = t[e];
      }
      v[4 * kHoldMaxGroup] = meta[lane];
      hold_put(n_held, v);
      ++n_held;
      wave_lds_fence();
      return true;
    }
  };
  // a later wave's first piece, begun by an earlier wave: parked for the merge
  auto park = [&](int ps, float M, float Lsum) {
    if (wave == 0) return;       // never: wave 0's pieces all begin inside its run
    const int v = wave - 1;
    f32x4* base = sm.pool + v * slot_f4;
    if (col < G) {
#pragma unroll
      for (int cc = 0; cc < DB; ++cc) base[(cc * G + col) * 4 + grp] = acc[cc];
      if (grp == 0) reinterpret_cast<float2*>(base + kp4)[col] = make_float2(M, Lsum);
    }
    if (lane == 0) sm.park_start[v] = ps;
  };
  auto full_sum = [&]() {
    const float l = xor_add<16>(l_run);
    return xor_add<32>(l);
  };

  // this wave's real tiles
  const int wa = ra + static_cast<int>(static_cast<long long>(rb - ra) * wave / W);
  const int wb = ra + static_cast<int>(static_cast<long long>(rb - ra) * (wave + 1) / W);

  // the piece holding real tile x of sequence s, as the share sees it: [ps, pe)
  auto piece_of = [&](int s, int x, int& ps, int& pe) {
    const int R0 = uniform(sm.preR[s]), R1 = uniform(sm.preR[s + 1]);
    if constexpr (PARTS) {
      if (single_seq(s)) {
        ps = R0;
        pe = R1;
      } else {
        ps = R0 + (x - R0) / P16 * P16;
        pe = min(ps + P16, R1);
      }
    } else {
      ps = max(R0, ra);
      pe = min(R1, rb);
    }
  };

  bool merger = false;        // this wave begins a piece that later waves continue
  int p_s = 0, ps = 0, pe = 0;
  float kept_l = 0.f;
  const int bs = a.block_size, mbps = a.max_blocks_per_seq;
  if (wa < wb) {
    unsigned char* ldsK = sm.tiles + wave * 2 * TILE_BYTES;
    unsigned char* ldsV = ldsK + TILE_BYTES;
    // the group's query rows as the B operand of S^T = K Q^T: lane (col, grp) holds
    // dims 32*ks + 8*grp .. +7 of head kvh*G + col (zero for col >= G)
    auto load_q = [&](int s, u32x4 (&q)[KS]) {
      const uint16_t* qrow = a.q + ((size_t)s * Hq + (size_t)kvh * G + col) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        q[ks] = u32x4{0, 0, 0, 0};
        if (col < G) q[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
      }
    };
    // cursor: sequence, tile within it, its tile count and length
    auto advance = [&](int& s, int& k, int& n, int& L) {
      if (++k >= n) {
        do { ++s; } while (s < S - 1 && uniform(sm.preR[s + 1]) == uniform(sm.preR[s]));
        k = 0;
        n = tiles_of(s);
        L = uniform(sm.len[s]);
      }
    };
    int cs = seq_at(sm.preR, wa), ck = wa - uniform(sm.preR[cs]);
    int cn = tiles_of(cs), cL = uniform(sm.len[cs]);
    u32x4 qc[KS];
    load_q(cs, qc);
    const int2 pg0 = tile_pages(a.bt, cs, kTile * ck, cL, bs, mbps);
    int ns = cs, nk = ck, nn = cn, nL = cL;
    int2 pg_next = make_int2(0, 0);
    if (wa + 1 < wb) {
      advance(ns, nk, nn, nL);
      pg_next = tile_pages(a.bt, ns, kTile * nk, nL, bs, mbps);
    }
    u32x4 rk[LOADS], rv[LOADS];
    {
      size_t lo_, hi_;
      tile_offsets(pg0, kTile * ck, kvh, Hkv, bs, D, lo_, hi_);
      load_tile<D>(a.kc + lo_, a.kc + hi_, lane, rk);
      load_tile<D>(a.vc + lo_, a.vc + hi_, lane, rv);
    }
    p_s = cs;
    piece_of(cs, wa, ps, pe);

    for (int x = wa; x < wb; ++x) {
      // The lane index is made opaque here so that the per-lane LDS addresses derived
      // from it are recomputed each tile instead of being held across the loop, which
      // keeps the register count down (191 VGPRs instead of 245, with 64 AGPRs, at
      // head_dim 256).
      lane = threadIdx.x & 63;
      asm volatile("" : "+v"(lane));
      col = lane & 15;
      grp = lane >> 4;
      // stage tile x in this wave's LDS slot
      wave_lds_fence();
#pragma unroll
      for (int jj = 0; jj < LOADS; ++jj) {
        const int cidx = jj * 64 + lane;
        const int row = cidx / Z::kChunks;
        *reinterpret_cast<u32x4*>(ldsK + Z::byte_off(row, cidx % Z::kChunks)) = rk[jj];
        *reinterpret_cast<u32x4*>(ldsV + ZV::byte_off(row, cidx % Z::kChunks)) = rv[jj];
      }
      wave_lds_fence();
      // tile x + 1 while x is consumed; the page ids of x + 2
      const bool more = x + 1 < wb;
      const bool new_seq = more && ns != cs;
      if (more) {
        size_t lo_, hi_;
        tile_offsets(pg_next, kTile * nk, kvh, Hkv, bs, D, lo_, hi_);
        load_tile<D>(a.kc + lo_, a.kc + hi_, lane, rk);
        load_tile<D>(a.vc + lo_, a.vc + hi_, lane, rv);
      }
      int s2 = ns, k2 = nk, n2 = nn, L2 = nL;
      if (x + 2 < wb) {
        advance(s2, k2, n2, L2);
        pg_next = tile_pages(a.bt, s2, kTile * k2, L2, bs, mbps);
      }

      // S^T[token, head] = sum_d K[token, d] Q[head, d]
      const int t0 = kTile * ck;
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(ldsK + Z::byte_off(col, 4 * ks + grp));
        st = DT::mfma_qk(kop, qc[ks], st);
      }
      // the next tile begins another sequence: its query rows replace this one's,
      // which the QK^T products above were the last to use
      if (new_seq) load_q(ns, qc);
      // online softmax in base 2; this lane holds head `col`, tokens t0 + 4*grp + e
      const int tk = t0 + 4 * grp;
      float xv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[e] = (tk + e < cL) ? st[e] * a.scale_log2 : kNegInf;
      float mx = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
      mx = xor_max<16>(mx);
      mx = xor_max<32>(mx);
      // Lazy rescale: the running max moves only when a head's tile max exceeds it by
      // more than 2^kLazyRescaleLog2 (a wave-uniform branch); otherwise the tile's
      // probabilities are taken against the old max (each at most 2^8, inside f16
      // and bf16) and the accumulators keep their scale.  The first tile of a piece
      // always moves it (the running max is -inf and every head has a key there).
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int cc = 0; cc < DB; ++cc) acc[cc] *= alpha;
      }
      u32x2 p_hi, p_lo;
      l_run += prob_operands<DT>(xv, m_run, p_hi, p_lo);
      // O^T[d, head] += sum_t V[t, d] P[head, t]: V^T read transposed out of the tile
      const bool tail = t0 + kTile > cL;
      uint32_t keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;   // masks slots past the end
      if (tail) {
        const int nv = cL - tk;
        keep_lo = (nv > 0 ? 0x0000ffffu : 0u) | (nv > 1 ? 0xffff0000u : 0u);
        keep_hi = (nv > 2 ? 0x0000ffffu : 0u) | (nv > 3 ? 0xffff0000u : 0u);
      }
      const int vrow = 4 * grp + (col >> 2);
#pragma unroll
      for (int cc = 0; cc < DB; ++cc) {
        const int vcol = 16 * cc + 4 * (col & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(ldsV + ZV::byte_off(vrow, vcol >> 3) + (vcol & 7) * 2));
        u32x2 vop = __builtin_bit_cast(u32x2, raw);
        vop.x &= keep_lo;
        vop.y &= keep_hi;
        acc[cc] = pv_mfma<DT>(vop, p_hi, p_lo, acc[cc]);
      }

      // the piece ends with this tile and the wave goes on: finish it from registers
      // (or park it, if an earlier wave began it) and start the next one
      if (more && x + 1 == pe) {
        const float Ls = full_sum();
        if (ps >= wa) {
          const long long dest = dest_of(p_s, ps, pe);
          if (dest < 0 || !(pool_piece(dest, m_run, Ls) || hold_piece(dest, m_run, Ls)))
            write_piece(dest, m_run, Ls);
        } else {
          park(ps, m_run, Ls);
        }
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int cc = 0; cc < DB; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
        p_s = ns;
        piece_of(ns, x + 1, ps, pe);
      }
      cs = ns; ck = nk; cn = nn; cL = nL;
      ns = s2; nk = k2; nn = n2; nL = L2;
    }
    // the wave's last piece
    kept_l = full_sum();
    if (ps >= wa) {
      if (pe <= wb) write_piece(dest_of(p_s, ps, pe), m_run, kept_l);
      else merger = true;
    } else {
      park(ps, m_run, kept_l);
    }
  }
  if constexpr (HOLD) {
    // the wave's held records, written once its walk is over
    for (int k = 0; k < n_held; ++k) {
      float v[kHoldStride];
      hold_get(k, v);
      const unsigned lo = static_cast<unsigned>(
          __builtin_amdgcn_readlane(__float_as_int(v[4 * kHoldMaxGroup]), 2 * G));
      const unsigned hi = static_cast<unsigned>(
          __builtin_amdgcn_readlane(__float_as_int(v[4 * kHoldMaxGroup]), 2 * G + 1));
      const long long d = static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo);
#pragma unroll
      for (int i = 0; i < kHoldMaxGroup; ++i) {
        if (i < G) {
          const int jj = lane + 64 * i;
          const int cc = jj / (4 * G), rem = jj - cc * 4 * G;
          *reinterpret_cast<f32x4*>(a.ws_acc + rec_acc_index(cc, d, rem >> 2, G, a.records) +
                                    4 * (rem & 3)) =
              f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
        }
      }
      if (lane < 2 * G) reinterpret_cast<float*>(a.ws_ml + d * G)[lane] = v[4 * kHoldMaxGroup];
    }
  }
  // pieces cut by range boundaries: the first wave holding one merges the parked parts
  __syncthreads();
  if constexpr (PARTS) {
    // the pooled records, written by the whole workgroup
    const int used = min(uniform(sm.pool_next), n_slots);
    for (int sl = W - 1; sl < used; ++sl) {
      const f32x4* base = sm.pool + sl * slot_f4;
      const long long d = *reinterpret_cast<const long long*>(base + kp4 + 8);
      for (int i = tid; i < kp4; i += NT) {
        const int cc = i / (4 * G), rem = i - cc * 4 * G;
        *reinterpret_cast<f32x4*>(a.ws_acc + rec_acc_index(cc, d, rem >> 2, G, a.records) +
                                  4 * (rem & 3)) = base[i];
      }
      if (tid < G) a.ws_ml[d * G + tid] = reinterpret_cast<const float2*>(base + kp4)[tid];
    }
  }
  if (merger) {
    float M = m_run, Lsum = kept_l;
    for (int v = wave + 1; v < W; ++v) {
      if (uniform(sm.park_start[v - 1]) != ps) continue;   // no part of this piece
      const f32x4* base = sm.pool + (v - 1) * slot_f4;
      const float2 ml =
          col < G ? reinterpret_cast<const float2*>(base + kp4)[col] : make_float2(kNegInf, 0.f);
      const float Mn = fmaxf(M, ml.x);
      const float f = Mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float fv = Mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml.x - Mn);
      Lsum = Lsum * f + ml.y * fv;
#pragma unroll
      for (int cc = 0; cc < DB; ++cc) {
        const f32x4 pv = col < G ? base[(cc * G + col) * 4 + grp] : f32x4{0.f, 0.f, 0.f, 0.f};
        acc[cc] = acc[cc] * f + pv * fv;
      }
      M = Mn;
    }
    write_piece(dest_of(p_s, ps, pe), M, Lsum);
  }

  if constexpr (!PARTS) {
    // the sequence this share begins and later shares continue: phase 2 merges it
    if (tid == 0) {
      int2 job = make_int2(-1, 0);
      if (rb > ra) {
        const int s = seq_at(sm.preR, rb - 1);
        if (sm.preR[s] >= ra && sm.preR[s + 1] > rb)
          job = make_int2(s * Hkv + kvh,
                          static_cast<int>(share_holding(T, sm.pre[s + 1] - 1, NS, skew) - j + 1));
      }
      a.jobs[r] = job;
    }
  }
}

}  // namespace pa
