// Host side of libpagedattn: argument validation, the length-tiered plan, and the
// launches of the gfx950 kernels in pa_kernels.h.  C ABI in include/pagedattn.h.
//
// Tiering follows the three-tier decode dispatch on the page of commit b80fd2b
// (short sequences in one workgroup, long ones split into partitions merged in
// a second kernel), re-thresholded for 256 compute units: one pass only pays
// when the batch alone supplies enough workgroups; otherwise every sequence
// longer than one partition is split.  The partition size is an argument, as
// the page of commit 8d26e23 asks ("should be tunable"); 0 sizes partitions so
// the step's K/V is spread over one workgroup per compute unit.
#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <vector>

#include "pa_kernels.h"
#include "pa_prefill.h"
#include "pa_stream.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

#ifndef PA_WAVES
#define PA_WAVES 4
#endif
constexpr int kWaves = PA_WAVES;            // waves per phase-1 workgroup
// tokens: smallest automatic partition.  Small steps are latency-bound, so they
// are spread over more workgroups with one tile per wave; measured on 1 x 1024
// tokens (us/step hot): 256 -> 17.3, 128 -> 14.7, 64 -> 13.3, 32 -> 13.1.
constexpr int kMinAutoPartition = 64;
constexpr int kDefaultCUs = 256;            // MI355X
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kMinTilesPerWG = 4;         // balanced mode: at least one tile per wave
// XCD-paired shares: permille of a pair's mean the member on the even XCD takes
// in addition.  Measured on 4 x 102400 tokens with fixed partitions: per-XCD
// mean workgroup times even out at 80 (odd XCDs ~8-10% slower with equal
// shares), 258.4 -> 252.2 us/step.
constexpr int kDefaultXcdSkew = 80;
constexpr int kCusPerXcd = 32;             // MI355X: 8 XCDs of 32 CUs
// Balanced mode: tiles of streaming a piece's start costs (head_dim 256, one
// workgroup per CU).  Measured on 32 x U[512, 8192] with equal shares: a share
// holding two pieces ran 4.8 us (about 8 tiles) longer than one holding one.
// Scaled to other head sizes (a tile carries head_dim/256 of the bytes) and
// halved with two workgroups per CU (each streams at half the rate).
constexpr int kPieceCostTiles = 8;
// Per-wave streams: a piece that starts inside a wave's run costs a state flush and,
// for a new sequence, query rows loaded with its first tile; counted as one tile.
constexpr int kStreamPieceCost = 1;
constexpr int kBalancedSlices = 8;        // balanced phase 2: 16-wide slices per workgroup

// 16-wide head_dim slices one balanced phase-2 workgroup merges
constexpr int balanced_slices(int D) { return D / 16 < kBalancedSlices ? D / 16 : kBalancedSlices; }

struct Plan {
  bool balanced = false; // length-balanced split (partition_size 0) vs fixed partitions
  bool stream = false;   // phase 1 as per-wave streams (pa_phase1_stream_kernel)
  bool parts = false;    // stream kernel with an explicit partition size
  bool head_seq = false; // head-sequential ablation (fixed partitions)
  int P = 0;             // partition size (tokens), grid mode
  int T1 = 0;            // single-pass threshold (tokens), grid mode
  int max_parts = 0;     // partitions per (seq, kv head) slot; 0 = no phase 2, grid mode
  int max_seq_len = 0;   // resolved length bound
  int group = 0;         // query heads per workgroup
  int units = 0;         // head units per sequence (num_kv_heads, or num_heads)
  int num_wg = 0;        // phase-1 workgroups, balanced mode
  int xcd_skew = 0;      // XCD-paired shares (permille), 0 = equal shares
  int piece_cost = 0;    // balanced mode: virtual tiles per sequence start
  long long records = 0; // partial records in the workspace
  long long grid1 = 0, grid2 = 0;
  bool fused = false;    // partials merged in phase 1 (ticket counters), no phase 2
  int reduce_slices = 1;     // 16-wide head_dim slices per phase-2 workgroup
  size_t ws_acc_off = 0, ws_ml_off = 0, ws_jobs_off = 0, ws_bytes = 0;
};

// Ticket counters of the fused combine sit at the start of every workspace that
// holds records, whatever the plan, so a workspace cleared once stays valid for
// any later call: the other regions never overlap them.
constexpr size_t kTicketBytes = PA_WORKSPACE_TICKET_BYTES;
constexpr long long kMaxTickets = kTicketBytes / sizeof(unsigned);

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Validation shared by every entry point (pointers excepted).
int check_sizes(int S, int Hq, int Hkv, int D, int bs, int mbps, int max_len, int P, int dtype) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || mbps < 0) return PA_ERR_SHAPE;
  if (Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (P < 0 || P % 16 != 0) return PA_ERR_PARTITION;
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(D)) return PA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return PA_ERR_UNSUPPORTED;
  if (bs != 8 && bs % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (S > 0 && mbps < 1) return PA_ERR_SHAPE;
  const long long cap = static_cast<long long>(mbps) * bs;
  if (max_len > cap) return PA_ERR_SHAPE;
  if (cap > std::numeric_limits<int>::max()) return PA_ERR_SHAPE;
  return PA_OK;
}

// Resident phase-1 workgroups per CU the fixed partitions aim at.  Measured on
// 4 x 102400 tokens: with head_dim 256 and pages of 16 or more tokens one
// workgroup per CU streams fastest (6.5 TB/s; two: -3%); with head_dim 128 or 64,
// or 8-token pages, a tile carries fewer bytes per page or per softmax step and a
// second resident workgroup hides the per-tile latency (head_dim 64: 3.2 -> 5.4
// TB/s; 128: 4.7 -> 6.1; 8-token pages: 5.0 -> 5.9).
int workgroups_per_cu(int D, int bs) { return D >= 256 && bs >= 16 ? 1 : 2; }

// Resident workgroups per CU of the stream kernel: its LDS (tile slots, the parked
// states of three waves, the per-sequence prefixes) is 124 KiB at head_dim 256, so
// one; at head_dim 128 or 64 two.
int stream_workgroups_per_cu(int D) { return D >= 256 ? 1 : 2; }

// Fixed partition size when the caller passes 0 but the balanced split does not
// apply (equal lengths declared, a forced tier, or more sequences than it keeps
// in LDS): spread the step's K/V over `slots` workgroups (CUs times
// workgroups_per_cu).  The work estimate is num_seqs * max_seq_len tokens per KV
// head (exact for equal lengths), or the caller's total-token hint.
int auto_partition(long long S, int Hkv, int max_len, long long slots, long long total_hint) {
  const long long tokens = total_hint > 0 ? total_hint : S * max_len;
  long long p = (tokens * Hkv + slots - 1) / slots;
  p = (p + 15) / 16 * 16;
  if (p < kMinAutoPartition) p = kMinAutoPartition;
  if (p > max_len) p = (max_len + 15) / 16 * 16;
  if (p < 16) p = 16;
  return static_cast<int>(p);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int make_plan(int S, int Hq, int Hkv, int D, int bs, int mbps, int max_len, int P_req,
              const pa_options* opt, Plan& pl) {
  pl = Plan{};
  // per-query-head ablation: one workgroup per query head (each KV page is then
  // read once per query head instead of once per KV head)
  const bool per_qhead = opt && opt->per_query_head;
  // head-sequential ablation: the grouped fixed-partition grid, heads taken in turn
  pl.head_seq = opt && opt->head_sequential;
  pl.units = per_qhead ? Hq : Hkv;
  pl.group = Hq / pl.units;
  pl.max_seq_len = max_len > 0 ? max_len : mbps * bs;
  const int cus = (opt && opt->num_cus > 0) ? opt->num_cus : kDefaultCUs;
  const bool forced_tier = opt && opt->single_pass_max_len >= 0;
  // a host-side total equal to num_seqs * max_seq_len means every sequence is at
  // the bound: fixed partitions of one workgroup per CU are then exactly balanced
  // and need no device-side prefix of seq_lens, as long as there are no more
  // segments than workgroup slots (256 x 16384 tokens, 1024 segments: fixed
  // partitions of whole sequences 2617 us, the balanced split 2559 us)
  const long long hint = opt ? opt->total_tokens_hint : 0;
  const long long slots_all = static_cast<long long>(cus) * workgroups_per_cu(D, bs);
  const bool uniform = hint > 0 && hint == static_cast<long long>(S) * pl.max_seq_len &&
                       static_cast<long long>(S) * pl.units <= slots_all;
  // the balanced kernel keeps its prefix of (virtual) tiles in 32-bit integers
  const long long max_tiles = (pl.max_seq_len + 15) / 16;
  const long long tiles_bound = static_cast<long long>(S) * (max_tiles + 1024);
  pl.balanced = P_req == 0 && !forced_tier && !uniform && !per_qhead && !pl.head_seq &&
                S <= pa::kMaxBalancedSeqs && tiles_bound <= std::numeric_limits<int>::max();
  // per-wave streams (the balanced split, and explicit partition sizes): not with the
  // fused combine or the per-query-head ablation, which keep one workgroup per piece
  const bool stream_ok = !(opt && opt->stream_walk < 0) && !per_qhead && !pl.head_seq &&
                         !(opt && opt->fused_combine) && S <= pa::kMaxBalancedSeqs;
  const int pc_req = opt ? opt->piece_cost : 0;
  const int stream_pc = pc_req == 0 ? kStreamPieceCost : (pc_req < 0 ? 0 : (pc_req > 1024 ? 1024 : pc_req));
  int parts_T1 = 0;
  long long parts_max = 1;       // partitions of the longest sequence
  bool stream_parts = false;
  if (stream_ok && P_req > 0) {
    parts_T1 = forced_tier ? opt->single_pass_max_len : P_req;
    const long long P16 = P_req / 16;
    parts_max = pl.max_seq_len > parts_T1 ? (max_tiles + P16 - 1) / P16 : 1;
    // the kernel keeps virtual tiles (partitions x piece cost + tiles) in 32 bits
    stream_parts = static_cast<long long>(S) * (max_tiles + parts_max * stream_pc) <=
                   std::numeric_limits<int>::max();
  }
  // XCD-paired shares apply to automatic splits, and to the shares (not the
  // partitions) of explicit partition sizes on per-wave streams; the pages' dense
  // grid and the per-query-head ablation keep equal work per workgroup
  int skew = opt ? opt->xcd_skew : 0;
  skew = skew == 0 ? kDefaultXcdSkew : (skew < 0 ? 0 : (skew > 500 ? 500 : skew));
  if (per_qhead || (P_req != 0 && !stream_parts)) skew = 0;
  // a single-XCD partition of the device (32 CUs) has no second parity to pair with
  if (cus < 2 * kCusPerXcd) skew = 0;
  if (pl.balanced) {
    pl.stream = stream_ok;
    // shares x KV heads: workgroups_per_cu resident workgroups per CU (measured on
    // the batch and long workloads as for fixed partitions: one per CU at head_dim
    // 256 with 16-token pages, 4% faster cold on the batch than two), but at least
    // kMinTilesPerWG tiles per workgroup
    const long long tiles = static_cast<long long>(S) * max_tiles;
    long long ns = (tiles + kMinTilesPerWG - 1) / kMinTilesPerWG;
    const long long slots = static_cast<long long>(cus) *
                            (pl.stream ? stream_workgroups_per_cu(D) : workgroups_per_cu(D, bs));
    const long long ns_max = slots / Hkv > 0 ? slots / Hkv : 1;
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    pl.num_wg = static_cast<int>(ns * Hkv);
    pl.xcd_skew = ns % 2 == 0 ? skew : 0;     // shares pair up across XCD parities
    pl.piece_cost = pl.stream ? stream_pc
                    : pc_req == 0 ? kPieceCostTiles * 256 / D / workgroups_per_cu(D, bs)
                                  : (pc_req < 0 ? 0 : (pc_req > 1024 ? 1024 : pc_req));
    pl.records = 2LL * pl.num_wg;
    pl.grid1 = pl.num_wg;
    pl.grid2 = static_cast<long long>(pl.num_wg) * (D / 16 / balanced_slices(D));
    pl.reduce_slices = balanced_slices(D);
    pl.T1 = -1;
  } else if (stream_parts) {
    // the pages' partitions of P tokens, one partial each, walked by per-wave streams
    // over shares that end on partition boundaries
    pl.stream = pl.parts = true;
    pl.P = P_req;
    pl.T1 = parts_T1;
    if (pl.max_seq_len > pl.T1) pl.max_parts = (pl.max_seq_len + pl.P - 1) / pl.P;
    const long long slots = static_cast<long long>(cus) * stream_workgroups_per_cu(D);
    long long ns = slots / Hkv > 0 ? slots / Hkv : 1;
    const long long pieces = static_cast<long long>(S) * parts_max;
    if (ns > pieces) ns = pieces;
    if (ns < 1) ns = 1;
    pl.num_wg = static_cast<int>(ns * Hkv);
    pl.xcd_skew = ns % 2 == 0 ? skew : 0;
    pl.piece_cost = stream_pc;
    pl.grid1 = pl.num_wg;
    pl.records = static_cast<long long>(S) * pl.units * pl.max_parts;
  } else {
    pl.P = P_req > 0 ? P_req
                     : auto_partition(S, pl.units, pl.max_seq_len,
                                      static_cast<long long>(cus) * workgroups_per_cu(D, bs),
                                      hint);
    // a sequence that fits in one partition is served in one pass
    pl.T1 = forced_tier ? opt->single_pass_max_len : pl.P;
    if (pl.max_seq_len > pl.T1) pl.max_parts = (pl.max_seq_len + pl.P - 1) / pl.P;
    pl.xcd_skew = pl.max_parts >= 2 ? skew : 0;
    const long long parts = pl.max_parts > 0 ? pl.max_parts : 1;
    pl.grid1 = static_cast<long long>(S) * pl.units * parts;
    pl.records = static_cast<long long>(S) * pl.units * pl.max_parts;
  }
  if (!pl.balanced && pl.max_parts > 0) {
    // Phase 2 of fixed partitions: a workgroup takes `slices` 16-wide head_dim slices
    // of one segment and folds its partials kRedThreads / (4 * slices) * unroll at a
    // time.  Wider workgroups are fewer but need more rounds for a long segment.
    // Measured on MI355X (D 256, 6 heads per group, 16 to 256 segments of up to 400
    // partials): about 1 us per round of the longest segment and 6 ns per workgroup,
    // so the width with the least rounds * 1000 + workgroups * 6 (ns) is taken.
    const long long segs = static_cast<long long>(S) * pl.units;
    long long best_cost = std::numeric_limits<long long>::max();
    for (const int spw : {1, 2, 4, balanced_slices(D)}) {
      if (spw > balanced_slices(D)) continue;
      const int per_round = pa::kRedThreads / (4 * spw) * pa::reduce_unroll(pl.group);
      const long long rounds = (pl.max_parts + per_round - 1) / per_round;
      const long long wgs = segs * (D / 16 / spw);
      const long long cost = rounds * 1000 + wgs * 6;
      if (cost <= best_cost) {             // ties go to the wider workgroup
        best_cost = cost;
        pl.reduce_slices = spw;
      }
    }
    pl.grid2 = segs * (D / 16 / pl.reduce_slices);
  }
  if (pl.grid1 > std::numeric_limits<int>::max() || pl.grid2 > std::numeric_limits<int>::max())
    return PA_ERR_SHAPE;
  if (pl.records > 0) {
    const long long segments = static_cast<long long>(S) * pl.units;
    pl.fused = opt && opt->fused_combine && segments <= kMaxTickets;
    if (pl.fused) pl.grid2 = 0;
    const size_t recs = static_cast<size_t>(pl.records) * pl.group;   // (record, head) pairs
    pl.ws_acc_off = kTicketBytes;
    pl.ws_ml_off = pl.ws_acc_off + align256(recs * D * sizeof(float));
    pl.ws_bytes = pl.ws_ml_off + recs * sizeof(float2);
    if (pl.balanced) {
      pl.ws_jobs_off = align256(pl.ws_bytes);
      pl.ws_bytes = pl.ws_jobs_off + static_cast<size_t>(pl.num_wg) * sizeof(int2);
    }
  }
  return PA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Phase 2 is instantiated per group size so its loads can all be in flight at once.
template <int D, class DT, int G>
void launch_reduce_g(int slices, unsigned grid, hipStream_t stream, const pa::DecodeArgs& args) {
  const dim3 block(pa::kRedThreads);
  switch (slices) {
    case 1: hipLaunchKernelGGL((pa::pa_reduce_kernel<D, DT, G, 1>), dim3(grid), block, 0, stream, args); break;
    case 2: hipLaunchKernelGGL((pa::pa_reduce_kernel<D, DT, G, 2>), dim3(grid), block, 0, stream, args); break;
    case 4: hipLaunchKernelGGL((pa::pa_reduce_kernel<D, DT, G, 4>), dim3(grid), block, 0, stream, args); break;
    default:
      if constexpr (balanced_slices(D) > 4)
        hipLaunchKernelGGL((pa::pa_reduce_kernel<D, DT, G, balanced_slices(D)>), dim3(grid), block,
                           0, stream, args);
      break;
  }
}

template <int D, class DT>
int launch_reduce(int group, int slices, unsigned grid, hipStream_t stream,
                  const pa::DecodeArgs& args) {
  switch (group) {
    case 1: launch_reduce_g<D, DT, 1>(slices, grid, stream, args); break;
    case 2: launch_reduce_g<D, DT, 2>(slices, grid, stream, args); break;
    case 3: launch_reduce_g<D, DT, 3>(slices, grid, stream, args); break;
    case 4: launch_reduce_g<D, DT, 4>(slices, grid, stream, args); break;
    case 5: launch_reduce_g<D, DT, 5>(slices, grid, stream, args); break;
    case 6: launch_reduce_g<D, DT, 6>(slices, grid, stream, args); break;
    case 7: launch_reduce_g<D, DT, 7>(slices, grid, stream, args); break;
    case 8: launch_reduce_g<D, DT, 8>(slices, grid, stream, args); break;
    case 9: launch_reduce_g<D, DT, 9>(slices, grid, stream, args); break;
    case 10: launch_reduce_g<D, DT, 10>(slices, grid, stream, args); break;
    case 11: launch_reduce_g<D, DT, 11>(slices, grid, stream, args); break;
    case 12: launch_reduce_g<D, DT, 12>(slices, grid, stream, args); break;
    case 13: launch_reduce_g<D, DT, 13>(slices, grid, stream, args); break;
    case 14: launch_reduce_g<D, DT, 14>(slices, grid, stream, args); break;
    case 15: launch_reduce_g<D, DT, 15>(slices, grid, stream, args); break;
    case 16: launch_reduce_g<D, DT, 16>(slices, grid, stream, args); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <int D, class DT>
int launch_decode(const pa::DecodeArgs& args, const Plan& pl, hipStream_t stream,
                  const pa_options* opt) {
  if (opt && opt->phase1_begin) {
    if (hipEventRecord(opt->phase1_begin, stream) != hipSuccess) return PA_ERR_HIP;
  }
  if (pl.stream && pl.parts)
    hipLaunchKernelGGL((pa::pa_phase1_stream_kernel<D, DT, kWaves, true>),
                       dim3(static_cast<unsigned>(pl.grid1)), dim3(kWaves * 64), 0, stream, args);
  else if (pl.stream)
    hipLaunchKernelGGL((pa::pa_phase1_stream_kernel<D, DT, kWaves, false>),
                       dim3(static_cast<unsigned>(pl.grid1)), dim3(kWaves * 64), 0, stream, args);
  else if (pl.balanced)
    hipLaunchKernelGGL((pa::pa_phase1_balanced_kernel<D, DT, kWaves>),
                       dim3(static_cast<unsigned>(pl.grid1)), dim3(kWaves * 64), 0, stream, args);
  else if (pl.head_seq)
    hipLaunchKernelGGL((pa::pa_phase1_kernel<D, DT, kWaves, true>),
                       dim3(static_cast<unsigned>(pl.grid1)), dim3(kWaves * 64), 0, stream, args);
  else
    hipLaunchKernelGGL((pa::pa_phase1_kernel<D, DT, kWaves>),
                       dim3(static_cast<unsigned>(pl.grid1)), dim3(kWaves * 64), 0, stream, args);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (opt && opt->phase1_end) {
    if (hipEventRecord(opt->phase1_end, stream) != hipSuccess) return PA_ERR_HIP;
  }
  if (pl.grid2 > 0) {
    const int st = launch_reduce<D, DT>(pl.group, pl.reduce_slices, static_cast<unsigned>(pl.grid2),
                                        stream, args);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

}  // namespace

PA_API const char* paged_attn_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent sizes";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim must be 64, 128 or 256, group 1..16, block_size 8 "
             "or a multiple of 16, dtype f16 or bf16";
    case PA_ERR_PARTITION: return "PA_ERR_PARTITION: partition_size must be 0 or a multiple of 16";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch failed";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: pointer alignment (16 B for q and caches, 8 B for out, 256 B for workspace)";
    default: return "unknown pa_status_t";
  }
}

PA_API size_t paged_attn_workspace_size_ex(int num_seqs, int num_heads, int num_kv_heads,
                                           int head_dim, int block_size, int max_blocks_per_seq,
                                           int max_seq_len, int partition_size,
                                           const pa_options* opt) {
  if (check_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  max_seq_len, partition_size, PA_F16) != PA_OK)
    return static_cast<size_t>(-1);
  Plan pl;
  if (make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                max_seq_len, partition_size, opt, pl) != PA_OK)
    return static_cast<size_t>(-1);
  return pl.ws_bytes;
}

PA_API size_t paged_attn_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int max_blocks_per_seq,
                                        int max_seq_len, int partition_size) {
  return paged_attn_workspace_size_ex(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, max_seq_len, partition_size, nullptr);
}

namespace {

// Host mirror of the share boundaries of pa_phase1_stream_kernel with an explicit
// partition size (plan information only): shares of the step's virtual tiles
// (piece_cost per partition plus the real tiles), each boundary moved to the nearest
// partition boundary; returns how many shares hold real tiles.
long long stream_parts_busy_shares(const int32_t* lens, int S, const Plan& pl, int Hkv) {
  const long long P16 = pl.P / 16, c = pl.piece_cost, unit = c + P16;
  std::vector<long long> pre(S + 1, 0), preR(S + 1, 0);
  std::vector<bool> single(S, false);
  for (int s = 0; s < S; ++s) {
    long long L = lens[s] < pl.max_seq_len ? lens[s] : pl.max_seq_len;
    if (L < 0) L = 0;
    const long long n = (L + 15) / 16;
    single[s] = L <= pl.T1;
    const long long np = n == 0 ? 0 : (single[s] ? 1 : (n + P16 - 1) / P16);
    pre[s + 1] = pre[s] + np * c + n;
    preR[s + 1] = preR[s] + n;
  }
  const long long T = pre[S], NS = pl.num_wg / Hkv;
  auto seq_at = [&](long long x) {   // largest s < S with pre[s] <= x
    int s = 0, top = S - 1;
    while (s < top) {
      const int mid = (s + top + 1) / 2;
      if (pre[mid] <= x) s = mid; else top = mid - 1;
    }
    return s;
  };
  auto real_of_cut = [&](long long j) -> long long {
    const long long x = pa::share_cut(T, j, NS, pl.xcd_skew);
    if (x >= T) return preR[S];
    const int s = seq_at(x);
    const long long off = x - pre[s], cs = pre[s + 1] - pre[s], n = preR[s + 1] - preR[s];
    if (single[s]) return preR[s] + (2 * off >= cs ? n : 0);
    long long p = (2 * off + unit) / (2 * unit);
    const long long np = (n + P16 - 1) / P16;
    if (p > np) p = np;
    return preR[s] + (p * P16 < n ? p * P16 : n);
  };
  long long busy = 0;
  for (long long j = 0; j < NS; ++j)
    if (real_of_cut(j) < real_of_cut(j + 1)) ++busy;
  return busy;
}

}  // namespace

PA_API int paged_attn_plan(const int32_t* seq_lens_host, int num_seqs, int num_heads,
                           int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int max_seq_len, int partition_size,
                           int dtype, const pa_options* opt, pa_plan_info* info) {
  if (!info) return PA_ERR_NULL;
  int st = check_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, max_seq_len, partition_size, dtype);
  if (st != PA_OK) return st;
  Plan pl;
  st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 max_seq_len, partition_size, opt, pl);
  if (st != PA_OK) return st;
  *info = pa_plan_info{};
  info->partition_size = pl.P;
  info->single_pass_max_len = pl.T1;
  info->max_partitions = pl.max_parts;
  info->group = pl.group;
  info->phase1_workgroups = pl.grid1;
  info->phase2_workgroups = pl.grid2;
  info->reduce_slices = pl.grid2 > 0 ? pl.reduce_slices : 0;
  info->workspace_bytes = pl.ws_bytes;
  info->threads_per_workgroup = kWaves * 64;
  info->lds_bytes_phase1 = kWaves * 2 * pa::kTile * head_dim * 2;
  info->balanced = pl.balanced ? 1 : 0;
  info->fused = pl.fused ? 1 : 0;
  info->xcd_skew = pl.xcd_skew;
  info->piece_cost = pl.piece_cost;
  info->stream = pl.stream ? 1 : 0;
  info->head_sequential = pl.head_seq ? 1 : 0;
  if (seq_lens_host) {
    if (pl.balanced) {
      // host mirror of the device split: sequence s covers virtual tiles
      // [pre_s, pre_s + piece_cost + n) of T, its real ones last; share j takes
      // [share_cut(j), share_cut(j + 1)), one workgroup per KV head
      long long T = 0;
      for (int s = 0; s < num_seqs; ++s) {
        const int L = seq_lens_host[s] < pl.max_seq_len ? seq_lens_host[s] : pl.max_seq_len;
        T += L > 0 ? (L + 15) / 16 + pl.piece_cost : 0;   // virtual tiles
      }
      const long long NS = pl.num_wg / num_kv_heads;
      const int sk = pl.xcd_skew, pc = pl.piece_cost;
      long long start = 0;
      for (int s = 0; s < num_seqs; ++s) {
        const int L = seq_lens_host[s] < pl.max_seq_len ? seq_lens_host[s] : pl.max_seq_len;
        const long long n = L > 0 ? (L + 15) / 16 + pc : 0;   // virtual tiles
        if (n > 0 && pa::share_holding(T, start + pc, NS, sk) !=
                         pa::share_holding(T, start + n - 1, NS, sk))
          info->partitioned_seqs++;
        else
          info->single_pass_seqs++;
        start += n;
      }
      for (long long j = 0; j < NS; ++j)
        if (pa::share_cut(T, j, NS, sk) < pa::share_cut(T, j + 1, NS, sk))
          info->active_workgroups += num_kv_heads;
    } else {
      for (int s = 0; s < num_seqs; ++s) {
        const int L = seq_lens_host[s] < pl.max_seq_len ? seq_lens_host[s] : pl.max_seq_len;
        if (L <= pl.T1) {
          info->single_pass_seqs++;
          info->active_workgroups += num_kv_heads;
        } else {
          info->partitioned_seqs++;
          info->active_workgroups += static_cast<long long>(num_kv_heads) *
                                     ((L + pl.P - 1) / pl.P);
        }
      }
      if (pl.parts)
        info->active_workgroups =
            num_kv_heads * stream_parts_busy_shares(seq_lens_host, num_seqs, pl, num_kv_heads);
    }
  }
  return PA_OK;
}

PA_API int paged_attn_decode_ex(void* out, const void* q, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int num_seqs, int num_heads,
                                int num_kv_heads, int head_dim, int block_size, float scale,
                                int partition_size, void* workspace, hipStream_t stream,
                                int max_blocks_per_seq, int max_seq_len, int dtype,
                                size_t workspace_bytes, const pa_options* opt) {
  int st = check_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, max_seq_len, partition_size, dtype);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
      !aligned(out, 8) || !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  Plan pl;
  st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 max_seq_len, partition_size, opt, pl);
  if (st != PA_OK) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PA_ERR_ALIGN;
  }

  pa::DecodeArgs args{};
  args.out = out;
  args.q = static_cast<const uint16_t*>(q);
  args.kc = static_cast<const uint16_t*>(key_cache);
  args.vc = static_cast<const uint16_t*>(value_cache);
  args.bt = block_tables;
  args.seq_lens = seq_lens;
  char* ws = static_cast<char*>(workspace);
  args.ws_acc = pl.ws_bytes ? reinterpret_cast<float*>(ws + pl.ws_acc_off) : nullptr;
  args.tickets = pl.fused ? reinterpret_cast<unsigned*>(ws) : nullptr;
  args.ws_ml = pl.ws_bytes ? reinterpret_cast<float2*>(ws + pl.ws_ml_off) : nullptr;
  args.jobs = pl.balanced && pl.ws_bytes ? reinterpret_cast<int2*>(ws + pl.ws_jobs_off) : nullptr;
  args.records = pl.records;
  args.num_wg = pl.num_wg;
  args.xcd_skew = pl.xcd_skew;
  args.piece_cost = pl.piece_cost;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = pl.group;
  args.units = pl.units;
  args.kv_group = num_heads / num_kv_heads;
  args.block_size = block_size;
  args.max_blocks_per_seq = max_blocks_per_seq;
  args.max_seq_len = pl.max_seq_len;
  args.partition_size = pl.P;
  args.single_pass_max_len = pl.T1;
  args.max_parts = pl.max_parts;
  args.scale_log2 = scale * kLog2e;

  const bool f16 = dtype == PA_F16;
  switch (head_dim) {
    case 256: return f16 ? launch_decode<256, pa::F16>(args, pl, stream, opt)
                         : launch_decode<256, pa::BF16>(args, pl, stream, opt);
    case 128: return f16 ? launch_decode<128, pa::F16>(args, pl, stream, opt)
                         : launch_decode<128, pa::BF16>(args, pl, stream, opt);
    default: return f16 ? launch_decode<64, pa::F16>(args, pl, stream, opt)
                        : launch_decode<64, pa::BF16>(args, pl, stream, opt);
  }
}

PA_API int paged_attn_decode(void* out, const void* q, const void* key_cache,
                             const void* value_cache, const int32_t* block_tables,
                             const int32_t* seq_lens, int num_seqs, int num_heads,
                             int num_kv_heads, int head_dim, int block_size, float scale,
                             int partition_size, void* workspace, hipStream_t stream,
                             int max_blocks_per_seq, int max_seq_len, int dtype,
                             size_t workspace_bytes) {
  return paged_attn_decode_ex(out, q, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                              num_heads, num_kv_heads, head_dim, block_size, scale,
                              partition_size, workspace, stream, max_blocks_per_seq,
                              max_seq_len, dtype, workspace_bytes, nullptr);
}

namespace {

// Workspace of paged_attn_decode_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses its
// name as an address (on the host it is only a stand-in): the device address is
// taken once per device with hipGetSymbolAddress and kept in scratch_addr.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call
// made with that device current).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    scratch_addr[dev].store(p, std::memory_order_release);   // racing lookups store the same value
  }
  *out = p;
  return PA_OK;
}

}  // namespace

PA_API int paged_attn_decode_noalloc(void* out, const void* q, const void* key_cache,
                                     const void* value_cache, const int32_t* block_tables,
                                     const int32_t* seq_lens, int num_seqs, int num_heads,
                                     int num_kv_heads, int head_dim, int block_size, float scale,
                                     int partition_size, hipStream_t stream,
                                     int max_blocks_per_seq, int max_seq_len, int dtype) {
  int st = check_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, max_seq_len, partition_size, dtype);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  Plan pl;
  st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 max_seq_len, partition_size, nullptr, pl);
  if (st != PA_OK) return st;
  if (pl.ws_bytes > kScratchBytes) return PA_ERR_WORKSPACE;
  // Every region this plan reads (partial records, balanced jobs) is written by the
  // same call before it is read, so the array needs no clearing between calls; the
  // ticket area is used only by the fused combine, which this entry point never runs.
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_on_current_device(&ws);
    if (st != PA_OK) return st;
  }
  return paged_attn_decode_ex(out, q, key_cache, value_cache, block_tables, seq_lens, num_seqs,
                              num_heads, num_kv_heads, head_dim, block_size, scale,
                              partition_size, ws, stream, max_blocks_per_seq, max_seq_len, dtype,
                              pl.ws_bytes > 0 ? kScratchBytes : 0, nullptr);
}

PA_API int paged_attn_workspace_init(void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace) return PA_ERR_NULL;
  if (!aligned(workspace, 256)) return PA_ERR_ALIGN;
  const size_t n = (workspace_bytes < kTicketBytes ? workspace_bytes : kTicketBytes) / 16;
  if (n == 0) return PA_OK;
  hipLaunchKernelGGL(pa::pa_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, stream, static_cast<pa::u32x4*>(workspace), n);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

namespace {

template <int D, class DT>
void launch_prefill(const pa::PrefillArgs& args, unsigned grid, hipStream_t stream) {
  const dim3 block(pa::kPrefillWaves * 64);
  if (args.block_size == 8)
    hipLaunchKernelGGL((pa::pa_prefill_kernel<D, DT, 1>), dim3(grid), block, 0, stream, args);
  else
    hipLaunchKernelGGL((pa::pa_prefill_kernel<D, DT, 2>), dim3(grid), block, 0, stream, args);
}

// Division by the page size as a multiply-high and a shift (Granlund-Montgomery
// with a 31-bit dividend): with k = ceil(log2 bs) and m = floor(2^(31+k) / bs) + 1
// (below 2^32), t / bs == (t * m) >> (31 + k) for every 0 <= t < 2^31.
void page_divider(int bs, unsigned& magic, int& shift) {
  int k = 0;
  while ((1LL << k) < bs) ++k;
  magic = static_cast<unsigned>((1ULL << (31 + k)) / static_cast<unsigned long long>(bs) + 1);
  shift = k - 1;
}

}  // namespace

PA_API int paged_attn_prefill(void* out, const void* q, const void* k_new, const void* v_new,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, const int32_t* ctx_lens,
                              const int32_t* query_start, int num_seqs, int num_heads,
                              int num_kv_heads, int head_dim, int block_size, float scale,
                              int max_blocks_per_seq, int max_query_len, int max_ctx_len,
                              int dtype, hipStream_t stream) {
  int st = check_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, max_ctx_len, 0, dtype);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale) || max_query_len < 0 || max_ctx_len < 0) return PA_ERR_SHAPE;
  // the kernel keeps the byte stride of a cache page (num_kv_heads rows of
  // block_size x head_dim) and the byte offset of a 32-row step of the new keys in
  // 32-bit registers
  const unsigned long long row_block_bytes = static_cast<unsigned long long>(num_kv_heads) *
                                             (block_size > 32 ? block_size : 32) * head_dim * 2;
  if (row_block_bytes >= (1ULL << 32)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_new || !v_new || !key_cache || !value_cache || !block_tables ||
      !ctx_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(out, 8) || !aligned(block_tables, 4) ||
      !aligned(ctx_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  const int G = num_heads / num_kv_heads;
  const long long col_blocks =
      (static_cast<long long>(max_query_len) * G + pa::kPrefillCols - 1) / pa::kPrefillCols;
  const long long units = static_cast<long long>(num_seqs) * num_kv_heads;
  const long long upx = (units + pa::kXcds - 1) / pa::kXcds;
  const long long grid = pa::kXcds * upx * col_blocks;
  if (grid > std::numeric_limits<int>::max() || col_blocks > std::numeric_limits<int>::max())
    return PA_ERR_SHAPE;
  pa::PrefillArgs args{};
  args.out = out;
  args.q = static_cast<const uint16_t*>(q);
  args.k_new = static_cast<const uint16_t*>(k_new);
  args.v_new = static_cast<const uint16_t*>(v_new);
  args.kc = static_cast<const uint16_t*>(key_cache);
  args.vc = static_cast<const uint16_t*>(value_cache);
  args.bt = block_tables;
  args.ctx_lens = ctx_lens;
  args.qstart = query_start;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = G;
  args.block_size = block_size;
  page_divider(block_size, args.bs_magic, args.bs_shift);
  args.max_blocks_per_seq = max_blocks_per_seq;
  args.max_query_len = max_query_len;
  args.max_ctx_len = max_ctx_len;
  args.col_blocks = static_cast<int>(col_blocks);
  // the kernel takes |scale| into the exponent and negates Q for a negative scale; a
  // zero scale is passed as 2^-100, with which every exponent is below 2^-50 in
  // magnitude and rounds to weight 1 in fp32, the uniform weights a zero scale means
  args.scale_log2 = scale * kLog2e;
  if (args.scale_log2 == 0.f) args.scale_log2 = 0x1p-100f;
  const unsigned g = static_cast<unsigned>(grid);
  const bool f16 = dtype == PA_F16;
  switch (head_dim) {
    case 256: f16 ? launch_prefill<256, pa::F16>(args, g, stream)
                  : launch_prefill<256, pa::BF16>(args, g, stream); break;
    case 128: f16 ? launch_prefill<128, pa::F16>(args, g, stream)
                  : launch_prefill<128, pa::BF16>(args, g, stream); break;
    default: f16 ? launch_prefill<64, pa::F16>(args, g, stream)
                 : launch_prefill<64, pa::BF16>(args, g, stream); break;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

PA_API int paged_attn_read_probe(const void* src, size_t chunk_bytes, const long long* order,
                                 long long num_chunks, int num_workgroups, unsigned* sink,
                                 hipStream_t stream) {
  if (chunk_bytes != 4096 && chunk_bytes != 8192 && chunk_bytes != 16384) return PA_ERR_UNSUPPORTED;
  if (num_chunks < 0 || num_workgroups < 1 || num_workgroups > (1 << 20)) return PA_ERR_SHAPE;
  if (num_chunks == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (!aligned(src, 16) || !aligned(sink, 4) || (order && !aligned(order, 8))) return PA_ERR_ALIGN;
  const auto* s = static_cast<const pa::u32x4*>(src);
  const dim3 grid(static_cast<unsigned>(num_workgroups));
  if (chunk_bytes == 4096)
    hipLaunchKernelGGL(pa::pa_read_probe_kernel<4096>, grid, dim3(256), 0, stream, s, order,
                       num_chunks, sink);
  else if (chunk_bytes == 8192)
    hipLaunchKernelGGL(pa::pa_read_probe_kernel<8192>, grid, dim3(256), 0, stream, s, order,
                       num_chunks, sink);
  else
    hipLaunchKernelGGL(pa::pa_read_probe_kernel<16384>, grid, dim3(256), 0, stream, s, order,
                       num_chunks, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

PA_API int paged_attn_gather_probe(void* k_out, void* v_out, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* seq_lens, int num_seqs, int num_kv_heads,
                                   int head_dim, int block_size, int max_blocks_per_seq,
                                   int max_seq_len, hipStream_t stream) {
  int st = check_sizes(num_seqs, num_kv_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, max_seq_len, 0, PA_F16);
  if (st != PA_OK) return st;
  if (max_seq_len <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!k_out || !v_out || !key_cache || !value_cache || !block_tables || !seq_lens)
    return PA_ERR_NULL;
  if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16))
    return PA_ERR_ALIGN;
  const long long grid = static_cast<long long>(num_seqs) * num_kv_heads;
  if (grid > std::numeric_limits<int>::max()) return PA_ERR_SHAPE;
  pa::GatherArgs g{static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out),
                   static_cast<const uint16_t*>(key_cache),
                   static_cast<const uint16_t*>(value_cache), block_tables, seq_lens,
                   num_seqs, num_kv_heads, block_size, max_blocks_per_seq, max_seq_len};
  const dim3 blocks(static_cast<unsigned>(grid));
  if (head_dim == 256)
    hipLaunchKernelGGL(pa::pa_gather_kernel<256>, blocks, dim3(256), 0, stream, g);
  else if (head_dim == 128)
    hipLaunchKernelGGL(pa::pa_gather_kernel<128>, blocks, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(pa::pa_gather_kernel<64>, blocks, dim3(256), 0, stream, g);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
