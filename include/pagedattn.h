/*
 * libpagedattn — GQA-grouped, partitioned paged-attention decode for MI355X (gfx950).
 *
 * One call computes, for every sequence s and query head h,
 *
 *     out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K_t) V_t ,   t in [0, seq_lens[s])
 *
 * where token t is read from physical page block_tables[s][t / block_size] at
 * slot t % block_size, and query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Method (pages of commits 8d26e23 "docs", b80fd2b "paged_attn.py" and
 * 87a19d2 "paged_attention_v2_triton.py"):
 *   - grid on KV heads, not query heads: one workgroup serves the whole group of
 *     query heads that share a KV head, so each K/V page is read once
 *     (8d26e23, "Key design change");
 *   - phase 1 produces, per (sequence, KV head, partition), the compound partial
 *     (max_score, exp_sum, weighted_v[head_dim]) for every query head of the
 *     group (8d26e23, compound type and phase-1 kernel);
 *   - phase 2 merges the partials with the flash-attention rescale
 *     alpha = exp(m_i - m_new), beta = exp(m_ij - m_new) (8d26e23 phase-2 kernel;
 *     87a19d2 online-softmax fix);
 *   - a length-tiered dispatch runs short sequences in one pass and splits long
 *     ones into partitions (b80fd2b, three-tier decode dispatch; 8d26e23, the
 *     partition size should be tunable);
 *   - optionally, the merge runs inside phase 1 instead of a second kernel: the
 *     cross-partition combine that is level 3 of the three-level decomposition
 *     (8d26e23), the last workgroup of a sequence found by an atomic ticket.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers unless a parameter says "host".
 *   - The caller owns every buffer.  The library never allocates or frees device
 *     memory, never synchronises the device or the stream, and keeps no pointer
 *     after returning.  Apart from paged_attn_decode_noalloc's per-device scratch
 *     array and the cache of its address, it has no mutable global state:
 *     concurrent calls on different streams are safe when their `out` and
 *     `workspace` differ.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously.  All host-side validation happens before the
 *     first HIP call; a rejected call enqueues nothing.
 *   - Errors are returned as pa_status_t.  There is no fallback path: a shape
 *     the kernels do not support is rejected, never served another way.
 *   - Device faults (for example a page id outside the pool, which the library
 *     cannot see) surface at the caller's next synchronisation.
 *
 * Layouts (all contiguous, row-major):
 *   q, out        [num_seqs][num_heads][head_dim]                       dtype
 *   key_cache     [num_blocks][num_kv_heads][block_size][head_dim]      dtype
 *   value_cache   [num_blocks][num_kv_heads][block_size][head_dim]      dtype
 *   block_tables  [num_seqs][max_blocks_per_seq]                        int32
 *   seq_lens      [num_seqs]                                            int32
 *   One (page, KV head) is one contiguous block_size*head_dim chunk.
 *   Entries of a block-table row at or past ceil(seq_lens[s]/block_size) are
 *   never read; slots at or past seq_lens[s] in the last page are never used
 *   (they may hold NaN).
 *
 * Supported shapes: head_dim 64, 128 or 256; num_heads / num_kv_heads (the
 * group) 1..16; block_size 8 or a multiple of 16; partition_size 0 (automatic)
 * or a positive multiple of 16; dtype f16 or bf16 (q, caches and out share it).
 * Pointers q, key_cache and value_cache must be 16-byte aligned, out 8-byte
 * aligned and workspace 256-byte aligned (every torch allocation is).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes at the start of every non-empty workspace reserved for the ticket
 * counters of the fused combine (pa_options.fused_combine). */
#define PA_WORKSPACE_TICKET_BYTES 65536

/* Size of the device-resident workspace of paged_attn_decode_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum pa_dtype_t {
    PA_F16 = 0,
    PA_BF16 = 1
} pa_dtype_t;

typedef enum pa_status_t {
    PA_OK = 0,
    PA_ERR_NULL = 1,         /* a required pointer is NULL                       */
    PA_ERR_SHAPE = 2,        /* inconsistent sizes (heads, lengths, table)       */
    PA_ERR_UNSUPPORTED = 3,  /* valid but not built: head_dim, group, dtype, bs  */
    PA_ERR_PARTITION = 4,    /* partition_size not 0 and not a multiple of 16    */
    PA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required          */
    PA_ERR_HIP = 6,          /* a kernel launch failed                           */
    PA_ERR_ALIGN = 7         /* a pointer is not aligned as required             */
} pa_status_t;

/* Tuning and instrumentation knobs for paged_attn_decode_ex.  Zero-initialise
 * and set what you need; a NULL options pointer means all defaults. */
typedef struct pa_options {
    /* Sequences with seq_len <= single_pass_max_len run in one pass (one
     * workgroup per (sequence, KV head), output written directly); longer ones
     * are partitioned.  < 0: automatic (= the partition size: a sequence that fits
     * in one partition is one pass); 0: partition every sequence (phase 2 always
     * runs). */
    int single_pass_max_len;
    /* Compute units assumed by the automatic choices; <= 0 means 256 (MI355X). */
    int num_cus;
    /* Sum of seq_lens if the caller knows it on the host (0 = unknown).  Only
     * used when partition_size is 0: a total of num_seqs * max_seq_len (every
     * sequence at the bound) selects fixed partitions of one workgroup per CU
     * instead of the device-side balanced split, when num_seqs * num_kv_heads
     * does not exceed the workgroup slots (256 CUs x w, w as below); with a
     * forced tier it sizes the automatic partitions. */
    long long total_tokens_hint;
    /* Ablation only: 1 launches one workgroup per query head instead of one per
     * KV head (the GQA-unaware grid; each KV page is read once per query head).
     * Uses fixed partitions (partition_size, or 0 for one workgroup per CU). */
    int per_query_head;
    /* 1: merge the partials of each partitioned sequence inside phase 1 (the
     * workgroup that finishes a sequence's last partial merges them, found by a
     * device-scope atomic ticket) instead of launching phase 2.  The ticket
     * counters occupy the first PA_WORKSPACE_TICKET_BYTES of the workspace: they
     * must be zero before the first fused call on a workspace
     * (paged_attn_workspace_init), and every fused call that completes leaves
     * them zero.  Calls sharing a workspace must not overlap.  Ignored (phase 2
     * runs) when num_seqs * num_kv_heads (num_heads with per_query_head)
     * exceeds PA_WORKSPACE_TICKET_BYTES / 4. */
    int fused_combine;
    /* Automatic splits only (partition_size 0): the hardware hands out
     * workgroup i to XCD i mod 8, and the workgroups of the odd XCDs of MI355X
     * stream K/V ~8-10% slower than those of the even ones, so shares are paired
     * across XCD parities and the even member takes this many permille of the
     * pair's mean more (the odd one as many less).  0 = default (80); negative =
     * equal shares; at most 500; off when num_cus is below 64 (one XCD).  Share
     * boundaries stay fixed for given sizes, so results do not depend on timing. */
    int xcd_skew;
    /* Length-balanced split only: the tiles of streaming that starting a piece
     * (a sequence's part inside a share) is counted as when the step is cut into
     * shares, so shares that start more pieces get fewer tiles.  0 = default
     * (8 x 256 / head_dim, halved where two workgroups share a CU); negative =
     * none (equal tiles per share). */
    int piece_cost;
    /* If non-NULL, hipEventRecord(phase1_begin/phase1_end, stream) is issued
     * immediately before/after the phase-1 kernel (instrumentation only). */
    hipEvent_t phase1_begin;
    hipEvent_t phase1_end;
    /* Phase-1 walk for explicit partition sizes and the length-balanced split.
     * 0 (default): per-wave streams where supported (up to 1024 sequences, not with
     * the fused combine or the per-query-head ablation): every wave of a workgroup
     * streams its own contiguous run of tiles across pieces, finishing a piece
     * that lies inside it from registers, and only pieces cut between waves are
     * merged, once, at the end;
     * with an explicit partition size, shares end on partition boundaries so each
     * partition still yields one partial.  Negative:
     * one workgroup per piece with a merge of its waves after every piece (the
     * pages' dense (sequence, KV head, partition) grid for explicit partition
     * sizes). */
    int stream_walk;
    /* Ablation only: 1 processes the group's query heads one after another inside
     * each workgroup (page of commit 8d26e23, phase-1 kernel): every staged K/V tile
     * is taken once per query head, re-read from LDS, with the MFMA operands of the
     * other heads zeroed.  Bitwise equal to the grouped pass with the same partitions;
     * uses fixed partitions (partition_size, or 0 as with equal lengths declared). */
    int head_sequential;
} pa_options;

/* What a call will launch; filled by paged_attn_plan. */
typedef struct pa_plan_info {
    int partition_size;        /* resolved partition size, tokens           */
    int single_pass_max_len;   /* resolved tier threshold, tokens           */
    int max_partitions;        /* partitions per (sequence, KV head) slot   */
    int group;                 /* query heads per KV head                   */
    long long phase1_workgroups;   /* grid of the phase-1 kernel            */
    long long phase2_workgroups;   /* grid of the phase-2 kernel (0 = none) */
    long long active_workgroups;   /* phase-1 workgroups that do work (needs host lengths) */
    int single_pass_seqs;      /* sequences served in one pass (needs host lengths) */
    int partitioned_seqs;      /* sequences split into partitions (needs host lengths) */
    size_t workspace_bytes;    /* bytes of workspace the call needs         */
    int threads_per_workgroup; /* phase-1 block size                        */
    int lds_bytes_phase1;      /* LDS of the phase-1 tile slots             */
    int balanced;              /* 1: length-balanced split (partition_size 0) */
    int fused;                 /* 1: partials merged in phase 1, no phase-2 launch */
    int xcd_skew;              /* XCD-paired shares in use (permille), 0 = equal */
    int piece_cost;            /* balanced split: tiles a piece start counts as */
    int stream;                /* 1: phase 1 walks per-wave streams (pa_options.stream_walk) */
    int head_sequential;       /* 1: the head-sequential ablation (pa_options.head_sequential) */
    int reduce_slices;         /* 16-wide head_dim slices per phase-2 workgroup (0 = no phase 2) */
} pa_plan_info;

/*
 * Bytes of device workspace paged_attn_decode needs for these sizes (0 when every
 * sequence can run in a single pass).  The pages keep the decode's buffers
 * preallocated and reuse them across calls so the hot call allocates nothing
 * (page of commit b80fd2b, paged_attn.py, the caching-allocator passage); here the
 * caller owns that buffer, sized by this call.  What it holds is the phase-1
 * compound partial of the page of commit 8d26e23 (attention_partial: max_score,
 * exp_sum, weighted_v).  Besides the sizes of the spec call it takes
 * num_kv_heads (the grid is on KV heads, so the partial count depends on it),
 * block_size and max_blocks_per_seq (the table capacity bounds the length when
 * max_seq_len <= 0, and the automatic split depends on the page size).  max_seq_len <= 0 means "unknown", and the
 * table capacity max_blocks_per_seq*block_size is used.  Returns (size_t)-1 for
 * arguments paged_attn_decode would reject.
 *
 * The workspace starts with PA_WORKSPACE_TICKET_BYTES of ticket counters (used
 * only by the fused combine, never touched otherwise), then holds, for each
 * (sequence, query head, partition), the phase-1 partial: weighted_v as head_dim
 * fp32 values, then (max_score, exp_sum) as two fp32 values, with max_score in
 * base-2 units (log2(e)*scale*q.k).
 */
size_t paged_attn_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int max_seq_len,
                                 int partition_size);

size_t paged_attn_workspace_size_ex(int num_seqs, int num_heads, int num_kv_heads,
                                    int head_dim, int block_size, int max_blocks_per_seq,
                                    int max_seq_len, int partition_size,
                                    const pa_options* opt);

/*
 * Decode attention for one step of a batch (the whole hot path: phase 1 with the
 * length-tiered dispatch, then phase 2 for partitioned sequences).  Page of commit
 * 8d26e23: the grid on KV heads ("Key design change"), the phase-1 kernel writing
 * one attention_partial per (sequence, KV head, partition) for the group's query
 * heads, the phase-2 kernel merging them with the flash-attention rescale; page of
 * commit 87a19d2: that rescale (the online-softmax fix); page of commit b80fd2b:
 * the length-tiered dispatch (three-tier decode dispatch).
 *
 *   out                 [num_seqs][num_heads][head_dim] dtype, written (device)
 *   q                   [num_seqs][num_heads][head_dim] dtype (device)
 *   key_cache/value_cache  paged caches, layout above (device)
 *   block_tables        [num_seqs][max_blocks_per_seq] int32 (device)
 *   seq_lens            [num_seqs] int32 (device); seq_len <= 0 gives a zero row.
 *                       Values above max_seq_len are treated as max_seq_len.
 *   num_seqs            >= 0 (0 is a no-op)
 *   num_heads, num_kv_heads   query and KV heads; num_heads % num_kv_heads == 0
 *   head_dim, block_size      see "Supported shapes"
 *   scale               multiplies q.k in fp32 (typically 1/sqrt(head_dim))
 *   partition_size      tokens per phase-1 partition of a long sequence (a positive
 *                       multiple of 16: the pages' fixed-partition grid), or 0:
 *                       automatic.  Automatic is the length-balanced split (the
 *                       step's tiles cut on the device into shares of about equal
 *                       cost, see pa_options.piece_cost and xcd_skew; one
 *                       workgroup per share and KV head, w per CU as below) for up
 *                       to 1024 sequences; with equal lengths declared through
 *                       pa_options.total_tokens_hint (and no more segments than
 *                       workgroup slots), more sequences, or a forced
 *                       tier, it is fixed partitions of ceil(num_seqs *
 *                       max_seq_len * num_kv_heads / (256 * w)) tokens rounded up
 *                       to 16, at least 64 and at most max_seq_len, where w (the
 *                       resident workgroups per CU aimed at) is 1 for head_dim 256
 *                       with block_size >= 16 and 2 otherwise
 *   workspace           device scratch of workspace_bytes bytes (may be NULL when
 *                       paged_attn_workspace_size(...) == 0); not read before written
 *   stream              hipStream_t to enqueue on
 *   max_blocks_per_seq  row stride of block_tables (entries)
 *   max_seq_len         host-known upper bound of seq_lens; <= 0 means
 *                       max_blocks_per_seq*block_size.  Sizes the grid.
 *   dtype               pa_dtype_t of q, the caches and out
 *   workspace_bytes     size of workspace, checked against the requirement
 * Returns PA_OK or the first error found.
 */
int paged_attn_decode(void* out, const void* q, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      float scale, int partition_size, void* workspace, hipStream_t stream,
                      int max_blocks_per_seq, int max_seq_len, int dtype,
                      size_t workspace_bytes);

/* paged_attn_decode with tuning/instrumentation options (opt may be NULL): the
 * tier threshold and partition choices the page of commit 8d26e23 says should be
 * tunable, the in-kernel combine (its level 3), and the ablation of its grid. */
int paged_attn_decode_ex(void* out, const void* q, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, int num_seqs, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, float scale,
                         int partition_size, void* workspace, hipStream_t stream,
                         int max_blocks_per_seq, int max_seq_len, int dtype,
                         size_t workspace_bytes, const pa_options* opt);

/*
 * Prefill over a paged context (the prefix path of the page of commit b80fd2b,
 * paged_attn.py: one online softmax over the cached context gathered by block
 * id, then over the current chunk under the causal mask).  For sequence s, the
 * new tokens n = 0 .. Q-1, Q = query_start[s+1] - query_start[s], sit at rows
 * r = query_start[s] + n of q, k_new and v_new; query head h of new token n
 * attends to the ctx_lens[s] tokens in the paged caches (KV head
 * h / (num_heads / num_kv_heads), as in decode) and to the new tokens j <= n:
 *
 *     out[r,h,:] = sum_u softmax_u(scale * q[r,h,:] . K_u) V_u
 *
 *   out                 [T][num_heads][head_dim] dtype, written (device); T = query_start[num_seqs]
 *   q                   [T][num_heads][head_dim] dtype (device)
 *   k_new, v_new        [T][num_kv_heads][head_dim] dtype (device): the chunk's own keys
 *                       and values (not read from the caches)
 *   key_cache/value_cache, block_tables   the paged context, layouts as for decode
 *   ctx_lens            [num_seqs] int32 (device): cached tokens per sequence (<= 0: none;
 *                       values above max_ctx_len are treated as max_ctx_len)
 *   query_start         [num_seqs + 1] int32 (device), non-decreasing, query_start[0] = 0
 *   max_query_len       host-known bound of the chunk lengths (sizes the grid; longer
 *                       chunks are cut to it); 0 (no new tokens) is a no-op, and the
 *                       row pointers q, k_new, v_new and out may then be NULL
 *   max_ctx_len         host-known bound of ctx_lens, <= max_blocks_per_seq*block_size
 *   scale               any finite value (a negative one is applied by negating q, which
 *                       is exact; zero gives every kept key the same weight)
 * Shapes, dtypes and alignment as for decode (k_new and v_new 16-byte aligned).
 * No workspace.  Returns PA_OK or the first error found.
 */
int paged_attn_prefill(void* out, const void* q, const void* k_new, const void* v_new,
                       const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* ctx_lens,
                       const int32_t* query_start, int num_seqs, int num_heads,
                       int num_kv_heads, int head_dim, int block_size, float scale,
                       int max_blocks_per_seq, int max_query_len, int max_ctx_len, int dtype,
                       hipStream_t stream);

/*
 * paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, plan, kernels and results as
 * paged_attn_decode with the same sizes (and no options); the workspace is a
 * file-scope device array of PA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held
 * until the process ends, whose address is looked up (hipGetSymbolAddress) on the
 * first call made with a device current.  The call allocates nothing and calls no
 * allocating routine.  Work runs on the current device: `stream` must belong to it.
 * A plan needing more than PA_NOALLOC_SCRATCH_BYTES of workspace (the bound covers
 * every plan of partition_size 0 with up to 1024 sequences; explicit partition
 * sizes need num_seqs * num_kv_heads * ceil(max_seq_len / partition_size) *
 * (num_heads / num_kv_heads) * (4 * head_dim + 8) bytes plus 64 KiB) returns
 * PA_ERR_WORKSPACE before any work is enqueued.  Every region a call reads is
 * written by that call first, so nothing needs clearing between calls; calls that
 * overlap on one GPU (other streams, other host threads) share the array and race:
 * the caller serialises them.  Returns PA_OK or the first error found.
 */
int paged_attn_decode_noalloc(void* out, const void* q, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* seq_lens, int num_seqs, int num_heads,
                              int num_kv_heads, int head_dim, int block_size, float scale,
                              int partition_size, hipStream_t stream, int max_blocks_per_seq,
                              int max_seq_len, int dtype);

/*
 * Workspace set-up for the in-kernel cross-partition combine (the level-3 combine
 * of the three-level decomposition, page of commit 8d26e23).
 * Clears the ticket area (the first min(workspace_bytes,
 * PA_WORKSPACE_TICKET_BYTES) bytes) of a workspace with a kernel on `stream`, as
 * the fused combine (pa_options.fused_combine) needs before the first call on a
 * new workspace, or after a call that failed.  workspace: device pointer,
 * 256-byte aligned (NULL only with workspace_bytes 0).  Returns PA_OK,
 * PA_ERR_NULL, PA_ERR_ALIGN or PA_ERR_HIP.
 */
int paged_attn_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Human-readable text for a pa_status_t (static storage, never NULL).  Errors are
 * returned, never served by a fallback path (the try/except fallbacks of the page
 * of commit b80fd2b are what this interface does not do). */
const char* paged_attn_status_str(int status);

/*
 * Host-only planning (no HIP call, usable without a GPU), the length-tiered
 * dispatch of the page of commit b80fd2b (three-tier decode dispatch) and the grid
 * of the page of commit 8d26e23 ((sequence, KV head, partition)): fills *info with the
 * grid, tier threshold, partition size and workspace a decode call with the same
 * arguments would use.  seq_lens_host (host pointer, may be NULL) adds the
 * per-sequence tier counts and the number of phase-1 workgroups that do work.
 * Returns the status paged_attn_decode would return from validation
 * (pointer arguments excepted).
 */
int paged_attn_plan(const int32_t* seq_lens_host, int num_seqs, int num_heads,
                    int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                    int max_seq_len, int partition_size, int dtype, const pa_options* opt,
                    pa_plan_info* info);

/*
 * Test hook for the block-table gather (the addressing and 16-byte page loads of
 * phase 1, without the attention math), the gather of K/V by block id of the page
 * of commit b80fd2b (paged_attn.py, rewrite item 1): writes the K and V rows of tokens
 * t < seq_lens[s] to k_out/v_out, laid out [num_seqs][num_kv_heads][max_seq_len]
 * [head_dim] (16-bit elements copied bit for bit; other slots are not written).
 * max_seq_len must be > 0 and <= max_blocks_per_seq*block_size.
 */
int paged_attn_gather_probe(void* k_out, void* v_out, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, int num_seqs, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq,
                            int max_seq_len, hipStream_t stream);

/*
 * Measurement hook: the read bandwidth the decode is bounded by.  The pages' case
 * for the KV-head grid is the K/V bytes read (page of commit 8d26e23, "Key design
 * change": 6x fewer), so the decode's roofline is HBM read bandwidth; this call
 * measures what the device delivers to the same access pattern (the phase-1 load
 * form: nontemporal 16-byte loads, 1 KiB contiguous per instruction, two chunks in
 * flight per wave).  It reads num_chunks chunks of chunk_bytes bytes (4096, 8192
 * or 16384: one (page, KV head) block of the caches) from src, chunk i at
 * src + order[i] * chunk_bytes, or at src + i * chunk_bytes when order is NULL,
 * spread over num_workgroups workgroups of 256 threads, and writes one XOR fold
 * per workgroup to sink[num_workgroups] (so no load is dead).
 *   src    device, 16-byte aligned, at least (max index + 1) * chunk_bytes bytes
 *   order  device int64 [num_chunks] or NULL; every entry must index a chunk of src
 *          (not checked: an entry outside src faults the device)
 * Returns PA_OK, PA_ERR_UNSUPPORTED (chunk size), PA_ERR_SHAPE, PA_ERR_NULL,
 * PA_ERR_ALIGN or PA_ERR_HIP.
 */
int paged_attn_read_probe(const void* src, size_t chunk_bytes, const long long* order,
                          long long num_chunks, int num_workgroups, unsigned* sink,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
