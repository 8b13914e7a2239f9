"""C-ABI boundary and host planner tests (CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import gqa_aware_paged_amd as pa
from gqa_aware_paged_amd import build as pa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_design_sizes.txt")


@pytest.fixture(scope="module")
def lib():
    if pa_build.is_stale():
        pa_build.build()
    return pa.lib()


def golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    return vals


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pa.SYMBOLS)


def test_status_strings(lib):
    for code in range(8):
        s = lib.paged_attn_status_str(code).decode()
        assert s.startswith("PA_")
    assert "unknown" in lib.paged_attn_status_str(99).decode()


FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: every call below fails validation


def call(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=24, Hkv=4, D=256, bs=16,
             scale=0.0625, P=512, ws=None, stream=None, mbps=64, maxlen=0, dtype=0, wsb=0)
    a.update(kw)
    return lib.paged_attn_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["sl"], a["S"],
                                 a["Hq"], a["Hkv"], a["D"], a["bs"], a["scale"], a["P"], a["ws"],
                                 a["stream"], a["mbps"], a["maxlen"], a["dtype"], a["wsb"])


def test_validation_errors_before_any_launch(lib):
    # S=2, Hkv=4 -> small batch -> every sequence longer than one partition is split,
    # so a workspace is required and the calls below stop at validation.
    assert call(lib, q=None) == 1                    # PA_ERR_NULL
    assert call(lib, Hkv=5) == 2                     # 24 % 5 -> PA_ERR_SHAPE
    assert call(lib, D=96) == 3                      # PA_ERR_UNSUPPORTED
    assert call(lib, Hq=68, Hkv=4) == 3              # group 17 > 16
    assert call(lib, bs=24) == 3                     # block size neither 8 nor a multiple of 16
    assert call(lib, bs=8, mbps=128) == 5            # 8 is supported (then: workspace missing)
    assert call(lib, D=64) == 5                      # head_dim 64 is supported
    assert call(lib, dtype=2) == 3
    assert call(lib, P=24) == 4                      # PA_ERR_PARTITION
    assert call(lib, P=-16) == 4
    assert call(lib, maxlen=64 * 16 + 1) == 2        # longer than the table row
    assert call(lib, scale=float("nan")) == 2
    assert call(lib) == 5                            # workspace missing -> PA_ERR_WORKSPACE
    need = lib.paged_attn_workspace_size(2, 24, 4, 256, 16, 64, 0, 512)
    assert call(lib, ws=FAKE, wsb=need - 1) == 5
    assert call(lib, ws=ctypes.c_void_p(0x10010), wsb=need) == 7    # workspace not 256-B aligned
    assert call(lib, q=ctypes.c_void_p(0x10008)) == 7               # q not 16-B aligned
    assert call(lib, S=0) == 0                                      # empty batch: no-op


def test_workspace_size_formula(lib):
    S, Hq, Hkv, D, bs, mbps, P = 4, 24, 4, 256, 16, 6400, 512
    n = lib.paged_attn_workspace_size(S, Hq, Hkv, D, bs, mbps, 102400, P)
    parts = 102400 // P
    acc = S * Hq * parts * D * 4
    tickets = 65536                      # PA_WORKSPACE_TICKET_BYTES, first in every workspace
    assert n == tickets + ((acc + 255) // 256) * 256 + S * Hq * parts * 8
    # explicit partitions: every sequence fits one partition -> one pass, no workspace
    assert lib.paged_attn_workspace_size(256, 24, 4, 256, 32, 512, 16384, 16384) == 0
    # balanced split (partition_size 0): two records per phase-1 workgroup + a job each
    nw = 256
    recs = 2 * nw * 6
    acc = tickets + ((recs * 256 * 4 + 255) // 256) * 256
    ml = ((acc + recs * 8 + 255) // 256) * 256
    assert lib.paged_attn_workspace_size(256, 24, 4, 256, 32, 512, 16384, 0) == ml + nw * 8
    assert lib.paged_attn_workspace_size(2, 24, 5, 256, 16, 64, 0, 512) == ctypes.c_size_t(-1).value


def test_plan_matches_pages_grid(lib):
    """One 100K-token sequence with 512-token partitions: 200 partitions and a grid
    of 4 KV heads x 200 = 800 workgroups instead of 24 x 200 = 4800 (the dense grid,
    stream_walk -1).  The default walks the same 800 partitions, one partial each,
    with per-wave streams on one workgroup per CU."""
    g = golden()
    L, P = g["long_seq_tokens"], g["partition_size"]
    args = ([L], g["num_q_heads"], g["num_kv_heads"], g["tile_head_dim"], 16, L // 16, L, P)
    info = pa.plan(*args, single_pass_max_len=0, stream_walk=-1)
    assert info["stream"] == 0
    assert info["max_partitions"] == g["num_partitions"]
    assert info["phase1_workgroups"] == g["blocks_per_kv_head_grid"]
    assert info["phase1_workgroups"] * info["group"] == g["blocks_per_q_head_grid"]
    assert info["group"] == g["gqa_ratio"] == g["kv_reads_saved_factor"]
    assert info["active_workgroups"] == 800
    assert info["partitioned_seqs"] == 1
    # per-wave streams: the same partitions and partial records, 64 shares x 4 KV heads
    st = pa.plan(*args, single_pass_max_len=0)
    assert st["stream"] == 1 and st["max_partitions"] == g["num_partitions"]
    assert st["phase1_workgroups"] == 256 and st["active_workgroups"] == 256
    assert st["workspace_bytes"] == info["workspace_bytes"]
    assert st["phase2_workgroups"] == info["phase2_workgroups"] == 4 * 16
    # the head-sequential ablation keeps the grouped grid (heads taken in turn inside it)
    hs = pa.plan(*args, single_pass_max_len=0, head_sequential=True)
    assert hs["head_sequential"] == 1 and hs["stream"] == 0
    assert hs["phase1_workgroups"] == g["blocks_per_kv_head_grid"]
    # the per-query-head ablation restores the pages' "before" grid
    info_q = pa.plan(*args, single_pass_max_len=0, per_query_head=True)
    assert info_q["phase1_workgroups"] == g["blocks_per_q_head_grid"] and info_q["stream"] == 0
    assert info_q["group"] == 1 and info_q["workspace_bytes"] == info["workspace_bytes"]
    # the same arithmetic for the 4-sequence long-context workload
    info4 = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, P, stream_walk=-1)
    assert info4["phase1_workgroups"] == 3200 and info4["phase2_workgroups"] == 4 * 4 * 16
    st4 = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, P)
    assert st4["phase1_workgroups"] == 256 and st4["phase2_workgroups"] == 4 * 4 * 16
    assert st4["xcd_skew"] == 80                # shares (whole partitions) paired by XCD
    # a partition per share at most: 3 sequences of 2 partitions -> 6 shares per KV head
    few = pa.plan([1024] * 3, 24, 4, 256, 16, 64, 1024, 512, single_pass_max_len=0)
    assert few["phase1_workgroups"] == 4 * 6 and few["active_workgroups"] == 4 * 6


def test_tier_thresholds(lib):
    g = golden()
    # explicit one-pass bound of 8192 tokens (the pages' short tier)
    lens = [g["single_pass_max_len"]] * 256 + [g["single_pass_max_len"] + 1] * 8
    info = pa.plan(lens, 24, 4, 256, 16, 1024, 0, 512,
                   single_pass_max_len=g["single_pass_max_len"])
    assert info["single_pass_max_len"] == g["single_pass_max_len"]
    assert info["single_pass_seqs"] == 256 and info["partitioned_seqs"] == 8
    # automatic tier: a sequence that fits in one partition runs in one pass
    info = pa.plan([512, 513, 8192], 24, 4, 256, 16, 512, 0, 512, stream_walk=-1)
    assert info["single_pass_max_len"] == 512
    assert info["single_pass_seqs"] == 1 and info["partitioned_seqs"] == 2
    assert info["active_workgroups"] == 4 * (1 + 2 + 16)
    st = pa.plan([512, 513, 8192], 24, 4, 256, 16, 512, 0, 512)
    assert st["stream"] == 1 and st["single_pass_seqs"] == 1 and st["partitioned_seqs"] == 2
    assert st["active_workgroups"] == 4 * (1 + 2 + 16)     # 19 pieces, 64 shares
    # explicit partition sizes
    for P in (256, 512, 1024):
        info = pa.plan([65536], 24, 4, 256, 16, 4096, 65536, P, single_pass_max_len=8192)
        assert info["max_partitions"] == 65536 // P
    info = pa.plan([100, 0, 7], 24, 4, 256, 16, 8, 100, 0, single_pass_max_len=100)
    assert info["single_pass_seqs"] == 3 and info["phase2_workgroups"] == 0


def test_balanced_split_plan(lib):
    """partition_size = 0: the step's tiles are cut into equal shares, one
    workgroup per CU at head_dim 256 with 16-token pages (two otherwise), whatever
    the length mix."""
    L = 102400
    info = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0)          # 4 x 100K tokens
    assert info["balanced"] == 1 and info["phase1_workgroups"] == 256
    assert info["active_workgroups"] == 256 and info["partitioned_seqs"] == 4
    assert info["phase2_workgroups"] == 256 * 2
    assert pa.plan([L] * 4, 24, 4, 128, 16, L // 16, L, 0)["phase1_workgroups"] == 512
    assert pa.plan([L] * 4, 24, 4, 256, 8, L // 8, L, 0, stream_walk=-1)["phase1_workgroups"] == 512
    # per-wave streams at head_dim 256 take 126 KiB of LDS: one workgroup per CU
    assert pa.plan([L] * 4, 24, 4, 256, 8, L // 8, L, 0)["phase1_workgroups"] == 256
    # 1024 segments of 1024 tiles over 256 workgroups: equal shares end on segment ends
    info = pa.plan([16384] * 256, 24, 4, 256, 32, 512, 16384, 0, xcd_skew=-1)
    assert info["phase1_workgroups"] == 256 and info["xcd_skew"] == 0
    assert info["single_pass_seqs"] == 256 and info["partitioned_seqs"] == 0
    # XCD-paired shares (4.32 and 3.68 sequences per pair of 8): one cut per pair
    info = pa.plan([16384] * 256, 24, 4, 256, 32, 512, 16384, 0)
    assert info["phase1_workgroups"] == 256 and info["xcd_skew"] == 80
    assert info["single_pass_seqs"] == 224 and info["partitioned_seqs"] == 32
    # short: one workgroup per 4 tiles (one per wave) of the length bound
    info = pa.plan([100] * 8, 24, 4, 256, 16, 8, 100, 0)
    assert info["phase1_workgroups"] == 4 * ((8 * 7 + 3) // 4)   # shares x KV heads
    # a mix of very short and very long sequences: the long ones are cut into many
    # shares; a short one is cut only where a share boundary happens to fall in it
    lens = [64] * 60 + [65536] * 4
    info = pa.plan(lens, 24, 4, 256, 16, 4096, 65536, 0)
    assert info["partitioned_seqs"] >= 4 and info["single_pass_seqs"] >= 50
    assert info["partitioned_seqs"] + info["single_pass_seqs"] == 64
    # zero-length sequences count as one pass
    info = pa.plan([0, 0, 5000], 24, 4, 256, 16, 400, 5000, 0)
    assert info["single_pass_seqs"] == 2 and info["partitioned_seqs"] == 1


def test_automatic_partition_size_for_256_cus(lib):
    """partition_size = 0 with equal lengths declared, a forced tier, or more
    sequences than the balanced split handles: fixed partitions for one workgroup
    per compute unit."""
    L = 102400
    info = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L)
    assert info["balanced"] == 0 and info["partition_size"] == 6400
    info = pa.plan([L] * 3 + [L - 1], 24, 4, 256, 16, L // 16, L, 0,
                   total_tokens_hint=4 * L - 1)
    assert info["balanced"] == 1
    info = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, single_pass_max_len=0)
    assert info["balanced"] == 0
    assert info["partition_size"] == 6400 and info["phase1_workgroups"] == 256
    info = pa.plan([L], 24, 4, 256, 16, L // 16, L, 0, single_pass_max_len=0)
    assert info["partition_size"] == 1600 and info["phase1_workgroups"] == 256
    info = pa.plan([16384] * 1100, 24, 4, 256, 32, 512, 16384, 0)   # too many for the split
    assert info["balanced"] == 0 and info["partition_size"] == 16384
    assert info["partitioned_seqs"] == 0 and info["workspace_bytes"] == 0
    # a tile prefix beyond 32 bits (1024 x 2^27 tokens): fixed partitions
    huge = pa.plan(None, 24, 4, 256, 16, 1 << 23, 1 << 27, 0, num_seqs=1024)
    assert huge["balanced"] == 0
    # equal lengths but more segments (256 x 4) than workgroup slots: balanced split
    info = pa.plan([16384] * 256, 24, 4, 256, 32, 512, 16384, 0, total_tokens_hint=256 * 16384)
    assert info["balanced"] == 1
    # a host-side total shrinks the partitions of an unequal batch
    lens = [64] * 1100 + [65536] * 4
    a = pa.plan(lens, 24, 4, 256, 16, 4096, 65536, 0)
    b = pa.plan(lens, 24, 4, 256, 16, 4096, 65536, 0, total_tokens_hint=sum(lens))
    per_cu = -(-sum(lens) * 4 // 256)
    assert a["partition_size"] == 65536
    assert b["partition_size"] == -(-per_cu // 16) * 16 and b["partitioned_seqs"] == 4
    # head_dim 128 / 64 and 8-token pages aim at two resident workgroups per CU
    for D, bs in ((128, 16), (64, 16), (256, 8)):
        info = pa.plan([L] * 4, 24, 4, D, bs, L // bs, L, 0, total_tokens_hint=4 * L)
        assert info["partition_size"] == 3200 and info["phase1_workgroups"] == 512


def test_tile_budget_against_pages(lib):
    """The pages size K and V tiles of 32 x 256 fp16 at 16 KB each, 32 KB of the
    48 KB SMEM budget.  Here each wave stages 16-token K and V tiles (8 KB each);
    four waves fill 64 KB of gfx950's 160 KB LDS, so two workgroups fit per CU."""
    g = golden()
    assert g["k_tile_tokens"] * g["tile_head_dim"] * 2 == g["k_tile_bytes_f16"]
    assert 2 * g["k_tile_bytes_f16"] == g["kv_tile_bytes_f16"] <= g["smem_budget_bytes"]
    assert g["gqa_ratio"] * g["tile_head_dim"] == g["group_live_registers"]
    info = pa.plan([1024], 24, 4, 256, 16, 64)
    assert info["lds_bytes_phase1"] == 4 * 2 * 16 * 256 * 2 == 65536
    assert 2 * (info["lds_bytes_phase1"] + 16 * 256 * 2) <= 160 * 1024
    assert info["threads_per_workgroup"] == 256


def test_plan_rejects_what_decode_rejects(lib):
    with pytest.raises(pa.PagedAttnError, match="PARTITION"):
        pa.plan([10], 24, 4, 256, 16, 4, 0, 40)
    with pytest.raises(pa.PagedAttnError, match="UNSUPPORTED"):
        pa.plan([10], 24, 4, 96, 16, 4, 0, 512)


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and fails loudly without its library."""
    src = open(os.path.join(ROOT, "gqa_aware_paged_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "raise RuntimeError" in src


def test_fused_combine_plan(lib):
    """The fused combine drops the phase-2 launch and keeps the workspace layout;
    it is declined when the ticket area cannot hold one counter per segment."""
    L, P = 102400, 512
    base = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, P, stream_walk=-1)
    fused = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, P, fused_combine=True)
    assert base["fused"] == 0 and base["phase2_workgroups"] == 4 * 4 * 16
    # the fused combine runs on one workgroup per piece (no per-wave streams)
    assert fused["stream"] == 0 and pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, P)["stream"] == 1
    assert fused["fused"] == 1 and fused["phase2_workgroups"] == 0
    assert fused["phase1_workgroups"] == base["phase1_workgroups"]
    assert fused["workspace_bytes"] == base["workspace_bytes"]
    bal = pa.plan([64] * 60 + [65536] * 4, 24, 4, 256, 16, 4096, 65536, 0, fused_combine=True)
    assert bal["balanced"] == 1 and bal["fused"] == 1 and bal["phase2_workgroups"] == 0
    # all sequences in one pass: nothing to merge, no workspace, nothing fused
    short = pa.plan([100] * 8, 24, 4, 256, 16, 8, 128, 128, fused_combine=True)
    assert short["workspace_bytes"] == 0 and short["fused"] == 0
    # 16384 counters: 4096 sequences x 4 KV heads fit, 683 x 24 query heads do not
    ok = pa.plan(None, 24, 4, 256, 16, 64, 1024, 256, num_seqs=4096, fused_combine=True)
    no = pa.plan(None, 24, 4, 256, 16, 64, 1024, 256, num_seqs=683, fused_combine=True,
                 per_query_head=True)
    assert ok["fused"] == 1 and no["fused"] == 0 and no["phase2_workgroups"] > 0


def test_workspace_init_validation(lib):
    """Error paths only (a valid call launches a kernel)."""
    stream = ctypes.c_void_p(0)
    assert lib.paged_attn_workspace_init(None, 0, stream) == 0          # nothing to clear
    assert lib.paged_attn_workspace_init(None, 4096, stream) == 1       # PA_ERR_NULL
    assert lib.paged_attn_workspace_init(ctypes.c_void_p(0x10010), 4096, stream) == 7


def prefill_call(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, qs=FAKE, S=2,
             Hq=24, Hkv=4, D=256, bs=16, scale=0.0625, mbps=64, mq=128, mc=1024, dtype=0,
             stream=None)
    a.update(kw)
    return lib.paged_attn_prefill(a["out"], a["q"], a["kn"], a["vn"], a["k"], a["v"], a["bt"],
                                  a["cl"], a["qs"], a["S"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                  a["scale"], a["mbps"], a["mq"], a["mc"], a["dtype"],
                                  a["stream"])


def test_prefill_validation_errors_before_any_launch(lib):
    """Every call here is rejected before a HIP call (or is an empty no-op)."""
    assert prefill_call(lib, kn=None) == 1                  # PA_ERR_NULL
    assert prefill_call(lib, qs=None) == 1
    assert prefill_call(lib, Hkv=5) == 2                    # PA_ERR_SHAPE
    assert prefill_call(lib, mc=64 * 16 + 1) == 2           # context longer than the table
    assert prefill_call(lib, mq=-1) == 2
    assert prefill_call(lib, scale=float("inf")) == 2
    assert prefill_call(lib, D=96) == 3                     # PA_ERR_UNSUPPORTED
    assert prefill_call(lib, bs=24) == 3
    assert prefill_call(lib, dtype=5) == 3
    assert prefill_call(lib, kn=ctypes.c_void_p(0x10008)) == 7   # PA_ERR_ALIGN
    assert prefill_call(lib, out=ctypes.c_void_p(0x10004)) == 7
    assert prefill_call(lib, S=0) == 0                      # nothing to do
    assert prefill_call(lib, mq=0) == 0
    # a cache page of 64 KV heads x 131072 slots x 256 dims is 2^32 bytes: its stride
    # does not fit the kernel's 32-bit page offsets, so the shape is refused
    assert prefill_call(lib, Hq=64, Hkv=64, bs=131072, mbps=1, mc=1024) == 3
    assert prefill_call(lib, Hq=64, Hkv=32, bs=131072, mbps=1, mc=1024, S=0) == 0


def test_read_probe_validation(lib):
    """The read probe rejects what it cannot run before any launch."""
    sink = FAKE
    P, L = ctypes.c_void_p, ctypes.c_longlong
    assert lib.paged_attn_read_probe(FAKE, 1000, None, L(4), 256, sink, None) == 3
    assert lib.paged_attn_read_probe(FAKE, 8192, None, L(4), 0, sink, None) == 2
    assert lib.paged_attn_read_probe(FAKE, 8192, None, L(-1), 256, sink, None) == 2
    assert lib.paged_attn_read_probe(None, 8192, None, L(4), 256, sink, None) == 1
    assert lib.paged_attn_read_probe(FAKE, 8192, None, L(4), 256, None, None) == 1
    assert lib.paged_attn_read_probe(P(0x10008), 8192, None, L(4), 256, sink, None) == 7
    assert lib.paged_attn_read_probe(FAKE, 8192, P(0x10004), L(4), 256, sink, None) == 7
    assert lib.paged_attn_read_probe(None, 8192, None, L(0), 256, None, None) == 0


def test_xcd_paired_shares_plan(lib):
    """Automatic splits pair their shares across XCD parities (default 80 permille);
    so do the shares of whole partitions that per-wave streams walk with an explicit
    partition size, while the pages' dense grid and the per-query-head ablation keep
    equal work per workgroup."""
    L = 102400
    hinted = pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L)
    assert hinted["balanced"] == 0 and hinted["max_partitions"] == 16
    assert hinted["xcd_skew"] == 80
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L,
                   xcd_skew=30)["xcd_skew"] == 30
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L,
                   xcd_skew=-1)["xcd_skew"] == 0
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L,
                   xcd_skew=900)["xcd_skew"] == 500
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 512, stream_walk=-1)["xcd_skew"] == 0
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 512)["xcd_skew"] == 80
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, total_tokens_hint=4 * L,
                   per_query_head=True)["xcd_skew"] == 0
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0)["xcd_skew"] == 80
    # a single-XCD partition (32 CUs) has nothing to pair across
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, num_cus=32)["xcd_skew"] == 0
    assert pa.plan([L] * 4, 24, 4, 256, 16, L // 16, L, 0, num_cus=64)["xcd_skew"] == 80
    # an odd number of shares per KV head cannot pair up
    odd = pa.plan([40] * 3, 24, 4, 256, 16, 3, 40, 0)
    assert odd["balanced"] == 1 and odd["phase1_workgroups"] == 4 * 3 and odd["xcd_skew"] == 0
    # a single partition per sequence has nothing to pair
    assert pa.plan([5000] * 2, 24, 4, 256, 16, 313, 5000, 0, total_tokens_hint=10000,
                   single_pass_max_len=1 << 20)["xcd_skew"] == 0


def _split_counts(lens, ns, skew, cost):
    """Sequences served in one pass / split, for ns shares per KV head cut at
    floor(T' * (1000 j + skew * (j odd)) / (1000 ns)) over T' virtual tiles, each
    sequence with tokens counting `cost` lead-in tiles before its real ones."""
    tiles = [(L + 15) // 16 for L in lens]
    T = sum(n + cost for n in tiles if n > 0)

    def cut(j):
        return T if j >= ns else T * (1000 * j + skew * (j & 1)) // (1000 * ns)

    def share(t):
        return max(j for j in range(ns) if cut(j) <= t)

    single = split = 0
    start = 0
    for n in tiles:
        if n == 0:
            single += 1
            continue
        first, last = start + cost, start + cost + n - 1
        if share(first) != share(last):
            split += 1
        else:
            single += 1
        start += n + cost
    return single, split


@pytest.mark.parametrize("seed", range(6))
def test_balanced_cut_matches_formula(lib, seed):
    """The planner's host mirror of the device cut (start cost + XCD pairing) agrees
    with the formula written out independently, for random length mixes."""
    import random
    rng = random.Random(seed)
    S = rng.choice([3, 17, 40, 100])
    lens = [rng.choice([0, rng.randint(1, 300), rng.randint(1, 20000)]) for _ in range(S)]
    max_len = max(max(lens), 16)
    mbps = (max_len + 15) // 16
    for skew, cost in ((-1, -1), (80, 8), (300, 3), (0, 40)):
        info = pa.plan(lens, 24, 4, 256, 16, mbps, max_len, 0, xcd_skew=skew, piece_cost=cost)
        assert info["balanced"] == 1
        ns = info["phase1_workgroups"] // 4
        sk, pc = info["xcd_skew"], info["piece_cost"]
        assert pc == (8 if cost == 0 else max(cost, 0))
        assert sk == (0 if ns % 2 else (80 if skew == 0 else max(skew, 0)))
        single, split = _split_counts(lens, ns, sk, pc)
        assert (info["single_pass_seqs"], info["partitioned_seqs"]) == (single, split), \
            (skew, cost, ns)


def test_phase2_width_follows_rounds_and_grid(lib):
    """Fixed partitions: the phase-2 workgroup width (16-wide slices) is the one with
    the least (rounds of the longest segment) x 1 us + workgroups x 6 ns: one slice
    for a few long segments, wider for many segments.  These are the widths measured
    fastest on MI355X for each case."""
    import workloads
    mixed, batch = list(workloads.mixed_lens()), list(workloads.batch_lens())

    def width(lens, P):
        mb = (max(lens) + 15) // 16
        info = pa.plan(lens, 24, 4, 256, 16, mb, max(lens), P)
        assert info["phase2_workgroups"] == len(lens) * 4 * (16 // info["reduce_slices"])
        return info["reduce_slices"]

    assert width([102400] * 4, 256) == 1 and width([102400] * 4, 512) == 1
    assert width(mixed, 256) == 4 and width(mixed, 512) == 4 and width(mixed, 1024) == 8
    assert width(batch, 256) == 8 and width(batch, 512) == 8
    # the balanced split's phase 2 always takes the widest workgroups; no phase 2 -> 0
    assert pa.plan(mixed, 24, 4, 256, 16, 4096, 65536, 0)["reduce_slices"] == 8
    assert pa.plan([10] * 3, 24, 4, 256, 16, 1, 10, 0, total_tokens_hint=30)["reduce_slices"] == 0
    # head_dim 64 has 4 slices in all
    assert pa.plan(mixed, 24, 4, 64, 16, 4096, 65536, 1024)["reduce_slices"] <= 4
