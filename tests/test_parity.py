"""GPU parity: the HIP decode against the fp64 CPU oracle, through the C ABI.

Tolerance: |gpu - oracle| <= max(2e-3, 1e-2 |oracle|) per element against the
unrounded oracle; bitwise where the mathematics fixes the result exactly.
"""
import math

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import oracle
import workloads
from helpers import assert_close, gpu_out, oracle_full, oracle_rows, say

pytestmark = pytest.mark.gpu

ALL_SINGLE = 1 << 30      # single_pass_max_len forcing one pass for every sequence
TIERS = {"auto": None, "partitioned": 0, "single": ALL_SINGLE}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


def run(w, tier=None, P=None, **kw):
    return pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                     partition_size=w.partition_size if P is None else P,
                     max_seq_len=w.max_seq_len, single_pass_max_len=tier, **kw)


def make(lens, **kw):
    kw.setdefault("device", "cuda")
    kw.setdefault("poison", True)
    kw.setdefault("scale", 1.0 / 16)
    return workloads.make_workload("case", lens, **kw)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tier", list(TIERS))
def test_tiny(tier):
    say(f"case tiny tier={tier}")
    w = workloads.tiny(device="cuda", poison=True)
    assert_close(gpu_out(run(w, TIERS[tier])), oracle_full(w), f"tiny/{tier}")


# partition_size 512 (the pages' grid) and 0 (the length-balanced split)
MODES = {"p512": 512, "balanced": 0}


def test_tiny_balanced():
    say("case tiny balanced")
    w = workloads.tiny(device="cuda", poison=True)
    assert pa.plan(list(w.seq_lens_host), 24, 4, 256, 16, w.max_blocks_per_seq,
                   w.max_seq_len, 0)["balanced"] == 1
    assert_close(gpu_out(run(w, P=0)), oracle_full(w), "tiny/balanced")


@pytest.mark.parametrize("mode", ["auto", "single", "balanced"])
def test_batch(mode):
    say(f"case batch mode={mode}")
    w = workloads.batch(device="cuda", poison=True)
    out = run(w, P=0) if mode == "balanced" else run(w, TIERS[mode])
    assert_close(gpu_out(out), oracle_full(w), f"batch/{mode}")


@pytest.mark.parametrize("mode", list(MODES))
def test_long_context_sampled(mode):
    say(f"case long 4x102400 {mode}, oracle on sequences 0 and 3")
    w = workloads.long_context(device="cuda", poison=True)
    out = gpu_out(run(w, P=MODES[mode]))
    rows = [(s, h) for s in (0, 3) for h in range(w.num_heads)]
    ref = oracle_rows(w, rows)
    got = np.stack([out[s, h] for s, h in rows])
    assert_close(got, ref, f"long/{mode}")


@pytest.mark.parametrize("P", [256, 512, 1024, 0])
def test_mixed_sampled(P):
    say(f"case mixed 64 seqs bf16 P={P}")
    w = workloads.mixed(device="cuda", poison=True, partition_size=P)
    out = gpu_out(run(w))
    order = np.argsort(w.seq_lens_host)
    seqs = [int(order[0]), int(order[20]), int(order[45]), int(order[-2]), int(order[-1])]
    rows = [(s, h) for s in seqs for h in range(w.num_heads)]
    ref = oracle_rows(w, rows)
    got = np.stack([out[s, h] for s, h in rows])
    assert_close(got, ref, f"mixed/P={P} lens={[int(w.seq_lens_host[s]) for s in seqs]}")


@pytest.mark.parametrize("mode", list(MODES))
def test_saturation_sampled(mode):
    say(f"case saturation 256x16384 bs=32 {mode}, 150000-page pool, oracle on 3 sequences")
    w = workloads.saturation(device="cuda", poison=False)
    out = gpu_out(run(w, P=MODES[mode]))
    rows = [(s, h) for s in (0, 137, 255) for h in range(w.num_heads)]
    ref = oracle_rows(w, rows)
    got = np.stack([out[s, h] for s, h in rows])
    assert_close(got, ref, f"saturation/{mode}")
    del w
    torch.cuda.empty_cache()


def test_balanced_many_short_sequences():
    """Hundreds of short segments per share, zero-length sequences in between."""
    say("case balanced: 300 short sequences with zeros")
    rng = np.random.default_rng(31)
    lens = rng.integers(0, 120, size=300)
    lens[::17] = 0
    w = make(list(lens), partition_size=0, seed=31)
    out = gpu_out(run(w, P=0))
    assert np.all(out[lens == 0] == 0)
    assert_close(out, oracle_full(w), "balanced/short")


def test_balanced_falls_back_above_sequence_cap():
    """More sequences than the balanced split keeps in LDS: fixed partitions."""
    say("case 1100 sequences, partition_size 0")
    lens = [5 + (i * 37) % 200 for i in range(1100)]
    w = make(lens, num_heads=8, num_kv_heads=4, head_dim=128, scale=1 / math.sqrt(128),
             partition_size=0, seed=32)
    assert pa.plan(lens, 8, 4, 128, 16, w.max_blocks_per_seq, w.max_seq_len, 0)["balanced"] == 0
    assert_close(gpu_out(run(w, P=0)), oracle_full(w), "fallback")


# ---------------------------------------------------------------------------
# shapes, dtypes, partitions, tiers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("P", [16, 32, 256, 1024])
def test_partition_sizes(dtype, bs, P):
    if P % bs and P < bs:
        pass  # a partition may cover part of a page: still legal (multiple of 16)
    say(f"case partitions dtype={dtype} bs={bs} P={P}")
    w = make([1, 17, 300, 1000, 2100], dtype=dtype, block_size=bs, partition_size=P)
    assert_close(gpu_out(run(w, 0)), oracle_full(w), f"{dtype}/bs{bs}/P{P}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("heads", [(8, 8), (16, 8), (16, 4), (32, 4), (64, 4), (16, 1)])
@pytest.mark.parametrize("tier", ["single", "partitioned", "balanced"])
def test_head_shapes(D, heads, tier):
    Hq, Hkv = heads
    say(f"case heads Hq={Hq} Hkv={Hkv} D={D} tier={tier}")
    w = make([5, 260, 777], num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             scale=1 / math.sqrt(D), partition_size=256)
    out = run(w, P=0) if tier == "balanced" else run(w, TIERS[tier])
    assert_close(gpu_out(out), oracle_full(w), f"Hq{Hq}/Hkv{Hkv}/D{D}/{tier}")


@pytest.mark.parametrize("bs", [8, 16, 48])
@pytest.mark.parametrize("tier", ["single", "partitioned", "balanced"])
def test_edge_lengths(tier, bs):
    lens = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025,
            0, 2]
    say(f"case edge lengths tier={tier} bs={bs}")
    w = make(lens, partition_size=512, block_size=bs)
    out = gpu_out(run(w, P=0) if tier == "balanced" else run(w, TIERS[tier]))
    assert np.all(out[0] == 0) and np.all(out[20] == 0)
    assert_close(out, oracle_full(w), f"edges/{tier}")


def test_outlier_rows_rescale():
    """Whole K rows x20 on 1% of tokens: the running max jumps often."""
    say("case outlier rows")
    w = make([3000, 4500], partition_size=512, q_mult=2.0)
    rng = np.random.default_rng(5)
    nb = w.num_blocks
    mask = torch.from_numpy(rng.random((nb, 1, 16, 1)) < 0.01).to("cuda")
    w.key_cache.copy_(torch.where(mask, w.key_cache * 20, w.key_cache))
    for tier in ("single", "partitioned"):
        assert_close(gpu_out(run(w, TIERS[tier])), oracle_full(w), f"outliers/{tier}")


# ---------------------------------------------------------------------------
# exact results
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_seq_len_one_is_v_bitwise(dtype):
    say(f"case L=1 dtype={dtype}")
    w = make([1, 1, 1], dtype=dtype)
    for tier in ("single", "partitioned", "balanced"):
        out = run(w, P=0) if tier == "balanced" else run(w, TIERS[tier])
        torch.cuda.synchronize()
        g = w.num_heads // w.num_kv_heads
        for s in range(3):
            page = int(w.block_tables_host[s, 0])
            for h in range(w.num_heads):
                assert torch.equal(out[s, h], w.value_cache[page, h // g, 0]), (tier, s, h)


def test_q_zero_gives_mean():
    say("case q=0")
    w = make([7, 100, 1300], partition_size=256)
    w.q.zero_()
    for tier in ("single", "partitioned"):
        assert_close(gpu_out(run(w, TIERS[tier])), oracle_full(w), f"q0/{tier}")


def test_power_of_two_scale_bitwise():
    say("case (2q, scale/2)")
    w = make([40, 900], partition_size=256)
    a = run(w, 0).clone()
    w2 = make([40, 900], partition_size=256)
    w2.q.copy_((w.q.float() * 2).to(w.q.dtype))
    w2.scale = w.scale / 2
    b = run(w2, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_deterministic_and_relabel_invariant():
    say("case determinism + page relabelling")
    w = workloads.batch(device="cuda", poison=True)
    a = run(w).clone()
    b = run(w).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c0 = run(w, P=0).clone()
    c1 = run(w, P=0).clone()
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(3))
    inv = torch.argsort(perm)
    kc = w.key_cache[perm.cuda()]
    vc = w.value_cache[perm.cuda()]
    bt = inv[torch.from_numpy(w.block_tables_host.astype(np.int64))].to(torch.int32).cuda()
    c = pa.decode(w.q, kc, vc, bt, w.seq_lens, w.scale, partition_size=w.partition_size,
                  max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_needle_high_page_ids():
    """Needles in pages whose element offsets exceed 2^32 (a 150,000-page pool of
    32-token pages): each query selects one token, so out == V[needle] exactly."""
    say("case needle at high page ids")
    NB, Hkv, bs, D, Hq = 150000, 4, 32, 256, 24
    kc = torch.empty((NB, Hkv, bs, D), dtype=torch.float16, device="cuda")
    vc = torch.empty_like(kc)
    L = 4096
    nblk = L // bs
    pages = torch.arange(NB - 2 * nblk, NB, dtype=torch.int64).flip(0)   # the top of the pool
    bt = pages.view(2, nblk).to(torch.int32).cuda().contiguous()
    g = torch.Generator(device="cuda").manual_seed(9)
    used = pages.cuda()
    kv = torch.randn((used.numel(), Hkv, bs, D), generator=g, device="cuda").half()
    kv[..., 0] = 0
    kc[used] = kv
    # V payload: dims 0-2 hold (page % 256, page // 256 % 256, slot), exact in fp16
    vv = torch.randn((used.numel(), Hkv, bs, D), generator=g, device="cuda").half()
    vv[..., 0] = (used % 256).view(-1, 1, 1).half()
    vv[..., 1] = ((used // 256) % 256).view(-1, 1, 1).half()
    vv[..., 2] = torch.arange(bs, device="cuda").view(1, 1, bs).half()
    vc[used] = vv
    q = torch.zeros((2, Hq, D), dtype=torch.float16, device="cuda")
    q[..., 0] = 32.0
    sl = torch.full((2,), L, dtype=torch.int32, device="cuda")
    for t in (0, 31, 32, 2047, L - 1):
        for s in range(2):
            page = int(bt[s, t // bs])
            kc[page, :, t % bs, 0] = 32.0
        for tier, P in ((ALL_SINGLE, 512), (0, 512), (None, 0)):
            out = pa.decode(q, kc, vc, bt, sl, 1.0 / 16, partition_size=P, max_seq_len=L,
                            single_pass_max_len=tier)
            torch.cuda.synchronize()
            for s in range(2):
                page = int(bt[s, t // bs])
                for h in range(Hq):
                    assert torch.equal(out[s, h], vc[page, h // 6, t % bs]), (t, s, h, tier)
        for s in range(2):
            kc[int(bt[s, t // bs]), :, t % bs, 0] = 0.0
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [256, 1024, 0])
def test_per_query_head_ablation(P):
    """One workgroup per query head computes each head's column exactly as the
    grouped workgroup of the same dense grid does (one workgroup per piece,
    stream_walk -1): with the same partitions the outputs agree bit for bit.
    (P = 0 sizes partitions per head unit, so only the oracle check applies.)"""
    say(f"case per-query-head ablation P={P}")
    w = make([1, 100, 700, 2000], partition_size=256)
    ablation = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                         partition_size=P, max_seq_len=w.max_seq_len, single_pass_max_len=0,
                         per_query_head=True)
    if P:
        grouped = run(w, 0, P=P, stream_walk=-1)
        torch.cuda.synchronize()
        assert torch.equal(grouped, ablation)
    assert_close(gpu_out(ablation), oracle_full(w), "per-query-head")


@pytest.mark.parametrize("P", [256, 1024, 0])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_sequential_ablation(P, dtype):
    """The group's query heads taken one after another per staged tile (the phase-1
    kernel of the page of commit 8d26e23): each head's column is computed exactly as
    in the grouped pass, so with the same partitions the outputs agree bit for bit
    (P = 0: the automatic fixed partitions of equal lengths declared, on both)."""
    say(f"case head-sequential ablation P={P} {dtype}")
    lens = [1, 100, 700, 2000] if P else [3000] * 3
    w = make(lens, partition_size=256, dtype=dtype, seed=60)
    kw = dict(partition_size=P, max_seq_len=w.max_seq_len)
    if P:
        kw["single_pass_max_len"] = 0
    else:
        kw["total_tokens_hint"] = int(sum(lens))
    info = pa.plan(lens, 24, 4, 256, 16, w.max_blocks_per_seq, w.max_seq_len, P,
                   head_sequential=True, **{k: v for k, v in kw.items()
                                             if k in ("single_pass_max_len", "total_tokens_hint")})
    assert info["head_sequential"] == 1 and info["stream"] == 0 and info["balanced"] == 0
    hs = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                   head_sequential=True, **kw)
    grouped = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                        stream_walk=-1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(hs, grouped)
    assert_close(gpu_out(hs), oracle_full(w), f"head-sequential/P{P}/{dtype}")


def test_workspace_reuse_and_stream():
    """A Decoder reuses one caller-owned workspace across calls and runs on a side stream."""
    say("case workspace reuse")
    w = make([300, 2000, 4000], partition_size=512)
    ref = oracle_full(w)
    dec = pa.Decoder(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                     w.max_blocks_per_seq, torch.float16, max_seq_len=w.max_seq_len,
                     partition_size=512, single_pass_max_len=0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            out = dec(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale)
    torch.cuda.current_stream().wait_stream(side)
    assert_close(gpu_out(out), ref, "decoder")


# ---------------------------------------------------------------------------
# XCD-paired shares (automatic splits)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("skew", [-1, 30, 80, 500])
def test_xcd_skew_balanced(skew):
    """Balanced split with paired shares of unequal size: a length mix with zero
    lengths; the result matches the oracle for any skew, and a repeat is bitwise
    identical."""
    say(f"case xcd skew balanced {skew}")
    w = make([5000, 0, 64, 12000, 700, 1, 9000, 33, 20000, 3], seed=80)
    info = pa.plan(list(w.seq_lens_host), 24, 4, 256, 16, w.max_blocks_per_seq, w.max_seq_len,
                   0, xcd_skew=skew)
    assert info["balanced"] == 1 and info["xcd_skew"] == max(skew, 0)
    out = run(w, P=0, xcd_skew=skew)
    assert_close(gpu_out(out), oracle_full(w), f"xcd/balanced/{skew}")
    assert torch.equal(out, run(w, P=0, xcd_skew=skew))


@pytest.mark.parametrize("lens", [[9000] * 3, [4200] * 2, [16 * 33] * 5])
@pytest.mark.parametrize("skew", [80, 500])
def test_xcd_skew_fixed(lens, skew):
    """Automatic fixed partitions (equal lengths declared) with paired partitions:
    an odd partition count leaves the last one unpaired, and a last pair past the
    length leaves an empty partial."""
    say(f"case xcd skew fixed lens={lens[0]}x{len(lens)} skew={skew}")
    w = make(lens, seed=81)
    hint = int(sum(lens))
    info = pa.plan(list(w.seq_lens_host), 24, 4, 256, 16, w.max_blocks_per_seq, w.max_seq_len,
                   0, total_tokens_hint=hint, xcd_skew=skew)
    assert info["balanced"] == 0 and info["max_partitions"] >= 2
    assert info["xcd_skew"] == skew
    out = run(w, P=0, total_tokens_hint=hint, xcd_skew=skew)
    assert_close(gpu_out(out), oracle_full(w), f"xcd/fixed/{lens[0]}/{skew}")


@pytest.mark.parametrize("cost", [-1, 3, 8, 60, 1000])
def test_piece_cost_balanced(cost):
    """Shares cut with a per-sequence virtual lead-in: with large values many
    shares hold lead-in tiles only, or cut a sequence right after its lead-in."""
    say(f"case piece cost {cost}")
    w = make([5000, 0, 64, 12000, 700, 1, 9000, 33, 20000, 3, 17, 160], seed=90)
    info = pa.plan(list(w.seq_lens_host), 24, 4, 256, 16, w.max_blocks_per_seq, w.max_seq_len,
                   0, piece_cost=cost)
    assert info["balanced"] == 1 and info["piece_cost"] == max(cost, 0)
    for skew in (-1, 0):
        out = run(w, P=0, piece_cost=cost, xcd_skew=skew)
        assert_close(gpu_out(out), oracle_full(w), f"piece_cost/{cost}/skew{skew}")
