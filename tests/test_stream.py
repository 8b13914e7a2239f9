"""Phase 1 as per-wave streams (pa_options.stream_walk 0, the default for the
length-balanced split and explicit partition sizes) and as one workgroup per piece
(stream_walk -1), against the oracle through the C ABI.

The stream walk cuts a share's tiles into one contiguous run per wave; a piece
inside a run is finished from registers, a piece cut between waves is parked and
merged after the kernel's one barrier, and with an explicit partition size the
shares end on partition boundaries.  The cases below put pieces everywhere those
rules branch: many pieces per wave, pieces spanning all four waves, fewer tiles
than waves, one-pass sequences longer than a partition, empty sequences, odd and
even share counts, large start costs."""
import math

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import workloads
from helpers import assert_close, gpu_out, oracle_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


def make(lens, **kw):
    kw.setdefault("device", "cuda")
    kw.setdefault("poison", True)
    kw.setdefault("scale", 1.0 / 16)
    return workloads.make_workload("stream", lens, **kw)


def run(w, P, **kw):
    return pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                     partition_size=P, max_seq_len=w.max_seq_len, **kw)


def plan(w, P, **kw):
    return pa.plan(list(w.seq_lens_host), w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                   w.max_blocks_per_seq, w.max_seq_len, P, **kw)


LENS = [5000, 0, 64, 12000, 700, 1, 9000, 33, 20000, 3, 17, 160, 2048, 0, 511, 513]


@pytest.mark.parametrize("walk", [0, -1], ids=["streams", "piece-per-workgroup"])
@pytest.mark.parametrize("P", [0, 16, 64, 256, 512, 1024])
def test_walks_mixed_lengths(walk, P):
    say(f"case walk={walk} P={P}")
    w = make(LENS, seed=200 + P)
    info = plan(w, P, stream_walk=walk)
    assert info["stream"] == (1 if walk == 0 else 0)
    out = run(w, P, stream_walk=walk)
    assert_close(gpu_out(out), oracle_full(w), f"walk{walk}/P{P}")
    assert torch.equal(out, run(w, P, stream_walk=walk)), "not deterministic"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("P", [0, 128])
@pytest.mark.parametrize("D,bs", [(64, 8), (64, 16), (128, 16), (128, 32), (256, 8), (256, 48)])
def test_stream_shapes(D, bs, P, dtype):
    say(f"case stream D={D} bs={bs} P={P} {dtype}")
    w = make([3000, 17, 0, 800, 4097, 250], head_dim=D, block_size=bs, num_heads=16,
             num_kv_heads=2, dtype=dtype, scale=1 / math.sqrt(D), seed=210 + D + bs)
    assert plan(w, P)["stream"] == 1
    assert_close(gpu_out(run(w, P)), oracle_full(w), f"stream/D{D}/bs{bs}/P{P}/{dtype}")


@pytest.mark.parametrize("cost", [-1, 1, 8, 100])
@pytest.mark.parametrize("P", [0, 256])
def test_stream_piece_cost(cost, P):
    """Large start costs leave shares of lead-in tiles only (balanced) or move share
    boundaries by whole partitions."""
    say(f"case stream piece cost {cost} P={P}")
    w = make(LENS, seed=230)
    info = plan(w, P, piece_cost=cost)
    assert info["stream"] == 1 and info["piece_cost"] == max(cost, 0)
    assert_close(gpu_out(run(w, P, piece_cost=cost)), oracle_full(w), f"cost{cost}/P{P}")


@pytest.mark.parametrize("skew", [-1, 80, 500])
def test_stream_partitions_xcd_paired(skew):
    """Explicit partitions stay whole; only which share takes the boundary partition
    follows the XCD pairing."""
    say(f"case stream partitions skew {skew}")
    w = make([9000, 9000, 4000, 300, 12000], seed=240)
    info = plan(w, 512, xcd_skew=skew)
    assert info["stream"] == 1 and info["xcd_skew"] == max(skew, 0)
    out = run(w, 512, xcd_skew=skew)
    assert_close(gpu_out(out), oracle_full(w), f"parts/skew{skew}")


@pytest.mark.parametrize("P", [0, 16])
def test_stream_many_short_sequences(P):
    """1024 sequences (the most the walk keeps in LDS) of 0..40 tokens: dozens of
    whole pieces inside every wave's run."""
    say(f"case stream 1024 short sequences P={P}")
    rng = np.random.default_rng(250)
    lens = rng.integers(0, 41, size=1024)
    lens[::37] = 0
    w = make(list(lens), num_heads=8, num_kv_heads=2, head_dim=128,
             scale=1 / math.sqrt(128), seed=250)
    assert plan(w, P)["stream"] == 1
    out = gpu_out(run(w, P))
    assert np.all(out[lens == 0] == 0)
    assert_close(out, oracle_full(w), f"short1024/P{P}")


@pytest.mark.parametrize("P", [0, 16, 512])
def test_stream_fewer_tiles_than_waves(P):
    """Shares of one to three tiles: some waves have no tiles at all."""
    say(f"case stream tiny shares P={P}")
    w = make([1, 2, 17, 40, 0, 9], seed=260)
    assert_close(gpu_out(run(w, P)), oracle_full(w), f"tiny-shares/P{P}")


@pytest.mark.parametrize("tier", [0, 2000, 1 << 30])
def test_stream_partitions_with_forced_tier(tier):
    """Explicit 256-token partitions with a forced one-pass bound: with 2000 and
    2^30, one-pass sequences longer than a partition are single pieces that shares
    never cut, however many waves they span."""
    say(f"case stream forced tier {tier}")
    w = make([1999, 2000, 2001, 300, 7000, 0, 256, 257], seed=270)
    info = plan(w, 256, single_pass_max_len=tier)
    assert info["stream"] == 1 and info["single_pass_max_len"] == tier
    assert_close(gpu_out(run(w, 256, single_pass_max_len=tier)), oracle_full(w),
                 f"forced-tier/{tier}")


def test_stream_relabel_invariant():
    say("case stream page relabelling")
    w = make(LENS, seed=280)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(4))
    inv = torch.argsort(perm)
    kc, vc = w.key_cache[perm.cuda()], w.value_cache[perm.cuda()]
    bt = inv[torch.from_numpy(w.block_tables_host.astype(np.int64))].to(torch.int32).cuda()
    for P in (0, 512):
        a = run(w, P)
        b = pa.decode(w.q, kc, vc, bt, w.seq_lens, w.scale, partition_size=P,
                      max_seq_len=w.max_seq_len)
        torch.cuda.synchronize()
        assert torch.equal(a, b), P


def test_stream_batch_and_long_workloads():
    """The batch workload in full and the long-context one on two sequences, with
    the default call (balanced split on streams) and 512-token partitions."""
    say("case stream batch + long")
    w = workloads.batch(device="cuda", poison=True)
    for P in (0, 512):
        assert_close(gpu_out(run(w, P)), oracle_full(w), f"batch/P{P}")
    del w
    from helpers import oracle_rows
    w = workloads.long_context(device="cuda", poison=True)
    rows = [(s, h) for s in (0, 3) for h in range(0, 24, 5)]
    ref = oracle_rows(w, rows)
    for P in (0, 512):
        out = gpu_out(run(w, P))
        assert_close(np.stack([out[s, h] for s, h in rows]), ref, f"long/P{P}")
