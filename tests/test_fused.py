"""GPU parity of the fused combine: partials merged inside phase 1 by the workgroup
that draws a segment's last ticket, with no phase-2 launch.

Same bar as the two-kernel path: |gpu - oracle| <= max(2e-3, 1e-2 |oracle|) per
element against the unrounded fp64 oracle, bitwise where the result is fixed.
"""
import math

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import workloads
from helpers import assert_close, gpu_out, oracle_full, oracle_rows, say

pytestmark = pytest.mark.gpu

TICKET_BYTES = 65536


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


def fused(w, P, tier=None, workspace=None, hint=0, **kw):
    return pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                     partition_size=P, max_seq_len=w.max_seq_len, single_pass_max_len=tier,
                     workspace=workspace, total_tokens_hint=hint, fused_combine=True, **kw)


def make(lens, **kw):
    kw.setdefault("device", "cuda")
    kw.setdefault("poison", True)
    kw.setdefault("scale", 1.0 / 16)
    return workloads.make_workload("case", lens, **kw)


def plan_of(w, P, tier=None, hint=0, **kw):
    return pa.plan(list(w.seq_lens_host), w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                   w.max_blocks_per_seq, w.max_seq_len, P, single_pass_max_len=tier,
                   total_tokens_hint=hint, fused_combine=True, **kw)


def test_tiny_partitioned():
    say("case fused tiny, 4 partitions of 256")
    w = workloads.tiny(device="cuda", poison=True)
    info = plan_of(w, 256, tier=0)
    assert info["fused"] == 1 and info["phase2_workgroups"] == 0 and info["max_partitions"] == 4
    assert_close(gpu_out(fused(w, 256, tier=0)), oracle_full(w), "fused/tiny")


@pytest.mark.parametrize("mode", ["p512", "uniform", "balanced"])
def test_long_context_sampled(mode):
    say(f"case fused long 4x102400 {mode}, oracle on sequences 1 and 2")
    w = workloads.long_context(device="cuda", poison=True)
    P, hint = {"p512": (512, 0), "uniform": (0, 4 * 102400), "balanced": (0, 0)}[mode]
    info = plan_of(w, P, hint=hint)
    assert info["fused"] == 1 and info["balanced"] == (mode == "balanced")
    out = gpu_out(fused(w, P, hint=hint))
    rows = [(s, h) for s in (1, 2) for h in range(w.num_heads)]
    assert_close(np.stack([out[s, h] for s, h in rows]), oracle_rows(w, rows), f"fused/long/{mode}")


@pytest.mark.parametrize("P", [256, 0])
def test_mixed_sampled(P):
    say(f"case fused mixed 64 seqs bf16 P={P}")
    w = workloads.mixed(device="cuda", poison=True, partition_size=P)
    out = gpu_out(fused(w, P))
    order = np.argsort(w.seq_lens_host)
    seqs = [int(order[0]), int(order[30]), int(order[50]), int(order[-2]), int(order[-1])]
    rows = [(s, h) for s in seqs for h in range(w.num_heads)]
    assert_close(np.stack([out[s, h] for s, h in rows]), oracle_rows(w, rows), f"fused/mixed/P={P}")


def test_batch_balanced():
    say("case fused batch balanced")
    w = workloads.batch(device="cuda", poison=True)
    assert_close(gpu_out(fused(w, 0)), oracle_full(w), "fused/batch")


def test_empty_shares_inside_a_sequence():
    """Fewer tiles than shares: empty shares inside the long sequence add identity
    records, and each draws a ticket.  Without the per-piece lead-in (piece_cost
    -1), which would add virtual tiles; with it, shares of lead-in tiles only."""
    say("case fused balanced, 48 tiles over 64 shares")
    lens = [16] * 10 + [600]
    w = make(lens, max_blocks_per_seq=4096, partition_size=0, seed=41)
    for cost in (-1, 0):
        info = pa.plan(lens, 24, 4, 256, 16, 4096, 65536, 0, fused_combine=True,
                       piece_cost=cost)
        assert info["balanced"] == 1 and info["fused"] == 1
        if cost < 0:
            assert info["active_workgroups"] < info["phase1_workgroups"]   # empty shares
        out = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                        partition_size=0, max_seq_len=65536, fused_combine=True,
                        piece_cost=cost)
        assert_close(gpu_out(out), oracle_full(w), f"fused/empty-shares/cost{cost}")


def test_single_record_segments():
    """Partitioned with one partition per sequence: the only partial is also the last."""
    say("case fused, one partition per sequence")
    w = make([1, 17, 300, 511, 512], partition_size=512, seed=42)
    info = plan_of(w, 512, tier=0)
    assert info["max_partitions"] == 1 and info["fused"] == 1
    assert_close(gpu_out(fused(w, 512, tier=0)), oracle_full(w), "fused/np=1")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("heads", [(8, 8), (16, 8), (32, 4), (64, 4), (16, 1)])
@pytest.mark.parametrize("P", [64, 0])
def test_head_shapes(D, heads, P):
    Hq, Hkv = heads
    say(f"case fused D={D} Hq={Hq} Hkv={Hkv} P={P}")
    w = make([1, 200, 1500, 3000], num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             scale=1 / math.sqrt(D), dtype="bf16" if Hq == 64 else "f16", seed=43 + D + Hq)
    assert_close(gpu_out(fused(w, P, tier=0 if P else None)), oracle_full(w),
                 f"fused/D={D}/{Hq}x{Hkv}/P={P}")


def test_zero_lengths():
    say("case fused, zero-length sequences among partitioned ones")
    lens = [0, 2000, 0, 1, 777, 0]
    w = make(lens, seed=44)
    for P in (128, 0):
        out = gpu_out(fused(w, P, tier=0 if P else None))
        assert np.all(out[[0, 2, 5]] == 0)
        assert_close(out, oracle_full(w), f"fused/zeros/P={P}")


def test_tickets_reset_and_workspace_reuse():
    """One workspace across plans of different layouts: every call is correct, the
    ticket area is zero after each, and a repeated call is bitwise identical."""
    say("case fused workspace reuse across plans")
    a = make([3000, 5000, 40], seed=45)
    b = make([64] * 30 + [9000], num_heads=16, num_kv_heads=2, head_dim=128,
             scale=1 / math.sqrt(128), seed=46)
    need = max(pa.workspace_size(3, 24, 4, 256, 16, a.max_blocks_per_seq, a.max_seq_len, 256),
               pa.workspace_size(31, 16, 2, 128, 16, b.max_blocks_per_seq, b.max_seq_len, 0),
               pa.workspace_size(3, 24, 4, 256, 16, a.max_blocks_per_seq, a.max_seq_len, 0,
                                 per_query_head=True))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                               # stale contents everywhere ...
    pa.workspace_init(ws)                        # ... then only the ticket area cleared
    ra, rb = oracle_full(a), oracle_full(b)
    first = None
    for i, (w, P, kw, ref) in enumerate([(a, 256, {}, ra), (b, 0, {}, rb),
                                         (a, 0, {"per_query_head": True}, ra), (a, 256, {}, ra),
                                         (b, 0, {}, rb)]):
        out = fused(w, P, tier=0 if P else None, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert int(ws[:TICKET_BYTES].count_nonzero()) == 0, f"tickets left set after call {i}"
        assert_close(gpu_out(out), ref, f"fused/reuse/{i}")
        if i == 0:
            first = out.clone()
        if i == 3:
            assert torch.equal(out, first)


def test_decoder_side_stream():
    say("case fused Decoder on a side stream")
    w = make([300, 2000, 4000], partition_size=512, seed=47)
    dec = pa.Decoder(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                     w.max_blocks_per_seq, torch.float16, max_seq_len=w.max_seq_len,
                     partition_size=512, single_pass_max_len=0, fused_combine=True)
    two = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                    partition_size=512, max_seq_len=w.max_seq_len, single_pass_max_len=0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs = [dec(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale).clone()
                for _ in range(3)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs)
    assert_close(gpu_out(outs[0]), oracle_full(w), "fused/decoder")
    # the two-kernel path folds in another order: equal within rounding, not bitwise
    assert_close(gpu_out(outs[0]), gpu_out(two).astype(np.float64), "fused vs two-kernel")
