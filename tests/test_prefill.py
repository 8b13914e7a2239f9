"""GPU parity of prefill over a paged context against the fp64 oracle, through
the C ABI: |gpu - oracle| <= max(2e-3, 1e-2 |oracle|) per element against the
unrounded oracle; bitwise where the result is fixed."""
import math

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import oracle
import workloads
from helpers import assert_close, gpu_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


def make(ctx, ql, **kw):
    kw.setdefault("device", "cuda")
    kw.setdefault("poison", True)
    return workloads.make_prefill("case", ctx, ql, **kw)


def run(w, **kw):
    c = w.ctx
    return pa.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache, c.block_tables,
                      c.seq_lens, w.query_start, c.scale, max(w.max_q_len, 1),
                      max(c.max_seq_len, 0), **kw)


def ref(w, rows=None):
    c = w.ctx
    return oracle.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache, c.block_tables_host,
                          c.seq_lens_host, w.query_start_host, c.scale, c.dtype, rows=rows)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bs", [8, 16, 32, 48, 64, 80])
def test_small_mixed(dtype, bs):
    say(f"case prefill small dtype={dtype} bs={bs}")
    w = make([0, 1, 15, 16, 17, 100, 333], [1, 7, 16, 17, 40, 3, 65], dtype=dtype,
             block_size=bs, seed=51)
    assert_close(gpu_out(run(w)), ref(w), f"prefill/{dtype}/bs{bs}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("heads", [(8, 8), (16, 8), (24, 4), (32, 4), (64, 4), (16, 1)])
def test_head_shapes(D, heads):
    Hq, Hkv = heads
    say(f"case prefill D={D} Hq={Hq} Hkv={Hkv}")
    w = make([50, 0, 260], [20, 33, 9], num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             scale=1 / math.sqrt(D), dtype="bf16" if Hq == 64 else "f16", seed=52 + D + Hq)
    assert_close(gpu_out(run(w)), ref(w), f"prefill/D{D}/{Hq}x{Hkv}")


@pytest.mark.parametrize("bs", [16, 48])
def test_step_boundaries(bs):
    """Context and chunk lengths on both sides of the 32-key steps: one to four
    context steps and one to four chunk steps, odd and even counts in both phases
    of the two-deep pipeline, context tails that leave the second tile of a step
    empty or partial."""
    ctx = [32, 33, 64, 65, 96, 97, 128, 16, 15, 1]
    ql = [32, 33, 64, 65, 96, 1, 2, 31, 97, 128]
    say(f"case prefill step boundaries bs={bs}")
    w = make(ctx, ql, block_size=bs, seed=58 + bs)
    assert_close(gpu_out(run(w)), ref(w), f"prefill/steps/bs{bs}")


def test_long_chunk_many_column_blocks():
    """A 300-token chunk over a 3000-token context: 29 column blocks per KV head,
    the causal bound moving across tiles and waves."""
    say("case prefill 2 x (3000 + 300)")
    w = make([3000, 1234], [300, 129], seed=53)
    assert_close(gpu_out(run(w)), ref(w), "prefill/long-chunk")


def test_empty_chunks_and_no_context():
    say("case prefill empty chunks")
    w = make([10, 0, 40, 0], [0, 5, 0, 1], seed=54)
    out = gpu_out(run(w))
    assert_close(out, ref(w), "prefill/empty")


def test_no_new_tokens_at_all():
    """Every chunk empty: no rows, so the row tensors are empty (NULL data pointers)
    whatever bound the caller passes; the call is a no-op."""
    say("case prefill no new tokens")
    w = make([58, 0, 300], [0, 0, 0], seed=56)
    assert w.q.shape[0] == 0
    out = run(w)                     # passes a bound of 1 with zero rows
    torch.cuda.synchronize()
    assert out.shape[0] == 0


def test_first_token_without_context_is_value_bitwise():
    say("case prefill first token = V")
    w = make([0, 0], [1, 4], seed=55, poison=False)
    out = run(w)
    torch.cuda.synchronize()
    for s in range(2):
        r = int(w.query_start_host[s])
        expect = w.v_new[r].repeat_interleave(w.ctx.num_heads // w.ctx.num_kv_heads, dim=0)
        assert torch.equal(out[r], expect)


def test_deterministic_and_relabel_invariant():
    say("case prefill determinism + page relabelling")
    w = make([700, 90], [50, 20], seed=56, poison=False)
    a = run(w).clone()
    b = run(w).clone()
    assert torch.equal(a, b)
    c = w.ctx
    perm = torch.randperm(c.num_blocks, generator=torch.Generator().manual_seed(3)).cuda()
    inv = torch.argsort(perm)
    kc, vc = c.key_cache[perm].contiguous(), c.value_cache[perm].contiguous()
    bt = inv[c.block_tables.long()].to(torch.int32).contiguous()
    d = pa.prefill(w.q, w.k_new, w.v_new, kc, vc, bt, c.seq_lens, w.query_start, c.scale,
                   w.max_q_len, c.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(a, d)


def test_chunked_prefill_workload_sampled():
    """The 4 x (16384 + 2048) chunked-prefill workload; the oracle on sampled rows."""
    say("case prefill 4 x (16384 + 2048), oracle on sampled rows")
    w = workloads.prefill_chunk(device="cuda", poison=True)
    out = gpu_out(run(w))
    rows = []
    for s in (0, 3):
        r0 = int(w.query_start_host[s])
        for n in (0, 1, 63, 64, 1000, 2047):
            for h in (0, 5, 6, 23):
                rows.append((r0 + n, h))
    got = np.stack([out[r, h] for r, h in rows])
    assert_close(got, ref(w, rows=rows), "prefill/chunk")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, -0.0, -1.0 / 16, -0.7, 1e-6])
def test_any_finite_scale(scale, dtype):
    """The kernel folds |scale| into the exponent and negates Q for a negative
    scale; a zero scale averages the kept keys uniformly.  All against the oracle,
    with poisoned slots past every context."""
    say(f"case prefill scale={scale} {dtype}")
    w = make([0, 1, 15, 16, 17, 100, 333], [1, 7, 16, 17, 40, 3, 65], dtype=dtype, seed=57,
             scale=scale)
    assert w.ctx.scale == scale
    assert_close(gpu_out(run(w)), ref(w), f"prefill/scale{scale}/{dtype}")
