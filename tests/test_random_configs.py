"""GPU parity over a seeded random sweep of supported configurations, in
combination.  Decode: head_dim, group size, page size, dtype, length mix (with
zero lengths), partition size, fused combine, XCD pairing and the per-sequence
start cost.  Prefill: head_dim, group size, page size, dtype, context and chunk
lengths (with empty ones).  Every case is compared with the fp64 oracle to the
usual bound."""
import math
import random

import pytest
import torch

import gqa_aware_paged_amd as pa
import oracle
import workloads
from helpers import assert_close, gpu_out, oracle_full, say

pytestmark = pytest.mark.gpu

N_CASES = 120
N_PREFILL = 60


def draw(seed):
    rng = random.Random(1000 + seed)
    D = rng.choice([64, 128, 256])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.choice([1, 2, 3, 4, 6, 8, 16])
    while Hkv * G > 64:
        G //= 2
    bs = rng.choice([8, 16, 32, 48])
    S = rng.choice([1, 2, 5, 13, 40])
    lens = [rng.choice([0, rng.randint(1, 40), rng.randint(1, 700), rng.randint(1, 5000)])
            for _ in range(S)]
    return dict(D=D, Hkv=Hkv, G=G, bs=bs, lens=lens,
                dtype=rng.choice(["f16", "bf16"]),
                P=rng.choice([0, 0, 0, 16, 64, 256, 512]),
                fused=rng.random() < 0.3,
                skew=rng.choice([-1, 0, 0, 300]),
                cost=rng.choice([-1, 0, 0, 20]),
                hint=rng.random() < 0.3)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_config(seed):
    c = draw(seed)
    say(f"case random {seed}: {c}")
    w = workloads.make_workload("case", c["lens"], num_heads=c["Hkv"] * c["G"],
                                num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                                dtype=c["dtype"], scale=1 / math.sqrt(c["D"]), seed=2000 + seed,
                                device="cuda", poison=True)
    hint = int(sum(max(L, 0) for L in c["lens"])) if c["hint"] else 0
    out = pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale,
                    partition_size=c["P"], max_seq_len=w.max_seq_len, total_tokens_hint=hint,
                    fused_combine=c["fused"], xcd_skew=c["skew"], piece_cost=c["cost"])
    assert_close(gpu_out(out), oracle_full(w), f"random/{seed}")


def draw_prefill(seed):
    rng = random.Random(5000 + seed)
    D = rng.choice([64, 128, 256])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.choice([1, 2, 3, 4, 6, 8, 16])
    while Hkv * G > 64:
        G //= 2
    S = rng.choice([1, 2, 3, 6])
    ctx = [rng.choice([0, rng.randint(1, 64), rng.randint(1, 1500)]) for _ in range(S)]
    ql = [rng.choice([0, 1, rng.randint(1, 40), rng.randint(1, 200)]) for _ in range(S)]
    return dict(D=D, Hkv=Hkv, G=G, bs=rng.choice([8, 16, 32, 48, 64]), ctx=ctx, ql=ql,
                dtype=rng.choice(["f16", "bf16"]))


@pytest.mark.parametrize("seed", range(N_PREFILL))
def test_random_prefill(seed):
    c = draw_prefill(seed)
    say(f"case random prefill {seed}: {c}")
    w = workloads.make_prefill("case", c["ctx"], c["ql"], num_heads=c["Hkv"] * c["G"],
                               num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                               dtype=c["dtype"], seed=3000 + seed, device="cuda", poison=True)
    cx = w.ctx
    out = pa.prefill(w.q, w.k_new, w.v_new, cx.key_cache, cx.value_cache, cx.block_tables,
                     cx.seq_lens, w.query_start, cx.scale, max(w.max_q_len, 1),
                     max(cx.max_seq_len, 0))
    ref = oracle.prefill(w.q, w.k_new, w.v_new, cx.key_cache, cx.value_cache,
                         cx.block_tables_host, cx.seq_lens_host, w.query_start_host, cx.scale,
                         cx.dtype)
    if ref.size:
        assert_close(gpu_out(out), ref, f"random-prefill/{seed}")
