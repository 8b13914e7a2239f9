"""Block-table indexing: the phase-1 gather must be bit-exact against the oracle's gather."""
import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import oracle
import workloads
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()


def check(w, what):
    Lcap = max(1, w.max_seq_len)
    k, v = pa.gather_probe(w.key_cache, w.value_cache, w.block_tables, w.seq_lens, Lcap)
    torch.cuda.synchronize()
    ko, vo = oracle.gather(w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host, Lcap)
    kb = k.cpu().view(torch.int16).numpy().view(np.uint16)
    vb = v.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kb, ko), f"{what}: K gather differs"
    assert np.array_equal(vb, vo), f"{what}: V gather differs"
    say(f"  {what}: gather bit-exact ({kb.size} elements each)")


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_gather_bit_exact(bs):
    say(f"case gather bs={bs}")
    w = workloads.make_workload("g", [0, 1, 15, 16, 17, 100, 1000, 3001], block_size=bs,
                                device="cuda", poison=True, seed=21)
    check(w, f"bs{bs}")


def test_gather_tiny_and_batch():
    say("case gather tiny + batch")
    check(workloads.tiny(device="cuda", poison=True), "tiny")
    check(workloads.batch(device="cuda", poison=True), "batch")


def test_gather_head_dim_128_shared_pages():
    say("case gather D=128, pages shared across sequences")
    w = workloads.make_workload("g", [64, 200, 333], head_dim=128, num_heads=16, num_kv_heads=8,
                                device="cuda", poison=True, seed=22, shared_prefix_blocks=3)
    check(w, "D128-shared")


@pytest.mark.parametrize("bs", [8, 16])
def test_gather_head_dim_64(bs):
    say(f"case gather D=64 bs={bs}")
    w = workloads.make_workload("g", [1, 8, 9, 24, 250, 1001], head_dim=64, num_heads=8,
                                num_kv_heads=2, block_size=bs, device="cuda", poison=True, seed=23)
    check(w, f"D64-bs{bs}")
