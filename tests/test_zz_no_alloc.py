"""paged_attn_decode_noalloc (workspace in a device-resident array, nothing
allocated by the call) against paged_attn_decode with a caller-owned workspace,
through the C ABI.  Same plan and kernels, so the outputs agree bit for bit, and
both are within the oracle's tolerance.  Two calls in a row, the second smaller,
show that what the first call left in the array does not leak into the second."""
import ctypes

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


def with_workspace(w, P):
    """paged_attn_decode (caller-owned workspace) through the C ABI."""
    lib = pa.lib()
    S, Hq, D = w.q.shape
    n = lib.paged_attn_workspace_size(S, Hq, w.num_kv_heads, D, w.block_size,
                                      w.max_blocks_per_seq, w.max_seq_len, P)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(w.q)
    st = lib.paged_attn_decode(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(w.q.data_ptr()),
        ctypes.c_void_p(w.key_cache.data_ptr()), ctypes.c_void_p(w.value_cache.data_ptr()),
        ctypes.c_void_p(w.block_tables.data_ptr()), ctypes.c_void_p(w.seq_lens.data_ptr()),
        S, Hq, w.num_kv_heads, D, w.block_size, w.scale, P, ctypes.c_void_p(ws.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), w.max_blocks_per_seq,
        w.max_seq_len, pa._DTYPE[w.q.dtype], n)
    assert st == 0, pa.PagedAttnError(st)
    return out


def no_alloc(w, P, out):
    """paged_attn_decode_noalloc through the C ABI, into a caller-owned out."""
    lib = pa.lib()
    S, Hq, D = w.q.shape
    return lib.paged_attn_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(w.q.data_ptr()),
        ctypes.c_void_p(w.key_cache.data_ptr()), ctypes.c_void_p(w.value_cache.data_ptr()),
        ctypes.c_void_p(w.block_tables.data_ptr()), ctypes.c_void_p(w.seq_lens.data_ptr()),
        S, Hq, w.num_kv_heads, D, w.block_size, w.scale, P,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), w.max_blocks_per_seq,
        w.max_seq_len, pa._DTYPE[w.q.dtype])


@pytest.mark.parametrize("P", [0, 512])
def test_two_calls_second_smaller(P):
    big = workloads.make_workload("big", [9000, 0, 3000, 17, 12000, 640, 1, 5000],
                                  scale=1.0 / 16, device="cuda", poison=True, seed=71)
    small = workloads.make_workload("small", [700, 33, 1500], scale=1.0 / 16, device="cuda",
                                    poison=True, seed=72)
    for w in (big, small):
        say(f"case noalloc P={P} lens={list(w.seq_lens_host)}")
        out = torch.full_like(w.q, float("nan"))
        assert no_alloc(w, P, out) == 0
        ref = with_workspace(w, P)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "noalloc differs from paged_attn_decode"
        assert_close(gpu_out(out), oracle_full(w), f"noalloc/P{P}/{w.name}")


def test_bf16_head_dim_128_and_python_binding():
    w = workloads.make_workload("bf16", [100, 4000, 2600], num_heads=16, num_kv_heads=2,
                                head_dim=128, dtype="bf16", scale=128 ** -0.5, device="cuda",
                                poison=True, seed=73)
    out = torch.empty_like(w.q)
    pa.decode_noalloc(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale, out,
                      max_seq_len=w.max_seq_len)
    ref = with_workspace(w, 0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert_close(gpu_out(out), oracle_full(w), "noalloc/bf16/D128")


def test_plan_beyond_the_array_is_rejected():
    """Explicit 16-token partitions of 64 x 8192 tokens need ~800 MB of partials:
    rejected with PA_ERR_WORKSPACE before anything is enqueued (out stays as it was)."""
    w = workloads.make_workload("huge-plan", [8192] * 64, num_heads=24, num_kv_heads=4,
                                head_dim=64, scale=0.125, device="cuda", seed=74)
    out = torch.zeros_like(w.q)
    assert no_alloc(w, 16, out) == 5
    torch.cuda.synchronize()
    assert bool((out == 0).all())
