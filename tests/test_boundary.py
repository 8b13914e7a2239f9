"""The plain spec entry point, paged_attn_decode (no options), called through
the C ABI with valid arguments, and checked against the oracle.  The Python binding
and the other tests go through paged_attn_decode_ex; this file shows the plain
call gives the same plan and results on the tiny, long-context and mixed
workloads (sampled rows for the large ones)."""
import ctypes

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
import workloads
from helpers import assert_close, gpu_out, oracle_full, oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


def plain_decode(w, P):
    """lib.paged_attn_decode with a workspace sized by lib.paged_attn_workspace_size."""
    lib = pa.lib()
    S, Hq, D = w.q.shape
    n = lib.paged_attn_workspace_size(S, Hq, w.num_kv_heads, D, w.block_size,
                                      w.max_blocks_per_seq, w.max_seq_len, P)
    assert n != ctypes.c_size_t(-1).value
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    out = torch.full_like(w.q, float("nan"))
    st = lib.paged_attn_decode(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(w.q.data_ptr()),
        ctypes.c_void_p(w.key_cache.data_ptr()), ctypes.c_void_p(w.value_cache.data_ptr()),
        ctypes.c_void_p(w.block_tables.data_ptr()), ctypes.c_void_p(w.seq_lens.data_ptr()),
        S, Hq, w.num_kv_heads, D, w.block_size, w.scale, P, ctypes.c_void_p(ws.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), w.max_blocks_per_seq,
        w.max_seq_len, pa._DTYPE[w.q.dtype], n)
    assert st == 0, pa.PagedAttnError(st)
    return out


@pytest.mark.parametrize("P", [512, 0])
def test_plain_call_tiny(P):
    say(f"case plain paged_attn_decode tiny P={P}")
    w = workloads.tiny(device="cuda", poison=True)
    out = plain_decode(w, P)
    assert_close(gpu_out(out), oracle_full(w), f"plain/tiny/P{P}")
    # the same plan as the binding's _ex path with no options: identical bits
    assert torch.equal(out, pa.decode(w.q, w.key_cache, w.value_cache, w.block_tables,
                                      w.seq_lens, w.scale, partition_size=P,
                                      max_seq_len=w.max_seq_len))


@pytest.mark.parametrize("P", [0, 512])
def test_plain_call_long_context_sampled(P):
    """partition_size 0 with no length hint is the length-balanced split."""
    say(f"case plain paged_attn_decode long 4x102400 P={P}")
    w = workloads.long_context(device="cuda", poison=True)
    out = gpu_out(plain_decode(w, P))
    rows = [(s, h) for s in (1, 2) for h in range(w.num_heads)]
    assert_close(np.stack([out[s, h] for s, h in rows]), oracle_rows(w, rows),
                 f"plain/long/P{P}")


@pytest.mark.parametrize("P", [0, 256, 512, 1024])
def test_plain_call_mixed_sampled(P):
    say(f"case plain paged_attn_decode mixed P={P}")
    w = workloads.mixed(device="cuda", poison=True, partition_size=P)
    out = gpu_out(plain_decode(w, P))
    order = np.argsort(w.seq_lens_host)
    seqs = [int(order[i]) for i in (1, 10, 30, 50, 62)]
    rows = [(s, h) for s in seqs for h in range(w.num_heads)]
    assert_close(np.stack([out[s, h] for s, h in rows]), oracle_rows(w, rows),
                 f"plain/mixed/P{P}")
