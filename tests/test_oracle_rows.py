"""Pins for the row-sampled oracle path that every full-size GPU parity check uses.

Large workloads stay on the device; the tests hand the oracle a compact host
copy of only the pages some sequences reference (Workload.host_pages renumbers
the block table into that copy) and evaluate only some (sequence, query head)
rows (oracle.decode_rows).  Both must give exactly what the full oracle gives
on the original pool: the same rows of orc_decode bit for bit, and the same
gathered K/V bits.  Everything here runs on the CPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import oracle_rows


def make(lens, bs, seed, dtype="f16", **kw):
    return workloads.make_workload("rows", lens, num_heads=12, num_kv_heads=3, head_dim=32,
                                   block_size=bs, dtype=dtype, seed=seed, scale=0.2, **kw)


def full(w):
    return oracle.decode(w.q, w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host,
                         w.scale, w.dtype)


CASES = {
    # block size, lengths (zeros, page-aligned and ragged), shared prefix pages, dtype
    "bs8": (8, [0, 1, 8, 9, 63, 200, 0, 77], 0, "f16"),
    "bs16": (16, [33, 0, 16, 500, 1, 250, 17], 0, "bf16"),
    "bs32": (32, [31, 32, 33, 400, 0, 96], 0, "f16"),
    "bs16-shared-prefix": (16, [100, 64, 300, 48, 129], 3, "f16"),
    "bs48-shared-prefix": (48, [200, 96, 47, 500], 2, "bf16"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_rows_over_compact_pages_equal_full_oracle(case):
    """oracle_rows (host_pages + decode_rows, as the GPU tests call it) equals the
    same rows of the full oracle bit for bit.  Catches a (sequence, head) swap or
    a wrong sequence-to-local-index map in the sampling, and a page renumbered to
    the wrong compact page (any off-by-one moves a whole page of keys)."""
    bs, lens, shared, dtype = CASES[case]
    w = make(lens, bs, seed=len(lens) * 7 + bs, dtype=dtype, shared_prefix_blocks=shared,
             poison=True)
    ref = full(w)
    rng = np.random.default_rng(bs + shared)
    S, Hq = w.num_seqs, w.num_heads
    # out of order, repeated, every head of one sequence, zero-length sequences included
    rows = [(int(s), int(h)) for s, h in zip(rng.integers(0, S, 40), rng.integers(0, Hq, 40))]
    rows += [(S - 1, h) for h in range(Hq)]
    rows += [(int(np.argmin(w.seq_lens_host)), 0), rows[0]]
    got = oracle_rows(w, rows)
    want = np.stack([ref[s, h] for s, h in rows])
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", list(CASES))
def test_host_pages_gathers_the_same_bits(case):
    """The compact pool with the renumbered table gathers bit for bit the K/V rows
    the original pool and table gather, for sequences listed out of order."""
    bs, lens, shared, dtype = CASES[case]
    w = make(lens, bs, seed=3 + bs, dtype=dtype, shared_prefix_blocks=shared, poison=True)
    seqs = list(np.random.default_rng(bs).permutation(w.num_seqs))[: max(2, w.num_seqs - 1)]
    kp, vp, bt, sl = w.host_pages(seqs)
    # only referenced pages are copied, each once, and every entry in use points into the copy
    nblk = [-(-int(w.seq_lens_host[s]) // bs) for s in seqs]
    distinct = np.unique(np.concatenate([w.block_tables_host[s, :n] for s, n in zip(seqs, nblk)]))
    assert kp.shape[0] == len(distinct) and vp.shape == kp.shape
    for i, n in enumerate(nblk):
        assert np.all((bt[i, :n] >= 0) & (bt[i, :n] < kp.shape[0]))
    assert np.array_equal(sl, w.seq_lens_host[seqs])
    Lcap = int(max(w.seq_lens_host.max(), 1))
    k_c, v_c = oracle.gather(kp, vp, bt, sl, Lcap)
    k_o, v_o = oracle.gather(w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host,
                             Lcap)
    assert np.array_equal(k_c, k_o[seqs]) and np.array_equal(v_c, v_o[seqs])


def test_rows_of_every_head_match_full_decode_on_compact_pool():
    """decode_rows over all (sequence, head) pairs equals decode on the same compact
    inputs (the selection machinery alone, no page renumbering involved)."""
    w = make([5, 120, 0, 333], 16, seed=41)
    kp, vp, bt, sl = w.host_pages(range(w.num_seqs))
    q = w.q.cpu()
    whole = oracle.decode(q, kp, vp, bt, sl, w.scale, w.dtype)
    rows = [(s, h) for s in range(w.num_seqs) for h in range(w.num_heads)][::-1]
    got = oracle.decode_rows(rows, q, kp, vp, bt, sl, w.scale, w.dtype)
    assert np.array_equal(got, np.stack([whole[s, h] for s, h in rows]))


def test_rows_reject_out_of_range_pairs():
    w = make([40, 7], 16, seed=42)
    args = (w.q, w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host, w.scale,
            w.dtype)
    for bad in ([(2, 0)], [(0, 12)], [(-1, 0)], [(0, -1)]):
        with pytest.raises(ValueError, match="bad shape"):
            oracle.decode_rows(bad, *args)


def test_compact_copy_of_nothing():
    """No sequence selected: an empty pool and table, and no rows."""
    w = make([10, 20], 16, seed=43)
    kp, vp, bt, sl = w.host_pages([])
    assert kp.shape[0] == 0 and vp.shape[0] == 0 and sl.shape == (0,)
    assert torch.is_tensor(kp) and bt.shape[0] == 0
