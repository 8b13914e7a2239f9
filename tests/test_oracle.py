"""Pins for the CPU oracle, checked against things other than itself.

Each test names the mistake it would catch.  Everything here runs on the CPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def small(lens, Hq=24, Hkv=4, D=64, bs=16, dtype="f16", seed=0, **kw):
    return workloads.make_workload("t", lens, num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                   block_size=bs, dtype=dtype, seed=seed, **kw)


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def run(w, **kw):
    return oracle.decode(w.q, w.key_cache, w.value_cache, w.block_tables_host,
                         w.seq_lens_host, w.scale, w.dtype, **kw)


def brute_force(w):
    """Independent unpaged attention: contiguous copy by numpy fancy indexing,
    log-sum-exp softmax, einsum over the group axis."""
    K = f64(w.key_cache)
    V = f64(w.value_cache)
    Q = f64(w.q)
    S, Hq, D = Q.shape
    g = Hq // w.num_kv_heads
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(w.seq_lens_host[s])
        if L <= 0:
            continue
        t = np.arange(L)
        pages = w.block_tables_host[s, t // w.block_size]
        Kc = K[pages, :, t % w.block_size, :]          # [L, Hkv, D]
        Vc = V[pages, :, t % w.block_size, :]
        Qg = Q[s].reshape(w.num_kv_heads, g, D)          # [Hkv, g, D]
        x = np.einsum("kgd,lkd->kgl", Qg, Kc) * w.scale  # [Hkv, g, L]
        lse = np.log(np.sum(np.exp(x - x.max(-1, keepdims=True)), -1, keepdims=True)) \
            + x.max(-1, keepdims=True)
        p = np.exp(x - lse)
        out[s] = np.einsum("kgl,lkd->kgd", p, Vc).reshape(Hq, D)
    return out


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_f16_conversion_exhaustive():
    """All 65536 binary16 patterns agree with numpy's float16 -> float64
    (catches a wrong exponent bias, subnormal scale or sign handling)."""
    raw = np.arange(65536, dtype=np.uint16)
    got = oracle.convert(raw, "f16")
    ref = raw.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_conversion_exhaustive():
    raw = np.arange(65536, dtype=np.uint16)
    got = oracle.convert(raw, "bf16")
    ref = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_round_to_single_rounding():
    """One RNE step from fp64: ties go to even, and values just above a tie
    round up (a cast through float32 would lose the 2^-40 and round down)."""
    x = np.array([1 + 2**-11, 1 + 3 * 2**-11, 1 + 2**-11 + 2**-40])
    assert f64(oracle.round_to(x, "f16")).tolist() == [1.0, 1 + 2**-9, 1 + 2**-10]
    y = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-40, 2.0**-134 * 3])
    assert f64(oracle.round_to(y, "bf16")).tolist() == [1.0, 1 + 2**-6, 1 + 2**-7, 2.0**-132]


# --------------------------------------------------------------------------
# the five checks the decode must satisfy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_brute_force_unpaged(dtype, bs):
    """(1) paged oracle == unpaged brute force on a contiguous copy."""
    w = small([1, 17, 100, 257], dtype=dtype, bs=bs, seed=3)
    assert rel_err(run(w), brute_force(w)) < 1e-12


def test_torch_sdpa_fp64():
    """softmax attention from a library routine on the gathered, head-expanded K/V."""
    w = small([33, 300], seed=4)
    ref = np.zeros((w.num_seqs, w.num_heads, w.head_dim))
    g = w.num_heads // w.num_kv_heads
    ko, vo = oracle.gather(w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host)
    for s in range(w.num_seqs):
        L = int(w.seq_lens_host[s])
        K = torch.from_numpy(oracle.convert(ko[s, :, :L], "f16")).repeat_interleave(g, 0)
        V = torch.from_numpy(oracle.convert(vo[s, :, :L], "f16")).repeat_interleave(g, 0)
        Q = w.q[s].to(torch.float64)[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=w.scale)
        ref[s] = o[:, 0, :].numpy()
    assert rel_err(run(w), ref) < 1e-12


def test_seq_len_one_is_v():
    """(2) L = 1: a single weight of exactly 1, so out == V[token 0] bit for bit."""
    w = small([1, 1], seed=5)
    out = run(w)
    g = w.num_heads // w.num_kv_heads
    for s in range(2):
        page = w.block_tables_host[s, 0]
        for h in range(w.num_heads):
            assert np.array_equal(out[s, h], f64(w.value_cache[page, h // g, 0]))


def test_constant_scores_mean():
    """(3) q = 0: every logit is 0, so out is the plain mean of V."""
    w = small([5, 64, 129], seed=6)
    w.q.zero_()
    out = run(w)
    ko, vo = oracle.gather(w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host)
    g = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        L = int(w.seq_lens_host[s])
        mean = oracle.convert(vo[s, :, :L], "f16").mean(axis=1)   # [Hkv, D]
        np.testing.assert_allclose(out[s], np.repeat(mean, g, 0), rtol=1e-13, atol=1e-15)


def test_page_permutation_invariance():
    """(4) relabel the physical pages (permute the pool, remap the table): identical output."""
    w = small([40, 77, 200], seed=7)
    out = run(w)
    rng = np.random.default_rng(8)
    NB = w.num_blocks
    perm = rng.permutation(NB)              # new page j holds old page perm[j]
    inv = np.argsort(perm)
    kc = w.key_cache[torch.from_numpy(perm)]
    vc = w.value_cache[torch.from_numpy(perm)]
    bt = inv[w.block_tables_host].astype(np.int32)
    out2 = oracle.decode(w.q, kc, vc, bt, w.seq_lens_host, w.scale, w.dtype)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("P", [16, 256, 512, 1024, "L"])
def test_partitioned_combine_equals_softmax(P):
    """(5) per-partition partials merged by the rescale rule == unpartitioned softmax,
    both by a sequential fold and by a one-shot merge."""
    lens = [1, 300, 1500, 2100]
    w = small(lens, Hq=6, Hkv=1, D=32, seed=9)
    ref = run(w)
    Pv = max(lens) if P == "L" else P
    m, l, acc = oracle.partials(w.q, w.key_cache, w.value_cache, w.block_tables_host,
                                w.seq_lens_host, w.scale, w.dtype, Pv)
    _, _, folded = oracle.fold_partials(m, l, acc)
    _, _, once = oracle.merge_once(m, l, acc)
    assert rel_err(folded, ref) < 1e-12
    assert rel_err(once, ref) < 1e-12


def test_combine_associative_and_identity():
    rng = np.random.default_rng(10)
    parts = [(rng.normal() * 5, rng.uniform(0.5, 30), rng.normal(size=8)) for _ in range(9)]
    ident = (-np.inf, 0.0, np.zeros(8))
    left = ident
    for p in parts:
        left = oracle.combine(left, p)
    # right fold and a random tree
    right = ident
    for p in reversed(parts):
        right = oracle.combine(p, right)
    items = list(parts)
    while len(items) > 1:
        i = rng.integers(0, len(items) - 1)
        items[i:i + 2] = [oracle.combine(items[i], items[i + 1])]
    for st in (right, items[0]):
        assert abs(st[0] - left[0]) == 0
        assert abs(st[1] - left[1]) / left[1] < 1e-13
        assert np.max(np.abs(st[2] - left[2])) < 1e-13
    # identity on either side returns the other operand untouched
    a = oracle.combine(ident, parts[0])
    b = oracle.combine(parts[0], ident)
    for st in (a, b):
        assert st[0] == parts[0][0] and st[1] == parts[0][1] and np.array_equal(st[2], parts[0][2])


@pytest.mark.parametrize("tile", [1, 16, 32, 100])
def test_pages_online_update_matches_definition(tile):
    """The tile-by-tile update exactly as the online-softmax fix writes it
    reaches the closed-form softmax."""
    rng = np.random.default_rng(11)
    x = rng.normal(size=333) * 6
    V = rng.normal(size=(333, 5))
    w = np.exp(x - x.max())
    ref = (w / w.sum()) @ V
    got = oracle.online_softmax_tiles(x, V, tile)
    assert np.max(np.abs(got - ref)) < 1e-13


def test_two_token_closed_form():
    """Logits 0 and 1 give weights 1/(1+e) and e/(1+e)."""
    x = np.array([0.0, 1.0])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    got = oracle.online_softmax_tiles(x, V, 1)
    assert abs(got[0] - 1 / (1 + math.e)) < 1e-16
    assert abs(got[1] - math.e / (1 + math.e)) < 1e-15
    # and the same through the paged C path: D = 2, q = (1, 0), K rows (0,*),(1,*)
    w = small([2], Hq=1, Hkv=1, D=2, bs=16, seed=12, scale=1.0)
    w.q[:] = torch.tensor([[[1.0, 0.0]]], dtype=torch.float16)
    page = w.block_tables_host[0, 0]
    w.key_cache[page, 0, 0] = torch.tensor([0.0, 5.0], dtype=torch.float16)
    w.key_cache[page, 0, 1] = torch.tensor([1.0, -3.0], dtype=torch.float16)
    w.value_cache[page, 0, 0] = torch.tensor([1.0, 0.0], dtype=torch.float16)
    w.value_cache[page, 0, 1] = torch.tensor([0.0, 1.0], dtype=torch.float16)
    out = run(w)[0, 0]
    assert abs(out[0] - 1 / (1 + math.e)) < 1e-16
    assert abs(out[1] - math.e / (1 + math.e)) < 1e-15


# --------------------------------------------------------------------------
# scale, GQA mapping, masking, degenerate cases
# --------------------------------------------------------------------------

def test_power_of_two_scale_trade():
    """(2q, scale/2) gives the same logits exactly: catches a scale applied twice,
    squared, or folded into q with rounding."""
    w = small([50, 130], seed=13)
    out = run(w)
    q2 = (w.q.to(torch.float32) * 2).to(w.q.dtype)
    out2 = oracle.decode(q2, w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host,
                         w.scale / 2, w.dtype)
    assert np.array_equal(out, out2)
    # a different scale must change the result
    out3 = oracle.decode(w.q, w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host,
                         w.scale * 2, w.dtype)
    assert not np.allclose(out, out3)


def test_gqa_equals_replicated_mha():
    """Query head h reads KV head h // (Hq/Hkv): replicating each KV head over its
    group and running with Hkv = Hq gives the same output bit for bit."""
    w = small([20, 90], seed=14)
    g = w.num_heads // w.num_kv_heads
    kc = w.key_cache.repeat_interleave(g, dim=1).contiguous()
    vc = w.value_cache.repeat_interleave(g, dim=1).contiguous()
    out = run(w)
    out_mha = oracle.decode(w.q, kc, vc, w.block_tables_host, w.seq_lens_host, w.scale, w.dtype)
    assert np.array_equal(out, out_mha)
    # heads of one group with identical queries give identical rows; other groups differ
    w.q[:, 0:g] = w.q[:, 0:1]
    out = run(w)
    for h in range(1, g):
        assert np.array_equal(out[:, h], out[:, 0])
    assert not np.allclose(out[:, g], out[:, 0])


def test_zero_length_gives_zeros():
    w = small([0, 10, 0], seed=15)
    out = run(w)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out[1])) and np.any(out[1] != 0)


def poison_outside(w):
    """Copies of the caches and table with NaN in every unreferenced page, in
    each last page's slots past the sequence end, and unused table entries
    pointed at a NaN page."""
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    bt = w.block_tables_host.copy()
    bs = w.block_size
    used = np.zeros(w.num_blocks, bool)
    for s in range(w.num_seqs):
        n = -(-int(w.seq_lens_host[s]) // bs)
        used[bt[s, :n]] = True
    unused = np.nonzero(~used)[0]
    assert len(unused) > 0
    kc[torch.from_numpy(unused)] = float("nan")
    vc[torch.from_numpy(unused)] = float("nan")
    for s in range(w.num_seqs):
        L = int(w.seq_lens_host[s])
        n = -(-L // bs)
        bt[s, n:] = unused[0]
        if L % bs:
            kc[bt[s, n - 1], :, L % bs:] = float("nan")
            vc[bt[s, n - 1], :, L % bs:] = float("nan")
    return kc, vc, bt


def test_nan_outside_sequence_has_no_effect():
    """NaN in unreferenced pages, tail slots and unused table entries: output bitwise unchanged."""
    w = small([17, 45, 64, 3], seed=16, max_blocks_per_seq=8)
    out = run(w)
    kc, vc, bt = poison_outside(w)
    out2 = oracle.decode(w.q, kc, vc, bt, w.seq_lens_host, w.scale, w.dtype)
    assert np.array_equal(out, out2)
    # and a NaN inside a sequence does reach its output (the poison is live)
    kc[w.block_tables_host[0, 0], 0, 0, 0] = float("nan")
    out3 = oracle.decode(w.q, kc, vc, bt, w.seq_lens_host, w.scale, w.dtype)
    assert np.isnan(out3[0, 0]).all() and not np.isnan(out3[1]).any()


def test_needle_selects_one_token():
    """q = 32 e0 and K[:, 0] = 0 except one needle token with K[...,0] = 32: logits
    are 64 vs 0, so out equals V[needle] after rounding to the dtype."""
    L = 300
    w = small([L], Hq=6, Hkv=1, D=32, seed=17, scale=1.0 / 16)
    w.q.zero_()
    w.q[0, :, 0] = 32.0
    w.key_cache[:, :, :, 0] = 0.0
    for needle in (0, 15, 16, 157, L - 1):
        kc = w.key_cache.clone()
        page = w.block_tables_host[0, needle // 16]
        kc[page, 0, needle % 16, 0] = 32.0
        out = oracle.decode(w.q, kc, w.value_cache, w.block_tables_host, w.seq_lens_host,
                            w.scale, w.dtype)
        vn = w.value_cache[page, 0, needle % 16]
        for h in range(6):
            assert torch.equal(oracle.round_to(out[0, h], "f16"), vn)


def test_oracle_rejects_bad_tables():
    w = small([40], seed=18)
    bt = w.block_tables_host.copy()
    bt[0, 1] = w.num_blocks          # out of the pool
    with pytest.raises(ValueError, match="page id"):
        oracle.decode(w.q, w.key_cache, w.value_cache, bt, w.seq_lens_host, w.scale, w.dtype)
    with pytest.raises(ValueError, match="capacity"):
        oracle.decode(w.q, w.key_cache, w.value_cache, w.block_tables_host,
                      np.array([10_000], np.int32), w.scale, w.dtype)


def test_partials_of_empty_partitions_are_identity():
    w = small([100, 600], Hq=2, Hkv=1, D=16, seed=19)
    m, l, acc = oracle.partials(w.q, w.key_cache, w.value_cache, w.block_tables_host,
                                w.seq_lens_host, w.scale, w.dtype, 256)
    assert m.shape[-1] == 3
    assert np.all(m[0, :, 1:] == -np.inf) and np.all(l[0, :, 1:] == 0)
    assert np.all(acc[0, :, 1:] == 0)
    assert np.all(np.isfinite(m[1]))
