"""Pins of the prefill oracle (CPU only): prefill over a paged context must agree
with definitions computed independently of it."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def case(ctx, ql, Hq=8, Hkv=2, D=64, bs=16, dtype="f16", seed=5, poison=False, scale=None):
    return workloads.make_prefill("pin", ctx, ql, num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  block_size=bs, dtype=dtype, seed=seed, poison=poison,
                                  scale=scale)


def run(w, **kw):
    c = w.ctx
    return oracle.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache, c.block_tables_host,
                          c.seq_lens_host, w.query_start_host, c.scale, c.dtype, **kw)


def values(t, dtype):
    return oracle.convert(oracle.bits(t), dtype)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_prefill_is_decode_over_the_extended_cache(bs):
    """New token n of a sequence with C cached tokens is decode over C + n + 1 tokens
    once the new keys are written into the cache after the context: same keys in
    the same order, so the two oracles agree bit for bit."""
    ctx, ql = [37, 0, 100, 16], [5, 3, 17, 1]
    w = case(ctx, ql, bs=bs, seed=6)
    c = w.ctx
    kb, vb = oracle.bits(c.key_cache).copy(), oracle.bits(c.value_cache).copy()
    NB, Hkv, _, D = kb.shape
    knb, vnb = oracle.bits(w.k_new), oracle.bits(w.v_new)
    rows = []                                    # per sequence: extended page list
    extra_k, extra_v = [], []
    for s, (C, Q) in enumerate(zip(ctx, ql)):
        pages = [int(p) for p in c.block_tables_host[s, : -(-C // bs)]]
        for n in range(Q):
            t = C + n
            if t // bs >= len(pages):            # a fresh page after the context's
                pages.append(NB + len(extra_k))
                extra_k.append(np.zeros((Hkv, bs, D), np.uint16))
                extra_v.append(np.zeros((Hkv, bs, D), np.uint16))
            p, slot = pages[t // bs], t % bs
            r = w.query_start_host[s] + n
            if p >= NB:
                extra_k[p - NB][:, slot] = knb[r]
                extra_v[p - NB][:, slot] = vnb[r]
            else:
                kb[p, :, slot] = knb[r]
                vb[p, :, slot] = vnb[r]
        rows.append(pages)
    kx = np.concatenate([kb] + [e[None] for e in extra_k]) if extra_k else kb
    vx = np.concatenate([vb] + [e[None] for e in extra_v]) if extra_v else vb
    MB = max(len(p) for p in rows)
    T = w.num_tokens
    bt = np.zeros((T, MB), np.int32)
    sl = np.zeros(T, np.int32)
    for s, (C, Q) in enumerate(zip(ctx, ql)):
        for n in range(Q):
            r = w.query_start_host[s] + n
            bt[r, : len(rows[s])] = rows[s]
            sl[r] = C + n + 1
    dec = oracle.decode(oracle.bits(w.q), kx, vx, bt, sl, c.scale, c.dtype)
    assert np.array_equal(run(w), dec)


def test_prefill_without_context_is_causal_sdpa():
    """No cached context: causal self-attention over the chunk, checked with torch's
    scaled_dot_product_attention in fp64 on head-expanded keys."""
    w = case([0, 0, 0], [1, 9, 33], Hq=12, Hkv=4, D=64, seed=7)
    out = run(w)
    q = torch.from_numpy(values(w.q, "f16"))
    k = torch.from_numpy(values(w.k_new, "f16")).repeat_interleave(3, dim=1)
    v = torch.from_numpy(values(w.v_new, "f16")).repeat_interleave(3, dim=1)
    for s in range(3):
        a, b = w.query_start_host[s], w.query_start_host[s + 1]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[a:b].transpose(0, 1), k[a:b].transpose(0, 1), v[a:b].transpose(0, 1),
            is_causal=True, scale=w.ctx.scale).transpose(0, 1).numpy()
        np.testing.assert_allclose(out[a:b], ref, rtol=1e-12, atol=1e-13)


def test_prefill_brute_force_with_context():
    """Context gathered with numpy fancy indexing, new keys appended, the causal
    mask as a boolean matrix, softmax through log-sum-exp."""
    ctx, ql = [50, 3, 0, 64], [7, 1, 4, 20]
    w = case(ctx, ql, Hq=6, Hkv=3, D=32, bs=16, dtype="bf16", seed=8)
    c = w.ctx
    K = values(c.key_cache, "bf16")
    V = values(c.value_cache, "bf16")
    q, kn, vn = values(w.q, "bf16"), values(w.k_new, "bf16"), values(w.v_new, "bf16")
    out = run(w)
    G = 2
    for s, (C, Q) in enumerate(zip(ctx, ql)):
        t = np.arange(C)
        pages = c.block_tables_host[s, t // 16]
        Kc = K[pages, :, t % 16]                       # [C, Hkv, D]
        Vc = V[pages, :, t % 16]
        a = w.query_start_host[s]
        Kall = np.concatenate([Kc, kn[a:a + Q]])      # [C+Q, Hkv, D]
        Vall = np.concatenate([Vc, vn[a:a + Q]])
        allowed = np.concatenate([np.ones((Q, C), bool), np.tril(np.ones((Q, Q), bool))], 1)
        for h in range(6):
            x = c.scale * np.einsum("nd,ud->nu", q[a:a + Q, h], Kall[:, h // G])
            x = np.where(allowed, x, -np.inf)
            lse = np.log(np.exp(x - x.max(1, keepdims=True)).sum(1, keepdims=True)) + \
                x.max(1, keepdims=True)
            ref = np.exp(x - lse) @ Vall[:, h // G]
            np.testing.assert_allclose(out[a:a + Q, h], ref, rtol=1e-12, atol=1e-13)


def test_first_new_token_without_context_is_its_value():
    w = case([0, 0], [1, 6], seed=9)
    out = run(w)
    vn = values(w.v_new, "f16")
    for s in range(2):
        r = w.query_start_host[s]
        for h in range(8):
            assert np.array_equal(out[r, h], vn[r, h // 4])


def test_page_relabelling_is_bitwise_invariant():
    w = case([70, 33], [9, 4], seed=10)
    c = w.ctx
    perm = np.random.default_rng(0).permutation(c.num_blocks)
    inv = np.argsort(perm)
    kb, vb = oracle.bits(c.key_cache), oracle.bits(c.value_cache)
    bt = c.block_tables_host.copy()
    ref = run(w)
    got = oracle.prefill(w.q, w.k_new, w.v_new, kb[perm], vb[perm], inv[bt].astype(np.int32),
                         c.seq_lens_host, w.query_start_host, c.scale, c.dtype)
    assert np.array_equal(got, ref)


def test_poisoned_pages_never_reach_the_output():
    """NaN in every unreferenced page and context tail slot, unused table entries
    pointing at a NaN page: any read outside the definition shows up as NaN."""
    w = case([31, 16, 0, 90], [4, 16, 3, 2], poison=True, seed=11)
    assert not np.isnan(run(w)).any()


def test_power_of_two_rescale_is_bitwise():
    w = case([40, 5], [6, 3], seed=12, scale=0.125)
    ref = run(w)
    w2 = case([40, 5], [6, 3], seed=12, scale=0.0625)
    w2.q = (w2.q.float() * 2).to(w2.q.dtype)
    assert np.array_equal(run(w2), ref)


def test_gqa_equals_replicated_mha():
    """Group 4 against the same keys replicated per query head (group 1)."""
    w = case([25, 0], [5, 7], Hq=8, Hkv=2, D=32, seed=13)
    c = w.ctx
    rep = lambda t: t.repeat_interleave(4, dim=1).contiguous()
    got = oracle.prefill(w.q, rep(w.k_new), rep(w.v_new), rep(c.key_cache), rep(c.value_cache),
                         c.block_tables_host, c.seq_lens_host, w.query_start_host, c.scale,
                         c.dtype)
    assert np.array_equal(got, run(w))


def test_selected_rows_match_full():
    w = case([12, 40], [3, 5], seed=14)
    full = run(w)
    rows = [(0, 0), (2, 7), (5, 3), (7, 1)]
    got = run(w, rows=rows)
    for i, (r, h) in enumerate(rows):
        assert np.array_equal(got[i], full[r, h])


def test_bad_tables_raise():
    w = case([40], [2], seed=15)
    c = w.ctx
    bt = c.block_tables_host.copy()
    bt[0, 1] = c.num_blocks + 5
    with pytest.raises(ValueError, match="page id"):
        oracle.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache, bt, c.seq_lens_host,
                       w.query_start_host, c.scale, c.dtype)
