"""CPU oracle for GQA paged-attention decode (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path (gqa_aware_paged_amd) never imports it and the
two share no code.

Contents
--------
decode / decode_rows / gather / partials
    ctypes wrappers over pa_oracle.c, the plain fp64 definition of decode
    attention with the block-table gather (see that file's header for the
    citations).
prefill
    The plain fp64 definition of prefill over a paged context (pa_oracle.c,
    orc_prefill): each new token attends to the cached context and, causally,
    to the new tokens up to itself.
combine / fold_partials / merge_once
    The partition merge.  The page of commit 8d26e23 (docs) defines the
    compound partial (max_score, exp_sum, weighted_v) and a combine that
    rescales like flash attention; the page of commit 87a19d2
    (paged_attention_v2_triton.py, the online-softmax fix) writes the rescale
    out: m_new = max(m_i, m_ij), alpha = exp(m_i - m_new),
    beta = exp(m_ij - m_new), l_new = alpha*l_i + beta*l_ij, and the
    accumulator is reweighted by alpha*l_i/l_new and beta*l_ij/l_new.
online_softmax_tiles
    The same update applied tile by tile to one row of logits, in the order
    and notation of the online-softmax fix on the page of commit 87a19d2.
round_to
    Round fp64 results to f16/bf16 with one round-to-nearest-even step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_SO = os.path.join(_HERE, "libpa_oracle.so")
DTYPE_CODE = {"f16": 0, "bf16": 1}
_lib_handle = None


def build(force: bool = True) -> str:
    """Compile pa_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, D, I, I, P]
        lib.orc_decode_rows.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, I, I, I, D, I, I]
        lib.orc_gather.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I]
        lib.orc_partials.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, I, I, I]
        lib.orc_convert.argtypes = [P, P, ctypes.c_int64, I]
        lib.orc_prefill.argtypes = [P, P, I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, I,
                                    I, P]
        for f in (lib.orc_decode, lib.orc_decode_rows, lib.orc_gather, lib.orc_partials,
                  lib.orc_prefill):
            f.restype = I
        lib.orc_convert.restype = None
        _lib_handle = lib
    return _lib_handle


_ERR = {-1: "bad shape", -2: "page id outside the pool", -3: "seq_len exceeds table capacity",
        -4: "out of memory"}


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle: {_ERR.get(rc, rc)}")


def bits(x) -> np.ndarray:
    """Raw 16-bit patterns of an f16/bf16 tensor (or a uint16 array), C-contiguous."""
    if isinstance(x, np.ndarray):
        if x.dtype == np.uint16:
            return np.ascontiguousarray(x)
        if x.dtype == np.float16:
            return np.ascontiguousarray(x).view(np.uint16)
        raise TypeError(x.dtype)
    t = x.detach().to("cpu").contiguous()
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(t.dtype)
    return t.view(torch.int16).numpy().view(np.uint16)


def _i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def convert(raw: np.ndarray, dtype: str) -> np.ndarray:
    raw = np.ascontiguousarray(raw, dtype=np.uint16)
    out = np.empty(raw.shape, np.float64)
    _lib().orc_convert(_p(raw), _p(out), raw.size, DTYPE_CODE[dtype])
    return out


def decode(q, key_cache, value_cache, block_tables, seq_lens, scale: float, dtype: str,
           threads: int = 0, return_threads: bool = False):
    """fp64 [S, Hq, D] = softmax(scale q K^T) V per query head, K/V gathered by block table."""
    qb, kb, vb = bits(q), bits(key_cache), bits(value_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, D = qb.shape
    NB, Hkv, bs, D2 = kb.shape
    assert D2 == D and vb.shape == kb.shape and sl.shape == (S,)
    MB = bt.shape[1] if bt.ndim == 2 else 0
    out = np.empty((S, Hq, D), np.float64)
    used = ctypes.c_int(0)
    _check(_lib().orc_decode(_p(out), _p(qb), _p(kb), _p(vb), _p(bt), _p(sl), S, Hq, Hkv,
                             D, bs, NB, MB, float(scale), DTYPE_CODE[dtype], int(threads),
                             ctypes.byref(used)))
    return (out, used.value) if return_threads else out


def decode_rows(rows: Sequence, q, key_cache, value_cache, block_tables, seq_lens,
                scale: float, dtype: str, threads: int = 0) -> np.ndarray:
    """fp64 [len(rows), D] for the (sequence, query head) pairs in `rows`."""
    qb, kb, vb = bits(q), bits(key_cache), bits(value_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    S, Hq, D = qb.shape
    NB, Hkv, bs, _ = kb.shape
    out = np.empty((r.shape[0], D), np.float64)
    _check(_lib().orc_decode_rows(_p(out), _p(r), r.shape[0], _p(qb), _p(kb), _p(vb), _p(bt),
                                  _p(sl), S, Hq, Hkv, D, bs, NB, bt.shape[1], float(scale),
                                  DTYPE_CODE[dtype], int(threads)))
    return out


def prefill(q, k_new, v_new, key_cache, value_cache, block_tables, ctx_lens, query_start,
            scale: float, dtype: str, rows: Optional[Sequence] = None,
            threads: int = 0, return_threads: bool = False):
    """fp64 prefill: q, k_new, v_new hold the new tokens of every sequence packed
    ([T, Hq, D] and [T, Hkv, D]; sequence s owns rows query_start[s] ..
    query_start[s+1]-1); ctx_lens[s] context tokens are in the paged caches.
    Returns [T, Hq, D], or [len(rows), D] for the (row, query head) pairs in rows."""
    qb, knb, vnb = bits(q), bits(k_new), bits(v_new)
    kb, vb = bits(key_cache), bits(value_cache)
    bt, cl, qs = _i32(block_tables), _i32(ctx_lens), _i32(query_start)
    T, Hq, D = qb.shape
    NB, Hkv, bs, D2 = kb.shape
    S = cl.shape[0]
    assert D2 == D and knb.shape == (T, Hkv, D) and vnb.shape == knb.shape
    assert qs.shape == (S + 1,) and int(qs[-1]) == T
    MB = bt.shape[1] if bt.ndim == 2 else 0
    if rows is None:
        r, n, out = None, 0, np.empty((T, Hq, D), np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n, out = r.shape[0], np.empty((r.shape[0], D), np.float64)
    used = ctypes.c_int(0)
    _check(_lib().orc_prefill(_p(out), None if r is None else _p(r), n, _p(qb), _p(knb),
                              _p(vnb), _p(kb), _p(vb), _p(bt), _p(cl), _p(qs), S, Hq, Hkv, D,
                              bs, NB, MB, float(scale), DTYPE_CODE[dtype], int(threads),
                              ctypes.byref(used)))
    return (out, used.value) if return_threads else out


def gather(key_cache, value_cache, block_tables, seq_lens, Lcap: Optional[int] = None):
    """Raw 16-bit K and V [S, Hkv, Lcap, D] of tokens t < seq_len (zeros elsewhere)."""
    kb, vb = bits(key_cache), bits(value_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    NB, Hkv, bs, D = kb.shape
    S = sl.shape[0]
    if Lcap is None:
        Lcap = int(sl.max()) if S else 0
    ko = np.zeros((S, Hkv, max(Lcap, 0), D), np.uint16)
    vo = np.zeros_like(ko)
    _check(_lib().orc_gather(_p(ko), _p(vo), _p(kb), _p(vb), _p(bt), _p(sl), S, Hkv, D, bs,
                             NB, bt.shape[1], Lcap))
    return ko, vo


def partials(q, key_cache, value_cache, block_tables, seq_lens, scale: float, dtype: str,
             partition_size: int, num_partitions: Optional[int] = None):
    """Per-partition (m, l, acc) by definition; m in natural-log units, acc normalised."""
    qb, kb, vb = bits(q), bits(key_cache), bits(value_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, D = qb.shape
    NB, Hkv, bs, _ = kb.shape
    P = int(partition_size)
    NP = num_partitions if num_partitions is not None else \
        max(1, max((int(L) + P - 1) // P for L in sl) if S else 1)
    m = np.empty((S, Hq, NP), np.float64)
    l = np.empty((S, Hq, NP), np.float64)
    acc = np.empty((S, Hq, NP, D), np.float64)
    _check(_lib().orc_partials(_p(m), _p(l), _p(acc), _p(qb), _p(kb), _p(vb), _p(bt), _p(sl),
                               S, Hq, Hkv, D, bs, NB, bt.shape[1], float(scale),
                               DTYPE_CODE[dtype], P, NP))
    return m, l, acc


# ---------------------------------------------------------------------------
# Partition merge, written from the rescale rule of the online-softmax fix.
# ---------------------------------------------------------------------------

def combine(a, b):
    """Merge two partials (m, l, acc) with acc normalised; (-inf, 0, 0) is the identity."""
    m_i, l_i, acc_i = a
    m_ij, l_ij, acc_ij = b
    if m_ij == -np.inf:
        return a
    if m_i == -np.inf:
        return b
    m_new = max(m_i, m_ij)
    alpha = np.exp(m_i - m_new)
    beta = np.exp(m_ij - m_new)
    l_new = alpha * l_i + beta * l_ij
    acc = acc_i * (alpha * l_i / l_new) + acc_ij * (beta * l_ij / l_new)
    return m_new, l_new, acc


def fold_partials(m, l, acc):
    """Sequential left fold of `combine` over the partition axis.

    m, l: [..., NP]; acc: [..., NP, D].  Returns (m, l, acc) with the partition
    axis folded away.  Rows whose every partition is empty come out as zeros.
    """
    lead = m.shape[:-1]
    D = acc.shape[-1]
    M = np.full(lead, -np.inf)
    Lsum = np.zeros(lead)
    A = np.zeros(lead + (D,))
    for idx in np.ndindex(*lead):
        st = (-np.inf, 0.0, np.zeros(D))
        for p in range(m.shape[-1]):
            st = combine(st, (m[idx + (p,)], l[idx + (p,)], acc[idx + (p,)]))
        M[idx], Lsum[idx], A[idx] = st
    return M, Lsum, A


def merge_once(m, l, acc):
    """One-shot merge over the partition axis: M = max m, w = l exp(m - M),
    out = sum w acc / sum w (zeros where no partition holds a token)."""
    M = np.max(m, axis=-1, keepdims=True)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(m), l * np.exp(m - safe), 0.0)
    W = w.sum(axis=-1)
    num = (w[..., None] * acc).sum(axis=-2)
    out = np.where(W[..., None] > 0, num / np.where(W > 0, W, 1.0)[..., None], 0.0)
    return M[..., 0], W, out


def online_softmax_tiles(x: np.ndarray, V: np.ndarray, tile: int) -> np.ndarray:
    """One query row: logits x [L] (already scaled), values V [L, D].

    Walks the row in tiles of `tile` tokens with the update of the
    online-softmax fix: p = exp(s - m_ij); l_ij = sum p; m_i_new =
    max(m_i, m_ij); alpha = exp(m_i - m_i_new); beta = exp(m_ij - m_i_new);
    l_i_new = alpha l_i + beta l_ij; acc = acc (alpha l_i / l_i_new) +
    (p beta / l_i_new) @ V.  Starts from (m_i, l_i, acc) = (-inf, 0, 0).
    """
    L, D = V.shape
    m_i, l_i, acc = -np.inf, 0.0, np.zeros(D)
    for t0 in range(0, L, tile):
        s = x[t0:t0 + tile]
        m_ij = np.max(s)
        p = np.exp(s - m_ij)
        l_ij = p.sum()
        m_i_new = max(m_i, m_ij)
        alpha = np.exp(m_i - m_i_new)      # exp(-inf) = 0 on the first tile
        beta = np.exp(m_ij - m_i_new)
        l_i_new = alpha * l_i + beta * l_ij
        acc = acc * (alpha * l_i / l_i_new) + (p * beta / l_i_new) @ V[t0:t0 + tile]
        m_i, l_i = m_i_new, l_i_new
    return acc


def round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp64 -> f16/bf16 with a single round-to-nearest-even step.

    f16 uses numpy's direct double->half conversion.  bf16 (8 significant
    bits, 8 exponent bits like binary32) is rounded here from its definition:
    scale by the bf16 spacing at x's exponent, round half to even, scale back;
    the result is exact in float32 and so converts to bf16 exactly.
    (A cast through float32 would round twice.)
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return torch.from_numpy(np.ascontiguousarray(x.astype(np.float16)))
    if dtype != "bf16":
        raise ValueError(dtype)
    _, e = np.frexp(x)                       # x = f * 2**e, 0.5 <= |f| < 1
    k = np.maximum(e - 8, -133)              # spacing 2**k; bf16 subnormals step by 2**-133
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.round(np.ldexp(x, -k)), k)
        r = np.where(np.isfinite(x), r, x)
        r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, x), r)
    return torch.from_numpy(np.ascontiguousarray(r.astype(np.float32))).to(torch.bfloat16)
