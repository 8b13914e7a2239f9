"""Seeded synthetic decode workloads for paged attention.

This module only draws random inputs; it contains none of the attention
arithmetic.  Both the CPU oracle (through the tests) and the GPU path consume
what it produces, so it imports neither of them.

Layouts (shared by every consumer):
  q            [num_seqs, num_heads, head_dim]                      f16 / bf16
  key_cache    [num_blocks, num_kv_heads, block_size, head_dim]     f16 / bf16
  value_cache  [num_blocks, num_kv_heads, block_size, head_dim]     f16 / bf16
  block_tables [num_seqs, max_blocks_per_seq]                       int32
  seq_lens     [num_seqs]                                           int32

Values are drawn as float32 N(0, 1) and rounded to the storage dtype with
round-to-nearest-even.  Physical page ids are a random permutation of the
pool, so no two logical blocks share a page unless a test asks for it.

The five named workloads follow the decode configurations the paged-attention
pages size their design for (one 100K-token sequence split into 200
partitions of 512 tokens, 24 query heads over 4 KV heads, head_dim 256,
16-token pages); their exact recipes are written out in each function.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor      # int32, same device as the caches
    seq_lens: torch.Tensor          # int32, same device as the caches
    seq_lens_host: np.ndarray       # int32 host copy
    block_tables_host: np.ndarray   # int32 host copy
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    partition_size: int
    dtype: str                      # "f16" | "bf16"
    trap_page: int = -1             # NaN-filled page used for unused table slots (or -1)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens_host.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables_host.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens_host.max()) if self.num_seqs else 0

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V that one decode step must read (exact tokens)."""
        esz = 2
        return int(np.clip(self.seq_lens_host, 0, None).astype(np.int64).sum()) * \
            self.num_kv_heads * self.head_dim * esz * 2

    def host_pages(self, seqs: Sequence[int]):
        """Compact host copy of the pages the given sequences reference.

        Returns (key_pool, value_pool, block_tables, seq_lens) on the CPU, with
        block-table entries renumbered into the compact pool.  Used to hand a
        bounded piece of a large device-resident workload to the CPU oracle.
        """
        seqs = list(seqs)
        bs = self.block_size
        nbs = [max(0, -(-int(self.seq_lens_host[s]) // bs)) for s in seqs]
        ids = np.concatenate([self.block_tables_host[s, :n] for s, n in zip(seqs, nbs)]) \
            if seqs else np.zeros(0, np.int64)
        uniq, inv = np.unique(ids.astype(np.int64), return_inverse=True)
        idx = torch.from_numpy(uniq).to(self.key_cache.device)
        kp = self.key_cache.index_select(0, idx).cpu()
        vp = self.value_cache.index_select(0, idx).cpu()
        mb = max(nbs) if nbs else 1
        bt = np.zeros((len(seqs), max(mb, 1)), np.int32)
        off = 0
        for i, n in enumerate(nbs):
            bt[i, :n] = inv[off:off + n]
            off += n
        sl = self.seq_lens_host[seqs].astype(np.int32)
        return kp, vp, bt, sl


def _normal(rng_or_gen, shape, device):
    """float32 N(0,1) of `shape`: numpy PCG64 on the CPU, torch's generator on a GPU."""
    if device == "cpu":
        return torch.from_numpy(rng_or_gen.standard_normal(shape, dtype=np.float32))
    out = torch.empty(shape, dtype=torch.float32, device=device)
    out.normal_(0.0, 1.0, generator=rng_or_gen)
    return out


def _fill_pool(pool: torch.Tensor, gen, device, outlier_frac: float, outlier_mult: float,
               seed: int):
    """Fill a [num_blocks, ...] pool in chunks with rounded N(0,1) values."""
    nb = pool.shape[0]
    per_page = int(np.prod(pool.shape[1:]))
    chunk = max(1, (1 << 26) // per_page)          # about 256 MB of float32 per chunk
    orng = np.random.Generator(np.random.PCG64(seed + 7)) if device == "cpu" else None
    ogen = None
    if device != "cpu" and outlier_frac > 0:
        ogen = torch.Generator(device=device)
        ogen.manual_seed(seed + 7)
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        x = _normal(gen, (b1 - b0,) + tuple(pool.shape[1:]), device)
        if outlier_frac > 0:
            if device == "cpu":
                u = torch.from_numpy(orng.random(x.shape, dtype=np.float32))
            else:
                u = torch.empty(x.shape, dtype=torch.float32, device=device)
                u.uniform_(0.0, 1.0, generator=ogen)
            x = torch.where(u < outlier_frac, x * outlier_mult, x)
        pool[b0:b1].copy_(x.to(pool.dtype))


def make_workload(name: str, seq_lens: Sequence[int], num_heads: int = 24,
                  num_kv_heads: int = 4, head_dim: int = 256, block_size: int = 16,
                  dtype: str = "f16", scale: Optional[float] = None,
                  partition_size: int = 512, pool_factor: float = 1.5,
                  num_blocks: Optional[int] = None, q_mult: float = 1.0,
                  outlier_frac: float = 0.0, outlier_mult: float = 20.0,
                  seed: int = 0, device: str = "cpu", poison: bool = False,
                  max_blocks_per_seq: Optional[int] = None,
                  shared_prefix_blocks: int = 0) -> Workload:
    """Build one seeded workload.

    poison=True writes NaN into every page no sequence references, into the
    slots past each sequence's length in its last page, and points unused
    block-table entries at a NaN page: a kernel that reads anything outside
    the tokens [0, seq_len) of its own pages then produces NaN.
    shared_prefix_blocks>0 makes every sequence's first blocks alias the same
    physical pages (legal read-only sharing).
    """
    tdt = DTYPES[dtype]
    lens = np.asarray(seq_lens, dtype=np.int64)
    S = len(lens)
    bs = block_size
    nblk = [max(0, -(-int(L) // bs)) for L in lens]
    need = sum(nblk) - max(0, S - 1) * min(shared_prefix_blocks, min(nblk) if nblk else 0)
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * max(need, 1))), 1) + (1 if poison else 0)
    mbps = max_blocks_per_seq or max(1, max(nblk) if nblk else 1)
    rng = np.random.Generator(np.random.PCG64(seed))
    if device == "cpu":
        gen = rng
    else:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed + 1000)

    # physical page assignment: a permutation of the pool; page perm[-1] is the trap page
    perm = rng.permutation(num_blocks).astype(np.int64)
    trap = int(perm[-1]) if poison else -1
    avail = perm[:-1] if poison else perm
    if need > len(avail):
        raise ValueError(f"pool of {num_blocks} pages cannot hold {need} pages")
    bt = np.full((S, mbps), trap if poison else 0, dtype=np.int32)
    cursor = 0
    shared = [int(x) for x in avail[:shared_prefix_blocks]] if shared_prefix_blocks else []
    cursor = len(shared)
    for s in range(S):
        k = 0
        if shared:
            k = min(len(shared), nblk[s])
            bt[s, :k] = shared[:k]
        m = nblk[s] - k
        bt[s, k:nblk[s]] = avail[cursor:cursor + m]
        cursor += m

    kv_shape = (num_blocks, num_kv_heads, bs, head_dim)
    kc = torch.empty(kv_shape, dtype=tdt, device=device)
    vc = torch.empty(kv_shape, dtype=tdt, device=device)
    _fill_pool(kc, gen, device, outlier_frac, outlier_mult, seed + 11)
    _fill_pool(vc, gen, device, outlier_frac, outlier_mult, seed + 13)
    q = (_normal(gen, (S, num_heads, head_dim), device) * q_mult).to(tdt)

    if poison:
        used = np.zeros(num_blocks, dtype=bool)
        for s in range(S):
            used[bt[s, :nblk[s]]] = True
        unused = torch.from_numpy(np.nonzero(~used)[0]).to(device)
        if unused.numel():
            kc.index_fill_(0, unused, float("nan"))
            vc.index_fill_(0, unused, float("nan"))
        for s in range(S):
            L = int(lens[s])
            if L > 0 and L % bs:
                last = int(bt[s, nblk[s] - 1])
                # a shared page may also be a non-last page of another sequence
                if shared and last in shared:
                    continue
                kc[last, :, L % bs:, :] = float("nan")
                vc[last, :, L % bs:, :] = float("nan")

    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    sl = lens.astype(np.int32)
    return Workload(name=name, q=q, key_cache=kc, value_cache=vc,
                    block_tables=torch.from_numpy(bt).to(device),
                    seq_lens=torch.from_numpy(sl).to(device),
                    seq_lens_host=sl, block_tables_host=bt,
                    num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    block_size=bs, scale=float(scale), partition_size=partition_size,
                    dtype=dtype, trap_page=trap)


# --------------------------------------------------------------------------
# The five named decode workloads.  Seeds are 1000 + id for lengths, tables
# and values.
# --------------------------------------------------------------------------

def tiny(device="cpu", poison=False, seed=1001):
    """1 seq x 1024 tokens, 24/4 heads, head_dim 256, 16-token pages, f16 N(0,1),
    scale 1/16, page ids a random permutation prefix of a 128-page pool, P=512."""
    return make_workload("tiny-1x1024", [1024], num_blocks=128 + (1 if poison else 0),
                         scale=1.0 / 16, partition_size=512, dtype="f16",
                         seed=seed, device=device, poison=poison)


def batch_lens(seed=1002):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(512, 8192, size=32, endpoint=True)


def batch(device="cpu", poison=False, seed=1002):
    """32 seqs, length uniform on [512, 8192], 24/4 heads, head_dim 256,
    16-token pages, f16 N(0,1), shared pool 1.5x the pages needed."""
    return make_workload("batch-32xU[512,8192]", batch_lens(seed), scale=1.0 / 16,
                         partition_size=512, dtype="f16", seed=seed, device=device,
                         poison=poison)


def long_context(device="cpu", poison=False, seed=1003, num_seqs=4, seq_len=102400,
                 head_dim=256, block_size=16):
    """4 seqs x 102400 tokens (200 partitions of 512), 24/4 heads, head_dim 256,
    16-token pages, f16; K, V ~ N(0,1); q = 8 N(0,1) so the softmax is peaked.
    head_dim and block_size may be changed for shape sweeps (scale 1/sqrt(head_dim))."""
    name = f"long-{num_seqs}x{seq_len}"
    if head_dim != 256 or block_size != 16:
        name += f"-D{head_dim}-bs{block_size}"
    return make_workload(name, [seq_len] * num_seqs, head_dim=head_dim, block_size=block_size,
                         scale=1.0 / math.sqrt(head_dim), partition_size=512, dtype="f16",
                         q_mult=8.0, seed=seed, device=device, poison=poison)


def mixed_lens(seed=1004, n=64):
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.uniform(math.log(64), math.log(65536), size=n)
    return np.clip(np.round(np.exp(u)), 64, 65536).astype(np.int64)


def mixed(device="cpu", poison=False, seed=1004, partition_size=512):
    """64 seqs, length log-uniform on [64, 65536], 24/4 heads, head_dim 256,
    16-token pages, bf16 N(0,1); partition size swept over {256, 512, 1024}."""
    return make_workload("mixed-64xlogU[64,65536]", mixed_lens(seed), scale=1.0 / 16,
                         partition_size=partition_size, dtype="bf16", seed=seed,
                         device=device, poison=poison)


def saturation(device="cpu", poison=False, seed=1005, num_seqs=256, seq_len=16384,
               num_blocks=150000):
    """256 seqs x 16384 tokens, 24/4 heads, head_dim 256, 32-token pages, f16
    N(0,1) with each K and V element independently x20 with probability 0.01,
    fully shuffled 150,000-page pool."""
    return make_workload(f"saturation-{num_seqs}x{seq_len}", [seq_len] * num_seqs,
                         block_size=32, num_blocks=num_blocks, scale=1.0 / 16,
                         partition_size=512, dtype="f16", outlier_frac=0.01,
                         outlier_mult=20.0, seed=seed, device=device, poison=poison)


@dataclasses.dataclass
class PrefillWorkload:
    """Prefill over a paged context: `ctx` holds the caches, block tables and
    context lengths (its seq_lens); the new tokens of every sequence are packed
    in q [T, Hq, D], k_new and v_new [T, Hkv, D], sequence s owning rows
    query_start[s] .. query_start[s+1]-1."""
    name: str
    ctx: Workload
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    query_start: torch.Tensor
    query_start_host: np.ndarray
    q_lens_host: np.ndarray

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_host[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens_host.max()) if len(self.q_lens_host) else 0


def make_prefill(name: str, ctx_lens: Sequence[int], q_lens: Sequence[int],
                 num_heads: int = 24, num_kv_heads: int = 4, head_dim: int = 256,
                 block_size: int = 16, dtype: str = "f16", scale: Optional[float] = None,
                 seed: int = 0, device: str = "cpu", poison: bool = False,
                 pool_factor: float = 1.5) -> PrefillWorkload:
    """Seeded prefill workload: the context part is make_workload(ctx_lens) (a
    context length of 0 gives a sequence with no cached tokens); the new tokens'
    q, k and v are N(0,1) rounded to the dtype."""
    ctx = make_workload(name, ctx_lens, num_heads=num_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, block_size=block_size, dtype=dtype, scale=scale,
                        seed=seed, device=device, poison=poison, pool_factor=pool_factor)
    ql = np.asarray(q_lens, dtype=np.int64)
    assert len(ql) == len(ctx_lens) and (ql >= 0).all()
    qs = np.zeros(len(ql) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(ql)
    T = int(qs[-1])
    tdt = DTYPES[dtype]
    if device == "cpu":
        gen = np.random.Generator(np.random.PCG64(seed + 500))
    else:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed + 1500)
    q = _normal(gen, (T, num_heads, head_dim), device).to(tdt)
    kn = _normal(gen, (T, num_kv_heads, head_dim), device).to(tdt)
    vn = _normal(gen, (T, num_kv_heads, head_dim), device).to(tdt)
    return PrefillWorkload(name=name, ctx=ctx, q=q, k_new=kn, v_new=vn,
                           query_start=torch.from_numpy(qs).to(device), query_start_host=qs,
                           q_lens_host=ql)


def prefill_chunk(device="cpu", poison=False, seed=1006, num_seqs=4, ctx_len=16384,
                  q_len=2048, head_dim=256, dtype="f16", block_size=16):
    """Chunked prefill: 4 sequences with 16384 cached context tokens each and a
    2048-token new chunk, 24/4 heads, head_dim 256, 16-token pages, f16 N(0,1),
    scale 1/sqrt(head_dim) (1/16); head_dim, dtype and block_size can be varied."""
    name = f"prefill-{num_seqs}x({ctx_len}+{q_len})"
    if (head_dim, dtype, block_size) != (256, "f16", 16):
        name += f"-D{head_dim}-{dtype}-bs{block_size}"
    return make_prefill(name, [ctx_len] * num_seqs, [q_len] * num_seqs, head_dim=head_dim,
                        block_size=block_size, dtype=dtype, scale=1.0 / math.sqrt(head_dim),
                        seed=seed, device=device, poison=poison)


NAMED = {"tiny": tiny, "batch": batch, "long": long_context, "mixed": mixed,
         "saturation": saturation}
