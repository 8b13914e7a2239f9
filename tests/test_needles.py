"""Bit-exact block-table indexing through the real decode walks (GPU, C ABI).

Query head h is 32 in dimension h and zero elsewhere (24 heads, head_dim 256).
K is zero in dimensions 0..23 except at one needle token t per (sequence, query
head), where K[t, kv head h // 6, dim h] = 64.  With scale 1/16 the needle's logit
is exactly 128 and every other token's exactly 0.  In the exact result every other
weight is e^-128 (2.6e-56), so out = V[needle] + d with |d| < 1e-51 here, less
than half the spacing of f16 or bf16 at any value, zero included: rounded to the
dtype the exact answer is the needle's V row itself.  On the GPU the base-2
probability 2^-184.7 is 0 in fp32, and a partition without the needle enters the
merge with weight exactly 0, so out[s, h] must equal that row bit for bit (a
logit of 64 would not do for bf16, whose probabilities keep e^-64).  One call
checks 24 token positions per sequence; the
calls move the needles so that every 16-token tile of every sequence holds one,
at changing slots, the last token of each sequence included.

Every used page lies above 2^32 elements of the pool (64-bit offsets), page ids
are shuffled, the pages next to the used ones, unused table entries and the slots
past each sequence's end hold NaN.  The V rows carry (page % 256, page / 256 % 256,
slot, KV head) in dimensions 0..3, so a mismatch names the row actually read.

The walks covered: the length-balanced split (equal or XCD-paired shares, with and
without the per-sequence start cost, with the fused combine), automatic fixed
partitions paired across XCDs (equal lengths declared, odd partition count), the
pages' explicit 512-token partitions, and one pass per sequence.
"""
import math

import numpy as np
import pytest
import torch

import gqa_aware_paged_amd as pa
from helpers import say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 24, 4, 256
G = HQ // HKV
ALL_SINGLE = 1 << 30


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.empty_cache()


class NeedlePool:
    """Caches whose used pages all sit above 2^32 elements, with needle-ready K."""

    def __init__(self, lens, bs, dtype, seed):
        self.lens = np.asarray(lens, np.int64)
        self.bs = bs
        self.tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        S = len(lens)
        nblk = [-(-int(L) // bs) if L > 0 else 0 for L in lens]
        need = sum(nblk)
        p0 = -(-(1 << 32) // (HKV * bs * D))          # first page at or above 2^32 elements
        self.nb = p0 + need + 8
        rng = np.random.default_rng(seed)
        used = p0 + rng.permutation(need)
        trap = p0 - 1
        mb = max(max(nblk), 1)
        bt = np.full((S, mb), trap, np.int32)
        off = 0
        for s, n in enumerate(nblk):
            bt[s, :n] = used[off:off + n]
            off += n
        assert int(used.min()) * HKV * bs * D >= (1 << 32) if need else True
        self.bt_host = bt
        dev = "cuda"
        shape = (self.nb, HKV, bs, D)
        self.kc = torch.empty(shape, dtype=self.tdt, device=dev)
        self.vc = torch.empty(shape, dtype=self.tdt, device=dev)
        # NaN around the used range: below it (the trap page included) and above it
        for c in (self.kc, self.vc):
            c[p0 - 8:p0].fill_(float("nan"))
            c[p0 + need:].fill_(float("nan"))
        g = torch.Generator(device=dev).manual_seed(seed)
        up = torch.from_numpy(used.astype(np.int64)).to(dev)
        k = torch.randn((need, HKV, bs, D), generator=g, device=dev)
        k[..., :HQ] = 0.0
        v = torch.randn((need, HKV, bs, D), generator=g, device=dev)
        v[..., 0] = (up % 256).view(-1, 1, 1).float()
        v[..., 1] = ((up // 256) % 256).view(-1, 1, 1).float()
        v[..., 2] = torch.arange(bs, device=dev).view(1, 1, bs).float()
        v[..., 3] = torch.arange(HKV, device=dev).view(1, HKV, 1).float()
        self.kc[up] = k.to(self.tdt)
        self.vc[up] = v.to(self.tdt)
        # slots past each sequence's end in its last page
        for s, L in enumerate(lens):
            if L > 0 and L % bs:
                last = int(bt[s, nblk[s] - 1])
                self.kc[last, :, L % bs:] = float("nan")
                self.vc[last, :, L % bs:] = float("nan")
        self.bt = torch.from_numpy(bt).to(dev)
        self.sl = torch.from_numpy(self.lens.astype(np.int32)).to(dev)
        self.q = torch.zeros((S, HQ, D), dtype=self.tdt, device=dev)
        for h in range(HQ):
            self.q[:, h, h] = 32.0
        self.max_len = int(self.lens.max())
        self.tiles = [-(-int(L) // 16) if L > 0 else 0 for L in lens]

    def calls(self):
        return -(-max(self.tiles) // HQ)

    def needles(self, c):
        """(seq, head, token) of call c: head h of sequence s takes tile (24c + h) mod
        n_s at slot (7k + 5h + 3c) mod 16, clamped to the last token."""
        out = []
        for s, n in enumerate(self.tiles):
            if n == 0:
                continue
            for h in range(HQ):
                k = (c * HQ + h) % n
                t = min(16 * k + (7 * k + 5 * h + 3 * c) % 16, int(self.lens[s]) - 1)
                out.append((s, h, t))
        return out

    def _index(self, nd):
        s = np.array([x[0] for x in nd]); h = np.array([x[1] for x in nd])
        t = np.array([x[2] for x in nd])
        pages = self.bt_host[s, t // self.bs].astype(np.int64)
        cols = [torch.from_numpy(a.astype(np.int64)).cuda()
                for a in (pages, h // G, t % self.bs, h)]
        return s, h, cols

    def check(self, c, what, **kw):
        nd = self.needles(c)
        s, h, (pg, kv, sl, dm) = self._index(nd)
        self.kc[pg, kv, sl, dm] = 64.0
        out = pa.decode(self.q, self.kc, self.vc, self.bt, self.sl, 1.0 / 16,
                        max_seq_len=self.max_len, **kw)
        exp = torch.zeros_like(out)
        exp[torch.from_numpy(s).cuda(), torch.from_numpy(h).cuda()] = self.vc[pg, kv, sl]
        torch.cuda.synchronize()
        self.kc[pg, kv, sl, dm] = 0.0
        same = (out == exp).all(dim=-1).cpu().numpy()       # +0 == -0
        if not same.all():
            bad = np.argwhere(~same)[:4]
            msg = []
            for bs_, bh in bad:
                hit = [x for x in nd if x[0] == bs_ and x[1] == bh]
                got = out[bs_, bh, :4].float().cpu().tolist()
                msg.append(f"(s={bs_}, h={bh}, needle t={hit[0][2] if hit else None}) read "
                           f"[page%256, page/256%256, slot, kvh]={got}")
            raise AssertionError(f"{what} call {c}: {int((~same).sum())} rows wrong: "
                                 + "; ".join(msg))


MIXED = [4101, 2000, 528, 777, 1, 17, 300, 4100, 0, 64, 1500, 33]

BALANCED = {
    "equal-shares": dict(xcd_skew=-1, piece_cost=-1),
    "equal-shares+start-cost": dict(xcd_skew=-1, piece_cost=8),
    "xcd-paired": dict(xcd_skew=80, piece_cost=-1),
    "xcd-paired+start-cost": dict(xcd_skew=80, piece_cost=8),
    "xcd-paired+start-cost+fused": dict(xcd_skew=80, piece_cost=8, fused_combine=True),
}


@pytest.mark.parametrize("walk", [0, -1], ids=["streams", "piece-per-workgroup"])
@pytest.mark.parametrize("bs,dtype", [(8, "bf16"), (16, "f16"), (32, "bf16")])
def test_needles_every_tile_mixed_lengths(bs, dtype, walk):
    """walk 0: per-wave streams (wave ranges, pieces cut between waves and merged,
    partitions kept whole per share); -1: one workgroup per piece."""
    say(f"case needles mixed lengths bs={bs} {dtype} walk={walk}")
    pool = NeedlePool(MIXED, bs, dtype, seed=bs)
    lens = list(pool.lens)
    for name, kw in BALANCED.items():
        info = pa.plan(lens, HQ, HKV, D, bs, pool.bt_host.shape[1], pool.max_len, 0,
                       xcd_skew=kw["xcd_skew"], piece_cost=kw["piece_cost"],
                       fused_combine=kw.get("fused_combine", False), stream_walk=walk)
        assert info["balanced"] == 1 and info["partitioned_seqs"] >= 6, info
        say(f"  balanced {name}: {info['phase1_workgroups']} workgroups, "
            f"{info['partitioned_seqs']} sequences cut, streams {info['stream']}")
        for c in range(pool.calls()):
            pool.check(c, f"bs{bs}/balanced/{name}/walk{walk}", partition_size=0,
                       stream_walk=walk, **kw)
    for name, kw in {"p512": dict(partition_size=512, single_pass_max_len=0),
                     "p64": dict(partition_size=64, single_pass_max_len=0),
                     "p512-auto-tier": dict(partition_size=512),
                     "single-pass": dict(partition_size=512, single_pass_max_len=ALL_SINGLE)
                     }.items():
        say(f"  {name}")
        for c in range(pool.calls()):
            pool.check(c, f"bs{bs}/{name}/walk{walk}", stream_walk=walk, **kw)
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bs,dtype", [(8, "f16"), (16, "bf16"), (32, "f16")])
def test_needles_every_tile_paired_fixed_partitions(bs, dtype):
    """Equal lengths declared through the host-side total: automatic fixed partitions
    paired across XCD parities (a 16-token cut inside each pair), an odd partition
    count per sequence so the last one is unpaired."""
    say(f"case needles paired fixed partitions bs={bs} {dtype}")
    # 4000 tokens: 21 partitions of 192 (one workgroup per CU); 8-token pages plan two
    # per CU, and 4040 tokens give 43 partitions of 96
    lens = [4040 if bs == 8 else 4000] * 3
    pool = NeedlePool(lens, bs, dtype, seed=100 + bs)
    hint = sum(lens)
    for skew, fused in ((80, False), (500, False), (80, True)):
        info = pa.plan(lens, HQ, HKV, D, bs, pool.bt_host.shape[1], pool.max_len, 0,
                       total_tokens_hint=hint, xcd_skew=skew, fused_combine=fused)
        assert info["balanced"] == 0 and info["xcd_skew"] == skew, info
        assert info["max_partitions"] % 2 == 1 and info["max_partitions"] >= 3, info
        say(f"  skew {skew} fused {fused}: partitions of {info['partition_size']}, "
            f"{info['max_partitions']} per sequence")
        for c in range(pool.calls()):
            pool.check(c, f"bs{bs}/paired/{skew}/{fused}", partition_size=0,
                       total_tokens_hint=hint, xcd_skew=skew, fused_combine=fused)
    del pool
    torch.cuda.empty_cache()
