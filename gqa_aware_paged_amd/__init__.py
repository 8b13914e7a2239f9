"""Python binding of libpagedattn (GQA-grouped paged-attention decode on MI355X).

Argument marshalling only: every step of the decode runs in the HIP kernels of
libpagedattn.so.  torch provides device memory and the current stream.  There
is no fallback: if the library is not built, or a call is rejected, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedattn.so")

PA_F16, PA_BF16 = 0, 1
_DTYPE = {torch.float16: PA_F16, torch.bfloat16: PA_BF16}
SYMBOLS = ("paged_attn_workspace_size", "paged_attn_workspace_size_ex", "paged_attn_decode",
           "paged_attn_decode_ex", "paged_attn_status_str", "paged_attn_plan",
           "paged_attn_gather_probe", "paged_attn_workspace_init", "paged_attn_prefill",
           "paged_attn_decode_noalloc", "paged_attn_read_probe")


class Options(ctypes.Structure):
    _fields_ = [("single_pass_max_len", ctypes.c_int), ("num_cus", ctypes.c_int),
                ("total_tokens_hint", ctypes.c_longlong), ("per_query_head", ctypes.c_int),
                ("fused_combine", ctypes.c_int), ("xcd_skew", ctypes.c_int),
                ("piece_cost", ctypes.c_int),
                ("phase1_begin", ctypes.c_void_p), ("phase1_end", ctypes.c_void_p),
                ("stream_walk", ctypes.c_int), ("head_sequential", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("partition_size", ctypes.c_int), ("single_pass_max_len", ctypes.c_int),
                ("max_partitions", ctypes.c_int), ("group", ctypes.c_int),
                ("phase1_workgroups", ctypes.c_longlong),
                ("phase2_workgroups", ctypes.c_longlong),
                ("active_workgroups", ctypes.c_longlong), ("single_pass_seqs", ctypes.c_int),
                ("partitioned_seqs", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t),
                ("threads_per_workgroup", ctypes.c_int), ("lds_bytes_phase1", ctypes.c_int),
                ("balanced", ctypes.c_int), ("fused", ctypes.c_int),
                ("xcd_skew", ctypes.c_int), ("piece_cost", ctypes.c_int),
                ("stream", ctypes.c_int), ("head_sequential", ctypes.c_int),
                ("reduce_slices", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpagedattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gqa_aware_paged_amd.build` "
                               "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.paged_attn_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        L.paged_attn_workspace_size.restype = Z
        L.paged_attn_workspace_size_ex.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(Options)]
        L.paged_attn_workspace_size_ex.restype = Z
        dec = [P, P, P, P, P, P, I, I, I, I, I, F, I, P, P, I, I, I, Z]
        L.paged_attn_decode.argtypes = dec
        L.paged_attn_decode.restype = I
        L.paged_attn_decode_ex.argtypes = dec + [ctypes.POINTER(Options)]
        L.paged_attn_decode_ex.restype = I
        L.paged_attn_status_str.argtypes = [I]
        L.paged_attn_status_str.restype = ctypes.c_char_p
        L.paged_attn_plan.argtypes = [P, I, I, I, I, I, I, I, I, I, ctypes.POINTER(Options),
                                      ctypes.POINTER(PlanInfo)]
        L.paged_attn_plan.restype = I
        L.paged_attn_gather_probe.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
        L.paged_attn_gather_probe.restype = I
        L.paged_attn_workspace_init.argtypes = [P, Z, P]
        L.paged_attn_workspace_init.restype = I
        L.paged_attn_prefill.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I,
                                         I, P]
        L.paged_attn_prefill.restype = I
        L.paged_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P, I, I, I]
        L.paged_attn_decode_noalloc.restype = I
        L.paged_attn_read_probe.argtypes = [P, Z, P, ctypes.c_longlong, I, P, P]
        L.paged_attn_read_probe.restype = I
        _lib = L
    return _lib


class PagedAttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(lib().paged_attn_status_str(status).decode())


def _check(status: int):
    if status != 0:
        raise PagedAttnError(status)


def _opts(single_pass_max_len: Optional[int], num_cus: int = 0,
          events: Optional[Tuple[int, int]] = None, total_tokens_hint: int = 0,
          per_query_head: bool = False, fused_combine: bool = False,
          xcd_skew: int = 0, piece_cost: int = 0, stream_walk: int = 0,
          head_sequential: bool = False) -> Options:
    o = Options()
    o.stream_walk = int(stream_walk)
    o.head_sequential = 1 if head_sequential else 0
    o.xcd_skew = int(xcd_skew)
    o.piece_cost = int(piece_cost)
    o.per_query_head = 1 if per_query_head else 0
    o.fused_combine = 1 if fused_combine else 0
    o.single_pass_max_len = -1 if single_pass_max_len is None else int(single_pass_max_len)
    o.num_cus = int(num_cus)
    o.total_tokens_hint = int(total_tokens_hint)
    if events is not None:
        o.phase1_begin, o.phase1_end = events
    return o


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def plan(seq_lens_host, num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
         max_blocks_per_seq: int, max_seq_len: int = 0, partition_size: int = 0,
         dtype: int = PA_F16, single_pass_max_len: Optional[int] = None,
         num_seqs: Optional[int] = None, num_cus: int = 0, total_tokens_hint: int = 0,
         per_query_head: bool = False, fused_combine: bool = False,
         xcd_skew: int = 0, piece_cost: int = 0, stream_walk: int = 0,
         head_sequential: bool = False) -> dict:
    """Host-only plan (no GPU needed).  seq_lens_host: sequence of ints or None."""
    arr = None
    if seq_lens_host is not None:
        n = len(seq_lens_host)
        arr = (ctypes.c_int32 * n)(*[int(x) for x in seq_lens_host])
        num_seqs = n
    info = PlanInfo()
    o = _opts(single_pass_max_len, num_cus, total_tokens_hint=total_tokens_hint,
              per_query_head=per_query_head, fused_combine=fused_combine, xcd_skew=xcd_skew,
              piece_cost=piece_cost, stream_walk=stream_walk, head_sequential=head_sequential)
    _check(lib().paged_attn_plan(arr, int(num_seqs or 0), num_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, max_seq_len, partition_size,
                                 dtype, ctypes.byref(o), ctypes.byref(info)))
    return info.as_dict()


def workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                   block_size: int, max_blocks_per_seq: int, max_seq_len: int = 0,
                   partition_size: int = 0, single_pass_max_len: Optional[int] = None,
                   total_tokens_hint: int = 0, num_cus: int = 0,
                   per_query_head: bool = False, stream_walk: int = 0,
                   fused_combine: bool = False, head_sequential: bool = False) -> int:
    o = _opts(single_pass_max_len, num_cus, total_tokens_hint=total_tokens_hint,
              per_query_head=per_query_head, stream_walk=stream_walk,
              fused_combine=fused_combine, head_sequential=head_sequential)
    n = lib().paged_attn_workspace_size_ex(num_seqs, num_heads, num_kv_heads, head_dim,
                                           block_size, max_blocks_per_seq, max_seq_len,
                                           partition_size, ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("paged_attn_workspace_size rejected the sizes")
    return int(n)


def workspace_init(workspace: torch.Tensor, stream: Optional[int] = None) -> None:
    """Clear the ticket area of a workspace for the fused combine (enqueued on
    `stream`, default the current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    _check(lib().paged_attn_workspace_init(_ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           ctypes.c_void_p(stream)))


class Decoder:
    """Holds the workspace of one decode configuration so the hot call allocates nothing.

    Mirrors the caller-owned workspace of the C ABI: allocate once, then call
    `__call__` every step.  With fused_combine the workspace's ticket area is
    cleared once here; every completed call leaves it clear.
    """

    def __init__(self, num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, max_blocks_per_seq: int, dtype: torch.dtype,
                 max_seq_len: int = 0, partition_size: int = 0,
                 single_pass_max_len: Optional[int] = None, total_tokens_hint: int = 0,
                 num_cus: int = 0, per_query_head: bool = False,
                 fused_combine: bool = False, xcd_skew: int = 0, piece_cost: int = 0,
                 stream_walk: int = 0, head_sequential: bool = False, device="cuda"):
        self.shape = (num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq)
        self.dtype = dtype
        self.max_seq_len = int(max_seq_len)
        self.partition_size = int(partition_size)
        self.opts = _opts(single_pass_max_len, num_cus, total_tokens_hint=total_tokens_hint,
                          per_query_head=per_query_head, fused_combine=fused_combine,
                          xcd_skew=xcd_skew, piece_cost=piece_cost, stream_walk=stream_walk,
                          head_sequential=head_sequential)
        nbytes = workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, max_seq_len, partition_size,
                                single_pass_max_len, total_tokens_hint, num_cus,
                                per_query_head, stream_walk, fused_combine, head_sequential)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.workspace_bytes = nbytes
        if fused_combine and nbytes > 0:
            workspace_init(self.workspace)
        self.out = torch.empty((num_seqs, num_heads, head_dim), dtype=dtype, device=device)

    def __call__(self, q, key_cache, value_cache, block_tables, seq_lens, scale: float,
                 out: Optional[torch.Tensor] = None, events: Optional[Tuple[int, int]] = None,
                 stream: Optional[int] = None) -> torch.Tensor:
        S, Hq, Hkv, D, bs, mbps = self.shape
        out = self.out if out is None else out
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        o = self.opts
        if events is not None:
            o = Options.from_buffer_copy(self.opts)
            o.phase1_begin, o.phase1_end = events
        _check(lib().paged_attn_decode_ex(
            _ptr(out), _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(seq_lens), S, Hq, Hkv, D, bs, float(scale), self.partition_size,
            _ptr(self.workspace), ctypes.c_void_p(stream), mbps, self.max_seq_len,
            _DTYPE[self.dtype], self.workspace_bytes, ctypes.byref(o)))
        return out


def _validate(q, key_cache, value_cache, block_tables, seq_lens):
    for name, t in (("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _DTYPE or key_cache.dtype != q.dtype or value_cache.dtype != q.dtype:
        raise ValueError("q, key_cache and value_cache must share dtype float16 or bfloat16")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if key_cache.shape != value_cache.shape or key_cache.dim() != 4 or q.dim() != 3:
        raise ValueError("q [S,Hq,D]; caches [num_blocks,Hkv,block_size,D]")


def decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
           partition_size: int = 0, max_seq_len: int = 0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, single_pass_max_len: Optional[int] = None,
           events: Optional[Tuple[int, int]] = None, total_tokens_hint: int = 0,
           per_query_head: bool = False, fused_combine: bool = False,
           xcd_skew: int = 0, piece_cost: int = 0, stream_walk: int = 0,
           head_sequential: bool = False) -> torch.Tensor:
    """One decode step: out[s,h] = softmax(scale q K^T) V over the paged caches.

    fused_combine: merge partitions inside phase 1; a workspace passed in must then
    have a clear ticket area (workspace_init, or a previous fused call)."""
    _validate(q, key_cache, value_cache, block_tables, seq_lens)
    S, Hq, D = q.shape
    _, Hkv, bs, _ = key_cache.shape
    mbps = block_tables.shape[1]
    need = workspace_size(S, Hq, Hkv, D, bs, mbps, max_seq_len, partition_size,
                          single_pass_max_len, total_tokens_hint, 0, per_query_head,
                          stream_walk, fused_combine, head_sequential)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if fused_combine:
            workspace_init(workspace)
    if out is None:
        out = torch.empty_like(q)
    o = _opts(single_pass_max_len, events=events, total_tokens_hint=total_tokens_hint,
              per_query_head=per_query_head, fused_combine=fused_combine, xcd_skew=xcd_skew,
              piece_cost=piece_cost, stream_walk=stream_walk, head_sequential=head_sequential)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().paged_attn_decode_ex(
        _ptr(out), _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(seq_lens), S, Hq, Hkv, D, bs, float(scale), int(partition_size), _ptr(workspace),
        ctypes.c_void_p(stream), mbps, int(max_seq_len), _DTYPE[q.dtype],
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        ctypes.byref(o)))
    return out


def decode_noalloc(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                   out: torch.Tensor, partition_size: int = 0, max_seq_len: int = 0,
                   stream: Optional[int] = None) -> torch.Tensor:
    """paged_attn_decode_noalloc: one decode step with the library's device-resident
    workspace (no allocation in the call; `out` is the caller's).  Calls that overlap
    on one GPU share that workspace and must be serialised by the caller."""
    _validate(q, key_cache, value_cache, block_tables, seq_lens)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    S, Hq, D = q.shape
    _, Hkv, bs, _ = key_cache.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().paged_attn_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(seq_lens), S, Hq, Hkv, D, bs, float(scale), int(partition_size),
        ctypes.c_void_p(stream), block_tables.shape[1], int(max_seq_len), _DTYPE[q.dtype]))
    return out


def prefill(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
            key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
            ctx_lens: torch.Tensor, query_start: torch.Tensor, scale: float,
            max_query_len: int, max_ctx_len: int, out: Optional[torch.Tensor] = None,
            stream: Optional[int] = None) -> torch.Tensor:
    """Prefill over a paged context: new token n of sequence s (row query_start[s] + n
    of q, k_new, v_new) attends to the ctx_lens[s] cached tokens and causally to
    the new tokens up to itself.  max_query_len / max_ctx_len are host-side bounds."""
    _validate(q, key_cache, value_cache, block_tables, ctx_lens)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("query_start", query_start)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype or query_start.dtype != torch.int32:
        raise ValueError("k_new/v_new share q's dtype; query_start is int32")
    T, Hq, D = q.shape
    _, Hkv, bs, _ = key_cache.shape
    S = ctx_lens.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != k_new.shape or query_start.shape != (S + 1,):
        raise ValueError("k_new/v_new [T, Hkv, D]; query_start [S+1]")
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().paged_attn_prefill(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(key_cache), _ptr(value_cache),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(query_start), S, Hq, Hkv, D, bs, float(scale),
        block_tables.shape[1], int(max_query_len) if T > 0 else 0, int(max_ctx_len),
        _DTYPE[q.dtype],
        ctypes.c_void_p(stream)))
    return out


def read_probe(src: torch.Tensor, chunk_bytes: int, order: Optional[torch.Tensor] = None,
               num_workgroups: int = 256, sink: Optional[torch.Tensor] = None,
               stream: Optional[int] = None) -> torch.Tensor:
    """Read every chunk of `src` (a device tensor of whole chunks) once, in order or
    in the order of `order` (device int64 permutation of the chunk indices); returns
    the per-workgroup XOR folds."""
    nbytes = src.numel() * src.element_size()
    if nbytes % chunk_bytes:
        raise ValueError("src must hold whole chunks")
    n = nbytes // chunk_bytes
    if order is not None:
        if order.dtype != torch.int64 or order.numel() != n or not order.is_cuda:
            raise ValueError("order must be a device int64 tensor with one entry per chunk")
    if sink is None:
        sink = torch.empty(num_workgroups, dtype=torch.int32, device=src.device)
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    _check(lib().paged_attn_read_probe(_ptr(src), chunk_bytes, _ptr(order), n, num_workgroups,
                                       _ptr(sink), ctypes.c_void_p(stream)))
    return sink


def gather_probe(key_cache: torch.Tensor, value_cache: torch.Tensor,
                 block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int):
    """Contiguous [S, Hkv, max_seq_len, D] copies of the K and V rows of tokens
    t < seq_len, gathered by the phase-1 addressing (slots past seq_len untouched,
    here zero-initialised)."""
    S = seq_lens.shape[0]
    _, Hkv, bs, D = key_cache.shape
    k_out = torch.zeros((S, Hkv, max_seq_len, D), dtype=key_cache.dtype, device=key_cache.device)
    v_out = torch.zeros_like(k_out)
    stream = torch.cuda.current_stream(key_cache.device).cuda_stream
    _check(lib().paged_attn_gather_probe(_ptr(k_out), _ptr(v_out), _ptr(key_cache),
                                         _ptr(value_cache), _ptr(block_tables), _ptr(seq_lens),
                                         S, Hkv, D, bs, block_tables.shape[1], int(max_seq_len),
                                         ctypes.c_void_p(stream)))
    return k_out, v_out
