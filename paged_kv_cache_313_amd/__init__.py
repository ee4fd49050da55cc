"""paged_kv_cache_313_amd -- PagedAttention's decode hot path for AMD MI355X.

Thin Python binding over ``libpagedkv.so`` (C ABI in ``include/pa.h`` and
``include/pa_block_manager.h``).  The functions here only marshal torch device
tensors into pointers and sizes and pass the current HIP stream; every step of
the path runs in the library's HIP kernels, and block allocation in its native
block manager (``BlockManager``).  There is no CPU or PyTorch fallback: if the library is missing or a
tensor is not on the GPU, the call raises.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import PA_PARTITION_BALANCED, PagedKVError, load  # noqa: F401
from .block_manager import BlockManager  # noqa: F401

__all__ = ["kv_append", "block_copy", "decode_attention", "decode_attention_noalloc", "prefill_attention",
           "decode_attention_hier",
           "prefill_attention_hier", "decode_workspace_bytes",
           "choose_partition", "swap_out", "swap_in", "swap_buffer", "stream_read", "PagedKVError", "load",
           "PA_PARTITION_BALANCED", "BlockManager", "debug_violations",
           "decode_attention_grouped", "prefix_groups"]

_DTYPES = {torch.float32: _lib.PA_F32, torch.float16: _lib.PA_F16, torch.bfloat16: _lib.PA_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libpagedkv has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check_out(out: torch.Tensor, query: torch.Tensor) -> None:
    """A caller-supplied output must have the query's shape, dtype and device:
    the kernels write exactly query.numel() elements of the query's dtype."""
    if not isinstance(out, torch.Tensor):
        raise TypeError("out must be a torch.Tensor")
    if tuple(out.shape) != tuple(query.shape) or out.dtype != query.dtype or out.device != query.device:
        raise ValueError(f"out must match the query: shape {tuple(query.shape)}, dtype {query.dtype}, device "
                         f"{query.device} (got {tuple(out.shape)}, {out.dtype}, {out.device})")


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def kv_append(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
              slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter ``key``/``value`` [T, Hkv, D] into the pools [NB, Hkv, bs, D] at
    ``slot_mapping`` (int64 [T], < 0 = skip)."""
    lib = load()
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    NB, Hkv, bs, D = k_pool.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or value.shape != key.shape or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch between key/value [T, Hkv, D] and pools [NB, Hkv, bs, D]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    if not (key.dtype == value.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("key, value and pools must share a dtype")
    st = lib.pa_kv_append(_dev(key, "key"), _dev(value, "value"), _dev(k_pool, "k_pool"),
                          _dev(v_pool, "v_pool"), _dev(slot_mapping, "slot_mapping"), T, Hkv, D, bs,
                          NB, _dtype_code(k_pool), _stream(k_pool, stream))
    _lib.check("pa_kv_append", st)


def block_copy(k_pool: torch.Tensor, v_pool: torch.Tensor, block_mapping: torch.Tensor,
               stream=None) -> None:
    """Copy-on-write: for each (src, dst) row of ``block_mapping`` (int32
    [N, 2]), block dst of both pools becomes a copy of block src."""
    lib = load()
    if block_mapping.dtype != torch.int32:
        raise TypeError("block_mapping must be int32")
    NB, Hkv, bs, D = k_pool.shape
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must match")
    N = block_mapping.numel() // 2
    if block_mapping.numel() != 2 * N:
        raise ValueError("block_mapping must be [N, 2]")
    st = lib.pa_block_copy(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                           _dev(block_mapping, "block_mapping"), N, Hkv, bs, D, NB,
                           _dtype_code(k_pool), _stream(k_pool, stream))
    _lib.check("pa_block_copy", st)


def _swap_args(k_pool, v_pool, block_ids, host):
    if block_ids.dtype != torch.int32:
        raise TypeError("block_ids must be int32")
    NB, Hkv, bs, D = k_pool.shape
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must match")
    n = block_ids.numel()
    if not isinstance(host, torch.Tensor) or host.is_cuda or not host.is_pinned():
        raise ValueError("host must be a pinned CPU tensor (pin_memory=True)")
    if not host.is_contiguous() or host.dtype != k_pool.dtype:
        raise ValueError("host must be contiguous and of the pools' dtype")
    if host.numel() < n * 2 * Hkv * bs * D:
        raise ValueError("host buffer smaller than [num_ids, 2, Hkv, bs, D]")
    return NB, Hkv, bs, D, n


def swap_buffer(num_ids: int, k_pool: torch.Tensor) -> torch.Tensor:
    """A pinned host buffer [num_ids, 2, Hkv, bs, D] for pa_swap_out / pa_swap_in."""
    NB, Hkv, bs, D = k_pool.shape
    return torch.empty((num_ids, 2, Hkv, bs, D), dtype=k_pool.dtype, pin_memory=True)


def swap_out(k_pool: torch.Tensor, v_pool: torch.Tensor, block_ids: torch.Tensor, host: torch.Tensor,
             stream=None) -> None:
    """Copy blocks ``block_ids`` (device int32 [n]) of both pools into the
    pinned, block-first host buffer ``host`` [n, 2, Hkv, bs, D] (K then V)."""
    lib = load()
    NB, Hkv, bs, D, n = _swap_args(k_pool, v_pool, block_ids, host)
    st = lib.pa_swap_out(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(block_ids, "block_ids"), n,
                         host.data_ptr(), Hkv, bs, D, NB, _dtype_code(k_pool), _stream(k_pool, stream))
    _lib.check("pa_swap_out", st)


def swap_in(host: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_ids: torch.Tensor,
            stream=None) -> None:
    """Write entry i of the pinned block-first host buffer into block
    ``block_ids[i]`` of both pools."""
    lib = load()
    NB, Hkv, bs, D, n = _swap_args(k_pool, v_pool, block_ids, host)
    st = lib.pa_swap_in(host.data_ptr(), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                        _dev(block_ids, "block_ids"), n, Hkv, bs, D, NB, _dtype_code(k_pool),
                        _stream(k_pool, stream))
    _lib.check("pa_swap_in", st)


def stream_read(buf: torch.Tensor, partials: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Measurement aid: read every byte of the contiguous device tensor
    ``buf`` once (pa_stream_read) and return the device uint32-valued int32
    tensor of per-workgroup XOR partials [PA_STREAM_READ_PARTIALS]."""
    lib = load()
    nbytes = buf.numel() * buf.element_size()
    if partials is None:
        partials = torch.empty(_lib.PA_STREAM_READ_PARTIALS, dtype=torch.int32, device=buf.device)
    if partials.dtype != torch.int32 or partials.numel() < _lib.PA_STREAM_READ_PARTIALS:
        raise ValueError(f"partials must be int32 with at least {_lib.PA_STREAM_READ_PARTIALS} entries")
    st = lib.pa_stream_read(_dev(buf, "buf"), nbytes, _dev(partials, "partials"), _stream(buf, stream))
    _lib.check("pa_stream_read", st)
    return partials


def debug_violations(clear: bool = True) -> int:
    """The PA_VIOLATION_* bits the kernels of a checked build (PA_DEBUG_CHECKS)
    met since the last clear; synchronises the device.  The normal build
    raises PagedKVError (PA_ERR_UNSUPPORTED)."""
    import ctypes
    flags = ctypes.c_uint32(0)
    _lib.check("pa_debug_violations", load().pa_debug_violations(ctypes.byref(flags), 1 if clear else 0))
    return int(flags.value)


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, partition_size: int) -> int:
    n = load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len, partition_size)
    if n == (1 << 64) - 1:
        raise ValueError("invalid arguments to pa_decode_workspace_bytes")
    return int(n)


def choose_partition(num_seqs: int, num_kv_heads: int, max_context_len: int, block_size: int) -> int:
    return int(load().pa_decode_choose_partition(num_seqs, num_kv_heads, max_context_len, block_size))


def decode_attention(query: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                     max_context_len: int, partition_size: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Single-query decode attention over the paged pools.

    query [S, Hq, D]; pools [NB, Hkv, bs, D]; block_tables int32 [S, MB];
    context_lens int32 [S]; ``max_context_len`` is a host-side upper bound of
    ``context_lens``.  ``partition_size``: 0 = no split, P > 0 = fixed
    P-token partitions, PA_PARTITION_BALANCED = balanced split, None = the
    library's choice.
    Returns ``out`` [S, Hq, D] in the query's dtype.
    """
    lib = load()
    S, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, max_blocks_per_seq] and context_lens [S]")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if partition_size is None:
        partition_size = choose_partition(S, Hkv, max_context_len, bs)
    if out is None:
        out = torch.empty_like(query)
    else:
        _check_out(out, query)
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pa_decode_attention(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                 _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                 _dev(context_lens, "context_lens"), S, Hq, Hkv, D, bs,
                                 block_tables.shape[1], NB, int(max_context_len), float(scale),
                                 int(partition_size), _dtype_code(query), ws_ptr, ws_bytes,
                                 _stream(query, stream))
    _lib.check("pa_decode_attention", st)
    return out


def decode_attention_grouped(query: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor, group_start: torch.Tensor,
                             group_shared: torch.Tensor, max_group_size: int, max_shared_len: int, scale: float,
                             max_context_len: int, partition_size: int = 512, out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_attention with fixed ``partition_size``-token partitions for a
    batch whose consecutive sequences share a prefix's blocks: group i is
    sequences group_start[i] .. group_start[i+1] - 1 (int32 [G + 1] on the
    GPU), whose first group_shared[i] tokens (int32 [G]) map to the same
    blocks.  ``max_group_size`` and ``max_shared_len`` are host bounds of the
    group sizes and of group_shared.  Same results as decode_attention with
    that partition size; see prefix_groups for deriving the groups."""
    lib = load()
    S, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"), (group_start, "group_start"),
                    (group_shared, "group_shared")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, max_blocks_per_seq] and context_lens [S]")
    G = group_shared.numel()
    if group_start.numel() != G + 1:
        raise ValueError("group_start must have one entry more than group_shared")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if out is None:
        out = torch.empty_like(query)
    else:
        _check_out(out, query)
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pa_decode_attention_grouped(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                         _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                         _dev(context_lens, "context_lens"), _dev(group_start, "group_start"),
                                         _dev(group_shared, "group_shared"), G, int(max_group_size),
                                         int(max_shared_len), S, Hq, Hkv, D, bs, block_tables.shape[1], NB,
                                         int(max_context_len), float(scale), int(partition_size),
                                         _dtype_code(query), ws_ptr, ws_bytes, _stream(query, stream))
    _lib.check("pa_decode_attention_grouped", st)
    return out


def prefix_groups(block_tables, context_lens, block_size: int, min_shared_blocks: int = 1):
    """Host helper: runs of consecutive sequences whose tables start with the
    same physical blocks (numpy int32 [S, MB] and [S]).  Returns
    (group_start int32 [G + 1], group_shared int32 [G] in tokens): a run
    holds the sequences that share at least ``min_shared_blocks`` leading
    blocks of their valid entries with the run's first sequence, and its
    shared length is the longest such common block prefix of all of them;
    a sequence that shares nothing with its neighbour is a group of one with
    no shared tokens."""
    import numpy as np
    tables = np.asarray(block_tables, dtype=np.int32)
    lens = np.asarray(context_lens, dtype=np.int64)
    S = tables.shape[0]
    nblk = (lens + block_size - 1) // block_size

    def common(a, b):   # leading valid blocks that sequences a and b both map to the same ids
        n = int(min(nblk[a], nblk[b]))
        diff = np.flatnonzero(tables[a, :n] != tables[b, :n])
        return int(diff[0]) if diff.size else n

    starts, shared = [0], []
    run = int(nblk[0]) if S else 0
    for s in range(1, S):
        c = min(common(starts[-1], s), run)
        if c >= min_shared_blocks:
            run = c
            continue
        shared.append(run * block_size if s - starts[-1] > 1 else 0)
        starts.append(s)
        run = int(nblk[s])
    if S:
        shared.append(run * block_size if S - starts[-1] > 1 else 0)
        starts.append(S)
    return np.asarray(starts, dtype=np.int32), np.asarray(shared, dtype=np.int32)


def decode_attention_noalloc(query: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                             max_context_len: int, partition_size: Optional[int] = None,
                             out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """decode_attention through pa_decode_attention_noalloc: no workspace
    argument, the split's partial results go to the library's static device
    scratch (PA_DECODE_SCRATCH_BYTES per GPU; calls on one GPU must not
    overlap).  ``out`` must be given (the call itself allocates nothing)."""
    lib = load()
    S, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, max_blocks_per_seq] and context_lens [S]")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if out is None:
        raise ValueError("decode_attention_noalloc needs a caller-allocated out")
    _check_out(out, query)
    if partition_size is None:
        partition_size = choose_partition(S, Hkv, max_context_len, bs)
    st = lib.pa_decode_attention_noalloc(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                         _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                         _dev(context_lens, "context_lens"), S, Hq, Hkv, D, bs,
                                         block_tables.shape[1], NB, int(max_context_len), float(scale),
                                         int(partition_size), _dtype_code(query), _stream(query, stream))
    _lib.check("pa_decode_attention_noalloc", st)
    return out


def prefill_attention(query: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
                      scale: float, max_query_len: int, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Causal attention of the packed new tokens ``query`` [T, Hq, D] over
    their sequences' paged contexts.  ``query_start`` int32 [S + 1] packs the
    sequences' new tokens; sequence s's are the last
    query_start[s+1] - query_start[s] of its context_lens[s] tokens (already
    appended).  ``max_query_len`` bounds the per-sequence count.  f16/bf16."""
    lib = load()
    T, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    S = context_lens.numel()
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"), (query_start, "query_start")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables must be [S, max_blocks_per_seq] and query_start [S + 1]")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if out is None:
        out = torch.empty_like(query)
    else:
        _check_out(out, query)
    st = lib.pa_prefill_attention(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                  _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                  _dev(context_lens, "context_lens"), _dev(query_start, "query_start"), S, T,
                                  Hq, Hkv, D, bs, block_tables.shape[1], NB, int(max_query_len), float(scale),
                                  _dtype_code(query), _stream(query, stream))
    _lib.check("pa_prefill_attention", st)
    return out


def _hier_args(small_tables, large_tables, num_large, S):
    for t, name in ((small_tables, "small_tables"), (large_tables, "large_tables"), (num_large, "num_large")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if (small_tables.dim() != 2 or large_tables.dim() != 2 or small_tables.shape[0] != S
            or large_tables.shape[0] != S or num_large.numel() != S):
        raise ValueError("small_tables [S, MS], large_tables [S, ML] and num_large [S] expected")


def decode_attention_hier(query, k_pool, v_pool, small_tables, large_tables, num_large, pages_per_large: int,
                          context_lens, scale: float, max_context_len: int, partition_size: Optional[int] = None,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """decode_attention over two-level tables: a sequence's first
    num_large[s] * H logical blocks are its large pages (large page P = blocks
    [P H, P H + H) of the pools), the rest its small blocks."""
    lib = load()
    S, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    _hier_args(small_tables, large_tables, num_large, S)
    if context_lens.dtype != torch.int32 or context_lens.numel() != S:
        raise ValueError("context_lens must be int32 [S]")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if partition_size is None:
        partition_size = choose_partition(S, Hkv, max_context_len, bs)
    if out is None:
        out = torch.empty_like(query)
    else:
        _check_out(out, query)
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pa_decode_attention_hier(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                      _dev(v_pool, "v_pool"), _dev(small_tables, "small_tables"),
                                      _dev(large_tables, "large_tables"), _dev(num_large, "num_large"),
                                      _dev(context_lens, "context_lens"), S, Hq, Hkv, D, bs, small_tables.shape[1],
                                      large_tables.shape[1], int(pages_per_large), NB, int(max_context_len),
                                      float(scale), int(partition_size), _dtype_code(query), ws_ptr, ws_bytes,
                                      _stream(query, stream))
    _lib.check("pa_decode_attention_hier", st)
    return out


def prefill_attention_hier(query, k_pool, v_pool, small_tables, large_tables, num_large, pages_per_large: int,
                           context_lens, query_start, scale: float, max_query_len: int,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """prefill_attention over two-level tables (see decode_attention_hier)."""
    lib = load()
    T, Hq, D = query.shape
    NB, Hkv, bs, D2 = k_pool.shape
    S = context_lens.numel()
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("head_dim mismatch between query and pools")
    _hier_args(small_tables, large_tables, num_large, S)
    if context_lens.dtype != torch.int32 or query_start.dtype != torch.int32 or query_start.numel() != S + 1:
        raise ValueError("context_lens int32 [S] and query_start int32 [S + 1] expected")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if out is None:
        out = torch.empty_like(query)
    else:
        _check_out(out, query)
    st = lib.pa_prefill_attention_hier(_dev(out, "out"), _dev(query, "query"), _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool"), _dev(small_tables, "small_tables"),
                                       _dev(large_tables, "large_tables"), _dev(num_large, "num_large"),
                                       _dev(context_lens, "context_lens"), _dev(query_start, "query_start"), S, T,
                                       Hq, Hkv, D, bs, small_tables.shape[1], large_tables.shape[1],
                                       int(pages_per_large), NB, int(max_query_len), float(scale),
                                       _dtype_code(query), _stream(query, stream))
    _lib.check("pa_prefill_attention_hier", st)
    return out
