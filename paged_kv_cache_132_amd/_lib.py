"""ctypes binding of libpa.so: argument marshalling only.

Every function takes torch tensors that already live on a HIP device, checks
that their shapes agree with each other, and passes raw device pointers plus
sizes to the C ABI on torch's current stream.  All arithmetic runs in the HIP
kernels; a missing or unloadable library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {
    0: "PA_OK", 1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_BAD_SHAPE", 3: "PA_ERR_BAD_DTYPE",
    4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_MISALIGNED", 6: "PA_ERR_WORKSPACE_TOO_SMALL", 7: "PA_ERR_HIP",
    8: "PA_ERR_POOL_EXHAUSTED", 9: "PA_ERR_UNKNOWN_SEQUENCE",
}
EXPORTED = ("pa_cache_write", "pa_cache_write_tokens", "pa_copy_blocks", "pa_decode", "pa_decode_partials",
            "pa_decode_merge", "pa_decode_write", "pa_decode_write_partials", "pa_decode_shared",
            "pa_decode_write_partials_shared", "pa_decode_workspace_size",
            "pa_decode_partition_size", "pa_decode_noalloc", "pa_decode_noalloc_max_workspace",
            "pa_prefill", "pa_prefill_write", "pa_status_string",
            "pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence", "pa_bm_append_token", "pa_bm_fork",
            "pa_bm_free_sequence", "pa_bm_take_copies", "pa_bm_sequence_length", "pa_bm_block_table",
            "pa_bm_ref_count", "pa_bm_stats_get")

_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_132_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        i32, f32, vp, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        lib.pa_cache_write.restype = ctypes.c_int
        lib.pa_cache_write.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp,
                                       i32, i32, i32, i32, i32, i32, f32, f32, vp]
        for fn in (lib.pa_decode, lib.pa_decode_partials, lib.pa_decode_merge):
            fn.restype = ctypes.c_int
            fn.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                           i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, vp, sz, vp]
        lib.pa_cache_write_tokens.restype = ctypes.c_int
        lib.pa_cache_write_tokens.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp,
                                              i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
        lib.pa_prefill.restype = ctypes.c_int
        lib.pa_prefill.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, vp]
        lib.pa_prefill_write.restype = ctypes.c_int
        lib.pa_prefill_write.argtypes = lib.pa_prefill.argtypes + [vp, vp, ctypes.c_int]
        lib.pa_copy_blocks.restype = ctypes.c_int
        lib.pa_copy_blocks.argtypes = [vp, i32, vp, i32, ctypes.c_int, i32, i32, i32, vp, i32, vp]
        for fn in (lib.pa_decode_write, lib.pa_decode_write_partials):
            fn.restype = ctypes.c_int
            fn.argtypes = lib.pa_decode.argtypes + [vp, vp, ctypes.c_int]
        lib.pa_decode_shared.restype = ctypes.c_int
        lib.pa_decode_shared.argtypes = lib.pa_decode.argtypes + [i32]
        lib.pa_decode_write_partials_shared.restype = ctypes.c_int
        lib.pa_decode_write_partials_shared.argtypes = lib.pa_decode_write_partials.argtypes + [i32]
        lib.pa_decode_workspace_size.restype = sz
        lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int, i32]
        lib.pa_decode_noalloc.restype = ctypes.c_int
        lib.pa_decode_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                          i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, vp]
        lib.pa_decode_noalloc_max_workspace.restype = sz
        lib.pa_decode_noalloc_max_workspace.argtypes = []
        lib.pa_decode_partition_size.restype = i32
        lib.pa_decode_partition_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int, i32]
        i64, u64, ip = ctypes.c_int64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_int32)
        lib.pa_bm_create.restype = vp
        lib.pa_bm_create.argtypes = [i32, i32, u64, ip]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_destroy.argtypes = [vp]
        lib.pa_bm_add_sequence.restype = ctypes.c_int
        lib.pa_bm_add_sequence.argtypes = [vp, i64, ip, i32, ip]
        lib.pa_bm_append_token.restype = ctypes.c_int
        lib.pa_bm_append_token.argtypes = [vp, i64, i32]
        lib.pa_bm_fork.restype = ctypes.c_int
        lib.pa_bm_fork.argtypes = [vp, i64, i64]
        lib.pa_bm_free_sequence.restype = ctypes.c_int
        lib.pa_bm_free_sequence.argtypes = [vp, i64]
        lib.pa_bm_take_copies.restype = i32
        lib.pa_bm_take_copies.argtypes = [vp, ip, i32]
        lib.pa_bm_sequence_length.restype = i32
        lib.pa_bm_sequence_length.argtypes = [vp, i64]
        lib.pa_bm_block_table.restype = i32
        lib.pa_bm_block_table.argtypes = [vp, i64, ip, i32]
        lib.pa_bm_ref_count.restype = i32
        lib.pa_bm_ref_count.argtypes = [vp, i32]
        lib.pa_bm_stats_get.restype = ctypes.c_int
        lib.pa_bm_stats_get.argtypes = [vp, vp]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [ctypes.c_int]
        _lib = lib
        return lib


def pa_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _check(status: int, what: str) -> None:
    if status != 0:
        name = load().pa_status_string(status).decode()
        raise RuntimeError(f"{what} failed: {name}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _pool_dims(kv_pool: torch.Tensor):
    if kv_pool.dim() != 5 or kv_pool.shape[1] != 2:
        raise ValueError("kv_pool must be [num_blocks, 2, block_size, num_kv_heads, head_dim]")
    if not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous")
    nb, _, bs, hkv, d = kv_pool.shape
    return int(nb), int(bs), int(hkv), int(d)


def _tables(block_tables: torch.Tensor, context_lens: torch.Tensor, num_seqs: int):
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [num_seqs, max_blocks_per_seq] tensor")
    if context_lens.shape != (num_seqs,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [num_seqs] tensor")
    return int(block_tables.shape[1])


def cache_write(kv_pool: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor,
                k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Write each sequence's newest token (t = context_lens[s] - 1) into kv_pool in place."""
    nb, bs, hkv, d = _pool_dims(kv_pool)
    if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (hkv, d):
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim] matching the pool")
    if not (key.is_contiguous() and value.is_contiguous()) or key.dtype != value.dtype:
        raise ValueError("key/value must be contiguous and of one dtype")
    B = int(key.shape[0])
    mb = _tables(block_tables, context_lens, B)
    st = load().pa_cache_write(_ptr(kv_pool), pa_dtype(kv_pool), _ptr(key), _ptr(value), pa_dtype(key),
                               _ptr(block_tables), _ptr(context_lens), B, hkv, d, bs, mb, nb,
                               float(k_scale), float(v_scale), _stream(stream))
    _check(st, "pa_cache_write")


def _cu(cu_seqlens: torch.Tensor, num_seqs: int) -> None:
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.shape != (num_seqs + 1,) or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 [num_seqs + 1] tensor")


def _max_new(cu_seqlens: torch.Tensor, max_new_tokens) -> int:
    """An upper bound on the per-sequence new-token counts; read from the
    device (a synchronisation) when the caller does not give one."""
    if max_new_tokens is not None:
        return int(max_new_tokens)
    if cu_seqlens.numel() < 2:
        return 0
    return int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())


def cache_write_tokens(kv_pool: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                       block_tables: torch.Tensor, context_lens: torch.Tensor, cu_seqlens: torch.Tensor,
                       k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Write packed new tokens (rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of key/value
    belong to sequence s, at positions context_lens[s] - n_s ..) into kv_pool in place."""
    nb, bs, hkv, d = _pool_dims(kv_pool)
    if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (hkv, d):
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim] matching the pool")
    if not (key.is_contiguous() and value.is_contiguous()) or key.dtype != value.dtype:
        raise ValueError("key/value must be contiguous and of one dtype")
    B = int(context_lens.shape[0])
    mb = _tables(block_tables, context_lens, B)
    _cu(cu_seqlens, B)
    st = load().pa_cache_write_tokens(_ptr(kv_pool), pa_dtype(kv_pool), _ptr(key), _ptr(value), pa_dtype(key),
                                      _ptr(block_tables), _ptr(context_lens), _ptr(cu_seqlens), B,
                                      int(key.shape[0]), hkv, d, bs, mb, nb, float(k_scale), float(v_scale),
                                      _stream(stream))
    _check(st, "pa_cache_write_tokens")


def prefill(query: torch.Tensor, kv_pool: torch.Tensor, block_tables: torch.Tensor,
            context_lens: torch.Tensor, cu_seqlens: torch.Tensor, scale: float, k_scale: float = 1.0,
            v_scale: float = 1.0, max_new_tokens: int | None = None, out: torch.Tensor | None = None,
            stream=None, new_key: torch.Tensor | None = None,
            new_value: torch.Tensor | None = None) -> torch.Tensor:
    """Causal attention of packed new queries [num_tokens, num_heads, head_dim] over
    their own sequences in the paged pool; returns out of query's shape and dtype.
    new_key / new_value ([num_tokens, num_kv_heads, head_dim]): write the new
    tokens in the same call (pa_prefill_write), as pa_cache_write_tokens would."""
    nb, bs, hkv, d = _pool_dims(kv_pool)
    if query.dim() != 3 or query.shape[2] != d or not query.is_contiguous():
        raise ValueError("query must be a contiguous [num_tokens, num_heads, head_dim] tensor")
    T, hq = int(query.shape[0]), int(query.shape[1])
    B = int(context_lens.shape[0])
    mb = _tables(block_tables, context_lens, B)
    _cu(cu_seqlens, B)
    if out is None:
        out = torch.empty_like(query)
    elif out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must match query")
    args = (_ptr(out), _ptr(query), pa_dtype(query), _ptr(kv_pool), pa_dtype(kv_pool),
            _ptr(block_tables), _ptr(context_lens), _ptr(cu_seqlens), B, T,
            _max_new(cu_seqlens, max_new_tokens), hq, hkv, d, bs, mb, nb, float(scale),
            float(k_scale), float(v_scale), _stream(stream))
    if new_key is None:
        st = load().pa_prefill(*args)
    else:
        if new_value is None or new_key.shape != (T, hkv, d) or new_value.shape != new_key.shape \
                or not (new_key.is_contiguous() and new_value.is_contiguous()) or new_value.dtype != new_key.dtype:
            raise ValueError("new_key/new_value must be contiguous [num_tokens, num_kv_heads, head_dim] of one dtype")
        st = load().pa_prefill_write(*args, _ptr(new_key), _ptr(new_value), pa_dtype(new_key))
    _check(st, "pa_prefill_write" if new_key is not None else "pa_prefill")
    return out


def copy_blocks(src_pool: torch.Tensor, dst_pool: torch.Tensor, block_mapping: torch.Tensor,
                stream=None) -> None:
    """dst_pool[d] = src_pool[s] for each row (s, d) of block_mapping (int32
    [num_pairs, 2] on the device).  Either pool may be pinned host memory
    (a swap); pass one tensor as both for copy-on-write inside a pool."""
    nb_s, bs, hkv, d = _pool_dims(src_pool)
    nb_d, bs_d, hkv_d, d_d = _pool_dims(dst_pool)
    if (bs, hkv, d) != (bs_d, hkv_d, d_d) or src_pool.dtype != dst_pool.dtype:
        raise ValueError("pools must have the same block geometry and dtype")
    if block_mapping.dtype != torch.int32 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2 \
            or not block_mapping.is_contiguous():
        raise ValueError("block_mapping must be a contiguous int32 [num_pairs, 2] tensor")
    st = load().pa_copy_blocks(_ptr(src_pool), nb_s, _ptr(dst_pool), nb_d, pa_dtype(src_pool), bs, hkv, d,
                               _ptr(block_mapping), int(block_mapping.shape[0]), _stream(stream))
    _check(st, "pa_copy_blocks")


def decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                          block_size: int, max_blocks_per_seq: int, kv_dtype: int,
                          partition_size: int = 0) -> int:
    n = load().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                        max_blocks_per_seq, kv_dtype, partition_size)
    if n == 0:
        raise RuntimeError("pa_decode_workspace_size: invalid arguments")
    return int(n)


def decode_partition_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                          block_size: int, max_blocks_per_seq: int, kv_dtype: int,
                          partition_size: int = 0) -> int:
    return int(load().pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                max_blocks_per_seq, kv_dtype, partition_size))


class Workspace:
    """A device workspace for pa_decode, grown on demand (its contents on
    entry do not matter, so one buffer serves calls of any size on one stream).

    A buffer is allocated on the stream the calls that use it launch on:
    when it grows, the caching allocator hands the old one out again only
    after the work already queued on that stream."""

    def __init__(self):
        self.buf: torch.Tensor | None = None

    def get(self, nbytes: int, device, stream=None) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device)):
                self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws: dict = {}


def decode(query: torch.Tensor, kv_pool: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
           out: torch.Tensor | None = None, workspace: torch.Tensor | Workspace | None = None,
           partition_size: int = 0, stream=None, phase: str = "both",
           new_key: torch.Tensor | None = None, new_value: torch.Tensor | None = None,
           run_size: int = 1) -> torch.Tensor:
    """Paged decode attention; returns out [num_seqs, num_heads, head_dim] of query's dtype.

    phase: "both" (pa_decode), "partials" (pa_decode_partials) or "merge"
    (pa_decode_merge, with the same arguments and workspace as the partials call).
    new_key / new_value ([num_seqs, num_kv_heads, head_dim], query dtype): write
    each sequence's newest token in the same pass (pa_decode_write /
    pa_decode_write_partials), as pa_cache_write would.
    run_size > 1: sequences share prefix blocks in aligned runs of that many
    (pa_decode_shared with phase "both", pa_decode_write_partials_shared with
    new_key / new_value and phase "partials")."""
    nb, bs, hkv, d = _pool_dims(kv_pool)
    if query.dim() != 3 or query.shape[2] != d or not query.is_contiguous():
        raise ValueError("query must be a contiguous [num_seqs, num_heads, head_dim] tensor")
    B, hq = int(query.shape[0]), int(query.shape[1])
    mb = _tables(block_tables, context_lens, B)
    if out is None:
        out = torch.empty_like(query)
    elif out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must match query")
    kvt = pa_dtype(kv_pool)
    need = decode_workspace_size(B, hq, hkv, d, bs, mb, kvt, partition_size)
    launch = torch.cuda.current_stream() if stream is None else stream
    if workspace is None:
        # one default workspace per (device, launch stream): calls on different
        # streams never share partials
        workspace = _default_ws.setdefault((query.device, launch.cuda_stream), Workspace())
    if isinstance(workspace, Workspace):
        ws = workspace.get(need, query.device, launch)
    else:
        ws = workspace
    extra = ()
    if run_size != 1 and phase != "merge":
        if (new_key is None) != (phase == "both"):
            raise ValueError("run_size: pa_decode_shared (phase 'both', no write) or "
                             "pa_decode_write_partials_shared (phase 'partials' with new_key / new_value)")
    if new_key is None:
        fn = {"both": load().pa_decode, "partials": load().pa_decode_partials,
              "merge": load().pa_decode_merge}[phase]
        if run_size != 1 and phase == "both":
            fn, extra = load().pa_decode_shared, (int(run_size),)
    else:
        if phase == "merge":
            raise ValueError("the fused write belongs to the attention pass, not the merge")
        if new_value is None or new_key.shape != (B, hkv, d) or new_value.shape != new_key.shape \
                or not (new_key.is_contiguous() and new_value.is_contiguous()) or new_value.dtype != new_key.dtype:
            raise ValueError("new_key/new_value must be contiguous [num_seqs, num_kv_heads, head_dim] of one dtype")
        fn = {"both": load().pa_decode_write, "partials": load().pa_decode_write_partials}[phase]
        extra = (_ptr(new_key), _ptr(new_value), pa_dtype(new_key))
        if run_size != 1:
            fn, extra = load().pa_decode_write_partials_shared, extra + (int(run_size),)
    st = fn(_ptr(out), _ptr(query), pa_dtype(query), _ptr(kv_pool), kvt,
            _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, bs, mb, nb,
            float(scale), float(k_scale), float(v_scale), int(partition_size),
            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream), *extra)
    _check(st, f"pa_decode ({phase})")
    return out


def decode_noalloc(query: torch.Tensor, kv_pool: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                   out: torch.Tensor | None = None, partition_size: int = 0, stream=None) -> torch.Tensor:
    """pa_decode_noalloc: paged decode with the library's fixed per-GPU
    workspace (the C call allocates nothing; pass `out` to allocate nothing
    here either).  Calls that may overlap on one GPU must be ordered."""
    nb, bs, hkv, d = _pool_dims(kv_pool)
    if query.dim() != 3 or query.shape[2] != d or not query.is_contiguous():
        raise ValueError("query must be a contiguous [num_seqs, num_heads, head_dim] tensor")
    B, hq = int(query.shape[0]), int(query.shape[1])
    mb = _tables(block_tables, context_lens, B)
    if out is None:
        out = torch.empty_like(query)
    elif out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must match query")
    st = load().pa_decode_noalloc(_ptr(out), _ptr(query), pa_dtype(query), _ptr(kv_pool), pa_dtype(kv_pool),
                                  _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, bs, mb, nb,
                                  float(scale), float(k_scale), float(v_scale), int(partition_size),
                                  _stream(stream))
    _check(st, "pa_decode_noalloc")
    return out

