"""ctypes binding of libpagedattn.so (declared in include/pa.h).

Argument marshalling only: each function takes torch tensors that already live
on the GPU, checks their element type, shape and contiguity, passes raw device
pointers and the current HIP stream to the C entry point of the same name, and
raises ``PaError`` on a nonzero status.  All computation happens in the HIP
kernels.  There is no fallback: if the library is missing, importing this
module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PAGEDATTN_LIB", os.path.join(_HERE, "libpagedattn.so"))

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_ERR_BUFFER = -4
PA_STATIC_SCRATCH_BYTES = 64 << 20   # include/pa.h: pa_decode_step_static's partials array
ERR_BLOCK_ID, ERR_CAPACITY, ERR_SLOT = 1, 2, 4

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first with __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950)")
lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _f32, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_SIGS = {
    "pa_slot_mapping": [_p, _p, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p, _p],
    "pa_kv_append": [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _p, _p],
    "pa_decode": [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                  _i32, _i32, _f32, _i32, _p, _p, _p, _p],
    "pa_merge_lse": [_p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p],
    "pa_gather_kv": [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                     _i32, _p, _p, _p, _p],
    "pa_shard_length": [_i32, _i32, _i32, _i32],
    "pa_max_partitions": [_i32, _i32, _i32, _i32],
    "pa_default_partition_tokens": [_i32, _i32, _i32, _i32, _i32, _i32],
    "pa_choose_partition_tokens": [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32],
    "pa_choose_partition_tokens_multi": [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32],
    "pa_kv_append_fp8": [_p, _p, _i32, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i64,
                         _p, _p],
    "pa_decode_fp8": [_p, _p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32,
                      _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p],
    "pa_slot_mapping_multi": [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p, _p],
    "pa_decode_multi": [_p, _i32, _p, _i32, _i32, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                        _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p],
    "pa_copy_blocks": [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _p, _p],
    "pa_kv_append_routed": [_p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                            _i32, _i64, _i32, _i32, _i32, _p, _p, _p],
    "pa_decode_step": [_p, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                       _i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p, _p],
    "pa_decode_step_static": [_p, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                              _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p,
                              _i32, _p, _p, _p],
    "pa_pool_add": [_p, _i64, _i64],
    "pa_pool_append": [_p, _i64, _i64, _p, _i32, _p],
    "pa_pool_fork": [_p, _i64, _i64],
    "pa_pool_finish": [_p, _i64],
    "pa_last_error": [],
}
for _name, _args in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_char_p if _name == "pa_last_error" else ctypes.c_int32
# pool calls whose result is not a status
for _name, _args, _res in (("pa_pool_create", [_i64, _i32], _p),
                           ("pa_pool_destroy", [_p], None),
                           ("pa_pool_num_free", [_p], _i64),
                           ("pa_pool_length", [_p, _i64], _i64),
                           ("pa_pool_num_blocks", [_p, _i64], _i64),
                           ("pa_pool_refcount", [_p, _i64], _i32),
                           ("pa_pool_table", [_p, _i64, _p, _i64], _i64)):
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

PA_ERR_EXHAUSTED, PA_ERR_SEQUENCE = -6, -7


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def _check(status: int):
    if status != 0:
        raise PaError(status, lib.pa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t, cache=False):
    """Element type code; a cache may also hold E4M3 codes (uint8)."""
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if cache and t.dtype == torch.uint8:
        return PA_FP8_E4M3
    raise TypeError(f"unsupported element type {t.dtype}")


def _need(t, dtype=None, dims=None, name="tensor"):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


# ------------------------------------------------------------------ host helpers
def pa_shard_length(context_len: int, n_shards: int, interleave: int, shard: int) -> int:
    return int(lib.pa_shard_length(context_len, n_shards, interleave, shard))


def pa_max_partitions(max_context_len: int, n_shards: int, interleave: int, partition_tokens: int) -> int:
    return int(lib.pa_max_partitions(max_context_len, n_shards, interleave, partition_tokens))


def pa_default_partition_tokens(n_seqs, n_kv_heads, max_context_len, n_shards, interleave, block_size) -> int:
    return int(lib.pa_default_partition_tokens(n_seqs, n_kv_heads, max_context_len, n_shards,
                                               interleave, block_size))


def pa_choose_partition_tokens(context_lens_host, n_q_heads, n_kv_heads, dk, dv, block_size,
                               dtype, latent, n_shards=1, interleave=1) -> int:
    """``context_lens_host``: host sequence of ints; ``dtype``: torch dtype of the cache
    (``torch.uint8`` = E4M3 codes read with bf16 queries)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    code = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}[dtype]
    return int(lib.pa_choose_partition_tokens(lens.ctypes.data_as(ctypes.c_void_p), int(lens.size),
                                              n_q_heads, n_kv_heads, dk, dv, block_size, code,
                                              int(bool(latent)), n_shards, interleave))


def pa_choose_partition_tokens_multi(context_lens_host, max_q_len, n_q_heads, n_kv_heads, dk, dv,
                                     block_size, dtype, latent, n_shards=1, interleave=1) -> int:
    """As ``pa_choose_partition_tokens``, for ``pa_decode_multi`` with grid bound
    ``max_q_len`` on new tokens per sequence (``n_q_heads`` unscaled)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    code = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}[dtype]
    return int(lib.pa_choose_partition_tokens_multi(lens.ctypes.data_as(ctypes.c_void_p),
                                                    int(lens.size), max_q_len, n_q_heads, n_kv_heads,
                                                    dk, dv, block_size, code, int(bool(latent)),
                                                    n_shards, interleave))


# ------------------------------------------------------------------ entry points
def pa_slot_mapping(block_table, context_lens, n_shards, interleave, block_size, n_blocks,
                    slot_mapping, err_flag=None):
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n = context_lens.shape[0]
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or slot_mapping.shape[0] != n:
        raise ValueError("block_table / context_lens / slot_mapping shapes disagree")
    _check(lib.pa_slot_mapping(_ptr(block_table), _ptr(context_lens), n, n_shards, interleave,
                               block_size, block_table.shape[2], n_blocks, _ptr(slot_mapping),
                               _ptr(err_flag), _stream(block_table)))


def pa_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, err_flag=None):
    _need(k_new, None, 3, "k_new")
    _need(k_cache, k_new.dtype, 4, "k_cache")
    _need(v_new, k_new.dtype, 3, "v_new")
    _need(v_cache, k_new.dtype, 4, "v_cache")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hkv, dk = k_new.shape
    nb, hkv2, bs, dk2 = k_cache.shape
    dv = 0 if v_new is None else v_new.shape[2]
    if hkv2 != hkv or dk2 != dk or slot_mapping.shape[0] != n:
        raise ValueError("k_new / k_cache / slot_mapping shapes disagree")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    _check(lib.pa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                            _ptr(slot_mapping), n, hkv, dk, dv, bs, nb, _dtype_code(k_new),
                            _ptr(err_flag), _stream(k_cache)))


def pa_decode(q, k_cache, v_cache, block_table, context_lens, n_shards, interleave,
              partition_tokens, max_partitions, scale, part_out, part_lse, dv=None, err_flag=None):
    _need(q, None, 3, "q")
    _need(k_cache, q.dtype, 4, "k_cache")
    _need(v_cache, q.dtype, 4, "v_cache")
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(part_out, torch.float32, 5, "part_out")
    _need(part_lse, torch.float32, 4, "part_lse")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hq, dk = q.shape
    nb, hkv, bs, dk2 = k_cache.shape
    if dv is None:
        dv = v_cache.shape[2] if v_cache is not None else dk
    if dk2 != dk:
        raise ValueError("q and k_cache head sizes differ")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    if tuple(part_out.shape) != (n, n_shards, max_partitions, hq, dv):
        raise ValueError(f"part_out must be {(n, n_shards, max_partitions, hq, dv)}")
    if tuple(part_lse.shape) != (n, n_shards, max_partitions, hq):
        raise ValueError(f"part_lse must be {(n, n_shards, max_partitions, hq)}")
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or context_lens.shape[0] != n:
        raise ValueError("block_table / context_lens shapes disagree with q")
    _check(lib.pa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                         _ptr(context_lens), n, hq, hkv, dk, dv, bs, nb, block_table.shape[2],
                         n_shards, interleave, partition_tokens, max_partitions, float(scale),
                         _dtype_code(q), _ptr(part_out), _ptr(part_lse), _ptr(err_flag),
                         _stream(q)))


def _scales(k_scale, v_scale, hkv, latent):
    _need(k_scale, torch.float32, 1, "k_scale")
    if latent:
        if v_scale is not None:
            raise ValueError("a latent cache takes no v_scale")
    else:
        _need(v_scale, torch.float32, 1, "v_scale")
        if v_scale is None or v_scale.numel() != k_scale.numel():
            raise ValueError("v_scale must match k_scale in size")
    n = k_scale.numel()
    if n not in (1, hkv):
        raise ValueError(f"need 1 or {hkv} scales, got {n}")
    return n


def pa_kv_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slot_mapping, err_flag=None):
    """E4M3 cache (uint8 codes): new rows (fp32 or bf16) quantised with per-head or
    per-tensor float32 scales."""
    _need(k_new, None, 3, "k_new")
    _need(k_cache, torch.uint8, 4, "k_cache")
    _need(v_new, k_new.dtype, 3, "v_new")
    _need(v_cache, torch.uint8, 4, "v_cache")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hkv, dk = k_new.shape
    nb, hkv2, bs, dk2 = k_cache.shape
    dv = 0 if v_new is None else v_new.shape[2]
    if hkv2 != hkv or dk2 != dk or slot_mapping.shape[0] != n:
        raise ValueError("k_new / k_cache / slot_mapping shapes disagree")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    ns = _scales(k_scale, v_scale, hkv, v_cache is None)
    _check(lib.pa_kv_append_fp8(_ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_cache),
                                _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), ns, _ptr(slot_mapping),
                                n, hkv, dk, dv, bs, nb, _ptr(err_flag), _stream(k_cache)))


def pa_kv_append_routed(k_new, v_new, k_cache, v_cache, block_table, context_lens, n_shards,
                        interleave, k_scale=None, v_scale=None, slot_mapping=None, err_flag=None):
    """Routing and append in one launch (one new token per sequence); ``slot_mapping``
    (int64 [n_seqs], optional) receives the slots.  A uint8 cache holds E4M3 codes and
    takes its scales."""
    _need(k_new, None, 3, "k_new")
    _need(k_cache, None, 4, "k_cache")
    _need(v_new, k_new.dtype, 3, "v_new")
    _need(v_cache, k_cache.dtype, 4, "v_cache")
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hkv, dk = k_new.shape
    nb, hkv2, bs, dk2 = k_cache.shape
    dv = 0 if v_new is None else v_new.shape[2]
    if hkv2 != hkv or dk2 != dk or context_lens.shape[0] != n or block_table.shape[0] != n:
        raise ValueError("k_new / k_cache / block_table / context_lens shapes disagree")
    if block_table.shape[1] != n_shards:
        raise ValueError(f"block_table must be [n_seqs][{n_shards}][max_blocks]")
    if slot_mapping is not None and slot_mapping.shape[0] != n:
        raise ValueError("slot_mapping must be [n_seqs]")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    ns = 0
    if k_cache.dtype == torch.uint8:
        ns = _scales(k_scale, v_scale, hkv, v_cache is None)
    elif k_cache.dtype != k_new.dtype:
        raise TypeError("k_new must have the cache's element type (or the cache be uint8 codes)")
    _check(lib.pa_kv_append_routed(_ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_cache),
                                   _ptr(v_cache), _dtype_code(k_cache, cache=True), _ptr(k_scale),
                                   _ptr(v_scale), ns, _ptr(block_table), _ptr(context_lens), n, hkv,
                                   dk, dv, bs, nb, block_table.shape[2], n_shards, interleave,
                                   _ptr(slot_mapping), _ptr(err_flag), _stream(k_cache)))


def pa_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, n_shards,
                  interleave, partition_tokens, max_partitions, scale, part_out, part_lse, dv=None,
                  err_flag=None):
    """pa_decode over an E4M3 cache (uint8 codes) with its scales."""
    _need(q, None, 3, "q")
    _need(k_cache, torch.uint8, 4, "k_cache")
    _need(v_cache, torch.uint8, 4, "v_cache")
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(part_out, torch.float32, 5, "part_out")
    _need(part_lse, torch.float32, 4, "part_lse")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hq, dk = q.shape
    nb, hkv, bs, dk2 = k_cache.shape
    if dv is None:
        dv = v_cache.shape[2] if v_cache is not None else dk
    if dk2 != dk:
        raise ValueError("q and k_cache head sizes differ")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    if tuple(part_out.shape) != (n, n_shards, max_partitions, hq, dv):
        raise ValueError(f"part_out must be {(n, n_shards, max_partitions, hq, dv)}")
    if tuple(part_lse.shape) != (n, n_shards, max_partitions, hq):
        raise ValueError(f"part_lse must be {(n, n_shards, max_partitions, hq)}")
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or context_lens.shape[0] != n:
        raise ValueError("block_table / context_lens shapes disagree with q")
    ns = _scales(k_scale, v_scale, hkv, v_cache is None)
    _check(lib.pa_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                             ns, _ptr(block_table), _ptr(context_lens), n, hq, hkv, dk, dv, bs, nb,
                             block_table.shape[2], n_shards, interleave, partition_tokens,
                             max_partitions, float(scale), _dtype_code(q), _ptr(part_out),
                             _ptr(part_lse), _ptr(err_flag), _stream(q)))


def pa_decode_step(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, n_shards,
                   interleave, partition_tokens, max_partitions, scale, part_out, part_lse,
                   k_scale=None, v_scale=None, slot_mapping=None, dv=None, err_flag=None):
    """Append of the new tokens and the attention in one call (``pa_decode_step``): the
    effect of ``pa_kv_append_routed`` then ``pa_decode`` (``pa_decode_fp8`` for a uint8
    cache of E4M3 codes, which takes its scales)."""
    call_decode_step(decode_step_args(q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                                      n_shards, interleave, partition_tokens, max_partitions, scale,
                                      part_out, part_lse, k_scale, v_scale, slot_mapping, dv,
                                      err_flag), q)


def call_decode_step(args, q):
    """``pa_decode_step`` on the arguments ``decode_step_args`` built, on ``q``'s device's
    current stream."""
    _check(lib.pa_decode_step(*args, _stream(q)))


def decode_step_args(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, n_shards,
                     interleave, partition_tokens, max_partitions, scale, part_out, part_lse,
                     k_scale=None, v_scale=None, slot_mapping=None, dv=None, err_flag=None):
    """The checks of ``pa_decode_step`` and its C arguments but the stream, as a list (a
    caller that passes the same tensors again can reuse it)."""
    _need(q, None, 3, "q")
    _need(k_new, None, 3, "k_new")
    _need(v_new, k_new.dtype, 3, "v_new")
    _need(k_cache, None, 4, "k_cache")
    _need(v_cache, k_cache.dtype, 4, "v_cache")
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(part_out, torch.float32, 5, "part_out")
    _need(part_lse, torch.float32, 4, "part_lse")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n, hq, dk = q.shape
    nb, hkv, bs, dk2 = k_cache.shape
    if dv is None:
        dv = v_cache.shape[2] if v_cache is not None else dk
    if dk2 != dk:
        raise ValueError("q and k_cache head sizes differ")
    if tuple(k_new.shape) != (n, hkv, dk):
        raise ValueError(f"k_new must be {(n, hkv, dk)}")
    if (v_new is None) != (v_cache is None) or (v_new is not None and tuple(v_new.shape) != (n, hkv, dv)):
        raise ValueError(f"v_new must be {(n, hkv, dv)} with a value cache, None without one")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    if tuple(part_out.shape) != (n, n_shards, max_partitions, hq, dv):
        raise ValueError(f"part_out must be {(n, n_shards, max_partitions, hq, dv)}")
    if tuple(part_lse.shape) != (n, n_shards, max_partitions, hq):
        raise ValueError(f"part_lse must be {(n, n_shards, max_partitions, hq)}")
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or context_lens.shape[0] != n:
        raise ValueError("block_table / context_lens shapes disagree with q")
    if slot_mapping is not None and slot_mapping.shape[0] != n:
        raise ValueError("slot_mapping must be [n_seqs]")
    ns = 0
    if k_cache.dtype == torch.uint8:
        ns = _scales(k_scale, v_scale, hkv, v_cache is None)
    elif k_cache.dtype != q.dtype or k_new.dtype != q.dtype:
        raise TypeError("q, k_new and the cache must share an element type (or the cache be uint8 codes)")
    return [_ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_cache), _ptr(v_cache),
            _dtype_code(k_cache, cache=True), _ptr(k_scale), _ptr(v_scale), ns, _ptr(block_table),
            _ptr(context_lens), n, hq, hkv, dk, dv, bs, nb, block_table.shape[2], n_shards, interleave,
            partition_tokens, max_partitions, float(scale), _dtype_code(q), _ptr(slot_mapping),
            _ptr(part_out), _ptr(part_lse), _ptr(err_flag)]


def pa_slot_mapping_multi(block_table, context_lens, query_start, n_shards, interleave, block_size,
                          n_blocks, slot_mapping, err_flag=None):
    """Slots of every new token; ``query_start`` int32 [n_seqs+1] on the GPU."""
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(query_start, torch.int32, 1, "query_start")
    _need(slot_mapping, torch.int64, 1, "slot_mapping")
    _need(err_flag, torch.int32, None, "err_flag")
    n = context_lens.shape[0]
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or query_start.shape[0] != n + 1:
        raise ValueError("block_table / context_lens / query_start shapes disagree")
    _check(lib.pa_slot_mapping_multi(_ptr(block_table), _ptr(context_lens), _ptr(query_start), n,
                                     slot_mapping.shape[0], n_shards, interleave, block_size,
                                     block_table.shape[2], n_blocks, _ptr(slot_mapping),
                                     _ptr(err_flag), _stream(block_table)))


def pa_decode_multi(q, query_start, max_q_len, k_cache, v_cache, block_table, context_lens, n_shards,
                    interleave, partition_tokens, max_partitions, scale, part_out, part_lse,
                    k_scale=None, v_scale=None, dv=None, err_flag=None):
    """Several new tokens per sequence (causal among them): ``q [rows][Hq][dk]``,
    ``query_start`` int32 [n_seqs+1]; an E4M3 cache (uint8) takes its scales."""
    _need(q, None, 3, "q")
    _need(k_cache, None, 4, "k_cache")
    _need(v_cache, k_cache.dtype, 4, "v_cache")
    _need(query_start, torch.int32, 1, "query_start")
    _need(block_table, torch.int32, 3, "block_table")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(part_out, torch.float32, 5, "part_out")
    _need(part_lse, torch.float32, 4, "part_lse")
    _need(err_flag, torch.int32, None, "err_flag")
    rows, hq, dk = q.shape
    nb, hkv, bs, dk2 = k_cache.shape
    n = context_lens.shape[0]
    if dv is None:
        dv = v_cache.shape[2] if v_cache is not None else dk
    if dk2 != dk:
        raise ValueError("q and k_cache head sizes differ")
    if v_cache is not None and tuple(v_cache.shape) != (nb, hkv, dv, bs):
        raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    if tuple(part_out.shape) != (rows, n_shards, max_partitions, hq, dv):
        raise ValueError(f"part_out must be {(rows, n_shards, max_partitions, hq, dv)}")
    if tuple(part_lse.shape) != (rows, n_shards, max_partitions, hq):
        raise ValueError(f"part_lse must be {(rows, n_shards, max_partitions, hq)}")
    if block_table.shape[0] != n or block_table.shape[1] != n_shards or query_start.shape[0] != n + 1:
        raise ValueError("block_table / context_lens / query_start shapes disagree")
    kv_code = _dtype_code(k_cache, cache=True)
    ns = 0
    if kv_code == PA_FP8_E4M3:
        ns = _scales(k_scale, v_scale, hkv, v_cache is None)
    _check(lib.pa_decode_multi(_ptr(q), _dtype_code(q), _ptr(query_start), rows, int(max_q_len),
                               _ptr(k_cache), _ptr(v_cache), kv_code, _ptr(k_scale), _ptr(v_scale),
                               ns, _ptr(block_table), _ptr(context_lens), n, hq, hkv, dk, dv, bs, nb,
                               block_table.shape[2], n_shards, interleave, partition_tokens,
                               max_partitions, float(scale), _ptr(part_out), _ptr(part_lse),
                               _ptr(err_flag), _stream(q)))


def pa_merge_lse(part_out, part_lse, out, lse=None):
    """``part_out [N][P...][Hq][dv]`` (any number of part axes), ``out [N][Hq][dv]``."""
    call_merge_lse(merge_lse_args(part_out, part_lse, out, lse), out)


def merge_lse_args(part_out, part_lse, out, lse=None):
    """The checks of ``pa_merge_lse`` and its C arguments but the stream, as a tuple (a
    caller that merges into the same tensors again can reuse it)."""
    _need(part_out, torch.float32, None, "part_out")
    _need(part_lse, torch.float32, None, "part_lse")
    _need(out, None, 3, "out")
    _need(lse, torch.float32, 2, "lse")
    n, hq, dv = out.shape
    n_parts = part_lse.numel() // max(n * hq, 1)
    if part_lse.numel() != n * n_parts * hq or part_out.numel() != n * n_parts * hq * dv:
        raise ValueError("part_out / part_lse / out sizes disagree")
    return (_ptr(part_out), _ptr(part_lse), n, n_parts, hq, dv, _ptr(out), _dtype_code(out), _ptr(lse))


def call_merge_lse(args, out):
    """``pa_merge_lse`` on the arguments ``merge_lse_args`` built, on ``out``'s device's
    current stream."""
    _check(lib.pa_merge_lse(*args, _stream(out)))


def pa_gather_kv(k_cache, v_cache, block_table, seq, shard, context_len, n_shards, interleave,
                 k_out, v_out, err_flag=None):
    _need(k_cache, None, 4, "k_cache")
    _need(v_cache, k_cache.dtype, 4, "v_cache")
    _need(block_table, torch.int32, 3, "block_table")
    _need(k_out, k_cache.dtype, 3, "k_out")
    _need(v_out, k_cache.dtype, 3, "v_out")
    _need(err_flag, torch.int32, None, "err_flag")
    nb, hkv, bs, dk = k_cache.shape
    dv = v_out.shape[2]
    L_r = pa_shard_length(context_len, n_shards, interleave, shard)
    if k_out.shape[0] < L_r or v_out.shape[0] < L_r:
        raise ValueError(f"k_out/v_out need {L_r} rows")
    _check(lib.pa_gather_kv(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), seq, shard,
                            context_len, hkv, dk, dv, bs, nb, block_table.shape[2], n_shards,
                            interleave, _dtype_code(k_cache, cache=True), _ptr(k_out), _ptr(v_out),
                            _ptr(err_flag), _stream(k_cache)))


def pa_copy_blocks(k_cache, v_cache, pairs, err_flag=None):
    """``pairs``: int64 GPU tensor ``[n][2]`` of (source, destination) block ids."""
    _need(k_cache, None, 4, "k_cache")
    _need(v_cache, k_cache.dtype, 4, "v_cache")
    _need(pairs, torch.int64, 2, "pairs")
    _need(err_flag, torch.int32, None, "err_flag")
    nb, hkv, bs, dk = k_cache.shape
    dv = 0
    if v_cache is not None:
        dv = v_cache.shape[2]
        if tuple(v_cache.shape) != (nb, hkv, dv, bs):
            raise ValueError("v_cache must be [n_blocks][n_kv_heads][dv][block_size]")
    if pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    _check(lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0], hkv, dk,
                              dv, bs, nb, _dtype_code(k_cache, cache=True), _ptr(err_flag),
                              _stream(k_cache)))


class PoolExhausted(PaError):
    """The pool has too few free blocks for the request; nothing changed."""


class BlockPool:
    """Host-side block accounting (pa_pool_* in include/pa.h).  Sequence ids are ints."""

    def __init__(self, n_blocks: int, block_size: int):
        self._h = lib.pa_pool_create(int(n_blocks), int(block_size))
        if not self._h:
            raise PaError(-2, lib.pa_last_error().decode())
        self.n_blocks = int(n_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            lib.pa_pool_destroy(h)

    @staticmethod
    def _status(rc):
        if rc == PA_ERR_EXHAUSTED:
            raise PoolExhausted(rc, lib.pa_last_error().decode())
        _check(rc)

    def add(self, seq: int, n_tokens: int = 0) -> None:
        self._status(lib.pa_pool_add(self._h, seq, n_tokens))

    def append(self, seq: int, n_tokens: int = 1):
        """Returns the copy-on-write block copies, a list of (source, destination)."""
        buf = (ctypes.c_int64 * 2)()
        made = ctypes.c_int32(0)
        self._status(lib.pa_pool_append(self._h, seq, n_tokens, buf, 1, ctypes.byref(made)))
        return [(int(buf[0]), int(buf[1]))] if made.value else []

    def fork(self, parent: int, child: int) -> None:
        self._status(lib.pa_pool_fork(self._h, parent, child))

    def finish(self, seq: int) -> None:
        self._status(lib.pa_pool_finish(self._h, seq))

    def num_free(self) -> int:
        return int(lib.pa_pool_num_free(self._h))

    def length(self, seq: int) -> int:
        return int(lib.pa_pool_length(self._h, seq))

    def num_blocks(self, seq: int) -> int:
        return int(lib.pa_pool_num_blocks(self._h, seq))

    def refcount(self, block: int) -> int:
        return int(lib.pa_pool_refcount(self._h, block))

    def table(self, seq: int):
        n = self.num_blocks(seq)
        if n < 0:
            raise PaError(PA_ERR_SEQUENCE, f"no sequence {seq}")
        buf = (ctypes.c_int32 * max(n, 1))()
        got = lib.pa_pool_table(self._h, seq, buf, n)
        if got != n:
            raise PaError(PA_ERR_SEQUENCE, f"pa_pool_table returned {got}")
        return [int(buf[j]) for j in range(n)]
