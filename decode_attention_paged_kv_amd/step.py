"""One decode step on one stream: slot routing, kv append, attention, LSE merge.

``DecodeStep`` owns the step's output and scratch tensors (allocated once, with
torch, for a maximum context length) and issues the library calls: routing, append and
attention in one call (``pa_decode_step``), then the merge.  A cache of
``torch.uint8`` holds E4M3 codes and takes its scales with each call (the ``_fp8``
entry points).
"""
from __future__ import annotations

import torch

from . import _lib as L


class DecodeStep:
    def __init__(self, n_seqs, n_q_heads, n_kv_heads, dk, dv, block_size, max_context_len,
                 n_shards=1, interleave=1, partition_tokens=0, scale=None, device="cuda",
                 out_dtype=torch.float32, context_lens_host=None, kv_dtype=torch.bfloat16,
                 latent=False):
        """``partition_tokens=0`` picks a size: from the host context lengths when given
        (``pa_choose_partition_tokens``), else from the longest context alone."""
        self.n_seqs, self.hq, self.hkv, self.dk, self.dv = n_seqs, n_q_heads, n_kv_heads, dk, dv
        self.block_size, self.n_shards, self.interleave = block_size, n_shards, interleave
        if not partition_tokens and context_lens_host is not None:
            partition_tokens = L.pa_choose_partition_tokens(context_lens_host, n_q_heads, n_kv_heads,
                                                            dk, dv, block_size, kv_dtype, latent,
                                                            n_shards, interleave)
        if not partition_tokens:
            partition_tokens = L.pa_default_partition_tokens(n_seqs, n_kv_heads, max_context_len,
                                                             n_shards, interleave, block_size)
        self.partition_tokens = partition_tokens
        self.max_partitions = max(1, L.pa_max_partitions(max_context_len, n_shards, interleave,
                                                         partition_tokens))
        self.scale = float(torch.tensor(scale if scale is not None else dk ** -0.5,
                                        dtype=torch.float32))
        dev = torch.device(device)
        P = self.max_partitions
        self.slot_mapping = torch.empty(n_seqs, dtype=torch.int64, device=dev)
        self.part_out = torch.empty(n_seqs, n_shards, P, n_q_heads, dv, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(n_seqs, n_shards, P, n_q_heads, dtype=torch.float32, device=dev)
        self.out, self.lse, self.direct = _outputs(self.part_out, self.part_lse, n_seqs, n_q_heads, dv,
                                                   n_shards, P, out_dtype, dev)
        self.err_flag = torch.zeros(1, dtype=torch.int32, device=dev)
        self._step_key, self._step_args = None, None   # see append_attend
        # the merge always reads and writes this object's own buffers: checked once
        self._merge_args = None if self.direct else L.merge_lse_args(self.part_out, self.part_lse,
                                                                      self.out, self.lse)

    def route(self, block_table, context_lens, n_blocks):
        L.pa_slot_mapping(block_table, context_lens, self.n_shards, self.interleave,
                          self.block_size, n_blocks, self.slot_mapping, self.err_flag)

    def append(self, k_new, v_new, k_cache, v_cache, k_scale=None, v_scale=None):
        if k_cache.dtype == torch.uint8:
            L.pa_kv_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, self.slot_mapping,
                               self.err_flag)
        else:
            L.pa_kv_append(k_new, v_new, k_cache, v_cache, self.slot_mapping, self.err_flag)

    def route_append(self, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                     k_scale=None, v_scale=None):
        """route() and append() in one launch (``pa_kv_append_routed``); the slots still
        land in ``slot_mapping``."""
        L.pa_kv_append_routed(k_new, v_new, k_cache, v_cache, block_table, context_lens,
                              self.n_shards, self.interleave, k_scale, v_scale, self.slot_mapping,
                              self.err_flag)

    def attend(self, q, k_cache, v_cache, block_table, context_lens, k_scale=None, v_scale=None):
        if k_cache.dtype == torch.uint8:
            L.pa_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                            self.n_shards, self.interleave, self.partition_tokens,
                            self.max_partitions, self.scale, self.part_out, self.part_lse,
                            dv=self.dv, err_flag=self.err_flag)
        else:
            L.pa_decode(q, k_cache, v_cache, block_table, context_lens, self.n_shards,
                        self.interleave, self.partition_tokens, self.max_partitions, self.scale,
                        self.part_out, self.part_lse, dv=self.dv, err_flag=self.err_flag)

    def merge(self):
        if not self.direct:
            L.call_merge_lse(self._merge_args, self.out)

    def append_attend(self, q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                      k_scale=None, v_scale=None):
        """route_append() then attend() in one call (``pa_decode_step``): one launch where
        the kernel can store the new rows itself; the slots land in ``slot_mapping``."""
        # The checked argument list is kept while the same tensors come back (same
        # objects, storage and shapes): the checks cost more host time than a small
        # step's launch.  The library checks every call again.
        ts = (q, k_new, v_new, k_cache, v_cache, block_table, context_lens, k_scale, v_scale)
        if not _same_tensors(ts, self._step_key):
            self._step_args = L.decode_step_args(q, k_new, v_new, k_cache, v_cache, block_table,
                                                 context_lens, self.n_shards, self.interleave,
                                                 self.partition_tokens, self.max_partitions,
                                                 self.scale, self.part_out, self.part_lse, k_scale,
                                                 v_scale, self.slot_mapping, self.dv, self.err_flag)
            self._step_key = _tensor_key(ts)
        L.call_decode_step(self._step_args, q)

    def __call__(self, q, k_new, v_new, k_cache, v_cache, block_table, context_lens, k_scale=None,
                 v_scale=None):
        """The whole step; returns ``(out, lse)`` (views of this object's buffers).  One
        launch with a single partition per sequence, else two (the merge)."""
        self.append_attend(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, k_scale,
                           v_scale)
        self.merge()
        return self.out, self.lse

    def capture(self, *args, **kwargs):
        """Record the whole step (the same arguments as a call) as a HIP graph and return
        it; ``graph.replay()`` then reruns the launches on whatever the argument
        tensors hold at that time.  The library allocates nothing and issues no memset,
        so the recorded launches are the step itself."""
        return capture_graph(lambda: self(*args, **kwargs))


def _tensor_key(ts):
    """What ``_same_tensors`` compares: each argument, its data address and shape."""
    return tuple((t, None, None) if t is None else (t, t.data_ptr(), t.shape) for t in ts)


def _same_tensors(ts, key):
    """True when ``ts`` are the very tensors ``key`` was taken of, still at the same
    addresses and shapes (a plain loop: this runs on every step)."""
    if key is None:
        return False
    for t, (t0, p0, s0) in zip(ts, key):
        if t is not t0 or (t is not None and (t.data_ptr() != p0 or t.shape != s0)):
            return False
    return True


def _outputs(part_out, part_lse, n_rows, hq, dv, n_shards, max_partitions, out_dtype, dev):
    """The step's output and LSE buffers.  With one shard, one partition and float32
    output they are views of the partials: the merge of a single part is the identity
    (weight exp(lse - lse) = 1) and the decode writes zeros into partition 0 of an empty
    sequence, so the merge launch is skipped (``direct``)."""
    if n_shards == 1 and max_partitions == 1 and out_dtype == torch.float32:
        return part_out.view(n_rows, hq, dv), part_lse.view(n_rows, hq), True
    return (torch.empty(n_rows, hq, dv, dtype=out_dtype, device=dev),
            torch.empty(n_rows, hq, dtype=torch.float32, device=dev), False)


def capture_graph(fn):
    """Run ``fn`` once to warm up, then record it into a ``torch.cuda.CUDAGraph`` (on a
    side stream, as graph capture requires)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


class MultiDecodeStep:
    """One step with several new tokens per sequence, each attending causally (the
    ``_multi`` entry points): routes and appends every new token's K/V, attends, and
    merges per row.  Sized for ``n_rows`` new tokens in total and at most
    ``max_q_len`` per sequence."""

    def __init__(self, n_seqs, n_rows, max_q_len, n_q_heads, n_kv_heads, dk, dv, block_size,
                 max_context_len, n_shards=1, interleave=1, partition_tokens=0, scale=None,
                 device="cuda", out_dtype=torch.float32, context_lens_host=None,
                 kv_dtype=torch.bfloat16, latent=False):
        self.n_seqs, self.n_rows, self.max_q = n_seqs, n_rows, max_q_len
        self.hq, self.hkv, self.dk, self.dv = n_q_heads, n_kv_heads, dk, dv
        self.block_size, self.n_shards, self.interleave = block_size, n_shards, interleave
        if not partition_tokens and context_lens_host is not None:
            partition_tokens = L.pa_choose_partition_tokens_multi(context_lens_host, max_q_len,
                                                                  n_q_heads, n_kv_heads, dk, dv,
                                                                  block_size, kv_dtype, latent,
                                                                  n_shards, interleave)
        if not partition_tokens:
            partition_tokens = L.pa_default_partition_tokens(n_seqs, n_kv_heads, max_context_len,
                                                             n_shards, interleave, block_size)
        self.partition_tokens = partition_tokens
        self.max_partitions = max(1, L.pa_max_partitions(max_context_len, n_shards, interleave,
                                                         partition_tokens))
        self.scale = float(torch.tensor(scale if scale is not None else dk ** -0.5,
                                        dtype=torch.float32))
        dev = torch.device(device)
        P = self.max_partitions
        self.slot_mapping = torch.empty(n_rows, dtype=torch.int64, device=dev)
        self.part_out = torch.empty(n_rows, n_shards, P, n_q_heads, dv, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(n_rows, n_shards, P, n_q_heads, dtype=torch.float32, device=dev)
        self.out, self.lse, self.direct = _outputs(self.part_out, self.part_lse, n_rows, n_q_heads, dv,
                                                   n_shards, P, out_dtype, dev)
        self.err_flag = torch.zeros(1, dtype=torch.int32, device=dev)
        self._merge_args = None if self.direct else L.merge_lse_args(self.part_out, self.part_lse,
                                                                      self.out, self.lse)

    def route(self, block_table, context_lens, query_start, n_blocks):
        L.pa_slot_mapping_multi(block_table, context_lens, query_start, self.n_shards,
                                self.interleave, self.block_size, n_blocks, self.slot_mapping,
                                self.err_flag)

    def append(self, k_new, v_new, k_cache, v_cache, k_scale=None, v_scale=None):
        if k_cache.dtype == torch.uint8:
            L.pa_kv_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, self.slot_mapping,
                               self.err_flag)
        else:
            L.pa_kv_append(k_new, v_new, k_cache, v_cache, self.slot_mapping, self.err_flag)

    def attend(self, q, query_start, k_cache, v_cache, block_table, context_lens, k_scale=None,
               v_scale=None):
        L.pa_decode_multi(q, query_start, self.max_q, k_cache, v_cache, block_table, context_lens,
                          self.n_shards, self.interleave, self.partition_tokens,
                          self.max_partitions, self.scale, self.part_out, self.part_lse,
                          k_scale=k_scale, v_scale=v_scale, dv=self.dv, err_flag=self.err_flag)

    def merge(self):
        if not self.direct:
            L.call_merge_lse(self._merge_args, self.out)

    def __call__(self, q, query_start, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                 k_scale=None, v_scale=None):
        """The whole step; returns ``(out, lse)`` per row (views of this object's buffers)."""
        self.route(block_table, context_lens, query_start, k_cache.shape[0])
        self.append(k_new, v_new, k_cache, v_cache, k_scale, v_scale)
        self.attend(q, query_start, k_cache, v_cache, block_table, context_lens, k_scale, v_scale)
        self.merge()
        return self.out, self.lse

    def capture(self, *args, **kwargs):
        """The whole step recorded as a HIP graph (see ``DecodeStep.capture``)."""
        return capture_graph(lambda: self(*args, **kwargs))
