"""Plain model of a decode step with several new tokens per sequence.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[KVB] ("Why does writing one token at a time duplicate work?") states the rule a
decode step follows: the new token's query is compared with the keys of every
token before it and of itself, and the values are weighted by the result; stored
rows never change.  A step may carry more than one new token of a sequence -- the
continuation of a long prompt split into chunks ([KVB], failure-mode paragraph on
chunked prefill; [AGX], execution-plane section: a per-step long-prefill token
threshold) or the verification of speculative tokens ([AGX], open-source kernel
contributions section) -- and the same rule then applies to each of them, which is
the causal mask among the new tokens.

Readings taken here:
* the ``n_b`` new tokens of sequence ``b`` are the last ``n_b`` of its context;
  ``context_lens[b] = L`` counts them, so new token ``i`` (0-based) sits at global
  position ``L - n_b + i`` and attends over positions ``0 .. L - n_b + i``;
* queries are packed as ``q [total new tokens][Hq][dk]``; rows
  ``query_start[b] .. query_start[b+1]-1`` belong to sequence ``b`` (``n_b`` may be 0);
* shards and partitions are those of the single-token step: a query sees, on
  shard ``r``, the shard's tokens whose global position it may attend to, which are
  a prefix of the shard's local order; every partition is cut at that prefix and a
  partition with nothing left is empty (output 0, LSE -inf), as in
  ``paged_attention.decode_partials``.
"""
from __future__ import annotations

import numpy as np

from . import paged_attention as pa


def query_counts(query_start) -> np.ndarray:
    qs = np.asarray(query_start, dtype=np.int64)
    return qs[1:] - qs[:-1]


def slot_mapping_multi(block_table, context_lens, query_start, n_shards: int, interleave: int,
                       block_size: int) -> np.ndarray:
    """Cache slot of every new token (row order of ``q``): new token ``i`` of
    sequence ``b`` is global token ``L - n_b + i``, placed by the same rule as a
    single new token (``paged_attention.token_home``)."""
    n = query_counts(query_start)
    out = np.empty(int(n.sum()), dtype=np.int64)
    row = 0
    for b, L in enumerate(np.asarray(context_lens)):
        for i in range(int(n[b])):
            pos = int(L) - int(n[b]) + i
            _, _, phys, off = pa.token_home(block_table[b], pos, n_shards, interleave, block_size)
            out[row] = phys * block_size + off
            row += 1
    return out


def decode_multi_partials(q, query_start, k_cache, v_cache, block_table, context_lens,
                          n_shards: int, interleave: int, block_size: int, partition_tokens: int,
                          max_partitions_: int, scale: float, dv: int):
    """Per-partition results of every new token.  Returns ``part_o
    [rows][S][Pmax][Hq][dv]`` and ``part_lse [rows][S][Pmax][Hq]``."""
    n = query_counts(query_start)
    rows, hq = q.shape[0], q.shape[1]
    part_o = np.zeros((rows, n_shards, max_partitions_, hq, dv))
    part_lse = np.full((rows, n_shards, max_partitions_, hq), pa.NEG_INF)
    row = 0
    for b, L in enumerate(np.asarray(context_lens)):
        L = int(L)
        for r in range(n_shards):
            K, V = pa.gather_shard(k_cache, v_cache, block_table[b], L, r, n_shards, interleave,
                                   block_size, dv)
            members = pa.shard_members(L, n_shards, interleave, r)
            for i in range(int(n[b])):
                pos = L - int(n[b]) + i
                seen = int(np.count_nonzero(members <= pos))     # a prefix of local order
                p = 0
                while p * partition_tokens < K.shape[0]:
                    lo = p * partition_tokens
                    hi = min((p + 1) * partition_tokens, seen)
                    if hi > lo:
                        part_o[row + i, r, p], part_lse[row + i, r, p] = pa.attention(
                            q[row + i], K[lo:hi], V[lo:hi], scale)
                    p += 1
        row += int(n[b])
    return part_o, part_lse


def decode_multi(q, query_start, k_cache, v_cache, block_table, context_lens, n_shards: int,
                 interleave: int, block_size: int, partition_tokens: int, max_partitions_: int,
                 scale: float, dv: int):
    """Every new token's output: its partials over all shards merged with
    ``paged_attention.merge_lse``.  Returns ``o [rows][Hq][dv]``, ``lse [rows][Hq]``
    and the partials."""
    part_o, part_lse = decode_multi_partials(q, query_start, k_cache, v_cache, block_table,
                                             context_lens, n_shards, interleave, block_size,
                                             partition_tokens, max_partitions_, scale, dv)
    rows, hq = q.shape[0], q.shape[1]
    o = np.zeros((rows, hq, dv))
    lse = np.full((rows, hq), pa.NEG_INF)
    for t in range(rows):
        o[t], lse[t] = pa.merge_lse(part_o[t].reshape(-1, hq, dv), part_lse[t].reshape(-1, hq))
    return o, lse, part_o, part_lse


def decode_step_multi(q, query_start, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                      n_shards: int, interleave: int, block_size: int, partition_tokens: int,
                      max_partitions_: int, scale: float, dv: int):
    """The whole step: store every new token's key and value in its slot, then
    attend (causally among the new tokens).  Returns a dict like
    ``paged_attention.decode_step``."""
    slots = slot_mapping_multi(block_table, context_lens, query_start, n_shards, interleave,
                               block_size)
    kc, vc = pa.kv_append(k_cache, v_cache, k_new, v_new, slots, block_size)
    o, lse, part_o, part_lse = decode_multi(q, query_start, kc, vc, block_table, context_lens,
                                            n_shards, interleave, block_size, partition_tokens,
                                            max_partitions_, scale, dv)
    return dict(slots=slots, k_cache=kc, v_cache=vc, o=o, lse=lse, part_o=part_o,
                part_lse=part_lse)
