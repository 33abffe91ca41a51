"""Plain fp64 NumPy oracle of one paged decode-attention step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py`` for who may call it and for
the page abbreviations [DCP], [KVB], [PA] used below).

Everything here is the plain definition, written for a reader to check by eye:
tokens are placed by enumerating them, K/V are gathered into contiguous arrays
through the block table, attention is an ordinary max-shifted softmax in fp64,
and partial results are merged with their log-sum-exp weights.  No blocking,
fusion or reordering beyond that.

Array conventions (the library's boundary uses the same ones):
* bf16 data is passed as ``uint16`` bit patterns; fp32 as ``float32``.  ``widen``
  turns either into float64 exactly.
* ``k_cache``: ``[n_blocks][n_kv_heads][block_size][dk]`` (token rows contiguous).
* ``v_cache``: ``[n_blocks][n_kv_heads][dv][block_size]`` (token index fastest),
  or ``None`` for the latent (MLA-style) cache, where V is the first ``dv``
  entries of each cached K row.
* ``block_table``: ``int32 [n_seqs][n_shards][max_blocks_per_shard]``; row
  ``[b][r]`` lists, in logical order, the physical blocks holding shard ``r``'s
  tokens of sequence ``b``.
* ``context_lens[b]`` counts every token of sequence ``b`` including the one the
  step appends (the new token sits at global position ``L - 1``).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------------
# element types
# ----------------------------------------------------------------------------------
def widen(x) -> np.ndarray:
    """Exact conversion to float64.

    ``uint16`` arrays are bf16 bit patterns: a bf16 value is the top half of the
    fp32 with the same bits, so shifting into the high half of a 32-bit word and
    reinterpreting gives the fp32 value, which float64 represents exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported element type {x.dtype}")


# ----------------------------------------------------------------------------------
# accounting: [KVB] "How KV-cache memory limits concurrency"; [PA] block-table section
# ----------------------------------------------------------------------------------
def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K and V one token occupies: one key and one value vector per KV
    head and per layer ([KVB], "How KV-cache memory limits concurrency"; the same
    product of factors is listed in [DCP]'s decode-bottleneck section)."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Fixed-size blocks that hold ``n_tokens`` when each block is filled before
    the next is taken ([PA], block-table section): the smallest count whose
    capacity reaches ``n_tokens``."""
    n = 0
    while n * block_size < n_tokens:
        n += 1
    return n


# ----------------------------------------------------------------------------------
# placement of tokens on shards: [DCP], DCP mechanism section
# ----------------------------------------------------------------------------------
def shard_of_token(i: int, n_shards: int, interleave: int) -> int:
    """Shard that holds global token ``i``.  [DCP] places tokens round-robin on
    the DCP ranks, ``interleave`` consecutive tokens at a time (interleave 1 puts
    token i on rank i mod S); tokens generated during decode follow the same rule."""
    return (i // interleave) % n_shards


def shard_members(L: int, n_shards: int, interleave: int, r: int) -> np.ndarray:
    """Global ids of the tokens of a length-``L`` sequence that live on shard
    ``r``, in ascending order.  The position of a token in this list is its local
    index in that shard (reading: a shard keeps its tokens in their global order;
    the pages do not print the per-rank listing)."""
    ids = np.arange(L, dtype=np.int64)
    return ids[(ids // interleave) % n_shards == r]


def shard_lengths(L: int, n_shards: int, interleave: int) -> np.ndarray:
    """Number of tokens on each shard, by enumeration."""
    return np.array([shard_members(L, n_shards, interleave, r).size for r in range(n_shards)],
                    dtype=np.int64)


def max_partitions(max_context_len: int, n_shards: int, interleave: int, partition_tokens: int) -> int:
    """Largest number of ``partition_tokens``-token partitions any shard needs for
    a sequence of at most ``max_context_len`` tokens."""
    longest = int(shard_lengths(max_context_len, n_shards, interleave).max()) if max_context_len > 0 else 0
    return blocks_needed(longest, partition_tokens)


# ----------------------------------------------------------------------------------
# block-table addressing: [PA] "A block table separates logical order from physical placement"
# ----------------------------------------------------------------------------------
def token_home(bt_b: np.ndarray, i: int, n_shards: int, interleave: int, block_size: int):
    """Where global token ``i`` of one sequence lives: (shard, local index,
    physical block, offset in block).  The shard comes from the placement rule,
    the local index is the count of earlier tokens on the same shard, and the
    block table row of that shard turns the logical block ``local // block_size``
    into a physical block ([PA], block-table section)."""
    r = shard_of_token(i, n_shards, interleave)
    local = int(np.count_nonzero((np.arange(i) // interleave) % n_shards == r))
    phys = int(bt_b[r][local // block_size])
    return r, local, phys, local % block_size


def slot_mapping(block_table: np.ndarray, context_lens: np.ndarray, n_shards: int,
                 interleave: int, block_size: int) -> np.ndarray:
    """Cache slot (``physical_block * block_size + offset``) of each sequence's new
    token, the one at global position ``L - 1`` ([KVB], "What does the KV cache
    hold?": the step stores the new token's key and value; [PA]: the current
    block is filled while it has room; [DCP]: new tokens follow the placement rule).
    A sequence with no tokens gets -1 ("no slot")."""
    out = np.empty(len(context_lens), dtype=np.int64)
    for b, L in enumerate(np.asarray(context_lens)):
        if L <= 0:                      # no token, nothing to place
            out[b] = -1
            continue
        _, _, phys, off = token_home(block_table[b], int(L) - 1, n_shards, interleave, block_size)
        out[b] = phys * block_size + off
    return out


def kv_append(k_cache: np.ndarray, v_cache, k_new: np.ndarray, v_new, slots: np.ndarray,
              block_size: int):
    """Store each new token's key and value rows into its slot, bit for bit
    ([KVB], "What does the KV cache hold?").  Returns new arrays; a negative slot
    means "no token" and is skipped.  ``v_cache is None`` is the latent cache,
    whose values are part of the stored key rows."""
    k_out = k_cache.copy()
    v_out = None if v_cache is None else v_cache.copy()
    for n, slot in enumerate(np.asarray(slots)):
        if slot < 0:
            continue
        blk, off = int(slot) // block_size, int(slot) % block_size
        k_out[blk, :, off, :] = k_new[n]
        if v_out is not None:
            v_out[blk, :, :, off] = v_new[n]
    return k_out, v_out


def copy_blocks(k_cache: np.ndarray, v_cache, pairs):
    """Copy whole physical blocks, bit for bit: for each (source, destination) pair
    every KV head's keys (and values, unless the cache is latent) of the source
    block overwrite the destination's.  This is the private copy a sequence takes
    before writing into a block it shares ([PA], "Sharing common blocks and
    copy-on-write").  Pairs apply in order; returns new arrays."""
    k_out = k_cache.copy()
    v_out = None if v_cache is None else v_cache.copy()
    for src, dst in pairs:
        k_out[int(dst)] = k_out[int(src)]
        if v_out is not None:
            v_out[int(dst)] = v_out[int(src)]
    return k_out, v_out


def _rows(k_cache, v_cache, phys: np.ndarray, off: np.ndarray, dv: int):
    k = k_cache[phys, :, off, :]                        # [n][Hkv][dk]
    if v_cache is None:
        v = k[:, :, :dv]
    else:
        v = v_cache[phys, :, :, off]                    # [n][Hkv][dv]
    return k, v


def gather_shard(k_cache, v_cache, bt_b: np.ndarray, L: int, r: int, n_shards: int,
                 interleave: int, block_size: int, dv: int):
    """K and V rows of shard ``r`` of one sequence, in local order, as stored
    (no conversion): ``[L_r][Hkv][dk]``, ``[L_r][Hkv][dv]``.  Logical block
    ``t // block_size`` of the shard is looked up in its block-table row; the
    offset is ``t % block_size`` ([PA], block-table section: attention follows the
    table to blocks that need not be adjacent)."""
    L_r = shard_members(L, n_shards, interleave, r).size
    t = np.arange(L_r, dtype=np.int64)
    phys = np.asarray(bt_b[r], dtype=np.int64)[t // block_size]
    return _rows(k_cache, v_cache, phys, t % block_size, dv)


def gather_sequence(k_cache, v_cache, bt_b: np.ndarray, L: int, n_shards: int,
                    interleave: int, block_size: int, dv: int):
    """All ``L`` K and V rows of one sequence in global token order, found one
    token at a time through its shard and block table."""
    dk = k_cache.shape[-1]
    hkv = k_cache.shape[1]
    K = np.empty((L, hkv, dk), dtype=k_cache.dtype)
    V = np.empty((L, hkv, dv), dtype=k_cache.dtype)
    for r in range(n_shards):
        members = shard_members(L, n_shards, interleave, r)
        k, v = gather_shard(k_cache, v_cache, bt_b, L, r, n_shards, interleave, block_size, dv)
        K[members] = k
        V[members] = v
    return K, V


# ----------------------------------------------------------------------------------
# attention: [KVB] "Why does writing one token at a time duplicate work?" and
# "What does the KV cache hold?"; LSE: [DCP] DCP mechanism and configuration sections
# ----------------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one decode query over stored keys and values, fp64.

    ``q``: ``[Hq][dk]``; ``K``: ``[L][Hkv][dk]``; ``V``: ``[L][Hkv][dv]`` (any
    element type ``widen`` accepts).  Query head ``h`` reads KV head
    ``h // (Hq // Hkv)`` (reading: contiguous GQA groups).  Scores are
    ``scale * q.k``; weights are their softmax over the ``L`` tokens; the output is
    the weighted sum of values and ``lse`` the natural log of the sum of
    ``exp(score)``.  With ``L == 0`` the output is 0 and ``lse`` is ``-inf``.

    Returns ``o [Hq][dv]`` and ``lse [Hq]`` in float64.
    """
    qd = widen(q)
    Kd = widen(K)
    Vd = widen(V)
    hq = qd.shape[0]
    L, hkv = Kd.shape[0], Kd.shape[1]
    dv = Vd.shape[-1]
    group = hq // hkv
    o = np.zeros((hq, dv))
    lse = np.full(hq, NEG_INF)
    if L == 0:
        return o, lse
    for h in range(hq):
        kvh = h // group
        s = float(scale) * (Kd[:, kvh, :] @ qd[h])
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        o[h] = (p @ Vd[:, kvh, :]) / l
        lse[h] = m + np.log(l)
    return o, lse


def merge_lse(part_o: np.ndarray, part_lse: np.ndarray):
    """Combine attention results computed over disjoint token sets.

    [DCP] (DCP mechanism section) gathers the LSE of each rank's partial result,
    reweights each partial output, and sums.  Written out: with
    ``lse = log(sum_p exp(lse_p))``, the weight of part ``p`` is
    ``exp(lse_p - lse)`` (its share of the softmax denominator) and
    ``o = sum_p w_p * o_p``.  Parts with ``lse_p = -inf`` hold no tokens and get
    weight 0; if every part is empty the result is ``o = 0``, ``lse = -inf``.

    ``part_o``: ``[P][Hq][dv]``, ``part_lse``: ``[P][Hq]``; returns ``o [Hq][dv]``,
    ``lse [Hq]`` in float64.
    """
    po = np.asarray(part_o, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    hq, dv = po.shape[1], po.shape[2]
    o = np.zeros((hq, dv))
    lse = np.full(hq, NEG_INF)
    for h in range(hq):
        live = np.isfinite(pl[:, h])
        if not live.any():
            continue
        m = pl[live, h].max()
        total = m + np.log(np.exp(pl[live, h] - m).sum())
        w = np.exp(pl[live, h] - total)
        o[h] = w @ po[live, h, :]
        lse[h] = total
    return o, lse


def decode_partials(q, k_cache, v_cache, block_table, context_lens, n_shards: int,
                    interleave: int, block_size: int, partition_tokens: int,
                    max_partitions_: int, scale: float, dv: int):
    """Per-partition results of one decode step.

    Each shard's local token list is cut into partitions of ``partition_tokens``
    consecutive local tokens (the last one may be short); each partition is a
    separate attention over its tokens ([DCP]: local attention on each rank's
    own tokens, returning output and LSE).  Unused partition slots hold
    ``o = 0``, ``lse = -inf``.

    Returns ``part_o [N][S][Pmax][Hq][dv]`` and ``part_lse [N][S][Pmax][Hq]``.
    """
    n = q.shape[0]
    hq = q.shape[1]
    part_o = np.zeros((n, n_shards, max_partitions_, hq, dv))
    part_lse = np.full((n, n_shards, max_partitions_, hq), NEG_INF)
    for b in range(n):
        L = int(context_lens[b])
        for r in range(n_shards):
            K, V = gather_shard(k_cache, v_cache, block_table[b], L, r, n_shards, interleave,
                                block_size, dv)
            L_r = K.shape[0]
            p = 0
            while p * partition_tokens < L_r:
                lo, hi = p * partition_tokens, min((p + 1) * partition_tokens, L_r)
                part_o[b, r, p], part_lse[b, r, p] = attention(q[b], K[lo:hi], V[lo:hi], scale)
                p += 1
    return part_o, part_lse


def decode(q, k_cache, v_cache, block_table, context_lens, n_shards: int, interleave: int,
           block_size: int, partition_tokens: int, max_partitions_: int, scale: float, dv: int):
    """Final output of one decode step: the partition partials of every shard of
    a sequence merged by ``merge_lse``.  Returns ``o [N][Hq][dv]``, ``lse [N][Hq]``
    and the partials."""
    part_o, part_lse = decode_partials(q, k_cache, v_cache, block_table, context_lens, n_shards,
                                       interleave, block_size, partition_tokens, max_partitions_,
                                       scale, dv)
    n, hq = q.shape[0], q.shape[1]
    o = np.zeros((n, hq, dv))
    lse = np.full((n, hq), NEG_INF)
    for b in range(n):
        o[b], lse[b] = merge_lse(part_o[b].reshape(-1, hq, dv), part_lse[b].reshape(-1, hq))
    return o, lse, part_o, part_lse


def decode_step(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, n_shards: int,
                interleave: int, block_size: int, partition_tokens: int, max_partitions_: int,
                scale: float, dv: int):
    """The whole step: route each new token to its slot, append its K/V, then
    attend over every stored token ([KVB], "What does the KV cache hold?").

    Returns a dict with ``slots``, the updated ``k_cache``/``v_cache``, ``o``,
    ``lse``, ``part_o`` and ``part_lse``.
    """
    slots = slot_mapping(block_table, context_lens, n_shards, interleave, block_size)
    kc, vc = kv_append(k_cache, v_cache, k_new, v_new, slots, block_size)
    o, lse, part_o, part_lse = decode(q, kc, vc, block_table, context_lens, n_shards, interleave,
                                      block_size, partition_tokens, max_partitions_, scale, dv)
    return dict(slots=slots, k_cache=kc, v_cache=vc, o=o, lse=lse, part_o=part_o,
                part_lse=part_lse)
