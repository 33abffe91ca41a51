"""Seeded synthetic inputs for paged decode attention.

This module builds the INPUTS of one decode step -- context lengths, block
tables over a shuffled shared pool, K/V cache contents, queries and the new
tokens' K/V -- and nothing else.  It holds none of the attention arithmetic
(no scores, softmax, merge or expected values).  Tests, ``bench.py`` and the
smoke check feed the same tensors to the HIP library and to the fp64 oracle.

Like the scheduler of a serving system, it decides where each token's K/V
lives: a sequence's tokens are dealt to ``n_shards`` shards ``interleave`` at
a time (token i on shard (i // interleave) % n_shards), each shard keeps its
tokens in global order, and each shard's tokens fill blocks taken from the
pool one after another.  Unused blocks, the unused tail slots of last blocks
and the slot of the token the step appends are NaN-poisoned, so a kernel that
reads a value it should not read produces NaN instead of a silently plausible
number.

The five workloads:
``tiny`` (1 sequence, fp32), ``batch`` (continuous-batching step, 64 ragged
sequences), ``long`` (8 sequences with log-normal lengths around 142K),
``dcp`` (one 200K sequence split into 4 interleaved shards) and ``latent``
(128 query heads on one 576-wide latent head, shared 2,048-token prefixes).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"
FP8 = "fp8"      # cache element type only: OCP E4M3 codes with float32 scales


@dataclass
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    dk: int
    dv: int
    block_size: int
    dtype: str                          # q and new K/V rows (and the cache unless kv_dtype)
    context_lens: np.ndarray            # int32 [N], includes the appended token
    n_shards: int = 1
    interleave: int = 1
    partition_tokens: int = 0           # 0 -> chosen by the library binding
    scale: float = 0.0                  # 0 -> 1/sqrt(dk), rounded to fp32
    latent: bool = False                # V is the first dv entries of each K row
    prefix_group: int = 1               # sequences per shared-prefix group
    prefix_tokens: int = 0              # shared prefix length (multiple of block_size)
    spare_frac: float = 0.10            # extra never-used blocks in the pool
    n_blocks: int = 0                   # physical pool size (0 -> computed)
    seed: int = 0
    kv_dtype: str = ""                  # "" -> same as dtype; FP8 -> E4M3 codes
    scale_per_head: bool = True         # FP8: one scale per KV head (else one per tensor)
    q_lens: np.ndarray = None           # int32 [N]: new tokens per sequence (None: one each)
    # filled by plan():
    block_table: np.ndarray = field(default=None, repr=False)
    live: np.ndarray = field(default=None, repr=False)       # bool [NB][bs]: holds a stored token
    token_id: np.ndarray = field(default=None, repr=False)   # int64 [NB][bs]: global id, -1 unused
    new_slot: np.ndarray = field(default=None, repr=False)   # int64 [rows]: slots of the appended tokens

    @property
    def n_seqs(self) -> int:
        return int(len(self.context_lens))

    @property
    def multi(self) -> bool:
        return self.q_lens is not None

    @property
    def query_start(self) -> np.ndarray:
        """int32 [N+1]: rows query_start[b] .. query_start[b+1]-1 of q are sequence b's."""
        n = self.q_lens if self.multi else np.ones(self.n_seqs, np.int64)
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)

    @property
    def n_rows(self) -> int:
        return int(self.query_start[-1])

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return {F32: 4, BF16: 2, FP8: 1}[self.cache_dtype]

    @property
    def scale_f32(self) -> float:
        s = self.scale if self.scale else 1.0 / np.sqrt(self.dk)
        return float(np.float32(s))

    @property
    def max_blocks_per_shard(self) -> int:
        return int(self.block_table.shape[2])

    def kv_bytes_per_token(self) -> int:
        """Bytes of K and V read per token per step (V counted once when it is
        part of the K row)."""
        per_head = self.dk if self.latent else self.dk + self.dv
        return self.n_kv_heads * per_head * self.kv_elem_bytes


def _split_counts(L: int, n_shards: int, interleave: int) -> np.ndarray:
    """How many of tokens 0..L-1 each shard receives when they are dealt
    ``interleave`` at a time."""
    ids = np.arange(L, dtype=np.int64)
    return np.bincount((ids // interleave) % n_shards, minlength=n_shards)


def plan(w: Workload) -> Workload:
    """Lay the workload's tokens out in a shuffled physical pool."""
    rng = np.random.default_rng([w.seed, 1])
    N, S, I, bs = w.n_seqs, w.n_shards, w.interleave, w.block_size
    counts = [_split_counts(int(L), S, I) for L in w.context_lens]
    nblk = [[-(-int(c) // bs) for c in cs] for cs in counts]
    maxblk = max(1, max(max(r) for r in nblk))
    shared_blocks = w.prefix_tokens // bs
    if w.prefix_tokens:
        # the shared prefix is whole blocks and every sequence appends after it,
        # so no step writes into a shared block
        assert S == 1 and w.prefix_tokens % bs == 0
        assert int(np.min(w.context_lens)) > w.prefix_tokens
    need = sum(sum(r) for r in nblk)
    if shared_blocks:
        n_groups = -(-N // w.prefix_group)
        need -= (N - n_groups) * shared_blocks
    nb = w.n_blocks or int(np.ceil(need * (1.0 + w.spare_frac))) + 1
    assert nb >= need
    w.n_blocks = nb
    order = iter(rng.permutation(nb).tolist())

    bt = np.full((N, S, maxblk), -1, dtype=np.int32)
    live = np.zeros((nb, bs), dtype=bool)
    tok = np.full((nb, bs), -1, dtype=np.int64)
    new_slot = np.empty(N, dtype=np.int64)
    multi_slots: list = []
    if w.multi:
        w.q_lens = np.asarray(w.q_lens, dtype=np.int32)
        assert w.q_lens.shape == (N,)
    prefix_of_group: dict = {}
    for b in range(N):
        L = int(w.context_lens[b])
        for r in range(S):
            for j in range(nblk[b][r]):
                if shared_blocks and j < shared_blocks:
                    key = (b // w.prefix_group, j)
                    if key not in prefix_of_group:
                        prefix_of_group[key] = next(order)
                    bt[b, r, j] = prefix_of_group[key]
                else:
                    bt[b, r, j] = next(order)
        # global ids of each shard's tokens, in order, into their slots
        ids = np.arange(L, dtype=np.int64)
        shard = (ids // I) % S
        for r in range(S):
            mine = ids[shard == r]
            loc = np.arange(mine.size)
            phys = bt[b, r, loc // bs].astype(np.int64)
            live[phys, loc % bs] = True
            tok[phys, loc % bs] = mine
        if w.multi:                     # the last q_lens[b] tokens are new
            n_new = int(w.q_lens[b])
            assert 0 <= n_new <= L
            for pos in range(L - n_new, L):
                r_new = (pos // I) % S
                loc_new = int(_split_counts(pos, S, I)[r_new])   # earlier tokens on that shard
                multi_slots.append(int(bt[b, r_new, loc_new // bs]) * bs + loc_new % bs)
            continue
        if L == 0:                      # an empty sequence appends nothing
            new_slot[b] = -1
            continue
        r_new = ((L - 1) // I) % S
        loc_new = int(counts[b][r_new]) - 1
        phys_new = int(bt[b, r_new, loc_new // bs])
        new_slot[b] = phys_new * bs + loc_new % bs
    if w.multi:
        new_slot = np.array(multi_slots, dtype=np.int64)
    # the appended tokens' slots hold nothing until kv_append writes them
    for s in new_slot[new_slot >= 0]:
        live[s // bs, s % bs] = False
    w.block_table, w.live, w.token_id, w.new_slot = bt, live, tok, new_slot
    return w


# --------------------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------------------
def tiny(context_len: int = 67, seed: int = 1) -> Workload:
    """1 sequence, 4 query heads on 1 KV head, head 64, fp32, 4-token blocks,
    context 67 (new token included), 17 logical blocks in a 64-block pool."""
    w = Workload("tiny", 4, 1, 64, 64, 4, F32, np.array([context_len], np.int32), n_blocks=64,
                 scale=0.125, seed=seed)
    return plan(w)


def batch(seed: int = 2) -> Workload:
    """Continuous-batching step: 64 sequences of prompt U[8,32] + generated U[16,96]
    tokens, 32 query / 8 KV heads, head 128, bf16, 16-token blocks."""
    rng = np.random.default_rng(seed)
    prompt = rng.integers(8, 33, 64)
    gen = rng.integers(16, 97, 64)
    return plan(Workload("batch", 32, 8, 128, 128, 16, BF16, (prompt + gen).astype(np.int32),
                         seed=seed))


def long_lengths(seed: int = 2, n: int = 8) -> np.ndarray:
    rng = np.random.default_rng(seed)
    L = np.clip(np.rint(rng.lognormal(np.log(142000.0), 0.5, n)), 16384, 200000)
    return L.astype(np.int32)


def long(seed: int = 2, partition_tokens: int = 4096) -> Workload:
    """Long-context decode: 8 sequences, log-normal lengths (median 142,000,
    sigma 0.5, clipped to [16,384, 200,000]), 32/8 heads, head 128, bf16,
    16-token blocks, 4,096-token split-KV partitions."""
    return plan(Workload("long", 32, 8, 128, 128, 16, BF16, long_lengths(seed),
                         partition_tokens=partition_tokens, seed=seed))


def dcp(interleave: int = 1, n_shards: int = 4, context_len: int = 200000, seed: int = 4,
        partition_tokens: int = 0) -> Workload:
    """One 200,000-token sequence, 64/8 heads, head 128, bf16, 16-token blocks,
    split into ``n_shards`` interleaved shards."""
    return plan(Workload(f"dcp_S{n_shards}_I{interleave}", 64, 8, 128, 128, 16, BF16,
                         np.array([context_len], np.int32), n_shards=n_shards,
                         interleave=interleave, partition_tokens=partition_tokens, seed=seed))


def latent(seed: int = 5, n_seqs: int = 32, lo: int = 4096, hi: int = 65536,
           q_len: int = 0) -> Workload:
    """Latent (MLA-style) cache: 32 sequences, 128 query heads on 1 KV head, key
    width 576 with the value the first 512 entries, context U[4,096, 65,536],
    bf16, 64-token blocks; groups of 4 sequences share a 2,048-token prefix.
    ``q_len`` > 0: each sequence's last ``q_len`` tokens are new (speculative
    verification, causal among themselves)."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi + 1, n_seqs).astype(np.int32)
    return plan(Workload(f"latent_spec{q_len}" if q_len else "latent", 128, 1, 576, 512, 64, BF16, L,
                         latent=True, prefix_group=4, prefix_tokens=2048, seed=seed,
                         q_lens=np.full(L.size, q_len, np.int32) if q_len else None))


def small(name: str, lens, hq: int, hkv: int, dk: int, dv: int, bs: int, dtype: str,
          n_shards: int = 1, interleave: int = 1, partition_tokens: int = 0, latent: bool = False,
          seed: int = 0, prefix_group: int = 1, prefix_tokens: int = 0, scale: float = 0.0,
          kv_dtype: str = "", scale_per_head: bool = True, q_lens=None) -> Workload:
    """Any small shape, for parity sweeps (``q_lens``: new tokens per sequence)."""
    return plan(Workload(name, hq, hkv, dk, dv, bs, dtype, np.asarray(lens, np.int32),
                         n_shards=n_shards, interleave=interleave,
                         partition_tokens=partition_tokens, latent=latent, seed=seed,
                         prefix_group=prefix_group, prefix_tokens=prefix_tokens, scale=scale,
                         kv_dtype=kv_dtype, scale_per_head=scale_per_head,
                         q_lens=None if q_lens is None else np.asarray(q_lens, np.int32)))


def speculative(seed: int = 2, q_len: int = 4) -> Workload:
    """Verification of speculative tokens on the long-context batch: the 8 log-normal
    sequences of ``long`` each bring ``q_len`` new tokens (the last of the context),
    causal among themselves; 32/8 heads, head 128, bf16, 16-token blocks."""
    L = long_lengths(seed)
    return plan(Workload(f"spec{q_len}", 32, 8, 128, 128, 16, BF16, L, seed=seed,
                         q_lens=np.full(L.size, q_len, np.int32)))


def with_fp8_cache(w: Workload, per_head: bool = True) -> Workload:
    """The same workload (same layout and seed) with an E4M3 cache."""
    import dataclasses

    w2 = dataclasses.replace(w, name=w.name + "_fp8", kv_dtype=FP8, scale_per_head=per_head)
    return w2


# --------------------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------------------
def make_tensors(w: Workload, device="cpu", fill: str = "normal", seed: int | None = None):
    """Torch tensors of the workload on ``device``.

    ``fill="normal"``: q, K, V and the new tokens' K/V are N(0,1) drawn in fp32
    and rounded to the workload's element type (round-to-nearest-even for bf16).
    ``fill="mean_probe"``: q = 0 (every score is 0) and the value of token t in
    dimension j is (31 t + j) mod 16, exactly representable in bf16, so the
    attention output is exactly the mean of the values.

    Returns a dict with ``q [N][Hq][dk]``, ``k_new [N][Hkv][dk]``,
    ``v_new [N][Hkv][dv]`` (None for latent), ``k_cache [NB][Hkv][bs][dk]``,
    ``v_cache [NB][Hkv][dv][bs]`` (None for latent), ``block_table``,
    ``context_lens`` and ``slot_mapping`` (int64, where the generator put the new
    tokens; the library computes its own).

    An FP8 cache (``w.kv_dtype == FP8``) holds uint8 E4M3 codes: fp32 normals times
    16 cast by torch's float8_e4m3fn conversion (values of roughly N(0, 16^2));
    unused slots hold the NaN code 0x7F.  The dict then also has ``k_scale`` and
    ``v_scale`` (float32, one per KV head or one per tensor, drawn from
    U[0.5, 2] / 16, so the stored values read back as roughly N(0, 1)); new rows
    and q stay in ``w.dtype``.  ``mean_probe`` is not available for FP8.
    """
    import torch

    dt = torch.float32 if w.dtype == F32 else torch.bfloat16
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(w.seed if seed is None else seed) * 1000003 + 7)
    N, Hq, Hkv, dk, dv, bs, NB = w.n_seqs, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size, w.n_blocks
    R = w.n_rows                        # query rows (one per new token)

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(dt)

    live = torch.from_numpy(w.live).to(dev)
    if w.cache_dtype == FP8:
        if fill != "normal":
            raise ValueError("an FP8 cache takes fill='normal' only")

        def codes(*shape):
            x = torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * 16.0
            return x.to(torch.float8_e4m3fn).view(torch.uint8)

        k_cache = codes(NB, Hkv, bs, dk)
        v_cache = None if w.latent else codes(NB, Hkv, dv, bs)
        q = randn(R, Hq, dk)
        k_new = randn(R, Hkv, dk)
        v_new = None if w.latent else randn(R, Hkv, dv)
        n_sc = Hkv if w.scale_per_head else 1
        k_scale = (0.5 + 1.5 * torch.rand(n_sc, generator=g, device=dev)) / 16.0
        v_scale = None if w.latent else (0.5 + 1.5 * torch.rand(n_sc, generator=g, device=dev)) / 16.0
        k_cache.masked_fill_(~live[:, None, :, None], 0x7F)
        if v_cache is not None:
            v_cache.masked_fill_(~live[:, None, None, :], 0x7F)
        return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                    k_scale=k_scale, v_scale=v_scale,
                    block_table=torch.from_numpy(w.block_table).to(dev),
                    context_lens=torch.from_numpy(w.context_lens.astype(np.int32)).to(dev),
                    slot_mapping=torch.from_numpy(w.new_slot).to(dev),
                    query_start=torch.from_numpy(w.query_start).to(dev))
    k_cache = randn(NB, Hkv, bs, dk)
    v_cache = None if w.latent else randn(NB, Hkv, dv, bs)
    q = randn(R, Hq, dk)
    k_new = randn(R, Hkv, dk)
    v_new = None if w.latent else randn(R, Hkv, dv)
    if fill == "mean_probe":
        if w.multi:
            raise ValueError("mean_probe is for one new token per sequence")
        q.zero_()
        tid = torch.from_numpy(w.token_id).to(dev)                    # [NB][bs]
        j = torch.arange(dv, device=dev)
        val = ((31 * tid[:, :, None] + j[None, None, :]) % 16).to(dt)  # [NB][bs][dv]
        if w.latent:
            k_cache[..., :dv] = val[:, None, :, :].expand(NB, Hkv, bs, dv)
        else:
            v_cache.copy_(val.transpose(1, 2)[:, None, :, :].expand(NB, Hkv, dv, bs))
        Lm1 = torch.from_numpy(np.maximum(w.context_lens.astype(np.int64) - 1, 0)).to(dev)
        newv = ((31 * Lm1[:, None] + j[None, :]) % 16).to(dt)         # [N][dv]
        if w.latent:
            k_new[..., :dv] = newv[:, None, :]
        else:
            v_new.copy_(newv[:, None, :].expand(N, Hkv, dv))
    elif fill != "normal":
        raise ValueError(fill)
    nan = float("nan")
    k_cache.masked_fill_(~live[:, None, :, None], nan)
    if v_cache is not None:
        v_cache.masked_fill_(~live[:, None, None, :], nan)
    return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                block_table=torch.from_numpy(w.block_table).to(dev),
                context_lens=torch.from_numpy(w.context_lens.astype(np.int32)).to(dev),
                slot_mapping=torch.from_numpy(w.new_slot).to(dev),
                query_start=torch.from_numpy(w.query_start).to(dev))
