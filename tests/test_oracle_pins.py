"""The fp64 oracle against brute force, closed forms, invariants, a library
routine and the pages' worked examples (CPU only)."""
import numpy as np
import pytest

import oracle_checks as oc
from oracle import block_manager as bm
from oracle import paged_attention as pa


@pytest.mark.parametrize("name", sorted(oc.ALL_CHECKS))
def test_pin(name):
    msg = oc.ALL_CHECKS[name]()
    assert msg is None, msg


def test_empty_attention_and_merge():
    o, lse = pa.attention(np.ones((2, 3)), np.zeros((0, 1, 3)), np.zeros((0, 1, 4)), 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # empty parts carry no weight; all-empty merges to (0, -inf)
    po = np.stack([np.full((2, 4), 7.0), np.zeros((2, 4))])
    pl = np.array([[0.5, -np.inf], [-np.inf, -np.inf]])
    o, lse = pa.merge_lse(po, pl)
    assert np.array_equal(o[0], po[0, 0]) and lse[0] == 0.5
    assert np.all(o[1] == 0) and lse[1] == -np.inf


def test_needle():
    """One key aligned with the query and scaled up dominates: the output is that
    token's value to within exp(-gap)."""
    r = np.random.default_rng(5)
    L, dk, dv = 300, 16, 8
    q = r.standard_normal((1, dk))
    K = 0.1 * r.standard_normal((L, 1, dk))
    V = r.standard_normal((L, 1, dv))
    pos = 173
    K[pos, 0] = 60.0 * q[0] / np.linalg.norm(q[0]) ** 2       # score 60 * scale
    o, lse = pa.attention(q, K, V, 1.0)
    assert np.max(np.abs(o[0] - V[pos, 0])) < 1e-20 + 10 * np.exp(-50)
    assert abs(lse[0] - 60.0) < 1e-12


def test_permutation_invariance():
    """The same logical content under two different physical placements gives
    bitwise identical results (the block table keeps order; placement is free)."""
    import workloads as wl

    outs = []
    for seed in (41, 42):
        w = wl.small("p", [13, 40], 4, 2, 8, 8, 4, wl.BF16, n_shards=2, interleave=3,
                     partition_tokens=8, seed=seed)
        r = np.random.default_rng(0)
        Kl = r.standard_normal((2, 40, 2, 8)).astype(np.float32)
        Vl = r.standard_normal((2, 40, 2, 8)).astype(np.float32)
        T = oc.tensors_np(w)
        kc = np.full_like(pa.widen(T["k_cache"]).astype(np.float32), np.nan)
        vc = np.full_like(pa.widen(T["v_cache"]).astype(np.float32), np.nan)
        for b in range(2):
            for r_ in range(2):
                for phys in w.block_table[b, r_]:
                    if phys < 0:
                        continue
                    for o in range(4):
                        i = w.token_id[phys, o]
                        if i >= 0 and w.live[phys, o]:
                            kc[phys, :, o, :] = Kl[b, i]
                            vc[phys, :, :, o] = Vl[b, i]
        q = r.standard_normal((2, 4, 8)).astype(np.float32)
        kn = np.stack([Kl[b, int(w.context_lens[b]) - 1] for b in range(2)])
        vn = np.stack([Vl[b, int(w.context_lens[b]) - 1] for b in range(2)])
        res = pa.decode_step(q, kn, vn, kc, vc, w.block_table, w.context_lens, 2, 3, 4, 8,
                             pa.max_partitions(40, 2, 3, 8), 0.25, 8)
        outs.append((res["o"], res["lse"]))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_kv_append_is_a_slot_copy():
    """After the append every slot holds what it held before except the new
    tokens' slots, which hold the new rows; read through a slot-major view."""
    import workloads as wl

    for w in (wl.small("a", [5, 9, 12], 4, 2, 8, 8, 4, wl.BF16, seed=3),
              wl.small("b", [20, 33], 8, 1, 12, 8, 8, wl.F32, latent=True, seed=4)):
        T = oc.tensors_np(w)
        kc, vc = pa.kv_append(T["k_cache"], T["v_cache"], T["k_new"], T["v_new"], w.new_slot,
                              w.block_size)
        NB, hkv, bs, dk = T["k_cache"].shape
        before = T["k_cache"].transpose(0, 2, 1, 3).reshape(NB * bs, hkv, dk).view(np.uint8)
        after = kc.transpose(0, 2, 1, 3).reshape(NB * bs, hkv, dk).view(np.uint8)
        changed = np.nonzero(np.any(before.reshape(NB * bs, -1) != after.reshape(NB * bs, -1), 1))[0]
        assert set(changed) <= set(w.new_slot.tolist())
        for n, s in enumerate(w.new_slot):
            assert np.array_equal(after[s], T["k_new"][n].view(np.uint8))
        if vc is not None:
            vb = T["v_cache"].transpose(0, 3, 1, 2).reshape(NB * bs, hkv, -1)
            va = vc.transpose(0, 3, 1, 2).reshape(NB * bs, hkv, -1)
            keep = np.ones(NB * bs, bool)
            keep[w.new_slot] = False
            assert np.array_equal(vb[keep].view(np.uint8), va[keep].view(np.uint8))
            for n, s in enumerate(w.new_slot):
                assert np.array_equal(va[s].view(np.uint8), T["v_new"][n].view(np.uint8))
    # a negative slot is padding and writes nothing
    k0 = np.zeros((2, 1, 4, 3), np.float32)
    k1, _ = pa.kv_append(k0, None, np.ones((1, 1, 3), np.float32), None, np.array([-1]), 4)
    assert np.array_equal(k0, k1)


# ---------------------------------------------------------------- the pages' worked examples
def test_block_reuse_example(golden):
    g = golden("pa_block_reuse_example.json")
    bs = g["block_size"]
    m = bm.BlockManager(16, bs)
    for name, n in g["requests"].items():
        m.add(name, n)
        assert m.num_blocks(name) == g["blocks"][name] == pa.blocks_needed(n, bs)
    assert sum(g["requests"].values()) == g["tokens_stored"]
    assert sum(m.num_blocks(k) for k in g["requests"]) * bs == g["slots_reserved"]
    assert sum(m.spare_slots(k) for k in g["requests"]) == g["slots_spare"]
    a_blocks = list(m.tables["A"])
    m.finish("A")
    assert m.num_free() == 16 - 3 and len(a_blocks) == g["A_blocks_returned_on_finish"]
    m.add("C", 1)                                   # C may take one of A's blocks
    assert m.tables["C"][0] in a_blocks or m.num_free() >= 1
    m.append("B", g["B_grows_to_without_new_block"] - g["requests"]["B"])
    assert m.num_blocks("B") == g["blocks"]["B"]
    m.append("B", 1)
    assert m.num_blocks("B") == g["B_blocks_at_13_tokens"]
    assert m.lengths["B"] == 13


def test_block_reuse_takes_freed_blocks():
    """With only the freed blocks left, a new request gets exactly those, in any
    position of the pool (no compaction)."""
    m = bm.BlockManager(5, 4)
    m.add("A", 6)
    m.add("B", 9)
    freed = set(m.tables["A"])
    m.finish("A")
    m.add("C", 8)
    assert set(m.tables["C"]) == freed
    with pytest.raises(bm.PoolExhausted):
        m.add("D", 1)


def test_copy_on_write():
    """A forked sequence shares every block; writing into the shared, not yet full
    last block copies it first, and only that block; a shared block is released
    only when its last user finishes."""
    m = bm.BlockManager(100, 64)
    m.add("P", 2050)                                 # 33 blocks, last holds 2 tokens
    for c in ("c1", "c2", "c3"):
        m.fork("P", c)
    assert all(m.refcount[b] == 4 for b in m.tables["P"])
    m.append("c1", 1)
    assert len(m.copies) == 1 and m.copies[0][0] == m.tables["P"][-1]
    assert m.tables["c1"][:-1] == m.tables["P"][:-1] and m.tables["c1"][-1] != m.tables["P"][-1]
    assert m.refcount[m.tables["P"][-1]] == 3
    # an aligned prefix (full last block) needs no copy: the append takes a new block
    m2 = bm.BlockManager(100, 64)
    m2.add("P", 2048)
    m2.fork("P", "c")
    m2.append("c", 1)
    assert m2.copies == [] and m2.num_blocks("c") == 33
    free0 = m.num_free()
    m.finish("P")
    assert m.num_free() == free0                     # still used by c2, c3 (and c1's prefix)
    for c in ("c1", "c2", "c3"):
        m.finish(c)
    assert m.num_free() == 100


def test_bytes_per_token_example(golden):
    g = golden("kvb_bytes_per_token.json")
    b = pa.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert b == g["bytes_per_token"] == g["kib_per_token"] * 1024
    assert b * g["request_tokens"] == g["mib_per_request"] * 2 ** 20
    # one layer of the 32/8/128 bf16 workloads: 4,096 B per token
    assert pa.kv_bytes_per_token(1, 8, 128, 2) == 4096


def test_dcp_interleave_example(golden):
    g = golden("dcp_interleave_example.json")
    S = g["dcp_size"]
    for i, r in g["interleave_1_first_tokens_rank"]:
        assert pa.shard_of_token(i, S, 1) == r
    for I in (1, 16):
        lens = pa.shard_lengths(g["request_tokens"], S, I)
        assert np.all(np.abs(lens - g["tokens_per_rank_approx"]) <= I)
        assert lens.sum() == g["request_tokens"]
        m0 = pa.shard_members(g["request_tokens"], S, I, 0)
        contiguous = m0[-1] - m0[0] + 1 == m0.size
        assert contiguous == g["contiguous_ranges"]


def test_shard_lengths_small():
    # a short sequence leaves later shards empty when L < S * I
    assert list(pa.shard_lengths(5, 4, 16)) == [5, 0, 0, 0]
    assert list(pa.shard_lengths(67, 4, 1)) == [17, 17, 17, 16]
    assert list(pa.shard_lengths(67, 4, 16)) == [19, 16, 16, 16]
    assert pa.max_partitions(200000, 4, 16, 1024) == 49
    assert pa.blocks_needed(0, 4) == 0 and pa.blocks_needed(6, 4) == 2 and pa.blocks_needed(9, 4) == 3
