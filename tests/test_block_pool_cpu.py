"""The native block pool (pa_pool_* in include/pa.h) against the oracle's
BlockManager, on the CPU: the page's worked example, then random sequences of
add / append / fork / finish.  The pool is all-or-nothing where the oracle stops
part-way, so an operation the pool refuses with PoolExhausted is checked to raise
in a copy of the oracle and is then left out of both."""
import copy
import ctypes

import numpy as np
import pytest

pytest.importorskip("torch")
P = pytest.importorskip("decode_attention_paged_kv_amd")
from oracle import block_manager as bm  # noqa: E402


def same_state(pool, m, seqs):
    assert pool.num_free() == m.num_free()
    for s in seqs:
        assert pool.table(s) == m.tables[s], s
        assert pool.length(s) == m.lengths[s]
        assert pool.num_blocks(s) == m.num_blocks(s)
    for b, r in m.refcount.items():
        assert pool.refcount(b) == r, b


def test_worked_example(golden):
    g = golden("pa_block_reuse_example.json")
    bs = g["block_size"]
    pool = P.BlockPool(16, bs)
    pool.add(0, g["requests"]["A"])
    pool.add(1, g["requests"]["B"])
    assert pool.num_blocks(0) == g["blocks"]["A"] and pool.num_blocks(1) == g["blocks"]["B"]
    spare = (pool.num_blocks(0) + pool.num_blocks(1)) * bs - g["tokens_stored"]
    assert spare == g["slots_spare"]
    pool.append(1, g["B_grows_to_without_new_block"] - g["requests"]["B"])
    assert pool.num_blocks(1) == g["blocks"]["B"]
    pool.append(1, 1)
    assert pool.num_blocks(1) == g["B_blocks_at_13_tokens"]
    free = pool.num_free()
    pool.finish(0)
    assert pool.num_free() - free == g["A_blocks_returned_on_finish"]


def test_copy_on_write_of_a_shared_last_block():
    pool = P.BlockPool(8, 4)
    pool.add(7, 6)                      # blocks 0, 1; block 1 half full
    pool.fork(7, 8)
    assert pool.refcount(0) == 2 and pool.refcount(1) == 2
    assert pool.append(8, 1) == [(1, 2)]  # child writes into the shared block: copy first
    assert pool.table(8) == [0, 2] and pool.refcount(1) == 1 and pool.refcount(2) == 1
    assert pool.append(7, 1) == []      # parent's block 1 is now its own
    assert pool.append(7, 2) == []      # fills block 1 then takes a new one
    assert pool.table(7) == [0, 1, 3]
    pool.fork(7, 9)                     # block 3 holds 1 token, shared
    pool.finish(7)
    assert pool.append(9, 1) == []      # sole owner again: no copy
    pool.finish(8)
    pool.finish(9)
    assert pool.num_free() == 8


def test_full_shared_last_block_needs_no_copy():
    pool = P.BlockPool(4, 4)
    pool.add(0, 4)
    pool.fork(0, 1)
    assert pool.append(1, 1) == []
    assert pool.table(1) == [0, 1] and pool.refcount(0) == 2


def test_exhaustion_changes_nothing():
    pool = P.BlockPool(3, 4)
    pool.add(0, 5)                      # 2 blocks
    pool.fork(0, 1)                     # shares both
    with pytest.raises(P.PoolExhausted):
        pool.append(1, 8)               # needs a copy plus 2 new blocks, 1 free
    assert pool.length(1) == 5 and pool.table(1) == [0, 1] and pool.num_free() == 1
    with pytest.raises(P.PoolExhausted):
        pool.add(2, 9)
    assert pool.length(2) == -1
    assert pool.append(1, 3) == [(1, 2)]  # copy only: fits


def test_errors():
    pool = P.BlockPool(4, 4)
    pool.add(0, 1)
    with pytest.raises(P.PaError) as e:
        pool.add(0, 1)
    assert e.value.status == -7
    for call in (lambda: pool.append(5, 1), lambda: pool.finish(5), lambda: pool.fork(5, 6),
                 lambda: pool.fork(0, 0)):
        with pytest.raises(P.PaError) as e:
            call()
        assert e.value.status == -7
    with pytest.raises(P.PaError) as e:
        pool.append(0, -1)
    assert e.value.status == -2
    assert pool.refcount(4) == -1 and pool.refcount(-1) == -1
    assert P.lib.pa_pool_create(-1, 4) is None and P.lib.pa_pool_create(4, 0) is None
    assert P.lib.pa_pool_add(None, 0, 0) == -1
    assert P.lib.pa_pool_num_free(None) == -1
    # a copy with no room to report it is refused before anything changes
    pool.fork(0, 1)
    made = ctypes.c_int32(-5)
    assert P.lib.pa_pool_append(pool._h, 1, 1, None, 0, ctypes.byref(made)) == -4
    assert pool.length(1) == 1 and pool.refcount(0) == 2
    # too small a table buffer
    buf = (ctypes.c_int32 * 1)()
    assert P.lib.pa_pool_table(pool._h, 0, buf, 0) == -1


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_oracle(seed):
    rng = np.random.default_rng(seed)
    n_blocks = int(rng.integers(8, 40))
    bs = int(rng.choice([1, 2, 4, 16]))
    pool = P.BlockPool(n_blocks, bs)
    m = bm.BlockManager(n_blocks, bs)
    live, next_id, refused = [], 0, 0
    for _ in range(400):
        op = rng.choice(["add", "append", "append", "append", "fork", "finish"])
        if op == "add" or not live:
            n = int(rng.integers(0, 3 * bs + 1))
            trial = copy.deepcopy(m)
            try:
                trial.add(next_id, n)
                ok_oracle = True
            except bm.PoolExhausted:
                ok_oracle = False
            try:
                pool.add(next_id, n)
                assert ok_oracle
                m = trial
                live.append(next_id)
            except P.PoolExhausted:
                assert not ok_oracle
                refused += 1
            next_id += 1
        elif op == "append":
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(1, 2 * bs + 2))
            trial = copy.deepcopy(m)
            before = len(trial.copies)
            try:
                trial.append(s, n)
                ok_oracle = True
            except bm.PoolExhausted:
                ok_oracle = False
            try:
                got = pool.append(s, n)
                assert ok_oracle
                assert got == trial.copies[before:]
                m = trial
            except P.PoolExhausted:
                assert not ok_oracle
                refused += 1
        elif op == "fork":
            s = live[int(rng.integers(len(live)))]
            pool.fork(s, next_id)
            m.fork(s, next_id)
            live.append(next_id)
            next_id += 1
        else:
            s = live.pop(int(rng.integers(len(live))))
            pool.finish(s)
            m.finish(s)
        same_state(pool, m, live)
    for s in live:
        pool.finish(s)
    assert pool.num_free() == n_blocks


def test_copy_blocks_rejects_bad_arguments_without_launch():
    vp = ctypes.c_void_p(0x1000)
    f = P.lib.pa_copy_blocks
    assert f(None, vp, vp, 1, 1, 64, 64, 4, 64, 0, None, None) == -1
    assert f(vp, vp, None, 1, 1, 64, 64, 4, 64, 0, None, None) == -1
    assert f(vp, vp, vp, -1, 1, 64, 64, 4, 64, 0, None, None) == -2
    assert f(vp, vp, vp, 1, 0, 64, 64, 4, 64, 0, None, None) == -2
    assert f(vp, vp, vp, 1, 1, 577, 64, 4, 64, 0, None, None) == -3
    assert f(vp, vp, vp, 1, 1, 64, 0, 4, 64, 0, None, None) == -3
    assert f(vp, vp, vp, 1, 1, 64, 64, 257, 64, 0, None, None) == -3
    assert f(vp, vp, vp, 1, 1, 64, 64, 4, 0, 0, None, None) == -2
    assert f(vp, vp, vp, 1, 1, 64, 64, 4, 64, 9, None, None) == -3
    assert P.lib.pa_last_error().decode() != ""
    assert f(vp, None, vp, 0, 1, 64, 0, 4, 64, 1, None, None) == 0   # nothing to copy
