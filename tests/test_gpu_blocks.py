"""Block copies and copy-on-write on the GPU against the oracle.

``pa_copy_blocks`` is compared bit for bit with the oracle's ``copy_blocks`` for
several cache layouts (word sizes 16, 4 and 2 bytes), with invalid pairs skipped
and flagged.  The end-to-end test drives the native block pool through a fork and
several decode steps: each step's copy-on-write copies go to ``pa_copy_blocks``,
then the library's step (route, append, attend, merge) runs on the pool's tables;
the oracle runs the same steps with its own block manager, block copy and decode.
Appends cross block boundaries on the way."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import bits_equal, compare_outputs, say, to_np
from oracle import block_manager as bm
from oracle import paged_attention as pa

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


def _rand(rng, shape, dtype):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dtype)


@pytest.mark.parametrize("dtype,hkv,dk,dv,bs,latent", [
    (torch.bfloat16, 8, 128, 128, 16, False),   # 32 KiB blocks, 16-byte words
    (torch.float32, 2, 64, 48, 4, False),
    (torch.bfloat16, 1, 576, 512, 64, True),    # latent cache: keys only
    (torch.bfloat16, 1, 3, 5, 1, False),        # 6- and 10-byte blocks: 2-byte words
    (torch.float32, 3, 1, 1, 1, False),         # 12-byte blocks: 4-byte words
])
def test_copy_blocks_bitexact(dtype, hkv, dk, dv, bs, latent):
    import decode_attention_paged_kv_amd as P

    say(f"[copy_blocks] {dtype} hkv={hkv} dk={dk} dv={dv} bs={bs} latent={latent}")
    rng = np.random.default_rng(hkv * 1000 + dk + bs)
    nb = 40
    k = _rand(rng, (nb, hkv, bs, dk), dtype)
    v = None if latent else _rand(rng, (nb, hkv, dv, bs), dtype)
    pairs = [(3, 7), (3, 9), (12, 12), (0, 38), (39, 1), (5, nb), (-1, 2)]
    valid = [(s, d) for s, d in pairs if 0 <= s < nb and 0 <= d < nb]
    k_ref, v_ref = pa.copy_blocks(to_np(k), to_np(v), valid)
    dev = torch.device("cuda")
    kd, vd = k.to(dev), None if v is None else v.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int64, device=dev), flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == P.ERR_BLOCK_ID
    assert bits_equal(to_np(kd), k_ref)
    if v is not None:
        assert bits_equal(to_np(vd), v_ref)


def test_copy_blocks_many_pairs():
    """4,096 copies in one call at the long-context layout (8 KV heads, head 128,
    16-token bf16 blocks)."""
    import decode_attention_paged_kv_amd as P

    rng = np.random.default_rng(5)
    nb, hkv, bs, d = 10240, 8, 16, 128
    say(f"[copy_blocks] {nb} blocks, 4096 pairs")
    g = torch.Generator().manual_seed(5)
    # arbitrary bit patterns (NaNs included): the copy must move bits, not values
    k = torch.randint(-32768, 32768, (nb, hkv, bs, d), dtype=torch.int16, generator=g).view(torch.bfloat16)
    v = torch.randint(-32768, 32768, (nb, hkv, d, bs), dtype=torch.int16, generator=g).view(torch.bfloat16)
    perm = rng.permutation(nb)
    src = rng.choice(perm[:4096], 4096)          # sources may repeat
    dst = perm[4096:8192]                        # destinations distinct, never a source
    pairs = np.stack([src, dst], axis=1).astype(np.int64)
    k_ref, v_ref = pa.copy_blocks(to_np(k), to_np(v), pairs)
    dev = torch.device("cuda")
    kd, vd = k.to(dev), v.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_copy_blocks(kd, vd, torch.from_numpy(pairs).to(dev), flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert bits_equal(to_np(kd), k_ref) and bits_equal(to_np(vd), v_ref)


@pytest.mark.parametrize("dtype,hq,hkv,dk,dv,bs,latent", [
    (wl.BF16, 32, 8, 128, 128, 16, False),
    (wl.F32, 4, 1, 64, 64, 4, False),
    (wl.BF16, 128, 1, 576, 512, 64, True),
])
def test_copy_on_write_decode_steps(dtype, hq, hkv, dk, dv, bs, latent):
    import decode_attention_paged_kv_amd as P

    say(f"[cow-steps] {dtype} hq={hq} hkv={hkv} dk={dk} dv={dv} bs={bs} latent={latent}")
    tdt = torch.bfloat16 if dtype == wl.BF16 else torch.float32
    rng = np.random.default_rng(bs * 7 + hq)
    dev = torch.device("cuda")
    nb, n_seqs, steps = 48, 4, 5
    L0 = 3 * bs - 2                              # last block of the prefix has 2 free slots
    kc = torch.zeros(nb, hkv, bs, dk, dtype=tdt)
    vc = None if latent else torch.zeros(nb, hkv, dv, bs, dtype=tdt)
    pool = P.BlockPool(nb, bs)
    man = bm.BlockManager(nb, bs)
    # the shared prefix, written through the library's append on one side and the
    # oracle's on the other
    pool.add(0, L0)
    man.add(0, L0)
    assert pool.table(0) == man.tables[0]
    t = np.arange(L0)
    slots = np.array(man.tables[0], np.int64)[t // bs] * bs + t % bs
    k_new = _rand(rng, (L0, hkv, dk), tdt)
    v_new = None if latent else _rand(rng, (L0, hkv, dv), tdt)
    k_ref, v_ref = pa.kv_append(to_np(kc), to_np(vc), to_np(k_new), to_np(v_new), slots, bs)
    kd, vd = kc.to(dev), None if vc is None else vc.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_kv_append(k_new.to(dev), None if v_new is None else v_new.to(dev), kd, vd,
                   torch.from_numpy(slots).to(dev), flag)
    for c in range(1, n_seqs):
        pool.fork(0, c)
        man.fork(0, c)
    max_len = L0 + steps
    max_blocks = -(-max_len // bs)
    Tp = 2 * bs
    step = P.DecodeStep(n_seqs, hq, hkv, dk, dv, bs, max_len, 1, 1, Tp, None, device=dev,
                        kv_dtype=tdt, latent=latent)
    n_copies = 0
    for it in range(steps):
        copies = []
        for s in range(n_seqs):
            got = pool.append(s, 1)
            before = len(man.copies)
            man.append(s, 1)
            assert got == man.copies[before:], (it, s)
            copies += got
        n_copies += len(copies)
        if copies:
            P.pa_copy_blocks(kd, vd, torch.tensor(copies, dtype=torch.int64, device=dev), flag)
            k_ref, v_ref = pa.copy_blocks(k_ref, v_ref, copies)
        bt = np.full((n_seqs, 1, max_blocks), -1, np.int32)
        lens = np.zeros(n_seqs, np.int32)
        for s in range(n_seqs):
            assert pool.table(s) == man.tables[s]
            bt[s, 0, :len(man.tables[s])] = man.tables[s]
            lens[s] = man.lengths[s]
        q = _rand(rng, (n_seqs, hq, dk), tdt)
        kn = _rand(rng, (n_seqs, hkv, dk), tdt)
        vn = None if latent else _rand(rng, (n_seqs, hkv, dv), tdt)
        step(q.to(dev), kn.to(dev), None if vn is None else vn.to(dev), kd, vd,
             torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev))
        torch.cuda.synchronize()
        ref = pa.decode_step(to_np(q), to_np(kn), to_np(vn), k_ref, v_ref, bt, lens, 1, 1, bs, Tp,
                             step.max_partitions, step.scale, dv)
        k_ref, v_ref = ref["k_cache"], ref["v_cache"]
        assert int(step.err_flag.item()) == 0 and int(flag.item()) == 0
        assert bits_equal(to_np(kd), k_ref), f"step {it}: k_cache"
        if v_ref is not None:
            assert bits_equal(to_np(vd), v_ref), f"step {it}: v_cache"
        compare_outputs(f"cow step {it}", dtype, to_np(step.out), to_np(step.lse), ref["o"],
                        ref["lse"])
    assert n_copies == n_seqs - 1                # only the first write into the shared block copies
    assert max(pool.num_blocks(s) for s in range(n_seqs)) == max_blocks
