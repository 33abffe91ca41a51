"""Pools larger than 4 GiB, with a workload's blocks at the top of the pool.

Byte offsets into such a pool pass 2^32 (and element offsets 2^31), so any 32-bit
offset arithmetic in a kernel would read or write the wrong place.  The same logical
content is placed twice: in a pool of its own size and at the highest block ids of a
pool of more than 4 GiB per tensor (the rest poisoned).  Placement does not change
the result, and the kernels reduce in logical order, so the whole step's output and
LSE must agree bit for bit, the appended rows must land at the same place relative
to the content, the poisoned part must be untouched, and the gather and block copy
must move the same bytes.  Covered: the bf16 MFMA kernel, the E4M3 cache, the latent
kernel and the generic one (fp32).  Also a batch of more than 65,535 (sequence, shard)
pairs, which the decode grids must take."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import check_large, run_library, say

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# name, workload, blocks in the large pool (each key cache > 4 GiB)
CASES = [
    ("bf16", lambda: wl.small("big_bf16", [700, 77, 1025], 32, 8, 128, 128, 16, wl.BF16,
                              partition_tokens=256, seed=21), 140_000),          # 32 KiB blocks
    ("e4m3", lambda: wl.small("big_e4m3", [700, 77, 1025], 32, 8, 128, 128, 16, wl.BF16,
                              partition_tokens=256, seed=22, kv_dtype=wl.FP8), 280_000),
    ("latent", lambda: wl.small("big_latent", [300, 1100], 16, 1, 576, 512, 64, wl.BF16,
                                partition_tokens=256, seed=23, latent=True), 60_000),  # 72 KiB
    ("generic_f32", lambda: wl.small("big_f32", [300, 41], 8, 2, 96, 80, 16, wl.F32,
                                     partition_tokens=64, seed=24), 720_000),     # 12 KiB keys
]
# Every case also passes 2^31 elements per tensor (bf16 2.3e9, E4M3 4.6e9, latent 2.2e9,
# fp32 keys 2.2e9).


_INT = {torch.float32: torch.int32, torch.bfloat16: torch.int16}


def _bits(t):
    """A view whose == compares bit patterns (NaN poison included)."""
    return t.view(_INT[t.dtype]) if t.dtype in _INT else t


def _poison_like(t):
    return 0x7F if t.dtype == torch.uint8 else float("nan")


def _big_copy(small, nb_big):
    """``small`` at the top of a pool of nb_big blocks, the rest poisoned."""
    if small is None:
        return None, 0
    nb = small.shape[0]
    big = torch.empty((nb_big,) + tuple(small.shape[1:]), dtype=small.dtype, device=small.device)
    off = nb_big - nb
    big[:off].fill_(_poison_like(small))
    big[off:].copy_(small)
    return big, off


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_content_at_the_top_of_a_large_pool(case):
    import decode_attention_paged_kv_amd as P

    name, make, nb_big = case
    w = make()
    say(f"[large pool] {name}: {nb_big} blocks")
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    kbig, off = _big_copy(T["k_cache"], nb_big)
    vbig, _ = _big_copy(T["v_cache"], nb_big)
    assert kbig.numel() * kbig.element_size() > 4 * GIB
    bt = T["block_table"]
    T_big = dict(T, k_cache=kbig, v_cache=vbig,
                 block_table=torch.where(bt >= 0, bt + off, bt).contiguous())

    small = run_library(w, T)            # appends into T's caches
    big = run_library(w, T_big)          # appends into the large pool
    assert int(small.err_flag.item()) == 0 and int(big.err_flag.item()) == 0
    assert torch.equal(_bits(small.out), _bits(big.out)), "output differs with the pool's placement"
    assert torch.equal(_bits(small.lse), _bits(big.lse)), "lse differs with the pool's placement"
    assert torch.equal(_bits(kbig[off:]), _bits(T["k_cache"])), "key rows differ after the append"
    if vbig is not None:
        assert torch.equal(_bits(vbig[off:]), _bits(T["v_cache"])), "value rows differ after the append"
    poison = _bits(torch.full((1,), _poison_like(kbig), dtype=kbig.dtype, device=dev))
    assert bool((_bits(kbig[:off]) == poison).all()), "the poisoned part of the pool was written"

    # the gather of the longest sequence, shard 0
    b = int(w.context_lens.argmax())
    L = int(w.context_lens[b])
    shape_k = (L, w.n_kv_heads, w.dk)
    outs = []
    for kc, vc, tbl in ((T["k_cache"], T["v_cache"], T["block_table"]),
                        (kbig, vbig, T_big["block_table"])):
        ko = torch.empty(shape_k, dtype=kc.dtype, device=dev)
        vo = torch.empty((L, w.n_kv_heads, w.dv), dtype=kc.dtype, device=dev)
        P.pa_gather_kv(kc, vc, tbl, b, 0, L, w.n_shards, w.interleave, ko, vo)
        outs.append((ko, vo))
    torch.cuda.synchronize()
    assert torch.equal(_bits(outs[0][0]), _bits(outs[1][0])), "gathered keys differ"
    assert torch.equal(_bits(outs[0][1]), _bits(outs[1][1])), "gathered values differ"

    # block copies from the top of the pool to block 0, and from there to the block below
    # the top (two calls: one call's pairs must not overlap)
    top = nb_big - 1
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    saved = kbig[top].clone()
    for pair in ([top, 0], [0, top - 1]):
        P.pa_copy_blocks(kbig, vbig, torch.tensor([pair], dtype=torch.int64, device=dev), flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert torch.equal(_bits(kbig[0]), _bits(saved)) and torch.equal(_bits(kbig[top - 1]), _bits(saved))
    del kbig, vbig, T_big, T
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kernel", ["gqa_bf16", "generic_f32"])
def test_more_than_65535_sequence_shard_pairs(kernel):
    """17,000 short sequences on 4 shards (68,000 (sequence, shard) pairs, past a 16-bit
    grid dimension): routing for every sequence, the append over the whole pool, and
    the attention of sampled sequences against the oracle; empty sequences among them."""
    rng = np.random.default_rng(17)
    lens = [int(x) for x in rng.integers(0, 48, 17_000)]
    lens[:3] = [0, 1, 47]
    if kernel == "gqa_bf16":
        w = wl.small("many_seqs_bf16", lens, 8, 2, 64, 64, 16, wl.BF16, n_shards=4, interleave=2,
                     partition_tokens=16, seed=31)
    else:
        w = wl.small("many_seqs_f32", lens, 4, 2, 40, 24, 8, wl.F32, n_shards=4, interleave=3,
                     partition_tokens=8, seed=32)
    assert w.n_seqs * w.n_shards > 65535
    sample = [0, 1, 2] + [int(x) for x in rng.integers(3, w.n_seqs, 5)] + [w.n_seqs - 1]
    check_large(w, sample)
