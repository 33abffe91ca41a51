"""Several new tokens per sequence (causal among them) on the GPU against the
oracle's ``multi_query``: slots and appended rows bit for bit, every partition's
output and LSE and the merged rows, on small workloads over the MFMA kernel
(bf16, head 64/128, E4M3 cache, DCP shards) and the generic one (fp32, odd
shapes, the latent cache), a whole sequence of new tokens (causal attention over
all of it), and the speculative-verification workload at full size."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import check_large, check_small, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# name, lens, q_lens, hq, hkv, dk, dv, bs, dtype, S, I, T, latent, kv_dtype
SMALL = [
    ("mq_gqa128", [1, 17, 300, 1000], [1, 4, 7, 3], 32, 8, 128, 128, 16, wl.BF16, 1, 1, 64, False, ""),
    ("mq_gqa_dcp", [900, 131], [5, 2], 64, 8, 128, 128, 16, wl.BF16, 4, 16, 64, False, ""),
    ("mq_gqa64_long_q", [70, 9, 400], [2, 0, 16], 16, 2, 64, 64, 32, wl.BF16, 1, 1, 64, False, ""),
    ("mq_gqa_fp8", [33, 520], [4, 4], 32, 8, 128, 128, 16, wl.BF16, 1, 1, 128, False, wl.FP8),
    ("mq_generic_f32", [30, 7, 99], [3, 1, 5], 6, 3, 40, 24, 8, wl.F32, 2, 3, 16, False, ""),
    ("mq_latent", [70, 200], [2, 3], 16, 1, 576, 512, 64, wl.BF16, 1, 1, 128, True, ""),
    ("mq_whole_sequence", [40, 77], [40, 77], 8, 2, 128, 128, 16, wl.BF16, 1, 1, 32, False, ""),
    ("mq_latent_fp8_empty", [70, 0, 9], [3, 0, 9], 16, 1, 576, 512, 64, wl.BF16, 1, 1, 64, True, wl.FP8),
    ("mq_dcp_fp8_d64", [200, 45], [6, 1], 16, 4, 64, 64, 16, wl.BF16, 3, 2, 32, False, wl.FP8),
    # 128 query heads on the latent cache: the matrix-core latent kernel, one unit per new
    # token -- ragged partitions; shards on which a new token sees none of a partition's
    # tokens; an E4M3 cache with an empty sequence and one whose tokens are all new
    ("mq_latent128", [129, 300, 700], [1, 4, 3], 128, 1, 576, 512, 64, wl.BF16, 1, 1, 128, True, ""),
    ("mq_latent128_dcp", [300, 90], [5, 2], 128, 1, 576, 512, 64, wl.BF16, 3, 2, 64, True, ""),
    ("mq_latent128_fp8", [70, 0, 9, 64], [3, 0, 9, 1], 128, 1, 576, 512, 64, wl.BF16, 1, 1, 64, True,
     wl.FP8),
    ("mq_latent192_dcp", [200, 77], [3, 2], 192, 1, 576, 512, 64, wl.BF16, 2, 1, 64, True, ""),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_multi_small(case):
    name, lens, q_lens, hq, hkv, dk, dv, bs, dt, S, I, T, latent, kv = case
    w = wl.small(name, lens, hq, hkv, dk, dv, bs, dt, n_shards=S, interleave=I, partition_tokens=T,
                 latent=latent, seed=sum(map(ord, name)) % 1000, kv_dtype=kv, q_lens=q_lens)
    check_small(w)


def test_multi_grid_bound_above_need():
    """max_q_len larger than any sequence's new tokens: the extra column chunks find no
    rows and exit; the result equals the tight bound's bit for bit."""
    import decode_attention_paged_kv_amd as P

    say("[multi] loose max_q_len")
    w = wl.small("mq_loose", [300, 70], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=64, seed=9,
                 q_lens=[2, 1])
    dev = torch.device("cuda")
    outs = []
    for max_q in (2, 9):
        T = wl.make_tensors(w, dev)
        step = P.MultiDecodeStep(w.n_seqs, w.n_rows, max_q, w.n_q_heads, w.n_kv_heads, w.dk, w.dv,
                                 w.block_size, 300, partition_tokens=64, scale=w.scale_f32, device=dev)
        step(T["q"], T["query_start"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
             T["block_table"], T["context_lens"])
        torch.cuda.synchronize()
        assert int(step.err_flag.item()) == 0
        outs.append((step.out.clone(), step.lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_multi_speculative_long():
    """The long-context batch with 4 new tokens per sequence, at full size."""
    w = wl.speculative(q_len=4)
    check_large(w)


def test_multi_latent_speculative():
    """The latent batch with 2 new tokens per sequence, at full size (the matrix-core
    latent kernel, one unit per new token)."""
    w = wl.latent(q_len=2)
    check_large(w)


def test_multi_latent_partners_timing_only():
    """The latent kernel keeps the units of two new tokens of one partition within a few
    tiles of each other through a progress array that every launch shares: it changes
    timing only.  With a full grid (the case where partners are paired), repeated runs of
    one step are bitwise equal, and two steps launched together on two streams -- sharing
    that array -- give bitwise what each gives alone."""
    import decode_attention_paged_kv_amd as P

    say("[multi] latent partners: repeated and concurrent launches")
    w = wl.small("mq_latent_pairs", [20000, 30000, 12000, 25000], 128, 1, 576, 512, 64, wl.BF16,
                 partition_tokens=512, latent=True, seed=21, q_lens=[2, 2, 3, 2])
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)

    def make():
        return P.MultiDecodeStep(w.n_seqs, w.n_rows, int(w.q_lens.max()), w.n_q_heads, w.n_kv_heads,
                                 w.dk, w.dv, w.block_size, int(w.context_lens.max()),
                                 partition_tokens=512, scale=w.scale_f32, device=dev, latent=True)

    a, b = make(), make()
    a(T["q"], T["query_start"], T["k_new"], T["v_new"], T["k_cache"], T.get("v_cache"),
      T["block_table"], T["context_lens"])   # the new rows are in the cache from here on
    args = (T["q"], T["query_start"], T["k_cache"], T.get("v_cache"), T["block_table"], T["context_lens"])
    torch.cuda.synchronize()

    def written(st):   # partition slots past a sequence's count keep whatever they held
        used = torch.isfinite(st.part_lse)
        return st.part_out[used].clone(), st.part_lse.clone()

    ref = written(a)
    assert ref[0].shape[0] > 0 and torch.isfinite(ref[0]).all()
    for _ in range(3):
        a.attend(*args)
        torch.cuda.synchronize()
        got = written(a)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        a.attend(*args)
    with torch.cuda.stream(s2):
        b.attend(*args)
    torch.cuda.synchronize()
    for st in (a, b):
        assert int(st.err_flag.item()) == 0
        got = written(st)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_multi_error_flag_on_too_many_new_tokens():
    """A sequence with more new tokens than context tokens is flagged and skipped; the
    others are computed."""
    import decode_attention_paged_kv_amd as P

    say("[multi-error] q_len > context")
    w = wl.small("mq_bad", [20, 50], 8, 2, 128, 128, 16, wl.BF16, partition_tokens=32, seed=5,
                 q_lens=[2, 3])
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    lens = T["context_lens"].clone()
    lens[0] = 1                                  # 2 new tokens, 1 context token
    step = P.MultiDecodeStep(w.n_seqs, w.n_rows, 3, w.n_q_heads, w.n_kv_heads, w.dk, w.dv,
                             w.block_size, 50, partition_tokens=32, device=dev)
    step.part_lse.fill_(123.0)
    step(T["q"], T["query_start"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
         T["block_table"], lens)
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) != 0
    assert torch.all(step.part_lse[:2] == 123.0)          # the bad sequence's rows untouched
    assert not torch.any(step.part_lse[2:] == 123.0)      # the good one's rows all written
