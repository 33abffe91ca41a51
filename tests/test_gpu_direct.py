"""One shard and one partition per sequence: the step skips the merge and returns the
partials themselves (a single part has weight exp(lse - lse) = 1, and the decode writes
zeros into partition 0 of an empty sequence).  The outputs must equal what
pa_merge_lse makes of the same partials, for the MFMA, generic and latent kernels (the
latent one also with an E4M3 cache) and for several new tokens per sequence, with empty sequences among them; and the whole
step is checked against the oracle (``check_small``)."""
import pytest
import torch

import workloads as wl
from gpu_harness import check_small, run_library, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# name, lens, hq, hkv, dk, dv, bs, dtype, T (>= every length), latent, q_lens, kv dtype
CASES = [
    ("gqa", [0, 17, 300, 1, 0], 32, 8, 128, 128, 16, wl.BF16, 320, False, None, ""),
    ("gqa_e4m3", [0, 90, 33], 32, 8, 128, 128, 16, wl.BF16, 96, False, None, wl.FP8),
    ("generic_f32", [5, 0, 130], 6, 3, 40, 24, 8, wl.F32, 136, False, None, ""),
    ("latent", [0, 65, 300], 16, 1, 576, 512, 64, wl.BF16, 320, True, None, ""),
    ("multi", [0, 40, 77], 32, 8, 128, 128, 16, wl.BF16, 80, False, [0, 3, 5], ""),
    # 128 heads on the latent cache: the matrix-core latent kernel
    ("latent128", [0, 65, 300], 128, 1, 576, 512, 64, wl.BF16, 320, True, None, ""),
    ("latent128_e4m3", [0, 65, 300], 128, 1, 576, 512, 64, wl.BF16, 320, True, None, wl.FP8),
    ("latent128_multi", [0, 65, 300], 128, 1, 576, 512, 64, wl.BF16, 320, True, [0, 2, 3], ""),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_direct_outputs_equal_the_merge(case):
    import decode_attention_paged_kv_amd as P

    name, lens, hq, hkv, dk, dv, bs, dt, T, latent, q_lens, kv = case
    say(f"[direct] {name}")
    w = wl.small(f"direct_{name}", lens, hq, hkv, dk, dv, bs, dt, partition_tokens=T, latent=latent,
                 seed=sum(map(ord, name)) % 1000, q_lens=q_lens, kv_dtype=kv)
    check_small(w)      # the step against the oracle
    dev = torch.device("cuda")
    T_ = wl.make_tensors(w, dev)
    step = run_library(w, T_)
    assert step.direct and step.max_partitions == 1
    assert int(step.err_flag.item()) == 0
    out = torch.empty_like(step.out)
    lse = torch.empty_like(step.lse)
    P.pa_merge_lse(step.part_out, step.part_lse, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(step.lse, lse), "lse differs from the merge of the partials"
    assert torch.equal(step.out, out), "output differs from the merge of the partials"
    empty = torch.isinf(lse)
    if q_lens is None:   # (every row of several new tokens sees at least its own token)
        assert bool(empty.any()), "the case should hold an empty row"
    assert bool((step.out[empty] == 0).all())
