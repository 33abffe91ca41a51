"""E4M3 (FP8) KV cache on the GPU against the oracle's ``fp8_kv``.

The append's codes are compared bit for bit (ties, subnormals, saturation, NaN,
per-head and per-tensor scales, fp32 and bf16 rows); the step is compared whole on
small workloads that reach the MFMA kernel (bf16 queries, head 64/128) and the
generic one (fp32 queries, odd shapes, the latent cache), and at full size on the
long-context and DCP workloads with an E4M3 cache."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import bits_equal, check_large, check_small, say, to_np
from oracle import fp8_kv as f8

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


def _probe_rows(n, width, rng):
    """Values that exercise the rounding: every code's value and the midpoints between
    neighbours (scaled by the scale later), random normals over many binades,
    saturation, infinities, NaN and signed zeros."""
    pos = f8.E4M3[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    special = np.array([448, 449, 463.9, 464, 1e6, np.inf, -np.inf, np.nan, 0.0, -0.0, 2.0 ** -10,
                        3 * 2.0 ** -11, 2.0 ** -12])
    base = np.concatenate([pos, -pos, mids, -mids, special])
    x = rng.standard_normal(n * width) * 2.0 ** rng.integers(-12, 9, n * width)
    x[:base.size] = base
    return x.reshape(n, width)


@pytest.mark.parametrize("new_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("per_head", [True, False])
def test_fp8_append_codes(new_dtype, per_head):
    import decode_attention_paged_kv_amd as P

    say(f"[fp8-append] {new_dtype} per_head={per_head}")
    rng = np.random.default_rng(7)
    n_tok, hkv, dk, dv, bs, nb = 40, 3, 64, 48, 16, 8
    # scale 1 for head 0 so the probe values hit ties and codes exactly; others arbitrary
    scales = np.array([1.0, 0.37, 3.1], np.float32)[:hkv if per_head else 1]
    k_rows = _probe_rows(n_tok * hkv, dk, rng).reshape(n_tok, hkv, dk)
    v_rows = _probe_rows(n_tok * hkv, dv, rng).reshape(n_tok, hkv, dv)
    k_new = torch.from_numpy(k_rows.astype(np.float32)).to(new_dtype)
    v_new = torch.from_numpy(v_rows.astype(np.float32)).to(new_dtype)
    slots = rng.permutation(nb * bs)[:n_tok].astype(np.int64)
    slots[3] = -1                                       # padding: writes nothing
    kc = torch.full((nb, hkv, bs, dk), 0x55, dtype=torch.uint8)
    vc = torch.full((nb, hkv, dv, bs), 0x55, dtype=torch.uint8)
    k_ref, v_ref = f8.kv_append(to_np(kc), to_np(vc), to_np(k_new), to_np(v_new), slots, bs,
                                scales, scales[::-1].copy())
    dev = torch.device("cuda")
    kd, vd = kc.to(dev), vc.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_kv_append_fp8(k_new.to(dev), v_new.to(dev), kd, vd, torch.from_numpy(scales).to(dev),
                       torch.from_numpy(scales[::-1].copy()).to(dev), torch.from_numpy(slots).to(dev),
                       flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert bits_equal(to_np(kd), k_ref), "key codes differ"
    assert bits_equal(to_np(vd), v_ref), "value codes differ"


# name, lens, hq, hkv, dk, dv, bs, q dtype, S, I, T, latent, per-head scales
SMALL = [
    ("f8_gqa128", [1, 17, 300, 1000], 32, 8, 128, 128, 16, wl.BF16, 1, 1, 256, False, True),
    ("f8_gqa64", [5, 64, 129], 16, 2, 64, 64, 32, wl.BF16, 1, 1, 64, False, True),
    ("f8_gqa_tensor_scale", [77, 513], 8, 8, 128, 128, 16, wl.BF16, 1, 1, 128, False, False),
    ("f8_gqa_dcp", [900, 31], 64, 8, 128, 128, 16, wl.BF16, 4, 16, 64, False, True),
    ("f8_generic_f32q", [1, 50, 130], 6, 3, 40, 24, 8, wl.F32, 1, 1, 32, False, True),
    ("f8_generic_bf16q", [3, 90], 5, 1, 96, 80, 16, wl.BF16, 2, 3, 32, False, False),
    ("f8_latent", [65, 300], 16, 1, 576, 512, 64, wl.BF16, 1, 1, 128, True, True),
    ("f8_empty_and_one", [0, 1, 17], 8, 2, 128, 128, 16, wl.BF16, 1, 1, 16, False, True),
    # 128 query heads on the latent cache: the matrix-core latent kernel
    ("f8_latent128", [129, 200, 700, 1500], 128, 1, 576, 512, 64, wl.BF16, 1, 1, 256, True, True),
    ("f8_latent128_edges", [0, 1, 65, 64], 128, 1, 576, 512, 64, wl.BF16, 1, 1, 64, True, False),
    ("f8_latent128_bs128", [65, 1000], 128, 1, 576, 512, 128, wl.BF16, 1, 1, 384, True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_small(case):
    name, lens, hq, hkv, dk, dv, bs, dt, S, I, T, latent, per_head = case
    w = wl.small(name, lens, hq, hkv, dk, dv, bs, dt, n_shards=S, interleave=I,
                 partition_tokens=T, latent=latent, seed=sum(map(ord, name)) % 1000,
                 kv_dtype=wl.FP8, scale_per_head=per_head)
    check_small(w)


def test_fp8_long():
    """8 sequences around 142K tokens, E4M3 cache, the benchmark's partition size."""
    w = wl.with_fp8_cache(wl.long(partition_tokens=0))
    check_large(w)


def test_fp8_latent():
    """The latent batch (32 sequences, 4K-64K tokens, 128 heads, shared prefixes) with an
    E4M3 cache, at full size."""
    w = wl.with_fp8_cache(wl.latent())
    check_large(w)


def test_fp8_latent_score_far_above_first_tile():
    """E4M3 latent cache: each sequence's appended token carries a key whose score is
    more than 64 log2 units above every other, so the partition holding it is redone
    against the exact max.  The scale (1/8) keeps the spike's code exact (40 -> 320)."""
    w = wl.small("f8_latent_spike", [150, 700], 128, 1, 576, 512, 64, wl.BF16, partition_tokens=512,
                 latent=True, seed=11, kv_dtype=wl.FP8, scale_per_head=False)

    def spike(T):
        T["k_scale"].fill_(0.125)
        T["q"][:, :, 0] += 30.0
        T["k_new"][:, :, 0] = 40.0

    step, ref = check_small(w, tweak=spike)
    assert ref["lse"].min() > 44.0


def test_fp8_dcp():
    w = wl.with_fp8_cache(wl.dcp(16))
    check_large(w, [0])


def test_fp8_block_copy():
    """pa_copy_blocks moves E4M3 codes bit for bit."""
    import decode_attention_paged_kv_amd as P
    from oracle import paged_attention as pa

    g = torch.Generator().manual_seed(3)
    k = torch.randint(0, 256, (20, 8, 16, 128), dtype=torch.uint8, generator=g)
    v = torch.randint(0, 256, (20, 8, 128, 16), dtype=torch.uint8, generator=g)
    pairs = [(2, 5), (2, 6), (19, 0)]
    k_ref, v_ref = pa.copy_blocks(k.numpy(), v.numpy(), pairs)
    dev = torch.device("cuda")
    kd, vd = k.to(dev), v.to(dev)
    P.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int64, device=dev))
    torch.cuda.synchronize()
    assert bits_equal(to_np(kd), k_ref) and bits_equal(to_np(vd), v_ref)
