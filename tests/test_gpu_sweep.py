"""A seeded random sweep of small shapes through the whole step, against the oracle.

Each case draws element type (fp32, bf16, or an E4M3 cache with bf16/fp32 queries),
query and KV heads, head sizes (the MFMA kernel's 64/128 and odd ones), block size,
shards and interleave, partition size, context lengths (including 0 and 1), one or
several new tokens per sequence, and the latent cache; every case must pass the same
bars as the named workloads (``gpu_harness.check_small``).  The draws are fixed by the
seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import check_small

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


def draw(i):
    r = np.random.default_rng([2024, i])
    if r.random() < 0.5:             # a shape the matrix-core kernel takes
        hkv = int(r.choice([1, 2, 4, 8]))
        d = int(r.choice([64, 128]))
        bs = int(r.choice([16, 32, 64]))
        n = int(r.integers(1, 5))
        lens = [int(x) for x in r.integers(0, 900, n)]
        return dict(name=f"sweep{i}", lens=lens, hq=hkv * int(r.choice([1, 4, 5, 8, 16, 24])),
                    hkv=hkv, dk=d, dv=d, bs=bs, dt=wl.BF16,
                    kv=wl.FP8 if r.random() < 0.4 else "", S=int(r.choice([1, 1, 2, 4])),
                    I=int(r.choice([1, 16])), T=bs * int(r.integers(1, 9)), latent=False,
                    q_lens=[int(r.integers(0, min(L, 8) + 1)) for L in lens] if r.random() < 0.4 else None,
                    per_head=bool(r.random() < 0.7))
    latent = r.random() < 0.15
    kv = r.choice(["f32", "bf16", "fp8"], p=[0.25, 0.45, 0.30])
    dt = wl.F32 if kv == "f32" else (wl.F32 if (kv == "fp8" and r.random() < 0.3) else wl.BF16)
    if latent:
        hkv = 1
        hq = int(r.choice([1, 8, 16]))
        dk = int(r.choice([24, 64, 576]))
        dv = int(r.integers(1, dk + 1)) if dk != 576 else 512
    else:
        hkv = int(r.choice([1, 2, 3, 4, 8]))
        hq = hkv * int(r.choice([1, 2, 4, 5, 8, 16, 20]))
        d = int(r.choice([64, 128, 40, 96, 8]))
        dk = d
        dv = d if r.random() < 0.8 else int(r.integers(1, 129))
    bs = int(r.choice([16, 32, 64, 1, 3, 8]))
    S = int(r.choice([1, 1, 2, 3, 4]))
    I = int(r.choice([1, 2, 16]))
    n = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(0, 600, n)]
    if r.random() < 0.3:
        lens[0] = int(r.choice([0, 1]))
    T = bs * int(r.integers(1, max(2, 256 // bs) + 1))
    q_lens = None
    if r.random() < 0.35:
        q_lens = [int(r.integers(0, min(L, 6) + 1)) for L in lens]
    return dict(name=f"sweep{i}", lens=lens, hq=hq, hkv=hkv, dk=dk, dv=dv, bs=bs, dt=dt,
                kv=wl.FP8 if kv == "fp8" else "", S=S, I=I, T=T, latent=latent, q_lens=q_lens,
                per_head=bool(r.random() < 0.7))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = draw(i)
    w = wl.small(c["name"], c["lens"], c["hq"], c["hkv"], c["dk"], c["dv"], c["bs"], c["dt"],
                 n_shards=c["S"], interleave=c["I"], partition_tokens=c["T"], latent=c["latent"],
                 seed=100 + i, kv_dtype=c["kv"], scale_per_head=c["per_head"], q_lens=c["q_lens"])
    check_small(w)


# The VALU kernel stages each tile's keys and values through a fixed LDS buffer, so its
# tile holds fewer than 32 tokens when rows are long: 7 tokens at fp32 576/512 with a
# separate value cache, 14 for an fp32 latent cache of 576, 31 at fp32 128/128.  These
# cases put several such tiles (and a ragged last one) in each partition.
GENERIC_CASES = [
    dict(name="gen_f32_576_512", lens=[0, 1, 100, 333], hq=16, hkv=1, dk=576, dv=512, bs=16,
         dt=wl.F32, kv="", S=1, I=1, T=64, latent=False, q_lens=None),
    dict(name="gen_f32_latent576", lens=[700, 5, 64], hq=16, hkv=1, dk=576, dv=512, bs=64,
         dt=wl.F32, kv="", S=1, I=1, T=128, latent=True, q_lens=None),
    dict(name="gen_f32_128_multi", lens=[150, 40, 97], hq=8, hkv=2, dk=128, dv=128, bs=8,
         dt=wl.F32, kv="", S=2, I=16, T=96, latent=False, q_lens=[3, 1, 5]),
    dict(name="gen_bf16_96_g20", lens=[260, 1, 33], hq=40, hkv=2, dk=96, dv=96, bs=16,
         dt=wl.BF16, kv="", S=1, I=1, T=128, latent=False, q_lens=[2, 1, 4]),
    dict(name="gen_fp8_f32q_128", lens=[300, 77], hq=8, hkv=2, dk=128, dv=128, bs=16,
         dt=wl.F32, kv=wl.FP8, S=2, I=16, T=256, latent=False, q_lens=None),
]


@pytest.mark.parametrize("c", GENERIC_CASES, ids=[c["name"] for c in GENERIC_CASES])
def test_generic_tile_sizes(c):
    w = wl.small(c["name"], c["lens"], c["hq"], c["hkv"], c["dk"], c["dv"], c["bs"], c["dt"],
                 n_shards=c["S"], interleave=c["I"], partition_tokens=c["T"], latent=c["latent"],
                 seed=7, kv_dtype=c["kv"], q_lens=c["q_lens"])
    check_small(w)
