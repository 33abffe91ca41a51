"""HIP library vs the fp64 oracle on the GPU (parity proper).

Small workloads are compared whole: routing, append and gather bit for bit,
every partition's output and LSE, and the merged result.  The full-size
workloads run at their real sizes with the partition size the benchmark uses
and every sequence is compared with the oracle (see ``gpu_harness.check_large``)."""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import check_large, check_small, compare_outputs, run_library, say, to_np
from oracle import paged_attention as pa

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# ------------------------------------------------------------------ the named workloads
@pytest.mark.parametrize("L", [67, 68])
def test_tiny(L):
    """1 sequence, 4/1 heads, head 64, fp32, 4-token blocks, 64-block pool (context
    counted with and without an extra token, so both readings are covered)."""
    check_small(wl.tiny(context_len=L))


def test_tiny_single_partition_and_sharded():
    w = wl.tiny()
    check_small(w, partition_tokens=68)
    for I in (1, 16):
        check_small(wl.small(f"tiny_S4_I{I}", [67], 4, 1, 64, 64, 4, wl.F32, n_shards=4,
                             interleave=I, partition_tokens=8, scale=0.125, seed=1))


def test_batch():
    """Continuous-batching step: 64 ragged sequences, 32/8 heads, head 128, bf16."""
    check_small(wl.batch())


def test_long():
    """8 sequences, log-normal lengths around 142K, 4,096-token partitions."""
    check_large(wl.long())


@pytest.mark.parametrize("I", [1, 16])
def test_dcp(I):
    """One 200,000-token sequence in 4 interleaved shards."""
    check_large(wl.dcp(interleave=I))


@pytest.mark.parametrize("I", [1, 16])
def test_dcp_matches_unsharded(I):
    """The 200,000-token sequence merged from 4 interleaved shards equals the same
    sequence decoded unsharded (S = 1) on the GPU, and both equal the oracle ([DCP]
    DCP mechanism section: the LSE-weighted merge of the ranks' partial outputs is the
    attention over all tokens; its measuring section compares DCP size 1 with DCP
    enabled).  The S = 1 cache is built from the sharded one through pa_gather_kv, in
    global token order, into 12,500 fresh blocks."""
    import decode_attention_paged_kv_amd as P

    w = wl.dcp(interleave=I)
    say(f"[dcp-vs-s1] I={I}")
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    sharded = run_library(w, T)                   # appends the new token, then decodes
    assert int(sharded.err_flag.item()) == 0
    L, S, bs = int(w.context_lens[0]), w.n_shards, w.block_size
    # every token of the sequence, global order, from the appended sharded cache
    K = torch.empty(L, w.n_kv_heads, w.dk, dtype=torch.bfloat16, device=dev)
    V = torch.empty(L, w.n_kv_heads, w.dv, dtype=torch.bfloat16, device=dev)
    for r in range(S):
        Lr = P.pa_shard_length(L, S, I, r)
        kg = torch.empty(Lr, w.n_kv_heads, w.dk, dtype=torch.bfloat16, device=dev)
        vg = torch.empty(Lr, w.n_kv_heads, w.dv, dtype=torch.bfloat16, device=dev)
        P.pa_gather_kv(T["k_cache"], T["v_cache"], T["block_table"], 0, r, L, S, I, kg, vg,
                       sharded.err_flag)
        ids = torch.from_numpy(pa.shard_members(L, S, I, r)).to(dev)
        K[ids], V[ids] = kg, vg
    nb = -(-L // bs)
    k1 = torch.full((nb, w.n_kv_heads, bs, w.dk), float("nan"), dtype=torch.bfloat16, device=dev)
    v1 = torch.full((nb, w.n_kv_heads, w.dv, bs), float("nan"), dtype=torch.bfloat16, device=dev)
    t = torch.arange(L, device=dev)
    k1[t // bs, :, t % bs, :] = K
    v1[t // bs, :, :, t % bs] = V
    bt1 = torch.arange(nb, dtype=torch.int32, device=dev).reshape(1, 1, nb)
    one = P.DecodeStep(1, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, bs, L, 1, 1, 0, w.scale_f32,
                       device=dev, context_lens_host=w.context_lens)
    one(T["q"], T["k_new"], T["v_new"], k1, v1, bt1, T["context_lens"])
    torch.cuda.synchronize()
    assert int(one.err_flag.item()) == 0
    d_o = (one.out - sharded.out).abs().max().item()
    d_l = (one.lse - sharded.lse).abs().max().item()
    rel = ((one.out - sharded.out).double().norm() / one.out.double().norm()).item()
    say(f"  S=4 vs S=1: max|do|={d_o:.3g} max|dlse|={d_l:.3g} rel_l2={rel:.3g}")
    assert d_o <= 5e-3 and d_l <= 1e-3 and rel <= 1e-4
    # both against the oracle, from host copies of the contiguous sequence
    Kh, Vh = to_np(K), to_np(V)
    o_ref, lse_ref = pa.attention(to_np(T["q"][0]), Kh, Vh, w.scale_f32)
    for name, st in (("S=4 merged", sharded), ("S=1", one)):
        compare_outputs(f"dcp I={I} {name}", wl.BF16, to_np(st.out)[0], to_np(st.lse)[0], o_ref,
                        lse_ref)


def test_latent():
    """128 query heads on one 576-wide latent head, shared 2,048-token prefixes."""
    check_large(wl.latent())


def test_latent_16_heads():
    """The latent batch with 16 query heads (a tensor-parallel share of 128), at full size:
    the latent kernel pads its products to 128 rows and writes only the real ones."""
    check_large(dataclasses.replace(wl.latent(), n_q_heads=16, name="latent_h16"))


# name, lens, hq, hkv, S, I, T, kv dtype: fewer than 128 query heads per latent KV head
FEWER_HEADS = [
    ("latent_h16", [0, 1, 65, 700], 16, 1, 1, 1, 256, ""),
    ("latent_h64_2kv", [300, 129], 128, 2, 1, 1, 128, ""),
    ("latent_h32_e4m3", [70, 513], 32, 1, 1, 1, 128, wl.FP8),
    ("latent_h16_dcp", [300, 90], 16, 1, 3, 2, 64, ""),
    ("latent_h1", [33, 200], 1, 1, 1, 1, 64, ""),
    # more than 128 heads per KV head: units of 128 heads, the last one partial
    ("latent_h160", [0, 129, 300], 160, 1, 1, 1, 128, ""),
    ("latent_h256_2kv_e4m3", [65, 200], 512, 2, 1, 1, 64, wl.FP8),
]


@pytest.mark.parametrize("case", FEWER_HEADS, ids=[c[0] for c in FEWER_HEADS])
def test_latent_fewer_heads(case):
    name, lens, hq, hkv, S, I, T, kv = case
    w = wl.small(name, lens, hq, hkv, 576, 512, 64, wl.BF16, n_shards=S, interleave=I,
                 partition_tokens=T, latent=True, seed=sum(map(ord, name)) % 1000, kv_dtype=kv)
    check_small(w)


# ------------------------------------------------------------------ exact probes at full size
@pytest.mark.parametrize("make", [lambda: wl.long(), lambda: wl.dcp(interleave=16),
                                  lambda: wl.dcp(interleave=1), lambda: wl.latent()],
                         ids=["long", "dcp_I16", "dcp_I1", "latent"])
def test_mean_probe_full_size(make):
    """q = 0: every weight is exactly 1 (exp of a zero score, in any precision), values
    are small integers, so every sum is exact and the output is the exact mean of each
    sequence's values -- any dropped, repeated or misaddressed token moves it.  Every
    sequence of the workload is compared."""
    check_large(make(), fill="mean_probe")


@pytest.mark.parametrize("make", [lambda: wl.long(), lambda: wl.dcp(interleave=16),
                                  lambda: wl.dcp(interleave=1), lambda: wl.latent()],
                         ids=["long", "dcp_I16", "dcp_I1", "latent"])
def test_needle_full_size(make):
    """One token per sequence, at a random earlier position, gets key alpha*u (u the
    sequence's unit query, shared by all its heads; alpha*scale ~ 45, or 50 for the
    latent cache, while every other score stays below ~0.5), so its weight is all but 1
    among up to 200,000 tokens: the output must be that token's value row and the LSE
    its score.  Checks the block-table read at that exact position, its shard and
    partition, and the merge, at full size.  In the latent kernel a needle outside the
    first tile lies more than 64 log2 units above the reference max set by earlier
    tokens, so the partition is redone against the exact max."""
    import decode_attention_paged_kv_amd as P  # noqa: F401

    w = make()
    say(f"[needle] {w.name} N={w.n_seqs} S={w.n_shards} I={w.interleave}")
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    rng = np.random.default_rng(123)
    alpha = 50.0 / float(w.scale_f32) if w.latent else 512.0
    g = w.n_q_heads // w.n_kv_heads
    expect_o, expect_lse = [], []
    for b in range(w.n_seqs):
        L = int(w.context_lens[b])
        lo = w.prefix_tokens if w.prefix_tokens else 0        # outside a shared prefix
        i = int(rng.integers(lo, L - 1))                     # an old token (not the new one)
        _, _, phys, off = pa.token_home(w.block_table[b], i, w.n_shards, w.interleave, w.block_size)
        u = torch.randn(w.dk, generator=torch.Generator().manual_seed(b), dtype=torch.float32)
        u = (u / u.norm()).to(torch.bfloat16)
        k = (u.float() * alpha).to(torch.bfloat16)
        T["q"][b] = u.to(dev)                                # every head of the sequence
        T["k_cache"][phys, :, off, :] = k.to(dev)            # every KV head
        if w.latent:                                         # the value is the key's head
            v = k[:w.dv].float()[None, :].repeat(w.n_kv_heads, 1)
        else:
            v = T["v_cache"][phys, :, :, off].float().cpu()  # [Hkv][dv]
        s = float(np.float32(w.scale_f32)) * float((u.double() * k.double()).sum())
        expect_o.append(v.repeat_interleave(g, dim=0))       # [Hq][dv]
        expect_lse.append(s)
    step = run_library(w, T)
    assert int(step.err_flag.item()) == 0
    out = step.out.float().cpu()
    lse = step.lse.float().cpu()
    for b in range(w.n_seqs):
        d_o = (out[b] - expect_o[b]).abs().max().item()
        d_l = (lse[b] - expect_lse[b]).abs().max().item()
        # latent values reach ~150 (the needle's key is its value): the stated bf16 bar;
        # elsewhere |v| ~ 1 and the bar is 1e-4.  A misread row would be off by ~|v|.
        tol_o = 5e-3 if w.latent else 1e-4
        say(f"  seq {b}: max|o - v_needle| = {d_o:.3g} (tol {tol_o:.3g}), max|lse - s_needle| = {d_l:.3g}")
        assert d_o < tol_o, f"seq {b}: output is not the needle's value row"
        assert d_l < 1e-3, f"seq {b}: lse is not the needle's score"


# ------------------------------------------------------------------ shapes and edge cases
SWEEP = [
    # name, lens, hq, hkv, dk, dv, bs, dtype, S, I, T, latent, prefix(group, tokens)
    ("gqa128_ragged", [1, 15, 16, 17, 300, 1000], 32, 8, 128, 128, 16, wl.BF16, 1, 1, 256, False, None),
    ("gqa128_f32", [1, 33, 250], 32, 8, 128, 128, 16, wl.F32, 1, 1, 64, False, None),
    ("dcp_small_I1", [1, 5, 63, 64, 65, 700], 64, 8, 128, 128, 16, wl.BF16, 4, 1, 32, False, None),
    ("dcp_small_I16", [1, 5, 63, 64, 65, 700], 64, 8, 128, 128, 16, wl.BF16, 4, 16, 32, False, None),
    ("mha64", [3, 40, 129], 8, 8, 64, 64, 16, wl.BF16, 1, 1, 32, False, None),
    ("g8_d64", [70, 513], 64, 8, 64, 64, 16, wl.BF16, 1, 1, 128, False, None),
    ("bs1", [1, 2, 9], 4, 2, 32, 32, 1, wl.F32, 2, 3, 4, False, None),
    ("bs256", [1, 255, 256, 257, 900], 8, 2, 64, 64, 256, wl.BF16, 1, 1, 256, False, None),
    ("odd_dims", [7, 30], 6, 3, 40, 24, 8, wl.BF16, 3, 2, 8, False, None),
    ("empty_seqs", [0, 1, 0, 20], 8, 4, 64, 64, 16, wl.BF16, 2, 16, 16, False, None),
    ("latent_small", [129, 200, 700, 1500], 128, 1, 576, 512, 64, wl.BF16, 1, 1, 256, True, (4, 128)),
    ("latent_f32", [65, 300], 16, 1, 576, 512, 64, wl.F32, 1, 1, 128, True, None),
    ("gqa128_bs64_dcp", [1, 63, 64, 65, 640, 2000], 32, 8, 128, 128, 64, wl.BF16, 3, 4, 192, False, None),
    # the latent kernel with one tile per block, and with eight, on shards
    ("latent_bs32_dcp", [129, 700, 1500, 0], 128, 1, 576, 512, 32, wl.BF16, 2, 16, 256, True, None),
    ("latent_bs256", [300, 1500, 2100], 128, 1, 576, 512, 256, wl.BF16, 1, 1, 512, True, None),
]


@pytest.mark.parametrize("case", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep(case):
    name, lens, hq, hkv, dk, dv, bs, dt, S, I, T, latent, prefix = case
    pg, pt = prefix or (1, 0)
    w = wl.small(name, lens, hq, hkv, dk, dv, bs, dt, n_shards=S, interleave=I,
                 partition_tokens=T, latent=latent, prefix_group=pg, prefix_tokens=pt, seed=zlib.crc32(name.encode()) % 1000)
    check_small(w)


def test_partition_size_independence():
    """Different partition sizes give the same merged result (within tolerance): 69
    parts per row (the workgroup merge), 9 (the one-wave merge) and 1 (no merge)."""
    w = wl.small("tsz", [1100, 77], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=16, seed=5)
    outs = {}
    for T in (16, 128, 1104):
        outs[T], _ = check_small(w, partition_tokens=T)
    for T in (128, 1104):
        d = (outs[16].out - outs[T].out).abs().max().item()
        say(f"  partition 16 vs {T}: max|do|={d:.3g}")
        assert d < 1e-5


def test_deterministic_and_placement_invariant():
    """Two runs give bitwise identical results, and so do two different physical
    placements of the same logical content."""
    import decode_attention_paged_kv_amd as P

    outs = []
    for seed in (7, 8):
        w = wl.small("perm", [300, 41], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=64, seed=seed)
        T = wl.make_tensors(w, "cuda", seed=0)
        # rewrite the pools so token i of sequence b holds the same rows in both placements
        g = torch.Generator(device="cuda").manual_seed(123)
        Kl = torch.randn(2, 300, 8, 128, generator=g, device="cuda").to(torch.bfloat16)
        Vl = torch.randn(2, 300, 8, 128, generator=g, device="cuda").to(torch.bfloat16)
        tid = torch.from_numpy(w.token_id).cuda()
        own = torch.full_like(tid, -1)
        for b in range(2):
            for phys in w.block_table[b, 0]:
                if phys >= 0:
                    own[int(phys)] = b
        live = torch.from_numpy(w.live).cuda() & (own >= 0)
        pos = live.nonzero()
        bsel, i = own[pos[:, 0], pos[:, 1]], tid[pos[:, 0], pos[:, 1]]
        T["k_cache"][pos[:, 0], :, pos[:, 1], :] = Kl[bsel, i]
        T["v_cache"][pos[:, 0], :, :, pos[:, 1]] = Vl[bsel, i]
        Ls = torch.tensor([300, 41], device="cuda") - 1
        T["k_new"].copy_(Kl[torch.arange(2, device="cuda"), Ls])
        T["v_new"].copy_(Vl[torch.arange(2, device="cuda"), Ls])
        T["q"].copy_(torch.randn(2, 32, 128, generator=g, device="cuda").to(torch.bfloat16))
        runs = []
        for _ in range(2):
            step = P.DecodeStep(2, 32, 8, 128, 128, 16, 300, partition_tokens=64, device="cuda")
            out, lse = step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
                            T["block_table"], T["context_lens"])
            torch.cuda.synchronize()
            runs.append((out.clone(), lse.clone()))
        assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
        outs.append(runs[0])
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_bf16_output():
    """bf16 output: within half an ulp of bf16 plus the bf16 tolerance."""
    import decode_attention_paged_kv_amd as P
    from gpu_harness import to_np
    from oracle import paged_attention as pa

    w = wl.batch()
    Tc = wl.make_tensors(w, "cpu")
    T = {k: (None if v is None else v.cuda()) for k, v in Tc.items()}
    H = {k: to_np(v) for k, v in Tc.items()}
    step = P.DecodeStep(w.n_seqs, 32, 8, 128, 128, 16, int(w.context_lens.max()), device="cuda",
                        out_dtype=torch.bfloat16)
    out, lse = step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
                    T["context_lens"])
    ref = pa.decode_step(H["q"], H["k_new"], H["v_new"], H["k_cache"], H["v_cache"], w.block_table,
                         w.context_lens, 1, 1, 16, step.partition_tokens, step.max_partitions,
                         w.scale_f32, 128)
    o = pa.widen(to_np(out))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref["o"]), 1e-30))) - 8)
    assert np.all(np.abs(o - ref["o"]) <= half_ulp + 5e-3)


def test_error_flag_on_bad_block_id():
    """A block id outside the pool is skipped and reported in the error flag; the
    kernels still finish normally (the bound check is the kernels' own)."""
    import decode_attention_paged_kv_amd as P

    w = wl.small("bad", [40, 40], 8, 2, 64, 64, 16, wl.BF16, partition_tokens=16, seed=9)
    T = wl.make_tensors(w, "cuda")
    T["block_table"][1, 0, 1] = w.n_blocks + 5
    step = P.DecodeStep(2, 8, 2, 64, 64, 16, 40, partition_tokens=16, device="cuda")
    step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
         T["context_lens"])
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) & P.ERR_BLOCK_ID
    assert torch.isfinite(step.out[0]).all()


def test_latent_score_far_above_first_tile():
    """Each sequence's appended token carries a key whose score is ~120 (log2 units)
    above every other: the latent kernel, whose reference max comes from the first
    tile of a partition, has to redo that partition against the exact max.  In the
    700-token sequence only the second partition holds the spike."""
    w = wl.small("latent_spike", [150, 700], 128, 1, 576, 512, 64, wl.BF16, partition_tokens=512,
                 latent=True, seed=11)

    def spike(T):
        T["q"][:, :, 0] += 10.0
        T["k_new"][:, :, 0] = 200.0

    step, ref = check_small(w, tweak=spike)
    # every head's spike is > 64 log2 units (44 nats) above the other scores (< ~5 nats)
    assert ref["lse"].min() > 50.0


def test_error_flag_on_bad_block_id_latent():
    """Latent kernel: a tile whose block id is invalid is skipped (copied from zeros,
    weights 0) and reported; the outputs stay finite."""
    import decode_attention_paged_kv_amd as P

    w = wl.small("bad_latent", [300, 300], 128, 1, 576, 512, 64, wl.BF16, partition_tokens=128,
                 latent=True, seed=12)
    T = wl.make_tensors(w, "cuda")
    T["block_table"][1, 0, 2] = w.n_blocks + 5
    step = P.DecodeStep(2, 128, 1, 576, 512, 64, 300, partition_tokens=128, device="cuda",
                        kv_dtype=torch.bfloat16, latent=True)
    step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
         T["context_lens"])
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) & P.ERR_BLOCK_ID
    assert torch.isfinite(step.out).all()


def test_error_flag_on_short_table():
    """A context longer than the block table holds is reported, not read."""
    import decode_attention_paged_kv_amd as P

    w = wl.small("short", [40], 8, 2, 64, 64, 16, wl.BF16, partition_tokens=16, seed=9)
    T = wl.make_tensors(w, "cuda")
    lens = torch.tensor([90], dtype=torch.int32, device="cuda")      # table holds 48 tokens
    step = P.DecodeStep(1, 8, 2, 64, 64, 16, 96, partition_tokens=16, device="cuda")
    P.pa_decode(T["q"], T["k_cache"], T["v_cache"], T["block_table"], lens, 1, 1, 16,
                step.max_partitions, step.scale, step.part_out, step.part_lse, err_flag=step.err_flag)
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) & P.ERR_CAPACITY
