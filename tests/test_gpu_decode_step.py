"""pa_decode_step (the step's append and attention in one call) on the GPU.

Held bit for bit to the same step as two calls, pa_kv_append_routed then pa_decode (or
pa_decode_fp8): every byte of both caches, the slots, and every partial output and LSE
(the decode reads the same cache, so the results must be identical, not merely close).
The two-call path is itself held to the oracle by the routed-append and decode parity
tests.  Cases cover each decode kernel with the append fused (GQA bf16, the generic
kernel in fp32 and with an E4M3 cache or a latent view, E4M3, DCP shards with interleave,
the latent kernel) and the shapes that
keep the append a launch of its own (more than 16 query heads per KV head; more than 128
on the latent kernel), with empty, one-token and multi-partition sequences."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# name, lens, hq, hkv, dk, dv, bs, dtype, S, I, latent, kv dtype, partition tokens
CASES = [
    ("gqa_bf16", [1, 17, 300, 0, 1000], 32, 8, 128, 128, 16, wl.BF16, 1, 1, False, "", 64),
    ("gqa_g32_unfused", [5, 260, 0, 77], 64, 2, 128, 128, 16, wl.BF16, 1, 1, False, "", 128),
    ("generic_f32_dcp", [0, 1, 5, 130, 77], 6, 3, 40, 24, 8, wl.F32, 3, 2, False, "", 16),
    ("generic_e4m3", [0, 3, 40, 77, 130], 8, 2, 40, 24, 8, wl.BF16, 2, 4, False, wl.FP8, 32),
    ("generic_latent_f32", [1, 9, 66, 0, 200], 4, 1, 64, 48, 4, wl.F32, 1, 1, True, "", 16),
    ("gqa_dcp16", [900, 31, 16, 0], 64, 8, 128, 128, 16, wl.BF16, 4, 16, False, "", 96),
    ("gqa_e4m3", [33, 520, 0, 1], 32, 8, 128, 128, 16, wl.BF16, 1, 1, False, wl.FP8, 128),
    ("latent", [65, 300, 1, 0, 2000], 16, 1, 576, 512, 64, wl.BF16, 1, 1, True, "", 256),
    ("latent_e4m3", [70, 0, 9, 700], 16, 1, 576, 512, 64, wl.BF16, 1, 1, True, wl.FP8, 256),
    ("latent_256h_unfused", [70, 640], 256, 1, 576, 512, 64, wl.BF16, 1, 1, True, "", 256),
]


def _bits(t):
    return None if t is None else t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_step_equals_append_then_decode(case):
    import decode_attention_paged_kv_amd as P

    name, lens, hq, hkv, dk, dv, bs, dt, S, I, latent, kv, T_part = case
    say(f"[decode step] {name}")
    w = wl.small(name, lens, hq, hkv, dk, dv, bs, dt, n_shards=S, interleave=I, latent=latent,
                 partition_tokens=T_part, seed=sum(map(ord, name)) % 1000, kv_dtype=kv)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    ks, vs = T.get("k_scale"), T.get("v_scale")
    fp8 = T["k_cache"].dtype == torch.uint8
    n = w.n_seqs
    Pmax = max(1, P.pa_max_partitions(int(max(lens)), S, I, T_part))
    scale = float(w.scale_f32)

    def buffers():
        po = torch.full((n, S, Pmax, hq, dv), float("nan"), dtype=torch.float32, device=dev)
        pl = torch.full((n, S, Pmax, hq), float("nan"), dtype=torch.float32, device=dev)
        slots = torch.full((n,), 12345, dtype=torch.int64, device=dev)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
        return po, pl, slots, flag

    # two calls
    k2 = T["k_cache"].clone()
    v2 = None if T["v_cache"] is None else T["v_cache"].clone()
    po2, pl2, slots2, flag2 = buffers()
    P.pa_kv_append_routed(T["k_new"], T["v_new"], k2, v2, T["block_table"], T["context_lens"], S, I,
                          ks, vs, slots2, flag2)
    if fp8:
        P.pa_decode_fp8(T["q"], k2, v2, ks, vs, T["block_table"], T["context_lens"], S, I, T_part, Pmax,
                        scale, po2, pl2, dv=dv, err_flag=flag2)
    else:
        P.pa_decode(T["q"], k2, v2, T["block_table"], T["context_lens"], S, I, T_part, Pmax, scale, po2,
                    pl2, dv=dv, err_flag=flag2)

    # one call
    k1 = T["k_cache"].clone()
    v1 = None if T["v_cache"] is None else T["v_cache"].clone()
    po1, pl1, slots1, flag1 = buffers()
    P.pa_decode_step(T["q"], T["k_new"], T["v_new"], k1, v1, T["block_table"], T["context_lens"], S, I,
                     T_part, Pmax, scale, po1, pl1, k_scale=ks, v_scale=vs, slot_mapping=slots1, dv=dv,
                     err_flag=flag1)
    torch.cuda.synchronize()

    assert int(flag1.item()) == 0 and int(flag2.item()) == 0
    assert np.array_equal(to_np(slots1), to_np(slots2)), "slots differ"
    assert torch.equal(_bits(k1), _bits(k2)), "key cache differs"
    if v1 is not None:
        assert torch.equal(_bits(v1), _bits(v2)), "value cache differs"
    assert torch.equal(_bits(pl1), _bits(pl2)), "partial LSEs differ"
    assert torch.equal(_bits(po1), _bits(po2)), "partial outputs differ"


def test_decode_step_object_and_graph():
    """DecodeStep's call (pa_decode_step, then the merge when there are several parts)
    equals the step made of separate calls; its captured graph replays it exactly,
    with eager work in between, several times."""
    import decode_attention_paged_kv_amd as P

    say("[decode step] DecodeStep and graph")
    w = wl.small("step_obj", [300, 70, 1, 0, 900], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=128,
                 seed=11)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    Lmax = int(w.context_lens.max())
    mk = lambda: P.DecodeStep(w.n_seqs, 32, 8, 128, 128, 16, Lmax, partition_tokens=128,
                              scale=float(w.scale_f32), device=dev)
    ref = mk()
    k2, v2 = T["k_cache"].clone(), T["v_cache"].clone()
    ref.route_append(T["k_new"], T["v_new"], k2, v2, T["block_table"], T["context_lens"])
    ref.attend(T["q"], k2, v2, T["block_table"], T["context_lens"])
    ref.merge()
    step = mk()
    k1, v1 = T["k_cache"].clone(), T["v_cache"].clone()
    out, lse = step(T["q"], T["k_new"], T["v_new"], k1, v1, T["block_table"], T["context_lens"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(k1), _bits(k2)) and torch.equal(_bits(v1), _bits(v2))
    assert torch.equal(step.slot_mapping, ref.slot_mapping)
    assert torch.equal(_bits(out), _bits(ref.out)) and torch.equal(_bits(lse), _bits(ref.lse))

    k3, v3 = T["k_cache"].clone(), T["v_cache"].clone()
    g = step.capture(T["q"], T["k_new"], T["v_new"], k3, v3, T["block_table"], T["context_lens"])
    for rep in range(3):
        step.out.zero_()
        k3.copy_(T["k_cache"])
        v3.copy_(T["v_cache"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(k3), _bits(k2)) and torch.equal(_bits(v3), _bits(v2)), rep
        assert torch.equal(_bits(step.out), _bits(ref.out)), rep
        assert torch.equal(_bits(step.lse), _bits(ref.lse)), rep


@pytest.mark.parametrize("latent", [False, True], ids=["gqa", "latent"])
def test_decode_step_with_an_invalid_new_token_block(latent):
    """A sequence whose new token's table entry is invalid: the flag is raised, nothing is
    stored for it, its slot is -1 -- as in the two-call path -- and the other sequences
    append and attend as usual (caches, slots and outputs equal to the two-call path)."""
    import decode_attention_paged_kv_amd as P
    from oracle import paged_attention as pa

    if latent:
        w = wl.small("step_bad_latent", [300, 70, 900], 16, 1, 576, 512, 64, wl.BF16, latent=True,
                     partition_tokens=256, seed=31)
    else:
        w = wl.small("step_bad_gqa", [300, 70, 900, 5], 32, 8, 128, 128, 16, wl.BF16,
                     partition_tokens=128, seed=32)
    say(f"[decode step] invalid block, {w.name}")
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    n, hq, dv, bs = w.n_seqs, w.n_q_heads, w.dv, w.block_size
    nb = T["k_cache"].shape[0]
    T_part = w.partition_tokens
    Pmax = max(1, P.pa_max_partitions(int(w.context_lens.max()), 1, 1, T_part))
    b_bad = 2
    L_bad = int(w.context_lens[b_bad])
    bt = T["block_table"].clone()
    loc = int(pa.shard_lengths(L_bad, 1, 1)[0]) - 1
    bt[b_bad, 0, loc // bs] = nb + 7
    scale = float(w.scale_f32)

    def run(fused):
        k = T["k_cache"].clone()
        v = None if T["v_cache"] is None else T["v_cache"].clone()
        po = torch.full((n, 1, Pmax, hq, dv), float("nan"), dtype=torch.float32, device=dev)
        pl = torch.full((n, 1, Pmax, hq), float("nan"), dtype=torch.float32, device=dev)
        slots = torch.full((n,), 12345, dtype=torch.int64, device=dev)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
        if fused:
            P.pa_decode_step(T["q"], T["k_new"], T["v_new"], k, v, bt, T["context_lens"], 1, 1, T_part, Pmax,
                             scale, po, pl, slot_mapping=slots, dv=dv, err_flag=flag)
        else:
            P.pa_kv_append_routed(T["k_new"], T["v_new"], k, v, bt, T["context_lens"], 1, 1, None, None, slots,
                                  flag)
            P.pa_decode(T["q"], k, v, bt, T["context_lens"], 1, 1, T_part, Pmax, scale, po, pl, dv=dv,
                        err_flag=flag)
        torch.cuda.synchronize()
        return k, v, po, pl, slots, int(flag.item())

    k1, v1, po1, pl1, s1, f1 = run(True)
    k2, v2, po2, pl2, s2, f2 = run(False)
    assert f1 == f2 and f1 & P.ERR_BLOCK_ID, (f1, f2)
    assert int(s1[b_bad].item()) == -1 and torch.equal(s1, s2)
    assert torch.equal(_bits(k1), _bits(k2))
    if v1 is not None:
        assert torch.equal(_bits(v1), _bits(v2))
    assert torch.equal(_bits(pl1), _bits(pl2)) and torch.equal(_bits(po1), _bits(po2))


def test_decode_step_object_reuses_checked_arguments_safely():
    """DecodeStep keeps the checked argument list of its last call while the same tensors
    come back.  Calls on tensors A, then B, then A again each equal a fresh step on the
    same inputs bit for bit; a tensor of another shape in place of one of them is
    checked (and refused), not run on the old list."""
    import decode_attention_paged_kv_amd as P

    say("[decode step] argument reuse")
    dev = torch.device("cuda")
    w = wl.small("step_reuse", [300, 70, 1, 900], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=128,
                 seed=12)
    Lmax = int(w.context_lens.max())
    mk = lambda: P.DecodeStep(w.n_seqs, 32, 8, 128, 128, 16, Lmax, partition_tokens=128,
                              scale=float(w.scale_f32), device=dev)
    sets = [wl.make_tensors(w, dev, seed=s) for s in (1, 2)]
    caches = [(T["k_cache"].clone(), T["v_cache"].clone()) for T in sets]

    def args(j):
        T, (kc, vc) = sets[j], caches[j]
        return (T["q"], T["k_new"], T["v_new"], kc, vc, T["block_table"], T["context_lens"])

    step = mk()
    for j in (0, 1, 0):
        kc0, vc0 = caches[j][0].clone(), caches[j][1].clone()
        out, lse = step(*args(j))
        out, lse = out.clone(), lse.clone()
        fresh = mk()
        T = sets[j]
        ref_out, ref_lse = fresh(T["q"], T["k_new"], T["v_new"], kc0, vc0, T["block_table"],
                                 T["context_lens"])
        torch.cuda.synchronize()
        assert int(step.err_flag.item()) == 0
        assert torch.equal(_bits(out), _bits(ref_out)) and torch.equal(_bits(lse), _bits(ref_lse)), \
            f"call on set {j} differs"
        # (unused cache slots hold NaN poison: compare the bits)
        assert torch.equal(_bits(caches[j][0]), _bits(kc0)) and torch.equal(_bits(caches[j][1]), _bits(vc0)), \
            "appended rows differ"
    bad_q = sets[0]["q"][:, :16].contiguous()    # 16 query heads where the step has 32
    with pytest.raises((ValueError, P.PaError)):
        step(bad_q, *args(0)[1:])
