"""pa_kv_append_routed (routing and append in one launch) on the GPU.

Held bit for bit to the oracle (``slot_mapping`` then ``kv_append``, or ``fp8_kv``'s
append for an E4M3 cache) and to the library's two-call path (pa_slot_mapping, then
pa_kv_append / pa_kv_append_fp8): the slots it reports and every byte of both caches,
including the poisoned slots it must not touch.  Cases: bf16 and fp32 caches, DCP
shards with interleave, E4M3 caches with per-head and per-tensor scales from fp32 and
bf16 rows, the latent cache (no value tensor), empty and one-token sequences, and a
sequence whose table entry is invalid (flagged, nothing written for it)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import bits_equal, say, to_np
from oracle import fp8_kv as f8
from oracle import paged_attention as pa

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


# name, lens, hq, hkv, dk, dv, bs, dtype, S, I, latent, kv dtype, per-head scales
CASES = [
    ("bf16", [1, 17, 300, 0, 1000], 32, 8, 128, 128, 16, wl.BF16, 1, 1, False, "", True),
    ("f32_dcp", [0, 1, 5, 130, 77], 6, 3, 40, 24, 8, wl.F32, 3, 2, False, "", True),
    ("bf16_dcp16", [900, 31, 16], 64, 8, 128, 128, 16, wl.BF16, 4, 16, False, "", True),
    ("e4m3_head", [33, 520, 0, 1], 32, 8, 128, 128, 16, wl.BF16, 1, 1, False, wl.FP8, True),
    ("e4m3_tensor_f32", [3, 90, 64], 5, 1, 96, 80, 16, wl.F32, 2, 3, False, wl.FP8, False),
    ("latent", [65, 300, 1], 16, 1, 576, 512, 64, wl.BF16, 1, 1, True, "", True),
    ("latent_e4m3", [70, 0, 9], 16, 1, 576, 512, 64, wl.BF16, 1, 1, True, wl.FP8, True),
]


def _clone(t):
    return None if t is None else t.clone()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_routed_append_matches_oracle_and_two_calls(case):
    import decode_attention_paged_kv_amd as P

    name, lens, hq, hkv, dk, dv, bs, dt, S, I, latent, kv, per_head = case
    say(f"[routed append] {name}")
    w = wl.small(name, lens, hq, hkv, dk, dv, bs, dt, n_shards=S, interleave=I, latent=latent,
                 seed=sum(map(ord, name)) % 1000, kv_dtype=kv, scale_per_head=per_head)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    ks, vs = T.get("k_scale"), T.get("v_scale")
    fp8 = T["k_cache"].dtype == torch.uint8
    n = w.n_seqs
    nb = T["k_cache"].shape[0]

    # the oracle, from host copies taken before any append
    H = {k: to_np(T[k]) for k in ("k_new", "v_new", "k_cache", "v_cache", "block_table")}
    slots_ref = pa.slot_mapping(H["block_table"], w.context_lens, S, I, bs)
    if fp8:
        k_ref, v_ref = f8.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots_ref, bs,
                                    to_np(ks), to_np(vs))
    else:
        k_ref, v_ref = pa.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots_ref, bs)

    # two calls
    k2, v2 = _clone(T["k_cache"]), _clone(T["v_cache"])
    slots2 = torch.empty(n, dtype=torch.int64, device=dev)
    flag2 = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_slot_mapping(T["block_table"], T["context_lens"], S, I, bs, nb, slots2, flag2)
    if fp8:
        P.pa_kv_append_fp8(T["k_new"], T["v_new"], k2, v2, ks, vs, slots2, flag2)
    else:
        P.pa_kv_append(T["k_new"], T["v_new"], k2, v2, slots2, flag2)

    # one call
    k1, v1 = _clone(T["k_cache"]), _clone(T["v_cache"])
    slots1 = torch.full((n,), 12345, dtype=torch.int64, device=dev)
    flag1 = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_kv_append_routed(T["k_new"], T["v_new"], k1, v1, T["block_table"], T["context_lens"], S, I,
                          ks, vs, slots1, flag1)
    torch.cuda.synchronize()

    assert int(flag1.item()) == 0 and int(flag2.item()) == 0
    assert np.array_equal(to_np(slots1), slots_ref), "slots differ from the oracle's"
    assert np.array_equal(to_np(slots2), slots_ref)
    assert bits_equal(to_np(k1), k_ref), "key cache differs from the oracle's"
    assert bits_equal(to_np(k1), to_np(k2)), "key cache differs from the two-call path"
    if v1 is not None:
        assert bits_equal(to_np(v1), v_ref), "value cache differs from the oracle's"
        assert bits_equal(to_np(v1), to_np(v2)), "value cache differs from the two-call path"

    # without the slot output, and with a sequence whose table entry is invalid: that
    # sequence appends nothing (flag raised), the others as before
    b_bad = int(np.argmax(w.context_lens))
    L_bad = int(w.context_lens[b_bad])
    bt_bad = T["block_table"].clone()
    r_new = ((L_bad - 1) // I) % S
    loc = int(pa.shard_lengths(L_bad, S, I)[r_new]) - 1
    bt_bad[b_bad, r_new, loc // bs] = nb + 5
    k3, v3 = _clone(T["k_cache"]), _clone(T["v_cache"])
    flag3 = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_kv_append_routed(T["k_new"], T["v_new"], k3, v3, bt_bad, T["context_lens"], S, I, ks, vs,
                          None, flag3)
    torch.cuda.synchronize()
    assert int(flag3.item()) != 0, "an invalid block id must raise the flag"
    slots_bad = slots_ref.copy()
    slots_bad[b_bad] = -1
    if fp8:
        k_ref3, v_ref3 = f8.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots_bad,
                                      bs, to_np(ks), to_np(vs))
    else:
        k_ref3, v_ref3 = pa.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots_bad, bs)
    assert bits_equal(to_np(k3), k_ref3)
    if v3 is not None:
        assert bits_equal(to_np(v3), v_ref3)


def test_decode_step_uses_one_launch_for_routing_and_append():
    """DecodeStep's call gives the same caches, slots and outputs as the step run with
    separate routing and append calls."""
    import decode_attention_paged_kv_amd as P

    say("[routed append] DecodeStep")
    w = wl.small("routed_step", [300, 70, 1], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=64,
                 seed=8)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    outs = []
    for fused in (True, False):
        kc, vc = T["k_cache"].clone(), T["v_cache"].clone()
        step = P.DecodeStep(w.n_seqs, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size, 300,
                            partition_tokens=64, scale=w.scale_f32, device=dev)
        if fused:
            step(T["q"], T["k_new"], T["v_new"], kc, vc, T["block_table"], T["context_lens"])
        else:
            step.route(T["block_table"], T["context_lens"], kc.shape[0])
            step.append(T["k_new"], T["v_new"], kc, vc)
            step.attend(T["q"], kc, vc, T["block_table"], T["context_lens"])
            step.merge()
        torch.cuda.synchronize()
        assert int(step.err_flag.item()) == 0
        outs.append((kc, vc, step.slot_mapping.clone(), step.out.clone(), step.lse.clone()))
    for a, b in zip(*outs):
        assert bits_equal(to_np(a), to_np(b))
