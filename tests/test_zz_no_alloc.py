"""pa_decode_step_static (a decode step that allocates nothing; its partials live in the
library's fixed device array) against the entry points it stands in for: pa_decode_step
with caller-allocated partials, then pa_merge_lse.  Same kernels on the same inputs, so
the outputs, LSEs, slots and caches must be identical bit for bit.  Two calls in a row,
the second smaller (the array keeps the first call's contents), then a call whose
partials would not fit, which must fail with PA_ERR_BUFFER and launch nothing; and the
call recorded into a HIP graph (its use case), replayed several times with eager work in
between, each replay equal to the eager call."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


def _static_call(T, w, k_cache, v_cache, T_part, Pmax, out, lse, slots, flag):
    import decode_attention_paged_kv_amd._lib as L

    q = T["q"]
    n, hq, dk = q.shape
    nb, hkv, bs, _ = k_cache.shape
    return L.lib.pa_decode_step_static(
        L._ptr(q), L._ptr(T["k_new"]), L._ptr(T["v_new"]), L._dtype_code(T["k_new"]), L._ptr(k_cache),
        L._ptr(v_cache), L._dtype_code(k_cache, cache=True), None, None, 0, L._ptr(T["block_table"]),
        L._ptr(T["context_lens"]), n, hq, hkv, dk, w.dv, bs, nb, T["block_table"].shape[2], w.n_shards,
        w.interleave, T_part, Pmax, float(w.scale_f32), L._dtype_code(q), L._ptr(slots), L._ptr(out),
        L.PA_F32, L._ptr(lse), L._ptr(flag), L._stream(q))


def _one(name, lens, hq, hkv, S, I, T_part, seed):
    import decode_attention_paged_kv_amd as P

    say(f"[no-alloc step] {name}")
    w = wl.small(name, lens, hq, hkv, 128, 128, 16, wl.BF16, n_shards=S, interleave=I,
                 partition_tokens=T_part, seed=seed)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    n = w.n_seqs
    Pmax = max(1, P.pa_max_partitions(int(max(lens)), S, I, T_part))
    assert S * Pmax > 1, "the case must go through the merge"

    # the existing entry points, with partials the caller allocates
    k2, v2 = T["k_cache"].clone(), T["v_cache"].clone()
    po = torch.empty(n, S, Pmax, hq, w.dv, dtype=torch.float32, device=dev)
    pl = torch.empty(n, S, Pmax, hq, dtype=torch.float32, device=dev)
    out2 = torch.empty(n, hq, w.dv, dtype=torch.float32, device=dev)
    lse2 = torch.empty(n, hq, dtype=torch.float32, device=dev)
    slots2 = torch.empty(n, dtype=torch.int64, device=dev)
    flag2 = torch.zeros(1, dtype=torch.int32, device=dev)
    P.pa_decode_step(T["q"], T["k_new"], T["v_new"], k2, v2, T["block_table"], T["context_lens"], S, I,
                     T_part, Pmax, float(w.scale_f32), po, pl, slot_mapping=slots2, dv=w.dv,
                     err_flag=flag2)
    P.pa_merge_lse(po, pl, out2, lse2)

    # the static entry point
    k1, v1 = T["k_cache"].clone(), T["v_cache"].clone()
    out1 = torch.full((n, hq, w.dv), float("nan"), dtype=torch.float32, device=dev)
    lse1 = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
    slots1 = torch.full((n,), 12345, dtype=torch.int64, device=dev)
    flag1 = torch.zeros(1, dtype=torch.int32, device=dev)
    st = _static_call(T, w, k1, v1, T_part, Pmax, out1, lse1, slots1, flag1)
    torch.cuda.synchronize()
    assert st == 0, P.lib.pa_last_error().decode()
    assert int(flag1.item()) == 0 and int(flag2.item()) == 0
    assert torch.equal(slots1, slots2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), "outputs differ"
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32)), "LSEs differ"
    return T, w


def test_static_step_matches_the_allocating_entry_points_twice():
    _one("static_big", [900, 17, 2000, 1, 0, 600, 1400, 33] * 3, 32, 8, 1, 1, 128, 21)
    T, w = _one("static_small_dcp", [300, 5, 1, 800], 64, 8, 2, 16, 64, 22)

    # partials beyond the array: rejected before any launch, nothing written
    import decode_attention_paged_kv_amd as P

    dev = torch.device("cuda")
    n = w.n_seqs
    k, v = T["k_cache"].clone(), T["v_cache"].clone()
    out = torch.full((n, 64, w.dv), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((n, 64), 7.0, dtype=torch.float32, device=dev)
    slots = torch.full((n,), 5, dtype=torch.int64, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    import decode_attention_paged_kv_amd._lib as L

    Pmax = L.PA_STATIC_SCRATCH_BYTES // (n * 2 * 64 * (w.dv + 1) * 4) + 1
    st = _static_call(T, w, k, v, 64, Pmax, out, lse, slots, flag)
    torch.cuda.synchronize()
    assert st == L.PA_ERR_BUFFER
    assert "partials need" in P.lib.pa_last_error().decode()
    assert torch.equal(k.view(torch.int16), T["k_cache"].view(torch.int16))   # NaN-poisoned slots:
    assert torch.equal(v.view(torch.int16), T["v_cache"].view(torch.int16))   # compare the bits
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()) and bool((slots == 5).all())


def test_static_step_under_graph_capture():
    import decode_attention_paged_kv_amd as P

    say("[no-alloc step] graph capture")
    w = wl.small("static_graph", [700, 20, 1300, 0, 64], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=128,
                 seed=23)
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    n = w.n_seqs
    Pmax = max(1, P.pa_max_partitions(int(w.context_lens.max()), 1, 1, 128))
    k, v = T["k_cache"].clone(), T["v_cache"].clone()
    out = torch.empty(n, 32, w.dv, dtype=torch.float32, device=dev)
    lse = torch.empty(n, 32, dtype=torch.float32, device=dev)
    slots = torch.empty(n, dtype=torch.int64, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    assert _static_call(T, w, k, v, 128, Pmax, out, lse, slots, flag) == 0
    torch.cuda.synchronize()
    out_ref, lse_ref, k_ref, v_ref = out.clone(), lse.clone(), k.clone(), v.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        k.copy_(T["k_cache"])
        v.copy_(T["v_cache"])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            assert _static_call(T, w, k, v, 128, Pmax, out, lse, slots, flag) == 0
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        out.zero_()
        lse.zero_()
        k.copy_(T["k_cache"])
        v.copy_(T["v_cache"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        assert torch.equal(out.view(torch.int32), out_ref.view(torch.int32)), rep
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), rep
        assert torch.equal(k.view(torch.int16), k_ref.view(torch.int16)), rep
        assert torch.equal(v.view(torch.int16), v_ref.view(torch.int16)), rep
