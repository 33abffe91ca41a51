"""Run a workload through the HIP library and through the fp64 oracle, and
compare them.  Used by the ``gpu``-marked tests and by ``__graft_entry__.smoke``.

Tolerances, per input type:
* fp32 inputs: output max-abs 1e-5, LSE max-abs 1e-5;
* bf16 inputs: output max-abs 5e-3, LSE max-abs 1e-3;
plus a relative L2 bound on the whole output, ||o - o*|| / ||o*||, because at
long context the outputs are themselves only ~5e-3 in size (so max-abs 5e-3
alone would accept a zero output).  The relative bound comes from the kernels'
arithmetic: fp32 accumulation of exactly-widened inputs with the softmax
weights kept to >= 16 significant bits (every matrix-core kernel feeds them to the
value product as a bf16 high part plus a bf16 remainder) gives ~1e-6; the bound is
1e-4 on every path.
kv append, slot routing and the gather are compared bit for bit.

An E4M3 cache (``w.kv_dtype == FP8``) is compared with the oracle's ``fp8_kv``
step: the stored codes bit for bit, outputs with the tolerances of the query type
(the kernels read the same dequantised values the oracle does).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as wl
from oracle import fp8_kv as f8
from oracle import multi_query as mq
from oracle import paged_attention as pa

TOL = {wl.F32: dict(out=1e-5, lse=1e-5), wl.BF16: dict(out=5e-3, lse=1e-3)}
REL_L2 = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits_equal(a, b) -> bool:
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))


def run_library(w, T, partition_tokens=None, out_dtype=torch.float32):
    """One full step through the library on the current stream.  ``T`` holds GPU
    tensors from ``workloads.make_tensors`` (the caches are updated in place)."""
    import decode_attention_paged_kv_amd as P

    Tp = partition_tokens or w.partition_tokens or 0
    if w.multi:
        step = P.MultiDecodeStep(w.n_seqs, w.n_rows, max(1, int(w.q_lens.max())), w.n_q_heads,
                                 w.n_kv_heads, w.dk, w.dv, w.block_size, int(w.context_lens.max()),
                                 w.n_shards, w.interleave, Tp, w.scale_f32, device=T["q"].device,
                                 out_dtype=out_dtype, context_lens_host=w.context_lens,
                                 kv_dtype=T["k_cache"].dtype, latent=w.latent)
        step(T["q"], T["query_start"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
             T["block_table"], T["context_lens"], T.get("k_scale"), T.get("v_scale"))
        torch.cuda.synchronize()
        return step
    step = P.DecodeStep(w.n_seqs, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size,
                        int(w.context_lens.max()), w.n_shards, w.interleave, Tp, w.scale_f32,
                        device=T["q"].device, out_dtype=out_dtype,
                        context_lens_host=w.context_lens, kv_dtype=T["k_cache"].dtype,
                        latent=w.latent)
    out, lse = step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
                    T["block_table"], T["context_lens"], T.get("k_scale"), T.get("v_scale"))
    torch.cuda.synchronize()
    return step


def compare_outputs(name, dtype, o, lse, o_ref, lse_ref, rel_l2=REL_L2, partials=False):
    """Raise AssertionError with a message if the library's output misses the oracle's.
    For partition partials the output rows of empty partitions are unspecified (the
    library does not write them); merged outputs of empty rows must be exactly 0."""
    tol = TOL[dtype]
    out_tol = tol["out"]
    o = np.array(o, np.float64)
    lse = np.asarray(lse, np.float64)
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), ~empty), f"{name}: empty/nonempty pattern differs"
    assert np.all(lse[empty] == -np.inf), f"{name}: empty rows must have lse -inf"
    if partials:
        o[empty] = 0.0
    assert not np.isnan(o).any(), f"{name}: NaN in output"
    assert np.all(o[empty] == 0), f"{name}: empty rows must have output 0"
    d_o = np.max(np.abs(o - o_ref)) if o.size else 0.0
    d_l = np.max(np.abs(lse[~empty] - lse_ref[~empty])) if (~empty).any() else 0.0
    nrm = np.linalg.norm(o_ref)
    rel = np.linalg.norm(o - o_ref) / nrm if nrm > 0 else 0.0
    say(f"  {name}: max|do|={d_o:.3g} (tol {out_tol}) max|dlse|={d_l:.3g} (tol {tol['lse']}) "
        f"rel_l2={rel:.3g} (tol {rel_l2})")
    assert d_o <= out_tol, f"{name}: output max-abs {d_o:.3g} > {out_tol}"
    assert d_l <= tol["lse"], f"{name}: lse max-abs {d_l:.3g} > {tol['lse']}"
    assert rel <= rel_l2, f"{name}: output relative L2 {rel:.3g} > {rel_l2}"


def oracle_step(w, H, block_table, context_lens, Tp, Pmax, query_start=None):
    """The oracle's step on numpy inputs ``H`` (E4M3 caches through ``fp8_kv``; several
    new tokens per sequence through ``multi_query``, with ``query_start``)."""
    if w.multi:
        slots = mq.slot_mapping_multi(block_table, context_lens, query_start, w.n_shards,
                                      w.interleave, w.block_size)
        if w.cache_dtype == wl.FP8:
            kc, vc = f8.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots,
                                  w.block_size, H["k_scale"], H["v_scale"])
            kd, vd = f8.dequantize_cache(kc, vc, H["k_scale"], H["v_scale"])
        else:
            kc, vc = pa.kv_append(H["k_cache"], H["v_cache"], H["k_new"], H["v_new"], slots,
                                  w.block_size)
            kd, vd = kc, vc
        o, lse, part_o, part_lse = mq.decode_multi(H["q"], query_start, kd, vd, block_table,
                                                   context_lens, w.n_shards, w.interleave,
                                                   w.block_size, Tp, Pmax, w.scale_f32, w.dv)
        return dict(slots=slots, k_cache=kc, v_cache=vc, o=o, lse=lse, part_o=part_o,
                    part_lse=part_lse)
    if w.cache_dtype == wl.FP8:
        return f8.decode_step(H["q"], H["k_new"], H["v_new"], H["k_cache"], H["v_cache"],
                              H["k_scale"], H["v_scale"], block_table, context_lens, w.n_shards,
                              w.interleave, w.block_size, Tp, Pmax, w.scale_f32, w.dv)
    return pa.decode_step(H["q"], H["k_new"], H["v_new"], H["k_cache"], H["v_cache"],
                          block_table, context_lens, w.n_shards, w.interleave, w.block_size,
                          Tp, Pmax, w.scale_f32, w.dv)


def check_small(w, partition_tokens=None, fill="normal", rel_l2=REL_L2, seed=None, tweak=None):
    """Whole-workload parity: routing, append (whole pool, bitwise), gather
    (bitwise, every sequence and shard), partials and merged outputs.  ``tweak``,
    if given, edits the CPU tensors in place before both sides see them."""
    import decode_attention_paged_kv_amd as P

    say(f"[parity] {w.name} N={w.n_seqs} Hq={w.n_q_heads} Hkv={w.n_kv_heads} dk={w.dk} dv={w.dv} "
        f"bs={w.block_size} {w.dtype} S={w.n_shards} I={w.interleave} lens={list(w.context_lens)[:8]}")
    Tc = wl.make_tensors(w, "cpu", fill=fill, seed=seed)
    if tweak is not None:
        tweak(Tc)
    H = {k: to_np(v) for k, v in Tc.items()}
    dev = torch.device("cuda")
    T = {k: (None if v is None else v.to(dev)) for k, v in Tc.items()}
    step = run_library(w, T, partition_tokens)
    Tp, Pmax = step.partition_tokens, step.max_partitions
    ref = oracle_step(w, H, w.block_table, w.context_lens, Tp, Pmax, w.query_start)
    kdt = T["k_cache"].dtype
    assert int(step.err_flag.item()) == 0, f"{w.name}: device error flag {int(step.err_flag.item())}"
    assert np.array_equal(to_np(step.slot_mapping), ref["slots"]), f"{w.name}: slot mapping"
    assert bits_equal(to_np(T["k_cache"]), ref["k_cache"]), f"{w.name}: k_cache after append"
    if ref["v_cache"] is not None:
        assert bits_equal(to_np(T["v_cache"]), ref["v_cache"]), f"{w.name}: v_cache after append"
    # gather through the library's address generation
    for b in range(w.n_seqs):
        L = int(w.context_lens[b])
        for r in range(w.n_shards):
            Lr = P.pa_shard_length(L, w.n_shards, w.interleave, r)
            kg = torch.empty(max(Lr, 1), w.n_kv_heads, w.dk, dtype=kdt, device=dev)
            vg = torch.empty(max(Lr, 1), w.n_kv_heads, w.dv, dtype=kdt, device=dev)
            P.pa_gather_kv(T["k_cache"], T["v_cache"], T["block_table"], b, r, L, w.n_shards,
                           w.interleave, kg, vg, step.err_flag)
            kr, vr = pa.gather_shard(ref["k_cache"], ref["v_cache"], w.block_table[b], L, r,
                                     w.n_shards, w.interleave, w.block_size, w.dv)
            assert bits_equal(to_np(kg)[:Lr], kr) and bits_equal(to_np(vg)[:Lr], vr), \
                f"{w.name}: gather seq {b} shard {r}"
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) == 0
    compare_outputs(f"{w.name} partials", w.dtype, to_np(step.part_out), to_np(step.part_lse),
                    ref["part_o"], ref["part_lse"], rel_l2, partials=True)
    compare_outputs(f"{w.name} merged", w.dtype, to_np(step.out), to_np(step.lse), ref["o"],
                    ref["lse"], rel_l2)
    return step, ref


def check_large(w, sample_seqs=None, partition_tokens=None, fill="normal", rel_l2=REL_L2):
    """Full-size parity: the step runs at the workload's real size in the launch
    configuration the benchmark times; routing is compared for every sequence,
    the append for the whole pool (every slot but the new ones unchanged, the new
    ones equal to the new rows), and the attention of every sequence (or of
    ``sample_seqs`` when given), whose blocks are copied out of the pre-step pool
    and handed to the oracle one sequence at a time."""
    import decode_attention_paged_kv_amd as P

    if sample_seqs is None:
        sample_seqs = range(w.n_seqs)
    say(f"[parity-large] {w.name} N={w.n_seqs} sum(L)={int(w.context_lens.sum())} "
        f"S={w.n_shards} I={w.interleave} fill={fill} seqs={len(sample_seqs)}")
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev, fill=fill)
    k_before = T["k_cache"].clone()
    v_before = None if T["v_cache"] is None else T["v_cache"].clone()
    step = run_library(w, T, partition_tokens)
    assert int(step.err_flag.item()) == 0, f"{w.name}: device error flag"
    if w.multi:
        slots_ref = mq.slot_mapping_multi(w.block_table, w.context_lens, w.query_start, w.n_shards,
                                          w.interleave, w.block_size)
    else:
        slots_ref = pa.slot_mapping(w.block_table, w.context_lens, w.n_shards, w.interleave,
                                    w.block_size)
    assert np.array_equal(to_np(step.slot_mapping), slots_ref), f"{w.name}: slot mapping"
    # append: compare slot-major views on the device
    bs = w.block_size
    sl = torch.from_numpy(slots_ref).to(dev)

    def bits(x):
        return x.view({torch.bfloat16: torch.int16, torch.float32: torch.int32,
                       torch.uint8: torch.uint8}[x.dtype])

    def slot_major_k(x):            # [NB][Hkv][bs][dk] -> [NB*bs][Hkv*dk]
        return bits(x).permute(0, 2, 1, 3).reshape(x.shape[0] * bs, -1)

    def slot_major_v(x):            # [NB][Hkv][dv][bs] -> [NB*bs][Hkv*dv]
        return bits(x).permute(0, 3, 1, 2).reshape(x.shape[0] * bs, -1)

    fp8 = w.cache_dtype == wl.FP8
    for after, before, new, fn, sc in ((T["k_cache"], k_before, T["k_new"], slot_major_k, T.get("k_scale")),
                                       (T["v_cache"], v_before, T["v_new"], slot_major_v, T.get("v_scale"))):
        if after is None:
            continue
        A, B = fn(after), fn(before)
        changed = torch.nonzero((A != B).any(dim=1)).flatten().cpu().numpy()
        assert set(changed.tolist()) <= set(slots_ref.tolist()), f"{w.name}: append touched other slots"
        if fp8:     # the oracle's codes of the new rows under each head's scale
            hs = f8.head_scales(to_np(sc), w.n_kv_heads)
            want = f8.quantize(to_np(new), hs[None, :, None]).reshape(new.shape[0], -1)
            newbits = torch.from_numpy(want).to(dev)
        else:
            newbits = new.reshape(new.shape[0], -1).view(A.dtype)
        valid = sl >= 0                  # empty sequences append nothing (slot -1)
        assert torch.equal(A[sl[valid]], newbits[valid]), f"{w.name}: appended rows differ"
    del A, B
    Tp, Pmax = step.partition_tokens, step.max_partitions
    for b in sample_seqs:
        L = int(w.context_lens[b])
        ids = np.unique(w.block_table[b][w.block_table[b] >= 0])
        remap = {int(x): i for i, x in enumerate(ids)}
        bt_b = np.vectorize(lambda x: remap.get(int(x), -1))(w.block_table[b:b + 1])
        idx = torch.from_numpy(ids).to(dev)
        kc = to_np(k_before.index_select(0, idx))
        vc = None if v_before is None else to_np(v_before.index_select(0, idx))
        rows = slice(int(w.query_start[b]), int(w.query_start[b + 1]))   # this sequence's q rows
        kn = to_np(T["k_new"][rows])
        vn = None if T["v_new"] is None else to_np(T["v_new"][rows])
        qb = to_np(T["q"][rows])
        Hb = dict(q=qb, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc,
                  k_scale=to_np(T.get("k_scale")), v_scale=to_np(T.get("v_scale")))
        qs_b = np.array([0, rows.stop - rows.start], np.int32)
        ref = oracle_step(w, Hb, bt_b.astype(np.int32), w.context_lens[b:b + 1], Tp, Pmax, qs_b)
        # the gather of each shard, bit for bit
        for r in range(w.n_shards):
            Lr = P.pa_shard_length(L, w.n_shards, w.interleave, r)
            kg = torch.empty(max(Lr, 1), w.n_kv_heads, w.dk, dtype=T["k_cache"].dtype, device=dev)
            vg = torch.empty(max(Lr, 1), w.n_kv_heads, w.dv, dtype=T["k_cache"].dtype, device=dev)
            P.pa_gather_kv(T["k_cache"], T["v_cache"], T["block_table"], b, r, L, w.n_shards,
                           w.interleave, kg, vg, step.err_flag)
            kr, vr = pa.gather_shard(ref["k_cache"], ref["v_cache"], bt_b[0], L, r, w.n_shards,
                                     w.interleave, bs, w.dv)
            assert bits_equal(to_np(kg)[:Lr], kr) and bits_equal(to_np(vg)[:Lr], vr), \
                f"{w.name}: gather seq {b} shard {r}"
        compare_outputs(f"{w.name} seq {b} partials", w.dtype, to_np(step.part_out[rows]),
                        to_np(step.part_lse[rows]), ref["part_o"], ref["part_lse"], rel_l2,
                        partials=True)
        compare_outputs(f"{w.name} seq {b} merged", w.dtype, to_np(step.out[rows]),
                        to_np(step.lse[rows]), ref["o"], ref["lse"], rel_l2)
    torch.cuda.synchronize()
    assert int(step.err_flag.item()) == 0
    return step
