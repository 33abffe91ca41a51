"""The C-ABI library on the CPU: it loads, exports every entry point that
include/pa.h declares, its host helpers compute the placement closed forms, and
argument errors are reported without launching anything (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

pytest.importorskip("torch")
P = pytest.importorskip("decode_attention_paged_kv_amd")
from oracle import paged_attention as pa  # noqa: E402


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"pa_kv_append", "pa_decode", "pa_merge_lse", "pa_slot_mapping", "pa_gather_kv"} <= set(names)
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("L,S,I", [(0, 1, 1), (1, 4, 16), (67, 4, 1), (67, 4, 16), (200000, 4, 1),
                                   (200000, 4, 16), (1000, 3, 7), (5, 4, 16), (123457, 5, 3)])
def test_shard_length_matches_oracle(L, S, I):
    got = [P.pa_shard_length(L, S, I, r) for r in range(S)]
    assert got == list(pa.shard_lengths(L, S, I))
    for T in (1, 16, 1024):
        assert P.pa_max_partitions(L, S, I, T) == pa.max_partitions(L, S, I, T)


def test_host_helpers_reject_bad_arguments():
    assert P.pa_shard_length(10, 0, 1, 0) == -1
    assert P.pa_shard_length(10, 2, 0, 0) == -1
    assert P.pa_shard_length(10, 2, 1, 2) == -1
    assert P.pa_max_partitions(10, 1, 1, 0) == -1
    T = P.pa_default_partition_tokens(8, 8, 200000, 1, 1, 16)
    assert T > 0 and T % 16 == 0
    assert P.pa_default_partition_tokens(1, 8, 200000, 4, 16, 64) % 64 == 0


def _call_decode(**over):
    args = dict(q=1, k=1, v=1, bt=1, lens=1, n=1, hq=4, hkv=1, dk=64, dv=64, bs=4, nb=64, mb=17,
                S=1, I=1, T=4, P=17, scale=0.125, dt=0, po=1, pl=1)
    args.update(over)
    a = args
    vp = lambda x: None if x is None else ctypes.c_void_p(0x1000)  # never dereferenced: rejected first
    return P.lib.pa_decode(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]), vp(a["lens"]), a["n"],
                           a["hq"], a["hkv"], a["dk"], a["dv"], a["bs"], a["nb"], a["mb"], a["S"],
                           a["I"], a["T"], a["P"], a["scale"], a["dt"], vp(a["po"]), vp(a["pl"]),
                           None, None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(po=None), -1), (dict(dt=7), -3), (dict(hq=6, hkv=4), -2),
    (dict(dk=577), -3), (dict(dv=513), -3), (dict(v=None, dv=65), -2), (dict(bs=0), -3),
    (dict(bs=257), -3), (dict(S=0), -2), (dict(I=0), -2), (dict(T=6), -2), (dict(T=0), -2),
    (dict(P=0), -4), (dict(n=-1), -2), (dict(mb=0), -2),
])
def test_decode_rejects_bad_arguments_without_launch(over, status):
    assert _call_decode(**over) == status
    assert P.lib.pa_last_error().decode() != ""


def test_other_entry_points_reject_bad_arguments():
    vp = ctypes.c_void_p(0x1000)
    assert P.lib.pa_kv_append(None, None, vp, None, vp, 1, 1, 64, 64, 4, 64, 0, None, None) == -1
    assert P.lib.pa_kv_append(vp, vp, vp, None, vp, 1, 1, 64, 64, 4, 64, 0, None, None) == -1
    assert P.lib.pa_kv_append(vp, None, vp, None, vp, 1, 1, 64, 64, 4, 64, 5, None, None) == -3
    assert P.lib.pa_merge_lse(None, vp, 1, 1, 1, 64, vp, 0, None, None) == -1
    assert P.lib.pa_merge_lse(vp, vp, 1, 0, 1, 64, vp, 0, None, None) == -2
    assert P.lib.pa_merge_lse(vp, vp, 1, 1, 1, 1024, vp, 0, None, None) == -3
    assert P.lib.pa_slot_mapping(vp, vp, 1, 0, 1, 4, 17, 64, vp, None, None) == -2
    assert P.lib.pa_gather_kv(vp, vp, vp, 0, 4, 67, 1, 64, 64, 4, 64, 17, 4, 1, 0, vp, vp, None, None) == -2
    # zero-size work is accepted and launches nothing
    assert P.lib.pa_kv_append(vp, vp, vp, vp, vp, 0, 1, 64, 64, 4, 64, 0, None, None) == 0
    assert _call_decode(n=0) == 0


def test_choose_partition_tokens():
    import torch

    import workloads as wl

    for w in (wl.batch(), wl.dcp(16), wl.small("x", [5, 900], 8, 2, 64, 64, 32, wl.BF16)):
        T = P.pa_choose_partition_tokens(w.context_lens, w.n_q_heads, w.n_kv_heads, w.dk, w.dv,
                                         w.block_size, torch.bfloat16, w.latent, w.n_shards,
                                         w.interleave)
        assert T > 0 and T % w.block_size == 0
    lens = np.array([10], np.int32)
    assert P.lib.pa_choose_partition_tokens(None, 1, 4, 1, 64, 64, 4, 0, 0, 1, 1) == -1
    assert P.pa_choose_partition_tokens(lens, 6, 4, 64, 64, 4, torch.float32, False) == -1


def test_choose_partition_tokens_multi():
    """The multi-token chooser models pa_decode_multi's own launch: one new token gives
    the single-token choice; on the latent shape two new tokens double the latent
    kernel's units (the partition shrinks, never grows), where scaling the head count
    instead would leave the latent kernel's model."""
    import torch

    import workloads as wl

    for w in (wl.long(), wl.latent(), wl.small("x", [5, 900], 8, 2, 64, 64, 32, wl.BF16)):
        args = (w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size, torch.bfloat16, w.latent,
                w.n_shards, w.interleave)
        T1 = P.pa_choose_partition_tokens(w.context_lens, *args)
        assert P.pa_choose_partition_tokens_multi(w.context_lens, 1, *args) == T1
        T2 = P.pa_choose_partition_tokens_multi(w.context_lens, 2, *args)
        assert T2 > 0 and T2 % w.block_size == 0
        if w.latent:
            assert T2 <= T1
            scaled = P.pa_choose_partition_tokens(w.context_lens, 2 * w.n_q_heads, *args[1:])
            assert T2 != scaled
    lens = np.array([10], np.int32)
    assert P.pa_choose_partition_tokens_multi(lens, 0, 4, 1, 64, 64, 4, torch.bfloat16, False) == -1
    assert P.lib.pa_choose_partition_tokens_multi(None, 1, 2, 4, 1, 64, 64, 4, 0, 0, 1, 1) == -1


def test_fp8_entry_points_reject_bad_arguments():
    vp = ctypes.c_void_p(0x1000)
    ap = P.lib.pa_kv_append_fp8
    # k_new, v_new, new_dtype, k_cache, v_cache, k_scale, v_scale, n_scales, slots, n, hkv, dk, dv, bs, nb
    assert ap(vp, vp, 1, vp, vp, None, vp, 1, vp, 1, 2, 64, 64, 16, 8, None, None) == -1   # no k_scale
    assert ap(vp, vp, 1, vp, vp, vp, None, 1, vp, 1, 2, 64, 64, 16, 8, None, None) == -1   # no v_scale
    assert ap(vp, vp, 2, vp, vp, vp, vp, 1, vp, 1, 2, 64, 64, 16, 8, None, None) == -3     # fp8 rows
    assert ap(vp, vp, 1, vp, vp, vp, vp, 3, vp, 1, 2, 64, 64, 16, 8, None, None) == -2     # n_scales
    assert ap(vp, vp, 1, vp, vp, vp, vp, 2, vp, 0, 2, 64, 64, 16, 8, None, None) == 0      # nothing to do
    dp = P.lib.pa_decode_fp8

    def dec(**over):
        a = dict(q=vp, k=vp, v=vp, ks=vp, vs=vp, ns=1, bt=vp, lens=vp, n=1, hq=8, hkv=2, dk=64,
                 dv=64, bs=16, nb=8, mb=4, S=1, I=1, T=16, P=4, scale=0.125, dt=1)
        a.update(over)
        return dp(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["ns"], a["bt"], a["lens"], a["n"],
                  a["hq"], a["hkv"], a["dk"], a["dv"], a["bs"], a["nb"], a["mb"], a["S"], a["I"],
                  a["T"], a["P"], a["scale"], a["dt"], vp, vp, None, None)

    assert dec(ks=None) == -1
    assert dec(vs=None) == -1
    assert dec(v=None, vs=None, n=0) == 0                  # latent: no value scale needed
    assert dec(ns=3) == -2
    assert dec(dt=2) == -3                                 # queries are not E4M3
    assert dec(n=0) == 0
    assert P.pa_choose_partition_tokens(np.array([1000], np.int32), 8, 2, 64, 64, 16,
                                        __import__("torch").uint8, False) % 16 == 0


def test_multi_entry_points_reject_bad_arguments():
    vp = ctypes.c_void_p(0x1000)
    sm = P.lib.pa_slot_mapping_multi
    # bt, lens, qstart, n_seqs, n_rows, S, I, bs, mb, nb, slots, flag, stream
    assert sm(vp, vp, None, 1, 1, 1, 1, 16, 4, 8, vp, None, None) == -1
    assert sm(vp, vp, vp, 1, -1, 1, 1, 16, 4, 8, vp, None, None) == -2
    assert sm(vp, vp, vp, 1, 1, 0, 1, 16, 4, 8, vp, None, None) == -2
    assert sm(vp, vp, vp, 0, 0, 1, 1, 16, 4, 8, vp, None, None) == 0
    dm = P.lib.pa_decode_multi

    def dec(**over):
        a = dict(q=vp, qdt=1, qs=vp, rows=4, maxq=2, k=vp, v=vp, kvdt=1, ks=None, vs=None, ns=0,
                 bt=vp, lens=vp, n=2, hq=8, hkv=2, dk=128, dv=128, bs=16, nb=8, mb=4, S=1, I=1,
                 T=16, P=4, scale=0.1)
        a.update(over)
        return dm(a["q"], a["qdt"], a["qs"], a["rows"], a["maxq"], a["k"], a["v"], a["kvdt"], a["ks"],
                  a["vs"], a["ns"], a["bt"], a["lens"], a["n"], a["hq"], a["hkv"], a["dk"], a["dv"],
                  a["bs"], a["nb"], a["mb"], a["S"], a["I"], a["T"], a["P"], a["scale"], vp, vp, None,
                  None)

    assert dec(qs=None) == -1
    assert dec(maxq=0) == -2
    assert dec(rows=-1) == -2
    assert dec(kvdt=0) == -3                          # f32 cache with bf16 queries
    assert dec(kvdt=2) == -1                          # E4M3 cache without scales
    assert dec(kvdt=2, ks=vp, vs=vp, ns=3) == -2
    assert dec(maxq=1 << 20) == -2                    # launch grid too large
    assert dec(rows=0) == 0
    assert dec(n=0) == 0


def test_chooser_picks_long_partitions_for_long_contexts():
    """Long contexts spread over every compute unit in partitions of thousands of tokens,
    not a block or two (the per-partition cost would dominate)."""
    import torch

    import workloads as wl

    for w, hq in ((wl.dcp(1), 64), (wl.long(), 32), (wl.speculative(), 32 * 4)):
        for kv in (torch.bfloat16, torch.uint8):
            T = P.pa_choose_partition_tokens(w.context_lens, hq, w.n_kv_heads, w.dk, w.dv,
                                             w.block_size, kv, False, w.n_shards, w.interleave)
            assert 1024 <= T <= 16384, (w.name, kv, T)


def test_routed_append_rejects_bad_arguments():
    vp = ctypes.c_void_p(0x1000)
    ap = P.lib.pa_kv_append_routed

    def call(**over):
        # k_new, v_new, new_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale, n_scales,
        # block_table, context_lens, n_seqs, hkv, dk, dv, bs, nb, max_blocks, S, I, slots, flag
        a = dict(kn=vp, vn=vp, nd=1, kc=vp, vc=vp, cd=1, ks=None, vs=None, ns=0, bt=vp, lens=vp, n=4,
                 hkv=2, dk=64, dv=64, bs=16, nb=8, mb=4, S=1, I=1, slots=None, flag=None)
        a.update(over)
        return ap(*a.values(), None)

    assert call(n=0) == 0                          # nothing to do
    assert call(bt=None) == -1
    assert call(lens=None) == -1
    assert call(vn=None) == -1                     # v_new without v_cache
    assert call(nd=0) == -3                        # rows f32, cache bf16
    assert call(cd=7) == -3
    assert call(nd=2, cd=2) == -3                  # E4M3 rows
    assert call(cd=2) == -1                        # E4M3 cache without scales
    assert call(cd=2, ks=vp, vs=vp, ns=3) == -2    # 3 scales for 2 KV heads
    assert call(cd=2, ks=vp, vs=vp, ns=2, n=0) == 0
    assert call(S=0) == -2
    assert call(I=0) == -2
    assert call(bs=0) == -3
    assert call(mb=0) == -2
    assert call(dk=0) == -3
    assert call(n=-1) == -2
    assert "n_seqs" in P.lib.pa_last_error().decode()


def test_decode_rejects_a_grid_past_2_31():
    vp = ctypes.c_void_p(0x1000)
    # q, k, v, bt, lens, n, hq, hkv, dk, dv, bs, nb, mb, S, I, T, P, scale, dtype, po, pl, flag, stream
    st = P.lib.pa_decode(vp, vp, vp, vp, vp, 1 << 20, 8, 2, 64, 64, 16, 8, 4, 64, 1, 16, 64, 0.125, 1,
                         vp, vp, None, None)
    assert st == -2 and "exceeds 2^31-1" in P.lib.pa_last_error().decode()


def test_decode_step_rejects_bad_arguments():
    vp = ctypes.c_void_p(0x1000)
    ds = P.lib.pa_decode_step

    def call(**over):
        # q, k_new, v_new, new_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale, n_scales,
        # block_table, context_lens, n_seqs, hq, hkv, dk, dv, bs, nb, max_blocks, S, I, T, Pmax,
        # scale, q_dtype, slots, part_out, part_lse, flag
        a = dict(q=vp, kn=vp, vn=vp, nd=1, kc=vp, vc=vp, cd=1, ks=None, vs=None, ns=0, bt=vp, lens=vp,
                 n=4, hq=8, hkv=2, dk=64, dv=64, bs=16, nb=8, mb=4, S=1, I=1, T=64, P=4, scale=0.125,
                 qd=1, slots=None, po=vp, pl=vp, flag=None)
        a.update(over)
        return ds(*a.values(), None)

    assert call(n=0) == 0                          # nothing to do
    assert call(kn=None) == -1
    assert call(vn=None) == -1                     # v_new without v_cache
    assert call(q=None) == -1
    assert call(po=None) == -1
    assert call(nd=0) == -3                        # rows f32, cache and q bf16
    assert call(cd=0) == -3                        # cache f32, q bf16
    assert call(cd=7) == -3
    assert call(nd=2) == -3                        # E4M3 rows
    assert call(cd=2) == -1                        # E4M3 cache without scales
    assert call(cd=2, ks=vp, vs=vp, ns=3) == -2    # 3 scales for 2 KV heads
    assert call(cd=2, ks=vp, vs=vp, ns=2, n=0) == 0
    assert call(T=24) == -2                        # not a multiple of the block size
    assert call(S=0) == -2
    assert call(n=-1) == -2
    assert "n_seqs" in P.lib.pa_last_error().decode()
