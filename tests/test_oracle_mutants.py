"""Planted mistakes in the oracle must be caught by its pins.

Each case replaces one function of the oracle (on the CPU, in this process
only) with a plausible wrong version -- a dropped term, a wrong index, a wrong
sign, a transposed operand -- and requires at least one of the pin checks in
``oracle_checks`` to fail.  This shows the pins constrain every part of the
oracle, not only its happy path.
"""
import numpy as np
import pytest

import oracle_checks as oc
from oracle import fp8_kv as f8
from oracle import multi_query as mq
from oracle import paged_attention as pa

_attention = pa.attention
_merge = pa.merge_lse
_members = pa.shard_members
_gather_shard = pa.gather_shard
_kv_append = pa.kv_append
_copy_blocks = pa.copy_blocks
_quantize = f8.quantize
_dequantize_cache = f8.dequantize_cache
_E4M3 = f8.E4M3.copy()
_mq_partials = mq.decode_multi_partials
_mq_slots = mq.slot_mapping_multi


def _attn_variant(kind):
    def f(q, K, V, scale):
        qd, Kd, Vd = pa.widen(q), pa.widen(K), pa.widen(V)
        hq, L, hkv, dv = qd.shape[0], Kd.shape[0], Kd.shape[1], Vd.shape[-1]
        g = hq // hkv
        o = np.zeros((hq, dv))
        lse = np.full(hq, -np.inf)
        if L == 0:
            return o, lse
        for h in range(hq):
            kvh = h % hkv if kind == "head_map" else h // g
            sc = 1.0 if kind == "no_scale" else scale
            s = sc * (Kd[:, kvh, :] @ qd[h])
            m = s.max()
            p = np.exp(s - m)
            l = p.sum()
            if kind == "no_norm":
                o[h] = p @ Vd[:, kvh, :]
            elif kind == "values_reversed":
                o[h] = (p @ Vd[::-1, kvh, :]) / l
            else:
                o[h] = (p @ Vd[:, kvh, :]) / l
            lse[h] = np.log(l) if kind == "lse_no_max" else m + np.log(l)
            if kind == "lse_log2":
                lse[h] = m + np.log2(l)
        return o, lse
    return f


def _merge_variant(kind):
    def f(part_o, part_lse):
        po = np.asarray(part_o, np.float64)
        pl = np.asarray(part_lse, np.float64)
        if kind == "drop_last":
            po, pl = po[:-1], pl[:-1]
        hq, dv = po.shape[1], po.shape[2]
        o = np.zeros((hq, dv))
        lse = np.full(hq, -np.inf)
        for h in range(hq):
            live = np.isfinite(pl[:, h])
            if not live.any():
                continue
            m = pl[live, h].max()
            total = m + np.log(np.exp(pl[live, h] - m).sum())
            w = np.exp(total - pl[live, h]) if kind == "sign" else np.exp(pl[live, h] - total)
            if kind == "uniform":
                w = np.full(live.sum(), 1.0 / live.sum())
            o[h] = w @ po[live, h, :]
            lse[h] = total
        return o, lse
    return f


def _members_no_interleave(L, S, I, r):
    ids = np.arange(L, dtype=np.int64)
    return ids[ids % S == r]


def _members_blocked(L, S, I, r):
    ids = np.arange(L, dtype=np.int64)
    return ids[(ids * S) // max(L, 1) == r]          # contiguous ranges instead of round-robin


def _gather_offset_shift(k_cache, v_cache, bt_b, L, r, S, I, bs, dv):
    L_r = pa.shard_members(L, S, I, r).size
    t = np.arange(L_r, dtype=np.int64)
    phys = np.asarray(bt_b[r], dtype=np.int64)[t // bs]
    off = (t + 1) % bs
    return pa._rows(k_cache, v_cache, phys, off, dv)


def _gather_v_from_k(k_cache, v_cache, bt_b, L, r, S, I, bs, dv):
    k, v = _gather_shard(k_cache, v_cache, bt_b, L, r, S, I, bs, dv)
    return k, k[:, :, :dv]


def _append_wrong_offset(k_cache, v_cache, k_new, v_new, slots, bs):
    return _kv_append(k_cache, v_cache, k_new, v_new, np.asarray(slots) + 1, bs)


def _copy_keys_only(k_cache, v_cache, pairs):
    k, _ = _copy_blocks(k_cache, None, pairs)
    return k, None if v_cache is None else v_cache.copy()


def _copy_reversed(k_cache, v_cache, pairs):
    return _copy_blocks(k_cache, v_cache, [(d, s) for s, d in pairs])


def _copy_nothing(k_cache, v_cache, pairs):
    return k_cache.copy(), None if v_cache is None else v_cache.copy()


def _quantize_truncate(x, scale):
    """round toward zero instead of to nearest"""
    y = (f8.to_f32(x) / np.asarray(scale, np.float32)).astype(np.float32)
    a = np.abs(y).astype(np.float64)
    code = (np.searchsorted(f8._POS, a, side="right") - 1).clip(0, f8.MAX_CODE)
    code = np.where(np.isnan(y), f8.NAN_CODE, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def _quantize_ties_up(x, scale):
    """ties go to the larger magnitude instead of the even code"""
    codes = _quantize(x, scale)
    y = (f8.to_f32(x) / np.asarray(scale, np.float32)).astype(np.float64)
    mag = codes & 0x7F
    up = np.minimum(mag + 1, f8.MAX_CODE)
    tie = (mag < f8.MAX_CODE) & (np.abs(np.abs(y) - f8.E4M3[mag]) == np.abs(f8.E4M3[up] - np.abs(y))) \
        & (f8.E4M3[up] > np.abs(y))
    return np.where(tie, up | (codes & 0x80), codes).astype(np.uint8)


def _quantize_times_scale(x, scale):
    """multiplies by the scale instead of dividing"""
    return _quantize(x, 1.0 / np.asarray(scale, np.float32))


def _dequantize_v_unscaled(k_cache, v_cache, k_scale, v_scale):
    kd, vd = _dequantize_cache(k_cache, v_cache, k_scale, v_scale)
    if v_cache is not None:
        vd = f8.dequantize(v_cache, 1.0)
    return kd, vd


def _dequantize_heads_reversed(k_cache, v_cache, k_scale, v_scale):
    hkv = k_cache.shape[1]
    ks = f8.head_scales(k_scale, hkv)[::-1]
    vs = None if v_scale is None else f8.head_scales(v_scale, hkv)[::-1]
    return _dequantize_cache(k_cache, v_cache, ks, vs)


MUTANTS = {
    "attention.head_map": ("attention", _attn_variant("head_map")),
    "attention.no_scale": ("attention", _attn_variant("no_scale")),
    "attention.no_norm": ("attention", _attn_variant("no_norm")),
    "attention.values_reversed": ("attention", _attn_variant("values_reversed")),
    "attention.lse_no_max": ("attention", _attn_variant("lse_no_max")),
    "attention.lse_log2": ("attention", _attn_variant("lse_log2")),
    "merge.sign": ("merge_lse", _merge_variant("sign")),
    "merge.drop_last": ("merge_lse", _merge_variant("drop_last")),
    "merge.uniform": ("merge_lse", _merge_variant("uniform")),
    "shard.no_interleave": ("shard_members", _members_no_interleave),
    "shard.blocked": ("shard_members", _members_blocked),
    "gather.offset": ("gather_shard", _gather_offset_shift),
    "gather.v_from_k": ("gather_shard", _gather_v_from_k),
    "append.offset": ("kv_append", _append_wrong_offset),
    "copy.keys_only": ("copy_blocks", _copy_keys_only),
    "copy.reversed": ("copy_blocks", _copy_reversed),
    "copy.nothing": ("copy_blocks", _copy_nothing),
}
FP8_MUTANTS = {
    "fp8.truncate": ("quantize", _quantize_truncate),
    "fp8.ties_up": ("quantize", _quantize_ties_up),
    "fp8.times_scale": ("quantize", _quantize_times_scale),
    "fp8.v_unscaled": ("dequantize_cache", _dequantize_v_unscaled),
    "fp8.heads_reversed": ("dequantize_cache", _dequantize_heads_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    failures = []
    for check in oc.ALL_CHECKS.values():
        try:
            msg = check()
        except Exception as e:          # a crash is also a detection
            msg = f"raised {type(e).__name__}"
        if msg:
            failures.append(msg)
            break
    assert failures, f"planted mistake {name} passed every pin"


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS) + ["fp8.subnormal_table"])
def test_fp8_mutant_is_caught(name, monkeypatch):
    if name == "fp8.subnormal_table":
        bad = _E4M3.copy()
        bad[1:8] *= 2.0                                # subnormals with the wrong exponent
        bad[0x81:0x88] *= 2.0
        monkeypatch.setattr(f8, "E4M3", bad)
        monkeypatch.setattr(f8, "_POS", bad[:0x7F])
    else:
        attr, fn = FP8_MUTANTS[name]
        monkeypatch.setattr(f8, attr, fn)
    failures = []
    for check in oc.ALL_CHECKS.values():
        try:
            msg = check()
        except Exception as e:          # a crash is also a detection
            msg = f"raised {type(e).__name__}"
        if msg:
            failures.append(msg)
            break
    assert failures, f"planted mistake {name} passed every pin"


def _mq_shifted(shift):
    """the causal bound moved by ``shift`` positions (clipped to the context)"""
    def f(q, query_start, k_cache, v_cache, block_table, context_lens, S, I, bs, T, Pmax, scale, dv):
        n = mq.query_counts(query_start)
        rows, hq = q.shape[0], q.shape[1]
        po = np.zeros((rows, S, Pmax, hq, dv))
        pl = np.full((rows, S, Pmax, hq), -np.inf)
        row = 0
        for b, L in enumerate(np.asarray(context_lens)):
            L = int(L)
            for r in range(S):
                K, V = pa.gather_shard(k_cache, v_cache, block_table[b], L, r, S, I, bs, dv)
                members = pa.shard_members(L, S, I, r)
                for i in range(int(n[b])):
                    pos = min(L - int(n[b]) + i + shift, L - 1) if shift is not None else L - 1
                    seen = int(np.count_nonzero(members <= pos))
                    p = 0
                    while p * T < K.shape[0]:
                        lo, hi = p * T, min((p + 1) * T, seen)
                        if hi > lo:
                            po[row + i, r, p], pl[row + i, r, p] = pa.attention(q[row + i], K[lo:hi],
                                                                                 V[lo:hi], scale)
                        p += 1
            row += int(n[b])
        return po, pl
    return f


def _mq_rows_reversed(q, query_start, *args):
    qs = np.asarray(query_start)
    q2 = q.copy()
    for b in range(len(qs) - 1):
        q2[qs[b]:qs[b + 1]] = q[qs[b]:qs[b + 1]][::-1]
    return _mq_partials(q2, query_start, *args)


def _mq_slots_first_position(block_table, context_lens, query_start, S, I, bs):
    out = _mq_slots(block_table, context_lens, query_start, S, I, bs)
    return out[::-1].copy()


MQ_MUTANTS = {
    "mq.bound_plus1": ("decode_multi_partials", _mq_shifted(1)),
    "mq.bound_minus1": ("decode_multi_partials", _mq_shifted(-1)),
    "mq.no_causal": ("decode_multi_partials", _mq_shifted(None)),
    "mq.rows_reversed": ("decode_multi_partials", _mq_rows_reversed),
    "mq.slots_reversed": ("slot_mapping_multi", _mq_slots_first_position),
}


@pytest.mark.parametrize("name", sorted(MQ_MUTANTS))
def test_multi_query_mutant_is_caught(name, monkeypatch):
    attr, fn = MQ_MUTANTS[name]
    monkeypatch.setattr(mq, attr, fn)
    failures = []
    for check in oc.ALL_CHECKS.values():
        try:
            msg = check()
        except Exception as e:          # a crash is also a detection
            msg = f"raised {type(e).__name__}"
        if msg:
            failures.append(msg)
            break
    assert failures, f"planted mistake {name} passed every pin"
