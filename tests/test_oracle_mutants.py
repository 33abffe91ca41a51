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
from oracle import paged_attention as pa

_attention = pa.attention
_merge = pa.merge_lse
_members = pa.shard_members
_gather_shard = pa.gather_shard
_kv_append = pa.kv_append
_copy_blocks = pa.copy_blocks


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
