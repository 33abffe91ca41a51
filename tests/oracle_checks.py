"""Checks that pin the fp64 oracle to things other than itself.

Each check returns ``None`` when it holds and a short message when it does not,
so that the same checks serve the plain pin tests (``test_oracle_pins.py``) and
the planted-mistake tests (``test_oracle_mutants.py``), which replace one piece
of the oracle with a plausible wrong version and require some check to fail.

What each check compares against:
* ``bruteforce``     -- 40-digit ``decimal`` scalar loops (no NumPy) on tiny inputs,
                        with GQA handled by ``np.repeat`` of the KV heads (MHA form);
* ``closed_forms``   -- one token (output = its value, LSE = its score) and two
                        tokens (logistic weights, ``logaddexp``), via SciPy/NumPy;
* ``mean_probe``     -- all-zero query: exact rational mean of integer values, LSE = ln L;
* ``shift``          -- adding a constant c to every score leaves the output and
                        moves the LSE by c (built with an extra key dimension);
* ``sdpa``           -- the paged decode step equals the last row of full causal
                        attention over the contiguous sequence (PyTorch SDPA, fp64,
                        ``enable_gqa``), contiguous K/V rebuilt from the generator's
                        own record of which token sits in which slot;
* ``gather``         -- the oracle's gather equals that record, bit for bit;
* ``slots``          -- the oracle's slot for each new token equals the generator's;
* ``merge``          -- S interleaved shards merged equal the unsharded result, for
                        two partition sizes, and merging is associative;
* ``copy_on_write``  -- forked sequences appending through the block manager, with its
                        block copies applied, read back exactly their own rows (kept
                        in a per-sequence Python list);
* ``fp8_table``      -- the E4M3 code values equal torch's float8_e4m3fn decoding;
* ``fp8_rounding``   -- quantised codes equal torch's float8_e4m3fn cast inside the
                        range (ties, subnormals, bf16 inputs, four scales), the error is
                        within half an ulp, and the saturation/NaN readings hold;
* ``fp8_decode``     -- the E4M3 step equals causal SDPA (fp64) over K/V decoded by
                        torch and scaled per head, new rows cast by torch;
* ``multi_sdpa``     -- with several new tokens per sequence, each one's output equals
                        its row of causal SDPA (fp64) over the whole sequence;
* ``multi_as_prefixes`` -- each new token equals the single-token step on the sequence
                        cut after it, one new token per sequence is the single-token
                        step, and the new tokens' slots equal the generator's.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

import numpy as np

from oracle import paged_attention as pa


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------------
def bruteforce_attention(q, K, V, scale):
    """Scalar, 40-digit decimal softmax attention in MHA form: ``K``/``V`` are
    ``[L][Hq][d]`` (one KV row per query head).  Returns lists of Decimals."""
    getcontext().prec = 40
    hq, dk = len(q), len(q[0])
    L = len(K)
    dv = len(V[0][0])
    sc = Decimal(float(scale))
    out, lses = [], []
    for h in range(hq):
        e = []
        for t in range(L):
            s = Decimal(0)
            for d in range(dk):
                s += Decimal(float(q[h][d])) * Decimal(float(K[t][h][d]))
            e.append((sc * s).exp())
        den = sum(e, Decimal(0))
        row = []
        for j in range(dv):
            num = Decimal(0)
            for t in range(L):
                num += e[t] * Decimal(float(V[t][h][j]))
            row.append(num / den)
        out.append(row)
        lses.append(den.ln())
    return out, lses


def check_bruteforce(seeds=range(6)):
    for seed in seeds:
        r = _rng(seed)
        hkv = int(r.integers(1, 3))
        g = int(r.integers(1, 3))
        hq = hkv * g
        L = int(r.integers(1, 9))
        dk = int(r.integers(1, 5))
        dv = int(r.integers(1, 5))
        q = r.standard_normal((hq, dk)).astype(np.float32)
        K = r.standard_normal((L, hkv, dk)).astype(np.float32)
        V = r.standard_normal((L, hkv, dv)).astype(np.float32)
        scale = float(np.float32(r.uniform(0.2, 1.5)))
        o, lse = pa.attention(q, K, V, scale)
        Kx = np.repeat(K.astype(np.float64), g, axis=1)
        Vx = np.repeat(V.astype(np.float64), g, axis=1)
        ob, lb = bruteforce_attention(q.astype(np.float64), Kx, Vx, scale)
        ob = np.array([[float(x) for x in row] for row in ob])
        lb = np.array([float(x) for x in lb])
        if np.max(np.abs(o - ob)) > 1e-13 or np.max(np.abs(lse - lb)) > 1e-13:
            return f"bruteforce seed {seed}: |do|={np.max(np.abs(o - ob)):.3g} |dlse|={np.max(np.abs(lse - lb)):.3g}"
    return None


def check_closed_forms():
    from scipy.special import expit

    r = _rng(11)
    for dk, dv in ((3, 2), (8, 5)):
        q = r.standard_normal((2, dk))
        K = r.standard_normal((2, 1, dk))
        V = r.standard_normal((2, 1, dv))
        scale = 0.7
        # one token
        o, lse = pa.attention(q, K[:1], V[:1], scale)
        s0 = scale * np.array([np.dot(q[h], K[0, 0]) for h in range(2)])
        if not (np.array_equal(o, np.repeat(V[0], 2, axis=0)) and np.allclose(lse, s0, rtol=0, atol=1e-14)):
            return "single token: output must be its value and lse its score"
        # two tokens
        o, lse = pa.attention(q, K, V, scale)
        for h in range(2):
            a = scale * np.dot(q[h], K[0, 0])
            b = scale * np.dot(q[h], K[1, 0])
            want = expit(a - b) * V[0, 0] + expit(b - a) * V[1, 0]
            if np.max(np.abs(o[h] - want)) > 1e-14 or abs(lse[h] - np.logaddexp(a, b)) > 1e-14:
                return "two tokens: logistic weights / logaddexp mismatch"
    return None


def check_mean_probe():
    from fractions import Fraction

    r = _rng(12)
    for L in (1, 5, 37):
        hkv, g, dk, dv = 2, 3, 4, 6
        q = np.zeros((hkv * g, dk))
        K = r.standard_normal((L, hkv, dk))
        V = r.integers(-8, 9, (L, hkv, dv)).astype(np.float64)
        o, lse = pa.attention(q, K, V, 1.0)
        for h in range(hkv * g):
            kvh = np.repeat(np.arange(hkv), g)[h]
            for j in range(dv):
                exact = Fraction(int(V[:, kvh, j].sum()), L)
                if abs(o[h, j] - float(exact)) > 1e-14:
                    return f"mean probe L={L}: output is not the mean of V"
        if np.max(np.abs(lse - np.log(L))) > 1e-14:
            return f"mean probe L={L}: lse is not ln L"
    return None


def check_shift():
    r = _rng(13)
    L, hkv, g, dk, dv = 23, 2, 2, 5, 3
    q = r.standard_normal((hkv * g, dk))
    K = r.standard_normal((L, hkv, dk))
    V = r.standard_normal((L, hkv, dv))
    scale = 0.6
    o0, l0 = pa.attention(q, K, V, scale)
    for c in (3.25, -40.0):
        q1 = np.concatenate([q, np.full((hkv * g, 1), c / scale)], axis=1)
        K1 = np.concatenate([K, np.ones((L, hkv, 1))], axis=2)
        o1, l1 = pa.attention(q1, K1, V, scale)
        if np.max(np.abs(o1 - o0)) > 1e-12 or np.max(np.abs(l1 - (l0 + c))) > 1e-12:
            return f"shift by {c}: output must not move and lse must move by c"
    return None


# ----------------------------------------------------------------------------------
# paged path, using the input generator's own record of the layout
# ----------------------------------------------------------------------------------
def small_workloads():
    import workloads as wl

    return [
        wl.small("mha_f32", [1, 7, 30], 3, 3, 8, 8, 4, wl.F32, seed=21),
        wl.small("gqa_bf16", [5, 33, 17], 4, 2, 16, 16, 8, wl.BF16, partition_tokens=8, seed=22),
        wl.small("dcp_i1", [1, 3, 41, 64], 4, 2, 8, 8, 4, wl.BF16, n_shards=4, interleave=1,
                 partition_tokens=4, seed=23),
        wl.small("dcp_i3", [2, 29, 50], 2, 1, 8, 8, 4, wl.F32, n_shards=3, interleave=3,
                 partition_tokens=8, seed=24),
        wl.small("latent", [17, 70, 70, 131], 8, 1, 24, 16, 8, wl.BF16, latent=True,
                 prefix_group=2, prefix_tokens=16, partition_tokens=16, seed=25),
    ]


def tensors_np(w, fill="normal"):
    import torch
    import workloads as wl

    t = wl.make_tensors(w, "cpu", fill=fill)

    def conv(x):
        if x is None:
            return None
        if x.dtype == torch.bfloat16:
            return x.contiguous().view(torch.int16).numpy().view(np.uint16)
        return x.contiguous().numpy()

    return {k: conv(v) for k, v in t.items()}


def contiguous_from_generator(w, T, b):
    """Global-order K/V rows of sequence ``b`` rebuilt from the generator's
    token-id record (every slot of every block in the sequence's table row that
    holds one of its tokens), with the appended token taken from ``k_new``/``v_new``."""
    L = int(w.context_lens[b])
    kc, vc = T["k_cache"], T["v_cache"]
    hkv, dk, dv = w.n_kv_heads, w.dk, w.dv
    K = np.empty((L, hkv, dk), kc.dtype)
    V = np.empty((L, hkv, dv), kc.dtype)
    seen = np.zeros(L, bool)
    for r in range(w.n_shards):
        for phys in w.block_table[b, r]:
            if phys < 0:
                continue
            for o in range(w.block_size):
                i = w.token_id[phys, o]
                if i < 0 or i >= L or not w.live[phys, o]:
                    continue
                K[i] = kc[phys, :, o, :]
                V[i] = kc[phys, :, o, :dv] if vc is None else vc[phys, :, :, o]
                seen[i] = True
    K[L - 1] = T["k_new"][b]
    V[L - 1] = T["k_new"][b][:, :dv] if T["v_new"] is None else T["v_new"][b]
    seen[L - 1] = True
    assert seen.all()
    return K, V


def run_oracle_step(w, T, partition_tokens=None):
    Tp = partition_tokens or w.partition_tokens or 16
    pmax = pa.max_partitions(int(w.context_lens.max()), w.n_shards, w.interleave, Tp)
    return pa.decode_step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
                          w.block_table, w.context_lens, w.n_shards, w.interleave, w.block_size,
                          Tp, pmax, w.scale_f32, w.dv)


def check_sdpa():
    import torch
    import torch.nn.functional as F

    for w in small_workloads():
        T = tensors_np(w)
        res = run_oracle_step(w, T)
        for b in range(w.n_seqs):
            K, V = contiguous_from_generator(w, T, b)
            L = K.shape[0]
            r = _rng(100 + b)
            Q = r.standard_normal((L, w.n_q_heads, w.dk))
            Q[L - 1] = pa.widen(T["q"][b])
            qt = torch.from_numpy(Q).permute(1, 0, 2)[None]
            kt = torch.from_numpy(pa.widen(K)).permute(1, 0, 2)[None]
            vt = torch.from_numpy(pa.widen(V)).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale_f32,
                                                 enable_gqa=True)[0, :, L - 1, :].numpy()
            err = np.max(np.abs(res["o"][b] - ref))
            if not err <= 1e-12:
                return f"sdpa {w.name} seq {b}: |do|={err:.3g}"
    return None


def check_gather():
    for w in small_workloads():
        T = tensors_np(w)
        res = run_oracle_step(w, T)
        for b in range(w.n_seqs):
            K, V = contiguous_from_generator(w, T, b)
            Kg, Vg = pa.gather_sequence(res["k_cache"], res["v_cache"], w.block_table[b],
                                        int(w.context_lens[b]), w.n_shards, w.interleave,
                                        w.block_size, w.dv)
            if not (np.array_equal(K.view(np.uint8), Kg.view(np.uint8))
                    and np.array_equal(V.view(np.uint8), Vg.view(np.uint8))):
                return f"gather {w.name} seq {b}: bits differ from the generator's layout"
    return None


def check_slots():
    for w in small_workloads():
        s = pa.slot_mapping(w.block_table, w.context_lens, w.n_shards, w.interleave, w.block_size)
        if not np.array_equal(s, w.new_slot):
            return f"slots {w.name}: {s} vs generator {w.new_slot}"
    return None


def check_merge():
    import workloads as wl

    for I in (1, 5):
        w = wl.small("m", [1, 6, 77], 4, 2, 8, 8, 4, wl.F32, n_shards=4, interleave=I, seed=31)
        T = tensors_np(w)
        res = run_oracle_step(w, T, partition_tokens=4)
        res2 = run_oracle_step(w, T, partition_tokens=64)
        for b in range(w.n_seqs):
            K, V = contiguous_from_generator(w, T, b)
            o, lse = pa.attention(T["q"][b], K, V, w.scale_f32)
            for rr in (res, res2):
                if np.max(np.abs(rr["o"][b] - o)) > 1e-12 or np.max(np.abs(rr["lse"][b] - lse)) > 1e-12:
                    return f"merge I={I} seq {b}: shards merged != unsharded"
            # associativity: merge per shard, then merge the shard results
            po, pl = res["part_o"][b], res["part_lse"][b]
            per = [pa.merge_lse(po[r], pl[r]) for r in range(w.n_shards)]
            o2, l2 = pa.merge_lse(np.stack([x[0] for x in per]), np.stack([x[1] for x in per]))
            if np.max(np.abs(o2 - o)) > 1e-12 or np.max(np.abs(l2 - lse)) > 1e-12:
                return f"merge I={I} seq {b}: not associative"
    return None


def check_copy_on_write():
    """Forked sequences that each append their own tokens, with the block copies the
    block manager asks for carried out by ``copy_blocks``, read back through their
    tables exactly the rows written for them: the shared prefix, then their own.  The
    expected rows come from a per-sequence Python list, never from the cache."""
    from oracle import block_manager as bm

    for latent in (False, True):
        bs, hkv, dk, dv, nb = 4, 2, 3, 2, 24
        r = _rng(11)
        cache = {"k": np.zeros((nb, hkv, bs, dk), np.float32),
                 "v": None if latent else np.zeros((nb, hkv, dv, bs), np.float32)}
        m = bm.BlockManager(nb, bs)
        rows = {}                                     # seq -> list of (k_row, v_row)

        def write(seq, n):
            for _ in range(n):
                before = len(m.copies)
                m.append(seq, 1)
                cache["k"], cache["v"] = pa.copy_blocks(cache["k"], cache["v"], m.copies[before:])
                i = m.lengths[seq] - 1
                slot = m.tables[seq][i // bs] * bs + i % bs
                kn = r.standard_normal((1, hkv, dk)).astype(np.float32)
                vn = None if latent else r.standard_normal((1, hkv, dv)).astype(np.float32)
                cache["k"], cache["v"] = pa.kv_append(cache["k"], cache["v"], kn, vn,
                                                      np.array([slot]), bs)
                rows[seq].append((kn[0], kn[0][:, :dv] if latent else vn[0]))

        m.add("P")
        rows["P"] = []
        write("P", 6)
        for c in ("a", "b", "c"):
            m.fork("P", c)
            rows[c] = list(rows["P"])
        write("a", 3)
        write("b", 1)
        write("P", 2)
        m.fork("b", "d")
        rows["d"] = list(rows["b"])
        write("d", 5)
        write("b", 2)
        if len(m.copies) < 3:
            return "copy-on-write: the scenario made fewer copies than planned"
        for seq, want in rows.items():
            bt = np.full((1, 8), -1, np.int32)
            bt[0, :len(m.tables[seq])] = m.tables[seq]
            K, V = pa.gather_sequence(cache["k"], cache["v"], bt, m.lengths[seq], 1, 1, bs, dv)
            if not (np.array_equal(K, np.stack([x[0] for x in want]))
                    and np.array_equal(V, np.stack([x[1] for x in want]))):
                return f"copy-on-write (latent={latent}): sequence {seq} reads other rows"
    return None


# ----------------------------------------------------------------------------------
# FP8 (E4M3) cache: the oracle's code table and rounding against torch's float8_e4m3fn
# conversions, the format's error bound, and the step against SDPA on values decoded
# by torch
# ----------------------------------------------------------------------------------
def check_fp8_table():
    import torch

    from oracle import fp8_kv as f8

    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    if not np.array_equal(np.isnan(ref), np.isnan(f8.E4M3)):
        return "fp8 table: NaN codes differ from torch's float8_e4m3fn"
    fin = ~np.isnan(ref)
    if not np.array_equal(ref[fin], f8.E4M3[fin]) or f8.E4M3[0x7E] != 448.0:
        return "fp8 table: values differ from torch's float8_e4m3fn"
    return None


def _fp8_probe_values():
    """float32 values spanning every binade of E4M3, exact code values, the midpoints
    between neighbouring codes (ties), the subnormal range and signed zeros."""
    from oracle import fp8_kv as f8

    r = _rng(41)
    x = r.standard_normal(20000) * 2.0 ** r.integers(-14, 9, 20000)
    pos = f8.E4M3[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, pos, -pos, mids, -mids, [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    return x.astype(np.float32)


def check_fp8_rounding():
    import torch

    from oracle import fp8_kv as f8

    x = _fp8_probe_values()
    for s in (1.0, 0.37, 3.1, 2.0 ** -5):
        s32 = np.float32(s)
        y = torch.from_numpy(x) / torch.tensor(s32)
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = f8.quantize(x, s32)
        inside = np.abs(y.numpy()) < 448          # torch does not saturate; compared apart
        if not np.array_equal(got[inside], ref[inside]):
            return f"fp8 rounding (scale {s}): codes differ from torch's float8_e4m3fn cast"
        # the format's own bound: half a unit in the last place
        yv = y.numpy().astype(np.float64)
        err = np.abs(f8.E4M3[got[inside]] - yv[inside])
        bound = np.maximum(np.abs(yv[inside]) * 2.0 ** -4, 2.0 ** -10)
        if np.any(err > bound):
            return f"fp8 rounding (scale {s}): error above half an ulp"
    # bf16 input rows are widened exactly before the division
    xb = torch.from_numpy(x[:5000]).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    yb = xb.float() / torch.tensor(np.float32(0.37))
    ref = yb.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inside = np.abs(yb.numpy()) < 448
    if not np.array_equal(f8.quantize(bits, np.float32(0.37))[inside], ref[inside]):
        return "fp8 rounding: bf16 inputs"
    # saturation and NaN (the readings: +-448 beyond the range, NaN keeps its sign)
    sat = f8.quantize(np.array([448, 449, 463.9, 464, 1e6, np.inf, -np.inf, -500, np.nan,
                                -np.nan], np.float32), np.float32(1.0))
    if sat.tolist() != [0x7E] * 6 + [0xFE, 0xFE, 0x7F, 0xFF]:
        return f"fp8 saturation: {[hex(c) for c in sat]}"
    return None


def fp8_workloads():
    import workloads as wl

    return [
        wl.small("f8_gqa", [5, 33, 17], 4, 2, 16, 16, 8, wl.BF16, partition_tokens=8, seed=51,
                 kv_dtype=wl.FP8),
        wl.small("f8_tensor_scale", [9, 40], 6, 3, 8, 8, 4, wl.F32, partition_tokens=16, seed=52,
                 kv_dtype=wl.FP8, scale_per_head=False),
        wl.small("f8_dcp", [3, 41, 64], 4, 2, 8, 8, 4, wl.BF16, n_shards=4, interleave=3,
                 partition_tokens=4, seed=53, kv_dtype=wl.FP8),
        wl.small("f8_latent", [17, 70], 8, 1, 24, 16, 8, wl.BF16, latent=True, partition_tokens=16,
                 seed=54, kv_dtype=wl.FP8),
    ]


def check_fp8_decode():
    """The E4M3 step equals the last row of causal SDPA (fp64) over K/V decoded with
    torch's float8_e4m3fn conversion and multiplied by each head's scale; the
    appended token's rows are torch's cast of new_row / scale."""
    import torch
    import torch.nn.functional as F

    from oracle import fp8_kv as f8

    def decode_torch(codes, scales, head_axis):
        vals = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
        shape = [1] * vals.ndim
        shape[head_axis] = -1
        return vals * scales.astype(np.float64).reshape(shape)

    for w in fp8_workloads():
        T = tensors_np(w)
        Tp = w.partition_tokens
        pmax = pa.max_partitions(int(w.context_lens.max()), w.n_shards, w.interleave, Tp)
        res = f8.decode_step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
                             T["k_scale"], T["v_scale"], w.block_table, w.context_lens,
                             w.n_shards, w.interleave, w.block_size, Tp, pmax, w.scale_f32, w.dv)
        ks = np.resize(T["k_scale"], w.n_kv_heads).astype(np.float32)
        vs = None if T["v_scale"] is None else np.resize(T["v_scale"], w.n_kv_heads).astype(np.float32)
        for b in range(w.n_seqs):
            Kc, Vc = contiguous_from_generator(w, T, b)    # codes; the new row is raw input
            L = Kc.shape[0]
            K = np.empty(Kc.shape)
            V = np.empty(Vc.shape)
            K[:L - 1] = decode_torch(Kc[:L - 1], ks, 1)
            newk = torch.from_numpy(pa.widen(T["k_new"][b]).astype(np.float32))
            kq = (newk / torch.from_numpy(ks)[:, None]).to(torch.float8_e4m3fn)
            K[L - 1] = kq.double().numpy() * ks[:, None]
            if T["v_new"] is None:
                V[:] = K[:, :, :w.dv]
            else:
                V[:L - 1] = decode_torch(Vc[:L - 1], vs, 1)
                newv = torch.from_numpy(pa.widen(T["v_new"][b]).astype(np.float32))
                vq = (newv / torch.from_numpy(vs)[:, None]).to(torch.float8_e4m3fn)
                V[L - 1] = vq.double().numpy() * vs[:, None]
            r = _rng(200 + b)
            Q = r.standard_normal((L, w.n_q_heads, w.dk))
            Q[L - 1] = pa.widen(T["q"][b])
            qt = torch.from_numpy(Q).permute(1, 0, 2)[None]
            kt = torch.from_numpy(K).permute(1, 0, 2)[None]
            vt = torch.from_numpy(np.ascontiguousarray(V)).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale_f32,
                                                 enable_gqa=True)[0, :, L - 1, :].numpy()
            err = np.max(np.abs(res["o"][b] - ref))
            if not err <= 1e-12:
                return f"fp8 sdpa {w.name} seq {b}: |do|={err:.3g}"
    return None


# ----------------------------------------------------------------------------------
# several new tokens per sequence (causal among them)
# ----------------------------------------------------------------------------------
def multi_workloads():
    import workloads as wl

    return [
        wl.small("mq_gqa", [5, 33, 17, 9], 4, 2, 16, 16, 8, wl.BF16, partition_tokens=8, seed=61,
                 q_lens=[3, 5, 1, 0]),
        wl.small("mq_dcp", [40, 64, 7], 4, 2, 8, 8, 4, wl.F32, n_shards=3, interleave=2,
                 partition_tokens=4, seed=62, q_lens=[6, 2, 7]),
        wl.small("mq_latent", [17, 70], 8, 1, 24, 16, 8, wl.BF16, latent=True, partition_tokens=16,
                 seed=63, q_lens=[4, 4]),
    ]


def run_multi_step(w, T, partition_tokens=None):
    from oracle import multi_query as mq

    Tp = partition_tokens or w.partition_tokens or 16
    pmax = pa.max_partitions(int(w.context_lens.max()), w.n_shards, w.interleave, Tp)
    return mq.decode_step_multi(T["q"], w.query_start, T["k_new"], T["v_new"], T["k_cache"],
                                T["v_cache"], w.block_table, w.context_lens, w.n_shards,
                                w.interleave, w.block_size, Tp, pmax, w.scale_f32, w.dv)


def contiguous_multi(w, T, b):
    """Global-order K/V rows of sequence ``b`` from the generator's token record, with
    its new tokens (the last ``q_lens[b]``) taken from the new rows."""
    L, n = int(w.context_lens[b]), int(w.q_lens[b])
    kc, vc = T["k_cache"], T["v_cache"]
    K = np.empty((L, w.n_kv_heads, w.dk), kc.dtype)
    V = np.empty((L, w.n_kv_heads, w.dv), kc.dtype)
    seen = np.zeros(L, bool)
    for r in range(w.n_shards):
        for phys in w.block_table[b, r]:
            if phys < 0:
                continue
            for o in range(w.block_size):
                i = w.token_id[phys, o]
                if i < 0 or i >= L or not w.live[phys, o]:
                    continue
                K[i] = kc[phys, :, o, :]
                V[i] = kc[phys, :, o, :w.dv] if vc is None else vc[phys, :, :, o]
                seen[i] = True
    r0 = int(w.query_start[b])
    for i in range(n):
        K[L - n + i] = T["k_new"][r0 + i]
        V[L - n + i] = T["k_new"][r0 + i][:, :w.dv] if T["v_new"] is None else T["v_new"][r0 + i]
        seen[L - n + i] = True
    assert seen.all()
    return K, V


def check_multi_sdpa():
    """Each new token's output equals its row of full causal attention (PyTorch SDPA,
    fp64) over the contiguous sequence; the other rows get random queries."""
    import torch
    import torch.nn.functional as F

    for w in multi_workloads():
        T = tensors_np(w)
        res = run_multi_step(w, T)
        for b in range(w.n_seqs):
            n = int(w.q_lens[b])
            if n == 0:
                continue
            K, V = contiguous_multi(w, T, b)
            L = K.shape[0]
            r = _rng(300 + b)
            Q = r.standard_normal((L, w.n_q_heads, w.dk))
            r0 = int(w.query_start[b])
            Q[L - n:] = pa.widen(T["q"][r0:r0 + n])
            qt = torch.from_numpy(Q).permute(1, 0, 2)[None]
            kt = torch.from_numpy(pa.widen(K)).permute(1, 0, 2)[None]
            vt = torch.from_numpy(np.ascontiguousarray(pa.widen(V))).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale_f32,
                                                 enable_gqa=True)[0, :, L - n:, :].numpy()
            err = np.max(np.abs(res["o"][r0:r0 + n] - ref.transpose(1, 0, 2)))
            if not err <= 1e-12:
                return f"multi sdpa {w.name} seq {b}: |do|={err:.3g}"
    return None


def check_multi_as_prefixes():
    """New token i of a sequence gets exactly the single-token step's result on the
    sequence cut after it (same cache, same partitions), and one new token per
    sequence is the single-token step itself (slots included)."""
    import workloads as wl
    from oracle import multi_query as mq

    for w in multi_workloads():
        T = tensors_np(w)
        res = run_multi_step(w, T)
        Tp = w.partition_tokens or 16
        pmax = pa.max_partitions(int(w.context_lens.max()), w.n_shards, w.interleave, Tp)
        for b in range(w.n_seqs):
            n, L, r0 = int(w.q_lens[b]), int(w.context_lens[b]), int(w.query_start[b])
            for i in range(n):
                o, lse, _, _ = pa.decode(T["q"][r0 + i:r0 + i + 1], res["k_cache"], res["v_cache"],
                                         w.block_table[b:b + 1], np.array([L - n + i + 1]),
                                         w.n_shards, w.interleave, w.block_size, Tp, pmax,
                                         w.scale_f32, w.dv)
                if not (np.array_equal(o[0], res["o"][r0 + i]) and np.array_equal(lse[0], res["lse"][r0 + i])):
                    return f"multi {w.name} seq {b} token {i}: differs from the cut sequence"
    w1 = wl.small("mq_one", [5, 33, 17], 4, 2, 16, 16, 8, wl.BF16, partition_tokens=8, seed=64,
                  q_lens=[1, 1, 1])
    T = tensors_np(w1)
    res = run_multi_step(w1, T)
    ref = pa.decode_step(T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"],
                         w1.block_table, w1.context_lens, 1, 1, w1.block_size, 8,
                         pa.max_partitions(int(w1.context_lens.max()), 1, 1, 8), w1.scale_f32, w1.dv)
    if not (np.array_equal(res["slots"], ref["slots"]) and np.array_equal(res["o"], ref["o"])
            and np.array_equal(res["lse"], ref["lse"])):
        return "multi with one new token per sequence differs from the single-token step"
    for w in multi_workloads():
        if not np.array_equal(mq.slot_mapping_multi(w.block_table, w.context_lens, w.query_start,
                                                    w.n_shards, w.interleave, w.block_size),
                              w.new_slot):
            return f"multi slots {w.name} differ from the generator's"
    return None


ALL_CHECKS = {
    "bruteforce": check_bruteforce,
    "closed_forms": check_closed_forms,
    "mean_probe": check_mean_probe,
    "shift": check_shift,
    "sdpa": check_sdpa,
    "gather": check_gather,
    "slots": check_slots,
    "merge": check_merge,
    "copy_on_write": check_copy_on_write,
    "fp8_table": check_fp8_table,
    "fp8_rounding": check_fp8_rounding,
    "fp8_decode": check_fp8_decode,
    "multi_sdpa": check_multi_sdpa,
    "multi_as_prefixes": check_multi_as_prefixes,
}
