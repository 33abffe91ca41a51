"""Benchmark of one decode step of paged attention on one MI355X.

A step is the whole hot path on one stream: slot routing of the new tokens,
kv append and the partitioned attention (one launch, pa_decode_step: the workgroup
whose partition holds a sequence's new token stores it first), then the LSE merge
(skipped when every sequence is one partition).  Several new tokens per sequence:
routing, append, attention and merge as separate launches.  Inputs are seeded
synthetic tensors already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W]
                  [--config long|dcp1|dcp16|dcp_s1|batch|latent|latent_fp8|latent_spec2|tiny|long_fp8|dcp1_fp8|dcp16_fp8|spec4]
                  [--no-cpu-baseline] [--no-secondary] [--next] [--cpu-budget S]

The default workload is the long-context step (8 sequences, log-normal lengths
around 142K tokens), the configuration the HBM-roofline target is stated for.
The other synthetic workloads (tiny, batch, DCP I=1 and I=16, the same 200K
sequence unsharded, latent) follow under ``secondary``, each with its own rates,
decode roofline and oracle baseline; ``--next`` adds the E4M3 and multi-token
workloads, the same way.
``value`` is KV-read GB/s over the whole step (algorithmic bytes: every stored
K and V element of every sequence read once per step; one byte per element for the
``_fp8`` configurations, whose cache holds E4M3 codes).  ``roofline`` prices the
decode kernel alone (with the append it performs): the same algorithmic bytes over
its average launch time, measured with HIP events on its stream around K launches of
it, back to back, right after the timed region.
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
SETTLE_S = 0.25          # default seconds of untimed back-to-back steps after the warm-up
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16, published


def make_workload(name):
    import workloads as wl

    return {
        "long": lambda: wl.long(),
        "dcp1": lambda: wl.dcp(interleave=1),
        "dcp16": lambda: wl.dcp(interleave=16),
        "dcp_s1": lambda: wl.dcp(interleave=1, n_shards=1),
        "batch": lambda: wl.batch(),
        "latent": lambda: wl.latent(),
        "tiny": lambda: wl.tiny(),
        "long_fp8": lambda: wl.with_fp8_cache(wl.long(partition_tokens=0)),
        "dcp1_fp8": lambda: wl.with_fp8_cache(wl.dcp(interleave=1)),
        "dcp16_fp8": lambda: wl.with_fp8_cache(wl.dcp(interleave=16)),
        "latent_fp8": lambda: wl.with_fp8_cache(wl.latent()),
        "latent_spec2": lambda: wl.latent(q_len=2),
        "spec4": lambda: wl.speculative(q_len=4),
    }[name]()


DESCRIBE = {
    "long": "long-context decode: 8 seqs, L log-normal (median 142K, sigma 0.5, clip [16384, 200000]), "
            "32 q / 8 kv heads, d 128, bf16, block 16, split-KV partitions of 4096 tokens",
    "dcp1": "DCP emulation: 1 seq of 200000 tokens, 64 q / 8 kv heads, d 128, bf16, block 16, "
            "S=4 interleaved shards, I=1, partition size chosen by pa_choose_partition_tokens",
    "dcp16": "DCP emulation: 1 seq of 200000 tokens, 64 q / 8 kv heads, d 128, bf16, block 16, "
             "S=4 interleaved shards, I=16, partition size chosen by pa_choose_partition_tokens",
    "dcp_s1": "DCP reference: the same 200000-token sequence unsharded (S=1), 64 q / 8 kv heads, d 128, "
              "bf16, block 16, partition size chosen by pa_choose_partition_tokens",
    "batch": "continuous-batching step: 64 seqs, L = U[8,32] + U[16,96], 32 q / 8 kv heads, d 128, "
             "bf16, block 16",
    "latent": "latent (MLA-style) cache: 32 seqs, L U[4096, 65536], 128 q heads on 1 kv head, "
              "key 576 / value 512 (view), bf16, block 64, 2048-token prefixes shared by 4",
    "tiny": "1 seq, L 67, 4 q / 1 kv head, d 64, fp32, block 4",
    "long_fp8": "long-context decode with an E4M3 KV cache (per-KV-head scales): 8 seqs, L log-normal "
                "(median 142K, sigma 0.5, clip [16384, 200000]), 32 q / 8 kv heads, d 128, bf16 q, "
                "block 16, partition size chosen by pa_choose_partition_tokens",
    "dcp1_fp8": "DCP emulation with an E4M3 KV cache: 1 seq of 200000 tokens, 64 q / 8 kv heads, "
                "d 128, bf16 q, block 16, S=4 interleaved shards, I=1",
    "dcp16_fp8": "DCP emulation with an E4M3 KV cache: 1 seq of 200000 tokens, 64 q / 8 kv heads, "
                 "d 128, bf16 q, block 16, S=4 interleaved shards, I=16",
    "latent_fp8": "latent (MLA-style) cache in E4M3 (one scale for the single kv head): 32 seqs, "
                  "L U[4096, 65536], 128 q heads, key 576 / value 512 (view), bf16 q, block 64, "
                  "2048-token prefixes shared by 4",
    "latent_spec2": "speculative verification on the latent batch: 32 seqs, L U[4096, 65536], "
                    "2 new tokens per sequence attending causally, 128 q heads on the 576-wide latent "
                    "cache (value 512), bf16, block 64",
    "spec4": "speculative verification on the long-context batch: 8 seqs, L log-normal (median 142K), "
             "4 new tokens per sequence attending causally, 32 q / 8 kv heads, d 128, bf16, block 16, "
             "partition size chosen by pa_choose_partition_tokens",
}


# Source files that make up each decode kernel: a committed counter summary stays valid
# while these are unchanged.
KERNEL_FILES = {"decode_gqa_kernel": ["decode_gqa.hip", "pa_append.h", "pa_common.h", "pa_launch.h"],
                "decode_mla_kernel": ["decode_mla.hip", "pa_append.h", "pa_common.h", "pa_launch.h"],
                "decode_generic_kernel": ["decode_generic.hip", "pa_append.h", "pa_common.h", "pa_launch.h"]}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_paged_kv_amd", "csrc")
    for fn in sorted(KERNEL_FILES[kernel]):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(config, launches_bytes):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken of the current sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    kernel = d.get("kernel")
    if kernel not in KERNEL_FILES or d.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


_SPIN_RATE = []


def spin_cycles(ms):
    """The argument of torch.cuda._sleep that spins the GPU for about ``ms``
    milliseconds (its rate measured once per process)."""
    import torch

    if not _SPIN_RATE:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_RATE.append(1_000_000 / max(a.elapsed_time(b), 1e-3))   # argument units per ms
    return int(ms * _SPIN_RATE[0])


def time_gpu(w, T, step, steps, warmup, settle_s=SETTLE_S):
    import torch

    ks, vs = T.get("k_scale"), T.get("v_scale")
    nb = T["k_cache"].shape[0]
    if w.multi:
        qs = T["query_start"]
        args = (T["q"], qs, T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
                T["context_lens"], ks, vs)
        def prepare():   # routing, then the append
            step.route(T["block_table"], T["context_lens"], qs, nb)
            step.append(T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], ks, vs)
        attend = lambda: step.attend(T["q"], qs, T["k_cache"], T["v_cache"], T["block_table"],
                                     T["context_lens"], ks, vs)
    else:
        args = (T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
                T["context_lens"], ks, vs)
        def prepare():   # routing and append happen inside the decode launch (pa_decode_step)
            pass
        attend = lambda: step.append_attend(*args)
    for _ in range(warmup):
        step(*args)
    torch.cuda.synchronize()
    # Then more untimed steps until settle_s of back-to-back work has passed: the
    # compute-heavier kernels (E4M3 cache, latent cache) run ~10 % slower for the first
    # ~50 ms while the clocks come up.
    settle, s0 = 0, time.perf_counter()
    while time.perf_counter() - s0 < settle_s:
        for _ in range(10):
            step(*args)
        settle += 10
        torch.cuda.synchronize()
    # The timed region holds exactly the K steps.  The decode launch's own duration comes
    # from launches after it (below): an event record costs the host ~4.5 us, which inside
    # the timed loop would make the host, not the GPU, set the pace of short steps.
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        prepare()
        attend()
        step.merge()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    # Short steps (the host's enqueue time, ~20 us a step with the events, then exceeds the
    # GPU's): a bounded spin of ~50 us per step is queued first, so that the host has
    # enqueued these steps before the GPU reaches them and each event interval holds the
    # decode launch, not the host's time to enqueue it.  Long steps keep the GPU ahead of
    # the host by themselves (and a spin would let the clocks of power-limited kernels
    # drop before the measured launches).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if total_ms / steps < 0.1:
        torch.cuda._sleep(spin_cycles(50e-3 * steps))
    for i in range(steps):
        prepare()
        ev[i][0].record()
        attend()
        ev[i][1].record()
        step.merge()
    torch.cuda.synchronize()
    dec = sorted(a.elapsed_time(b) for a, b in ev)
    # The decode launch's average duration (what the roofline prices): K more decode
    # launches alone, back to back, between one event pair on the launch stream, behind
    # the same spin when launches are short.  The pairs above give the spread from launch
    # to launch, but each pair's markers add a few microseconds to a short launch.
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if total_ms / steps < 0.1:
        torch.cuda._sleep(spin_cycles(50e-3 * steps))
    b0.record()
    for i in range(steps):
        attend()
    b1.record()
    torch.cuda.synchronize()
    res = dict(total_ms=total_ms, wall_s=wall, decode_ms_mean=b0.elapsed_time(b1) / steps,
               decode_ms_pairs_mean=sum(dec) / len(dec), decode_ms_median=dec[len(dec) // 2],
               decode_ms_min=dec[0], settle_steps=settle)
    # After the timed region: the same step recorded once as a HIP graph and replayed
    # K times (reported separately; it removes the host's per-launch cost).
    graph = step.capture(*args)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    res["graph_ms_per_step"] = g0.elapsed_time(g1) / steps
    del graph
    # Cold: before each step a 2 GiB buffer is read (untimed), which evicts the 256 MB
    # Infinity Cache and the L2s, so the step's inputs come from HBM even when the whole
    # workload would fit in the caches.  A read, not a write: a written buffer leaves
    # dirty lines whose write-back would be charged to the step.
    flush = torch.ones(1 << 29, dtype=torch.float32, device=T["q"].device)
    sink = torch.zeros(1, dtype=torch.float32, device=T["q"].device)
    cold_step, cold_dec = [], []
    resident = int(w.context_lens.astype("int64").sum()) * w.kv_bytes_per_token() < (256 << 20)
    n_cold = max(steps, 50) if resident else steps      # small steps: more samples
    for i in range(n_cold):
        sink.add_(flush.sum())
        a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        a.record()
        prepare()
        b.record()
        attend()
        c.record()
        step.merge()
        d.record()
        cold_step.append((a, d))
        cold_dec.append((b, c))
    torch.cuda.synchronize()
    cs = sorted(x.elapsed_time(y) for x, y in cold_step)
    cd = sorted(x.elapsed_time(y) for x, y in cold_dec)
    res.update(cold_ms_per_step_median=cs[len(cs) // 2], cold_decode_ms_median=cd[len(cd) // 2],
               cold_decode_ms_min=cd[0], cold_iterations=n_cold)
    del flush, sink
    return res


def mfma_roofline(r):
    """The latent decode against the dense bf16 matrix-core peak: the attention's products
    counted once (``mfma_frac``), and the MFMA work the kernel issues for them
    (``mfma_frac_executed``: the value product twice, for the weights' bf16 pair)."""
    return {"mfma_tflops": round(r["tflops"], 2), "mfma_frac": round(r["tflops"] / MFMA_BF16_TFLOPS, 4),
            "mfma_tflops_executed": round(r["tflops_executed"], 2),
            "mfma_frac_executed": round(r["tflops_executed"] / MFMA_BF16_TFLOPS, 4)}


def timing_fields(t):
    """The per-iteration spread of the hot (cache-warm, back-to-back) decode launch, each
    between its own event pair (mean, median, min), and the cold (caches flushed before
    each step) step and decode launch, in ms."""
    keys = ("decode_ms_pairs_mean", "decode_ms_median", "decode_ms_min", "cold_ms_per_step_median",
            "cold_decode_ms_median", "cold_decode_ms_min")
    out = {k: round(t[k], 5) for k in keys}
    out["settle_steps"] = t["settle_steps"]
    out["cold_iterations"] = t["cold_iterations"]
    return out


def cpu_baseline(w, T, budget_s=12.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: whole
    sequences, in order, until ``budget_s`` of CPU time is spent, with as many BLAS
    threads as the process may use (its CPU affinity).  When the whole workload fits in a
    third of the budget it is timed three times (median reported) and once more on one
    thread."""
    import numpy as np
    import torch

    from oracle import fp8_kv as f8
    from oracle import paged_attention as pa

    def host(x):
        if x is None:
            return None
        x = x.detach().cpu().contiguous()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
    except Exception:             # without it the BLAS default stands
        threadpool_limits = None

    # each sequence's inputs, copied to the host outside the timed calls
    jobs = []
    for b in range(w.n_seqs):
        ids = np.unique(w.block_table[b][w.block_table[b] >= 0])
        remap = np.full(w.n_blocks, -1, np.int64)
        remap[ids] = np.arange(ids.size)
        bt = np.where(w.block_table[b:b + 1] >= 0, remap[np.maximum(w.block_table[b:b + 1], 0)], -1).astype(np.int32)
        idx = torch.from_numpy(ids).to(T["k_cache"].device)
        rows = slice(int(w.query_start[b]), int(w.query_start[b + 1]))
        jobs.append(dict(bt=bt, kc=host(T["k_cache"].index_select(0, idx)),
                         vc=None if T["v_cache"] is None else host(T["v_cache"].index_select(0, idx)),
                         q=host(T["q"][rows]), kn=host(T["k_new"][rows]),
                         vn=None if T["v_new"] is None else host(T["v_new"][rows]),
                         qs=np.array([0, rows.stop - rows.start], np.int32)))
        if sum(int(x) for x in w.context_lens[:b + 1]) > 3_000_000:   # more than the budget allows
            break
    Tp = w.partition_tokens or 4096

    def step(b):
        j = jobs[b]
        L = w.context_lens[b:b + 1]
        pmax = max(pa.max_partitions(int(L[0]), w.n_shards, w.interleave, Tp), 1)
        if w.multi:
            from oracle import multi_query as mq

            mq.decode_step_multi(j["q"], j["qs"], j["kn"], j["vn"], j["kc"], j["vc"], j["bt"], L,
                                 w.n_shards, w.interleave, w.block_size, Tp, pmax, w.scale_f32, w.dv)
        elif w.cache_dtype == "fp8":
            f8.decode_step(j["q"], j["kn"], j["vn"], j["kc"], j["vc"], host(T["k_scale"]),
                           host(T.get("v_scale")), j["bt"], L, w.n_shards, w.interleave,
                           w.block_size, Tp, pmax, w.scale_f32, w.dv)
        else:
            pa.decode_step(j["q"], j["kn"], j["vn"], j["kc"], j["vc"], j["bt"], L, w.n_shards,
                           w.interleave, w.block_size, Tp, pmax, w.scale_f32, w.dv)

    def one_pass(threads):
        done, elapsed, seqs = 0, 0.0, []
        limit = threadpool_limits(limits=threads) if threadpool_limits else contextlib.nullcontext()
        with limit:
            for b in range(len(jobs)):
                t = time.perf_counter()
                step(b)
                elapsed += time.perf_counter() - t
                done += int(w.context_lens[b])
                seqs.append(b)
                if elapsed >= budget_s:
                    break
        return done, elapsed, seqs

    done, elapsed, seqs = one_pass(cores)
    res = {"unit": "GB/s", "cores": int(cores), "kind": "oracle"}
    note = ""
    if len(seqs) == w.n_seqs and elapsed < budget_s / 6:
        # The whole workload is quick: each measurement repeats it for about a second,
        # the median of three measurements is reported, and one more runs on one thread.
        reps = max(1, int(1.0 / max(elapsed, 1e-4)))

        def per_pass(threads):
            return sum(one_pass(threads)[1] for _ in range(reps)) / reps

        elapsed = sorted(per_pass(cores) for _ in range(3))[1]
        res["value_1_thread"] = round(done * w.kv_bytes_per_token() / per_pass(1) / 1e9, 4)
        note = (f"; the whole step repeated {reps}x per measurement, median of 3 measurements; "
                f"value_1_thread: the same on one thread")
    res["value"] = round(done * w.kv_bytes_per_token() / elapsed / 1e9, 4)
    res["seq_steps_per_s"] = round(len(seqs) / elapsed, 4)
    res["s_per_pass"] = round(elapsed, 6)
    res["sample"] = (f"sequences {seqs[0]}..{seqs[-1]} of {w.n_seqs} of the same workload ({done} context "
                     f"tokens, full decode step in the fp64 NumPy oracle), {elapsed:.3f} s per pass on "
                     f"{cores} threads (the process's CPU affinity){note}")
    return res


# Workloads timed after the headline by default, and those ``--next`` adds.
SECONDARY = ("tiny", "batch", "dcp1", "dcp16", "dcp_s1", "latent")
NEXT = ("long_fp8", "dcp1_fp8", "dcp16_fp8", "latent_fp8", "latent_spec2", "spec4")


def run_config(name, steps, warmup, with_cpu, partition_tokens=0, settle_s=SETTLE_S, cpu_budget=12.0):
    import numpy as np
    import torch

    import decode_attention_paged_kv_amd as P
    import workloads as wl

    w = make_workload(name)
    if partition_tokens:
        w.partition_tokens = partition_tokens
    dev = torch.device("cuda", 0)
    T = wl.make_tensors(w, dev)
    if w.multi:
        step = P.MultiDecodeStep(w.n_seqs, w.n_rows, int(w.q_lens.max()), w.n_q_heads, w.n_kv_heads,
                                 w.dk, w.dv, w.block_size, int(w.context_lens.max()), w.n_shards,
                                 w.interleave, w.partition_tokens, w.scale_f32, device=dev,
                                 context_lens_host=w.context_lens, kv_dtype=T["k_cache"].dtype,
                                 latent=w.latent)
    else:
        step = P.DecodeStep(w.n_seqs, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size,
                            int(w.context_lens.max()), w.n_shards, w.interleave,
                            w.partition_tokens, w.scale_f32, device=dev,
                            context_lens_host=w.context_lens, kv_dtype=T["k_cache"].dtype,
                            latent=w.latent)
    if not w.partition_tokens:
        w.partition_tokens = step.partition_tokens
    cpu = cpu_baseline(w, T, cpu_budget) if with_cpu else None
    t = time_gpu(w, T, step, steps, warmup, settle_s)
    assert int(step.err_flag.item()) == 0, "device error flag set"
    assert torch.isfinite(step.out).all(), "non-finite output"
    kv_bytes = int(np.sum(w.context_lens.astype(np.int64))) * w.kv_bytes_per_token()
    ms = t["total_ms"] / steps
    dec_ms = t["decode_ms_mean"]
    achieved = kv_bytes / (dec_ms * 1e-3) / 1e9
    tokens = int(np.sum(w.context_lens.astype(np.int64)))
    new_tokens = w.n_rows
    res = dict(w=w, step=step, kv_bytes=kv_bytes, ms_per_step=ms, decode_ms=dec_ms,
               tokens_per_s_decode=tokens / (dec_ms * 1e-3),
               new_tokens_per_s=new_tokens / (ms * 1e-3),
               value=kv_bytes / (ms * 1e-3) / 1e9, seq_steps=w.n_seqs / (ms * 1e-3),
               achieved=achieved, timing=t, cpu=cpu)
    if w.latent:
        # the attention's own products (scores and weighted values, each counted once),
        # and the matrix-core work the kernel issues for them: the weights enter the value
        # product as a bf16 pair, two MFMAs per value operand
        flops = int(np.sum(w.context_lens.astype(np.int64))) * w.n_q_heads * 2 * (w.dk + w.dv)
        executed = int(np.sum(w.context_lens.astype(np.int64))) * w.n_q_heads * 2 * (w.dk + 2 * w.dv)
        res["tflops"] = flops / (dec_ms * 1e-3) / 1e12
        res["tflops_executed"] = executed / (dec_ms * 1e-3) / 1e12
    return res


def calibrate_copy(steps, nbytes=2 << 30):
    """A plain copy kernel of known size: reads and writes ``nbytes`` per launch.
    Its rocprofv3 FETCH_SIZE / WRITE_SIZE against ``nbytes`` give the counters'
    scale for the HBM traffic of the decode kernel."""
    import torch

    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return {"kernel": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
            "ms": round(ms, 5), "GBs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long", choices=sorted(DESCRIBE))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of further untimed steps after the warm-up, for the clocks to settle")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the --config workload (no 'secondary' block)")
    ap.add_argument("--next", action="store_true",
                    help="also time the E4M3 and multi-token workloads under 'secondary'")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time per workload for cpu_baseline (secondary: half)")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="override the workload's partition size (tokens)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 2 GiB device-to-device copy (reference for HBM counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU (DCP shards are emulated as "
              "partitions on a single device); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if a.calibrate_copy:
        print(json.dumps(calibrate_copy(a.steps)), flush=True)
        return
    r = run_config(a.config, a.steps, a.warmup, not a.no_cpu_baseline, a.partition_tokens, a.settle,
                   a.cpu_budget)
    w = r["w"]
    traffic = measured_traffic(a.config, r["kv_bytes"])
    line = {
        "metric": "paged decode-attention KV-read GB/s and % of MI355X HBM peak; seq-steps/s",
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle_s": a.settle,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q in a shuffled block pool)",
        "config": {"workload": DESCRIBE[a.config], "name": a.config, "n_seqs": w.n_seqs,
                   "context_tokens": int(w.context_lens.sum()), "max_context": int(w.context_lens.max()),
                   "partition_tokens": r["step"].partition_tokens,
                   "kv_cache": "e4m3 codes + float32 per-head scales" if w.cache_dtype == "fp8" else w.dtype,
                   "kv_bytes_per_step": r["kv_bytes"],
                   # pool slots read at least once (a shared prefix block counts once)
                   "kv_bytes_per_step_unique": int((w.token_id >= 0).sum()) * w.kv_bytes_per_token()},
        "hbm_frac": round(r["value"] / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(r["seq_steps"], 2),
        "decode_ms": round(r["decode_ms"], 5),
        "kv_tokens_per_s_decode": round(r["tokens_per_s_decode"], 1),
        "new_tokens_per_s": round(r["new_tokens_per_s"], 1),
        "graph_ms_per_step": round(r["timing"]["graph_ms_per_step"], 5),
        "timing": timing_fields(r["timing"]),
        "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "pa_decode",
                     "algorithmic_bytes_per_launch": r["kv_bytes"]},
        "cpu_baseline": r["cpu"],
    }
    if "tflops" in r:
        line["roofline"].update(mfma_roofline(r))
    if not a.no_secondary:
        import torch

        del r
        torch.cuda.empty_cache()
        sec = {}
        names = SECONDARY + (NEXT if a.next else ())
        for name in names:
            if name == a.config:
                continue
            with_cpu = not a.no_cpu_baseline
            s = run_config(name, a.steps, a.warmup, with_cpu, settle_s=a.settle, cpu_budget=a.cpu_budget / 2)
            sw = s["w"]
            sec[name] = {
                "workload": DESCRIBE[name],
                "kv_GBs_step": round(s["value"], 2),
                "seq_steps_per_s": round(s["seq_steps"], 2),
                "ms_per_step": round(s["ms_per_step"], 5),
                "decode_ms": round(s["decode_ms"], 5),
                "kv_tokens_per_s_decode": round(s["tokens_per_s_decode"], 1),
                "new_tokens_per_s": round(s["new_tokens_per_s"], 1),
                "graph_ms_per_step": round(s["timing"]["graph_ms_per_step"], 5),
                "partition_tokens": s["step"].partition_tokens,
                "kv_bytes_per_step": s["kv_bytes"],
                "dtype": "f32" if sw.dtype == "f32" else "bf16",
                "timing": timing_fields(s["timing"]),
                "roofline": {"bound": "hbm", "achieved": round(s["achieved"], 2), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(s["achieved"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic(name, s["kv_bytes"]), "kernel": "pa_decode",
                             "algorithmic_bytes_per_launch": s["kv_bytes"]},
                "cpu_baseline": s["cpu"],
            }
            if "tflops" in s:
                sec[name]["roofline"].update(mfma_roofline(s))
            del s
            torch.cuda.empty_cache()
            print(f"bench.py: {name} done", file=sys.stderr, flush=True)
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
