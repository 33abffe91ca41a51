"""A decode step recorded as a HIP graph and replayed: every replay, with the
program's own eager work and synchronisations in between, must give exactly the
eager step's results on the inputs it finds (the kernels are deterministic, so the
comparison is bit for bit), and the eager step itself is checked against the oracle
(``check_small``)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_harness import check_small, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_paged_kv_amd  # noqa: F401  (fails loudly if the library is missing)


def _step_for(P, w, T):
    kw = dict(device=T["q"].device, context_lens_host=w.context_lens, kv_dtype=T["k_cache"].dtype,
              latent=w.latent)
    if w.multi:
        return P.MultiDecodeStep(w.n_seqs, w.n_rows, int(w.q_lens.max()), w.n_q_heads, w.n_kv_heads,
                                 w.dk, w.dv, w.block_size, int(w.context_lens.max()), w.n_shards,
                                 w.interleave, w.partition_tokens, w.scale_f32, **kw)
    return P.DecodeStep(w.n_seqs, w.n_q_heads, w.n_kv_heads, w.dk, w.dv, w.block_size,
                        int(w.context_lens.max()), w.n_shards, w.interleave, w.partition_tokens,
                        w.scale_f32, **kw)


def _args(w, T):
    base = (T["q"], T["k_new"], T["v_new"], T["k_cache"], T["v_cache"], T["block_table"],
            T["context_lens"], T.get("k_scale"), T.get("v_scale"))
    if w.multi:
        return (T["q"], T["query_start"]) + base[1:]
    return base


@pytest.mark.parametrize("name", ["batch", "fp8_dcp", "multi"])
def test_graph_replays_match_eager(name):
    import decode_attention_paged_kv_amd as P

    if name == "batch":
        w = wl.batch()
    elif name == "fp8_dcp":
        w = wl.small("g_fp8", [900, 31], 64, 8, 128, 128, 16, wl.BF16, n_shards=4, interleave=16,
                     partition_tokens=64, seed=3, kv_dtype=wl.FP8)
    else:
        w = wl.small("g_multi", [300, 70], 32, 8, 128, 128, 16, wl.BF16, partition_tokens=64, seed=4,
                     q_lens=[4, 2])
    say(f"[graph] {w.name}")
    check_small(w)                                    # the eager path against the oracle
    dev = torch.device("cuda")
    T = wl.make_tensors(w, dev)
    step = _step_for(P, w, T)
    ref = _step_for(P, w, T)
    graph = step.capture(*_args(w, T))
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for it in range(4):
        # eager work between replays: new queries and new token rows in place
        T["q"].copy_(torch.randn(T["q"].shape, generator=g, device=dev).to(T["q"].dtype))
        T["k_new"].copy_(torch.randn(T["k_new"].shape, generator=g, device=dev).to(T["k_new"].dtype))
        if T["v_new"] is not None:
            T["v_new"].copy_(torch.randn(T["v_new"].shape, generator=g, device=dev).to(T["v_new"].dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_lse = step.out.clone(), step.lse.clone()
        ref(*_args(w, T))
        torch.cuda.synchronize()
        assert int(step.err_flag.item()) == 0 and int(ref.err_flag.item()) == 0
        assert torch.equal(got_out, ref.out), f"replay {it}: output differs from the eager step"
        assert torch.equal(got_lse, ref.lse), f"replay {it}: lse differs from the eager step"
        assert torch.isfinite(got_out).all()
