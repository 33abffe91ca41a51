"""fp64 CPU oracle for one decode step of attention over a block-table-paged KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never routes through it, and this package imports
nothing from the HIP library or its Python binding.

Sources (web pages; every function cites the page and section it follows):

* [DCP]  soroban.highreso.jp/article/techblog-engineer-choubunllm -- "Why long-context
  LLMs get slow: distributing the KV cache with Decode Context Parallelism".
  Sections used: the decode-bottleneck section (KV bytes per token, decode is a
  read of every past K/V), the DCP mechanism section (interleaved placement of
  tokens on ranks; the three-stage DCP decode step whose last stage reweights the
  partial outputs with the LSE values of online softmax), the DCP configuration
  section (the decode backend must return the LSE).
* [KVB]  qiita.com/systemdesignsimple/items/76d9c4d7ac4a80e2deff -- "KV cache and
  continuous batching".  Sections "What does the KV cache hold?" (a decode step
  appends the new token's key and value, then attends over everything stored),
  "Why does writing one token at a time duplicate work?" (the query is compared
  with all earlier keys and the values are weighted by the result; cached rows
  never change), and "How KV-cache memory limits concurrency" (bytes per token).
* [AGX]  agentlenshq.com/ja/blogs/5a6c5ce5-d812-4d7e-b52c-cb4a97581aac -- "vLLM AgentX
  release".  Sections used: execution plane (long prompts split by a per-step token
  threshold) and open-source kernel contributions (a speculative-verification path).
* [PA]   ai-compass.weeybrid.co.jp/algorizm/paged-attention/ -- "What is
  PagedAttention?".  Sections "A block table separates logical order from
  physical placement", "Reusing blocks freed when a request ends" (worked
  example with 4-token blocks) and "Sharing common blocks and copy-on-write".

Modules:
* ``paged_attention`` -- placement of tokens into shards and blocks, kv append,
  gather, softmax attention with LSE, partition partials and the LSE merge.
* ``block_manager``   -- fixed-size block accounting: free list, reuse,
  reference counts, copy-on-write.
* ``fp8_kv``          -- a cache stored as FP8 E4M3 codes with float32 scales per
  tensor or per KV head: quantise on append, dequantise on read (the pages name FP8
  storage of the cache; the format, scaling and rounding are readings stated there).
* ``multi_query``     -- a step with several new tokens per sequence, each attending
  causally (over everything before it and itself): slots, partials and merge.

Parity status of each function is stated in its docstring; every function here
is pinned by a CPU test in ``tests/test_oracle_*.py`` (none is "parity unpinned").
"""
from . import paged_attention, block_manager, fp8_kv, multi_query  # noqa: F401
