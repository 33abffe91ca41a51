"""Paged decode attention for AMD MI355X (gfx950): the Python face of libpagedattn.so.

``pa_*`` functions mirror the C ABI in ``include/pa.h`` one to one (see ``_lib``).
``DecodeStep`` strings the calls of one decode step together on one stream: slot
routing with the kv append (one launch), the partitioned attention and the LSE merge.
``MultiDecodeStep`` is the same step with several new tokens per sequence (causal
among them).  ``BlockPool`` is the host-side block accounting (fork, copy-on-write, reuse) whose
copies ``pa_copy_blocks`` carries out on the device.
"""
from ._lib import (  # noqa: F401
    ERR_BLOCK_ID, ERR_CAPACITY, ERR_SLOT, LIB_PATH, PA_BF16, PA_F32, PA_FP8_E4M3, BlockPool,
    PaError, PoolExhausted, lib, pa_choose_partition_tokens, pa_choose_partition_tokens_multi,
    pa_copy_blocks, pa_decode,
    pa_decode_fp8, pa_decode_multi, pa_decode_step, pa_default_partition_tokens, pa_gather_kv, pa_kv_append,
    pa_kv_append_fp8, pa_kv_append_routed, pa_max_partitions, pa_merge_lse, pa_shard_length,
    pa_slot_mapping, pa_slot_mapping_multi,
)
from .step import DecodeStep, MultiDecodeStep  # noqa: F401
