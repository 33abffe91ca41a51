/*
 * pa.h -- C ABI of one decode step of attention over a block-table-paged KV cache,
 * for AMD Instinct MI355X (gfx950).  Library: libpagedattn.so.
 *
 * Pages the operations follow (cited per entry point below):
 *  [KVB] qiita.com/systemdesignsimple/items/76d9c4d7ac4a80e2deff, "KV cache and
 *        continuous batching": a decode step stores the new token's key/value and
 *        then attends over every stored token (section "What does the KV cache
 *        hold?"); bytes per token (section "How KV-cache memory limits concurrency").
 *  [PA]  ai-compass.weeybrid.co.jp/algorizm/paged-attention/, "What is
 *        PagedAttention?": fixed-size blocks, a per-request block table from logical
 *        to physical blocks, attention reads KV through the table (section "A block
 *        table separates logical order from physical placement").
 *  [DCP] soroban.highreso.jp/article/techblog-engineer-choubunllm, "Why long-context
 *        LLMs get slow: distributing the KV cache with Decode Context Parallelism":
 *        tokens dealt to S shards `interleave` at a time; each shard attends over its
 *        own tokens and returns an output plus its softmax LSE; the partial outputs
 *        are reweighted with the LSEs and summed (DCP mechanism section); the decode
 *        backend must return the LSE (DCP configuration section).
 *  [AGX] agentlenshq.com/ja/blogs/5a6c5ce5-d812-4d7e-b52c-cb4a97581aac, "vLLM AgentX
 *        release": long prompts split by a per-step token threshold (execution-plane
 *        section) and a speculative-verification kernel path (open-source kernel
 *        contributions section), both steps with several new tokens per sequence.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless stated.
 *    The library allocates no device memory and keeps no pointer after returning.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream) and runs asynchronously; no call synchronises.
 *  - Return value: PA_OK (0) or a negative pa_status.  On an error detected on the
 *    host (null pointer, bad shape, unsupported combination, buffer too small)
 *    NOTHING is launched; pa_last_error() returns a message (per calling thread).
 *  - Data-dependent errors (a block id outside [0, n_blocks), a context longer than
 *    the block table holds, a slot outside the pool) are detected on the device:
 *    the offending token or block is skipped and, if `err_flag` is non-NULL, a
 *    nonzero value is stored in *err_flag (never cleared by the library).
 *  - Element types: PA_F32 (IEEE binary32) or PA_BF16 (bfloat16).  q, K and V of one
 *    call share one type, except for an E4M3 cache (pa_kv_append_fp8, pa_decode_fp8).
 *    Partial outputs and LSEs are always float32.
 *
 * Layout of the paged cache (one layer)
 * -------------------------------------
 *  k_cache  [n_blocks][n_kv_heads][block_size][dk]   a token's key row is contiguous
 *  v_cache  [n_blocks][n_kv_heads][dv][block_size]   token index fastest
 *  Latent (MLA-style) cache: v_cache == NULL; the value of a token is the first dv
 *  entries of its key row (dv <= dk), read from k_cache.
 *  slot = physical_block * block_size + offset_in_block.
 *
 * Sharding (DCP emulated on one GPU)
 * ----------------------------------
 *  Global token i (0-based) of a sequence lives on shard (i / interleave) % n_shards;
 *  each shard keeps its tokens in global order, so token i has local index
 *  (i / (interleave*n_shards))*interleave + i % interleave, and shard r of a length-L
 *  sequence holds  L_r = c*interleave + clamp(L - c*interleave*n_shards - r*interleave,
 *  0, interleave)  tokens with c = L / (interleave*n_shards).
 *  block_table  int32 [n_seqs][n_shards][max_blocks_per_shard]: row [b][r] lists the
 *  physical blocks of shard r of sequence b in logical order (entry j holds local
 *  tokens j*block_size .. j*block_size+block_size-1).  Unused entries are ignored.
 *  n_shards = 1 is the ordinary unsharded cache.
 *
 * context_lens  int32 [n_seqs]: tokens of each sequence INCLUDING the token this
 *  step appends, which sits at global position context_lens[b]-1.  0 = no tokens.
 */
#ifndef PAGEDATTN_PA_H
#define PAGEDATTN_PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL                          */
  PA_ERR_SHAPE = -2,        /* a size is out of range or sizes are inconsistent   */
  PA_ERR_UNSUPPORTED = -3,  /* valid but not implemented (dtype, head size, ...)  */
  PA_ERR_BUFFER = -4,       /* a caller buffer is too small for the request       */
  PA_ERR_HIP = -5,          /* the HIP runtime reported an error on launch        */
  PA_ERR_EXHAUSTED = -6,    /* a block pool has too few free blocks; nothing changed */
  PA_ERR_SEQUENCE = -7      /* a block pool does not know the sequence id, or the id
                               of a new sequence is already in use                  */
} pa_status;

/* PA_FP8_E4M3: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN; no infinities;
 * largest magnitude 448).  A cache element type only (see pa_kv_append_fp8). */
typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Largest supported sizes. */
#define PA_MAX_HEAD_DIM 576
#define PA_MAX_BLOCK_SIZE 256

/*
 * pa_slot_mapping -- cache slot of each sequence's new token ([DCP]: a token made
 * during decode is placed by the same interleave rule; [PA]: the current block is
 * filled while it has room, so the token goes to local offset (local index mod
 * block_size) of the block the table lists for it).
 *   block_table, context_lens : as above.
 *   slot_mapping (out)        : int64 [n_seqs]; slot of token context_lens[b]-1, or
 *                               -1 when context_lens[b] <= 0 or its block id is invalid
 *                               (then *err_flag is set).
 */
int pa_slot_mapping(const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                    int32_t n_shards, int32_t interleave, int32_t block_size,
                    int32_t max_blocks_per_shard, int64_t n_blocks, int64_t* slot_mapping,
                    int32_t* err_flag, void* stream);

/*
 * pa_kv_append -- store each new token's key and value into its slot, bit for bit
 * ([KVB], "What does the KV cache hold?").
 *   k_new  [n_tokens][n_kv_heads][dk];  v_new [n_tokens][n_kv_heads][dv] (NULL for the
 *   latent cache, where v_cache must be NULL too).
 *   slot_mapping int64 [n_tokens]: slot < 0 is padding and is skipped; a slot at or
 *   beyond n_blocks*block_size is skipped and sets *err_flag.  Two tokens with the
 *   same slot: the stored row is one of them, unspecified which.
 */
int pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int64_t* slot_mapping, int32_t n_tokens, int32_t n_kv_heads, int32_t dk,
                 int32_t dv, int32_t block_size, int64_t n_blocks, int32_t dtype,
                 int32_t* err_flag, void* stream);

/*
 * pa_kv_append_fp8 -- pa_kv_append for a cache stored as E4M3 codes (one byte per
 * element).  The KV cache may be kept in an 8-bit floating type so that a token takes
 * fewer bytes ([DCP], the passage that sets DCP beside KV-cache quantisation; element
 * size as a factor of bytes per token: [KVB], "How KV-cache memory limits
 * concurrency").  Element e of a new key row of KV head h is stored as the code of
 * k_new[e] / k_scale[h] (k_scale[0] when n_scales == 1): the quotient is formed in
 * float32 (IEEE division) and rounded to the nearest E4M3 value, ties to the even code;
 * magnitudes of 448 and above (and infinities) become +-448, NaN the NaN code.  Values
 * likewise with v_scale.  A stored code c reads back as value(c) * scale.
 *   k_new, v_new: [n_tokens][n_kv_heads][dk|dv] of new_dtype (PA_F32 or PA_BF16).
 *   k_cache, v_cache: uint8 codes in the layout of the paged cache.
 *   k_scale, v_scale: DEVICE float32 [n_scales], n_scales = 1 (per tensor) or
 *   n_kv_heads (per KV head); positive and finite (not checked).  v_scale and v_cache
 *   are NULL for the latent cache.  Slots as in pa_kv_append.
 */
int pa_kv_append_fp8(const void* k_new, const void* v_new, int32_t new_dtype, uint8_t* k_cache,
                     uint8_t* v_cache, const float* k_scale, const float* v_scale,
                     int32_t n_scales, const int64_t* slot_mapping, int32_t n_tokens,
                     int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
                     int64_t n_blocks, int32_t* err_flag, void* stream);

/*
 * pa_kv_append_routed -- pa_slot_mapping and then the append (pa_kv_append, or
 * pa_kv_append_fp8 for an E4M3 cache) in one launch, for a step with one new token per
 * sequence: sequence b's new token (global position context_lens[b]-1) is routed to its
 * shard, local index and block by the same rule, and its rows are stored exactly as the
 * two calls would store them.  Saves a launch per decode step.
 *   k_new, v_new: [n_seqs][n_kv_heads][dk|dv] of new_dtype (PA_F32 or PA_BF16); v_new
 *   and v_cache NULL for the latent cache.
 *   k_cache, v_cache: the paged cache of cache_dtype: PA_F32 or PA_BF16 (then equal to
 *   new_dtype) or PA_FP8_E4M3 (then k_scale, v_scale, n_scales as in pa_kv_append_fp8;
 *   otherwise they are ignored and may be NULL).
 *   block_table, context_lens, n_shards, interleave, max_blocks_per_shard: as in
 *   pa_slot_mapping.
 *   slot_mapping (out, optional): int64 [n_seqs], the slots pa_slot_mapping would write;
 *   NULL to skip.  An empty sequence or an invalid table entry appends nothing (the
 *   latter sets *err_flag).
 */
int pa_kv_append_routed(const void* k_new, const void* v_new, int32_t new_dtype, void* k_cache,
                        void* v_cache, int32_t cache_dtype, const float* k_scale,
                        const float* v_scale, int32_t n_scales, const int32_t* block_table,
                        const int32_t* context_lens, int32_t n_seqs, int32_t n_kv_heads, int32_t dk,
                        int32_t dv, int32_t block_size, int64_t n_blocks,
                        int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
                        int64_t* slot_mapping, int32_t* err_flag, void* stream);

/*
 * pa_decode -- attention of one query token per sequence over its paged K/V, split
 * into shards and partitions, each emitting an output and its LSE ([PA]: attention
 * follows the block table; [DCP]: local attention per shard returning output + LSE).
 *   q          [n_seqs][n_q_heads][dk]; query head h reads KV head h / (n_q_heads/n_kv_heads).
 *   partition_tokens T (> 0, a multiple of block_size): shard r of sequence b is cut
 *              into partitions of T consecutive LOCAL tokens; partition p covers local
 *              tokens [p*T, min((p+1)*T, L_r)).
 *   max_partitions Pmax: partition slots per shard in the outputs; must be at least
 *              pa_max_partitions(max context, n_shards, interleave, T) for the lengths
 *              passed (a longer context sets *err_flag and its excess is dropped).
 *   scale      multiplies q.k before the softmax.
 *   part_out   float32 [n_seqs][n_shards][Pmax][n_q_heads][dv]: softmax-weighted mean
 *              of the partition's values.  Rows of an empty partition are NOT written
 *              (their weight in any merge is zero; pa_merge_lse never reads them),
 *              except in partition 0 of a shard with no tokens, where they are 0 --
 *              so with one shard and Pmax = 1 the partials already are what
 *              pa_merge_lse would return (a single part has weight exactly 1).
 *   part_lse   float32 [n_seqs][n_shards][Pmax][n_q_heads]: natural log of the sum of
 *              exp(scale*q.k) over the partition; -inf for an empty partition.
 *   Unsupported: dk or dv outside [1, PA_MAX_HEAD_DIM], dv > 512, block_size outside
 *   [1, PA_MAX_BLOCK_SIZE], n_q_heads not a multiple of n_kv_heads.
 */
int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
              int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
              int64_t n_blocks, int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
              int32_t partition_tokens, int32_t max_partitions, float scale, int32_t dtype,
              float* part_out, float* part_lse, int32_t* err_flag, void* stream);

/*
 * pa_decode_step -- a decode step's append and attention in one call: the effect of
 * pa_kv_append_routed (one new token per sequence, the last of its context_lens[b]
 * tokens) followed by pa_decode / pa_decode_fp8 on the same stream, with the same
 * results -- the cache then holds the new rows bit for bit (E4M3: the same codes), and
 * the outputs are those of the decode over the appended cache.  A decode step stores
 * the new token's rows, then attends over everything stored ([KVB] "KV キャッシュは何を
 * 保持するのか?"); here the workgroup whose partition holds a sequence's new token stores
 * its rows before reading them, so the step is one launch.  When one partition of a KV
 * head is read by several workgroups (more than 16 query heads per KV head outside the
 * latent kernel, more than 128 on it) the append is a launch of its own first.
 *   k_new, v_new  [n_seqs][n_kv_heads][dk | dv] of new_dtype: the cache's element type,
 *              or PA_F32 / PA_BF16 rows quantised into an E4M3 cache; v_new NULL exactly
 *              when v_cache is (latent cache).
 *   k_cache, v_cache  the cache of cache_dtype, written (the new tokens' slots) and read.
 *   k_scale, v_scale, n_scales  as in pa_decode_fp8 when cache_dtype is PA_FP8_E4M3,
 *              otherwise ignored (may be NULL / 0).
 *   q_dtype    element type of q; equal to cache_dtype and new_dtype unless the cache is
 *              PA_FP8_E4M3.
 *   slot_mapping (out, optional)  int64 [n_seqs]: as in pa_kv_append_routed.
 *   The block receiving a new token must be private to its sequence (copy-on-write keeps
 *   a block that is written private), since other sequences' workgroups run meanwhile.
 *   Other arguments and the outputs: as in pa_decode.  Errors: as pa_kv_append_routed and
 *   pa_decode report them; nothing is launched on a rejected call.
 */
int pa_decode_step(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                   void* k_cache, void* v_cache, int32_t cache_dtype, const float* k_scale,
                   const float* v_scale, int32_t n_scales, const int32_t* block_table,
                   const int32_t* context_lens, int32_t n_seqs, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size, int64_t n_blocks,
                   int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
                   int32_t partition_tokens, int32_t max_partitions, float scale, int32_t q_dtype,
                   int64_t* slot_mapping, float* part_out, float* part_lse, int32_t* err_flag,
                   void* stream);

/*
 * pa_decode_step_static -- pa_decode_step followed by pa_merge_lse, allocating nothing:
 * for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The partial outputs and LSEs, which
 * the two calls take from the caller, live here in a fixed device array of the library,
 * PA_STATIC_SCRATCH_BYTES on each GPU, held from the library's load until the process
 * ends.  No allocator is called.
 *   out   [n_seqs][n_q_heads][dv] of out_dtype (PA_F32 or PA_BF16) and lse float32
 *         [n_seqs][n_q_heads]: as pa_merge_lse writes them (with one shard, one partition
 *         slot and out_dtype PA_F32 the decode writes them itself, one launch in all).
 *   Other arguments: as in pa_decode_step.
 *   The partials take n_seqs*n_shards*max_partitions*n_q_heads*(dv + 1)*4 bytes (output
 *   and LSE parts each rounded up to 256); a call needing more than
 *   PA_STATIC_SCRATCH_BYTES returns PA_ERR_BUFFER and launches nothing.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's contents
 *   (nothing in it needs to start at zero): calls that overlap on one GPU -- from several
 *   streams or host threads -- race, and the caller must order them.
 */
#define PA_STATIC_SCRATCH_BYTES (64u << 20)
int pa_decode_step_static(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                          void* k_cache, void* v_cache, int32_t cache_dtype, const float* k_scale,
                          const float* v_scale, int32_t n_scales, const int32_t* block_table,
                          const int32_t* context_lens, int32_t n_seqs, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
                          int64_t n_blocks, int32_t max_blocks_per_shard, int32_t n_shards,
                          int32_t interleave, int32_t partition_tokens, int32_t max_partitions,
                          float scale, int32_t q_dtype, int64_t* slot_mapping, void* out,
                          int32_t out_dtype, float* lse, int32_t* err_flag, void* stream);

/*
 * pa_decode_fp8 -- pa_decode over an E4M3 cache written by pa_kv_append_fp8: every
 * stored key (value) element is taken as value(code) * k_scale[h] (v_scale[h]; index 0
 * when n_scales == 1), for KV head h; the latent cache (v_cache == NULL) takes the
 * value from the key row, with k_scale.  q is of q_dtype (PA_F32 or PA_BF16); the other
 * arguments and the outputs are as in pa_decode.  Cache base addresses must be 16-byte
 * aligned.
 */
int pa_decode_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                  const float* k_scale, const float* v_scale, int32_t n_scales,
                  const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                  int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                  int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                  int32_t n_shards, int32_t interleave, int32_t partition_tokens,
                  int32_t max_partitions, float scale, int32_t q_dtype, float* part_out,
                  float* part_lse, int32_t* err_flag, void* stream);

/*
 * Several new tokens per sequence (multi-query decode).  A step may carry more than
 * one new token of a sequence -- a prompt continued in chunks ([KVB], failure-mode
 * paragraph on chunked prefill; [AGX], execution-plane section) or speculative tokens
 * to verify ([AGX], open-source kernel contributions section) -- and each follows the
 * decode rule of [KVB] ("Why does writing one token at a time duplicate work?"): it
 * attends over every earlier token and itself.  The n_b new tokens of sequence b are
 * the last n_b of its context (context_lens[b] counts them): new token i sits at
 * global position L - n_b + i and attends over positions 0 .. L - n_b + i (causal
 * among the new tokens).
 *   query_start  DEVICE int32 [n_seqs + 1], non-decreasing, query_start[0] = 0,
 *                query_start[n_seqs] = n_rows: rows query_start[b] .. query_start[b+1]-1
 *                of the packed arrays below are sequence b's new tokens in order.  A
 *                sequence whose rows fall outside [0, n_rows), or with more new tokens
 *                than context tokens (or than max_q_len), sets *err_flag and is skipped
 *                (its rows are not written).
 */

/*
 * pa_slot_mapping_multi -- the cache slot of every new token (slot_mapping int64
 * [n_rows], row order), by the same placement rule as pa_slot_mapping.  The new rows
 * then go to pa_kv_append (or pa_kv_append_fp8) with n_tokens = n_rows.
 */
int pa_slot_mapping_multi(const int32_t* block_table, const int32_t* context_lens,
                          const int32_t* query_start, int32_t n_seqs, int32_t n_rows,
                          int32_t n_shards, int32_t interleave, int32_t block_size,
                          int32_t max_blocks_per_shard, int64_t n_blocks, int64_t* slot_mapping,
                          int32_t* err_flag, void* stream);

/*
 * pa_decode_multi -- pa_decode with several new tokens per sequence, each attending
 * causally.  q [n_rows][n_q_heads][dk] of q_dtype; max_q_len: a bound on every
 * sequence's new tokens (it sizes the launch).  kv_dtype is q_dtype, or PA_FP8_E4M3
 * with k_scale/v_scale/n_scales as in pa_decode_fp8 (else those are ignored).
 *   part_out float32 [n_rows][n_shards][Pmax][n_q_heads][dv], part_lse float32
 *   [n_rows][n_shards][Pmax][n_q_heads]: as in pa_decode, per row; a partition holding
 *   none of the tokens a row may see has lse -inf.  pa_merge_lse with n_seqs = n_rows
 *   finishes the step.
 */
int pa_decode_multi(const void* q, int32_t q_dtype, const int32_t* query_start, int32_t n_rows,
                    int32_t max_q_len, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                    const float* k_scale, const float* v_scale, int32_t n_scales,
                    const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                    int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                    int32_t n_shards, int32_t interleave, int32_t partition_tokens,
                    int32_t max_partitions, float scale, float* part_out, float* part_lse,
                    int32_t* err_flag, void* stream);

/*
 * pa_merge_lse -- combine the partials of each (sequence, head) into the attention
 * over all its tokens ([DCP], DCP mechanism section: gather the LSEs, reweight each
 * partial output, sum).  With lse = log(sum_p exp(lse_p)), part p has weight
 * exp(lse_p - lse); parts with lse_p = -inf have weight 0; if every part is empty the
 * output is 0 and lse is -inf.  part_out rows of parts with lse_p = -inf are not read.
 *   part_out float32 [n_seqs][n_parts][n_q_heads][dv], part_lse float32
 *   [n_seqs][n_parts][n_q_heads] (pa_decode's outputs with n_parts = n_shards*Pmax).
 *   out      [n_seqs][n_q_heads][dv] of out_dtype (PA_F32, or PA_BF16 rounded to nearest
 *            even);  lse float32 [n_seqs][n_q_heads], may be NULL.
 */
int pa_merge_lse(const float* part_out, const float* part_lse, int32_t n_seqs, int32_t n_parts,
                 int32_t n_q_heads, int32_t dv, void* out, int32_t out_dtype, float* lse,
                 void* stream);

/*
 * pa_gather_kv -- copy the K/V rows of shard `shard` of sequence `seq` into contiguous
 * arrays in local token order, through the same block-table address generation
 * pa_decode uses ([PA], block-table section).  For checking the paged addressing.
 *   context_len: L of sequence `seq` (host value, the same as its context_lens entry).
 *   k_out [L_r][n_kv_heads][dk], v_out [L_r][n_kv_heads][dv] (v_out from the first dv
 *   entries of the key rows when v_cache is NULL); L_r = pa_shard_length(L, ...).
 *   Rows whose block id is invalid are left unwritten and set *err_flag.
 *   dtype PA_FP8_E4M3 copies the codes.
 */
int pa_gather_kv(const void* k_cache, const void* v_cache, const int32_t* block_table,
                 int32_t seq, int32_t shard, int32_t context_len, int32_t n_kv_heads, int32_t dk,
                 int32_t dv, int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                 int32_t n_shards, int32_t interleave, int32_t dtype, void* k_out, void* v_out,
                 int32_t* err_flag, void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks, for copy-on-write ([PA], "Sharing common
 * blocks and copy-on-write": before a sequence writes into a block other sequences
 * share, it gets its own copy).  For each pair i, block pairs[2i] (source) is copied to
 * block pairs[2i+1] (destination): all KV heads, the keys and, unless v_cache is NULL
 * (latent cache), the values; bit-exact.
 *   pairs: DEVICE int64 [n_pairs][2].  A pair with an id outside [0, n_blocks) is
 *   skipped and sets *err_flag; src == dst is a no-op.  Destinations must be distinct
 *   and must not be the source of another pair of the same call (else the content of
 *   those blocks is unspecified).  Sizes as in pa_kv_append; dtype may be PA_FP8_E4M3.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n_pairs,
                   int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size, int64_t n_blocks,
                   int32_t dtype, int32_t* err_flag, void* stream);

/*
 * Block pool -- host-side accounting of a shared pool of fixed-size blocks ([PA]):
 * each sequence has a table of physical blocks in logical order; a token goes into the
 * last block while it has room, else into a newly taken block (block-table section);
 * a finished sequence returns its blocks for anyone to reuse, nothing is compacted
 * ("Reusing blocks freed when a request ends"); sequences forked from a parent share its
 * blocks under a reference count, and a sequence about to write into a shared last
 * block first takes a copy of it ("Sharing common blocks and copy-on-write"); when the
 * pool runs out the request has to wait (limits section).
 * Policy of this library: free blocks are handed out first-in first-out (initially
 * 0, 1, .., n_blocks-1; a block whose count drops to 0 goes to the back).  All calls
 * are HOST calls on an object that is not thread-safe; sequence ids are any int64 the
 * caller chooses.  pa_pool_append is all-or-nothing: if the free blocks do not cover
 * the new blocks and copies it needs, it changes nothing and returns PA_ERR_EXHAUSTED.
 */
typedef struct pa_block_pool pa_block_pool;
/* NULL on invalid arguments or out of memory. */
pa_block_pool* pa_pool_create(int64_t n_blocks, int32_t block_size);
void pa_pool_destroy(pa_block_pool* pool);
/* a new sequence (id not in use) with n_tokens tokens to store (0 allowed) */
int pa_pool_add(pa_block_pool* pool, int64_t seq, int64_t n_tokens);
/* store n_tokens more tokens of `seq`.  Copy-on-write copies made on the way are
 * written to copies (HOST int64 [max_copies][2], (source, destination) block pairs, in
 * order; they go to pa_copy_blocks before the new tokens are written); *n_copies gets
 * their number (a single call makes at most one).  PA_ERR_BUFFER if max_copies is too
 * small (nothing changed). */
int pa_pool_append(pa_block_pool* pool, int64_t seq, int64_t n_tokens, int64_t* copies,
                   int32_t max_copies, int32_t* n_copies);
/* `child` (id not in use) starts with `parent`'s tokens, sharing its blocks */
int pa_pool_fork(pa_block_pool* pool, int64_t parent, int64_t child);
/* the sequence ends; blocks no other sequence uses become free */
int pa_pool_finish(pa_block_pool* pool, int64_t seq);
/* accounting: -1 on an unknown sequence or block */
int64_t pa_pool_num_free(const pa_block_pool* pool);
int64_t pa_pool_length(const pa_block_pool* pool, int64_t seq);
int64_t pa_pool_num_blocks(const pa_block_pool* pool, int64_t seq);
int32_t pa_pool_refcount(const pa_block_pool* pool, int64_t block);
/* the sequence's physical block ids in logical order into table (HOST int32
 * [capacity]); returns their number, or -1 (unknown sequence or capacity too small) */
int64_t pa_pool_table(const pa_block_pool* pool, int64_t seq, int32_t* table, int64_t capacity);

/* Host helpers (no device work).  Return -1 on invalid arguments. */
int32_t pa_shard_length(int32_t context_len, int32_t n_shards, int32_t interleave, int32_t shard);
int32_t pa_max_partitions(int32_t max_context_len, int32_t n_shards, int32_t interleave,
                          int32_t partition_tokens);

/*
 * pa_default_partition_tokens -- a partition size (a multiple of block_size) that
 * cuts the work of a step into enough (sequence, shard, partition, KV head) units to
 * keep all 256 compute units of an MI355X busy, preferring long partitions (fewer
 * partials to merge).  A heuristic of this library, not something the pages define.
 */
int32_t pa_default_partition_tokens(int32_t n_seqs, int32_t n_kv_heads, int32_t max_context_len,
                                    int32_t n_shards, int32_t interleave, int32_t block_size);

/*
 * pa_choose_partition_tokens -- a partition size for a step whose context lengths the
 * caller knows on the host (context_lens_host: HOST int32 [n_seqs]).  Picks the multiple
 * of block_size that minimises a model of how the kernel pa_decode would run for this
 * shape (latent != 0: value = first dv entries of the key row) is dispatched: the
 * busiest workgroup's tokens plus a fixed per-unit cost when the kernel keeps a resident
 * grid, else the busiest XCD's rounds of workgroups x (partition tokens + that cost),
 * with the kernel's occupancy and the device's compute-unit and XCD counts.  dtype
 * PA_FP8_E4M3 means an E4M3 cache read with bf16 queries (pa_decode_fp8).  A heuristic
 * of this library.  Returns -1 on invalid arguments.
 */
int32_t pa_choose_partition_tokens(const int32_t* context_lens_host, int32_t n_seqs,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                                   int32_t block_size, int32_t dtype, int32_t latent,
                                   int32_t n_shards, int32_t interleave);

/*
 * pa_choose_partition_tokens_multi -- the same choice for pa_decode_multi with
 * max_q_len (>= 1) as its grid bound on new tokens per sequence: the model takes the
 * launch pa_decode_multi makes (in the GQA and generic kernels the (new token, head)
 * pairs of a KV head share workgroups; the latent kernel takes one unit of work per new
 * token).  context_lens_host and the other arguments as in pa_choose_partition_tokens
 * (n_q_heads unscaled).  Returns -1 on invalid arguments.
 */
int32_t pa_choose_partition_tokens_multi(const int32_t* context_lens_host, int32_t n_seqs,
                                         int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t dk, int32_t dv, int32_t block_size, int32_t dtype,
                                         int32_t latent, int32_t n_shards, int32_t interleave);

/* Message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_PA_H */
