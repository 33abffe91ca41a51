// pa_api.cpp -- the C ABI declared in include/pa.h: argument validation, launch
// configuration and dispatch.  Nothing is launched when validation fails.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <vector>
#include <string>

#include "../../include/pa.h"
#include "pa_common.h"
#include "pa_launch.h"
#include "pa_dispatch.h"
#include "pa_error.h"

namespace pa {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(int32_t dt) { return dt == PA_F32 || dt == PA_BF16; }
bool valid_cache_dtype(int32_t dt) { return valid_dtype(dt) || dt == PA_FP8_E4M3; }
int64_t elem_bytes(int32_t dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : 1; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_placement(int32_t n_shards, int32_t interleave, int32_t block_size) {
  REQUIRE(n_shards >= 1 && n_shards <= 65535, PA_ERR_SHAPE, "n_shards=%d must be in [1, 65535]", n_shards);
  REQUIRE(interleave >= 1, PA_ERR_SHAPE, "interleave=%d must be >= 1", interleave);
  REQUIRE(int64_t(n_shards) * interleave <= (int64_t(1) << 30), PA_ERR_SHAPE,
          "n_shards*interleave=%lld too large", (long long)n_shards * interleave);
  REQUIRE(block_size >= 1 && block_size <= PA_MAX_BLOCK_SIZE, PA_ERR_UNSUPPORTED,
          "block_size=%d must be in [1, %d]", block_size, PA_MAX_BLOCK_SIZE);
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return pa::last_error(); }

int32_t pa_shard_length(int32_t context_len, int32_t n_shards, int32_t interleave, int32_t shard) {
  if (context_len < 0 || n_shards < 1 || interleave < 1 || shard < 0 || shard >= n_shards) return -1;
  if (int64_t(n_shards) * interleave > (int64_t(1) << 30)) return -1;
  return pa::shard_len(context_len, n_shards, interleave, shard);
}

int32_t pa_max_partitions(int32_t max_context_len, int32_t n_shards, int32_t interleave,
                          int32_t partition_tokens) {
  if (partition_tokens < 1) return -1;
  const int32_t longest = pa_shard_length(max_context_len, n_shards, interleave, 0);
  if (longest < 0) return -1;
  return (longest + partition_tokens - 1) / partition_tokens;
}

int32_t pa_default_partition_tokens(int32_t n_seqs, int32_t n_kv_heads, int32_t max_context_len,
                                    int32_t n_shards, int32_t interleave, int32_t block_size) {
  if (n_seqs < 1 || n_kv_heads < 1 || block_size < 1 || block_size > PA_MAX_BLOCK_SIZE) return -1;
  const int32_t longest = pa_shard_length(max_context_len, n_shards, interleave, 0);
  if (longest < 0) return -1;
  // Enough units for several workgroups per compute unit, partitions no longer
  // than 4,096 tokens and no shorter than 256 tokens (or one block).
  const int64_t want_units = 4 * 256;
  const int64_t rows = int64_t(n_seqs) * n_shards * n_kv_heads;
  int32_t T = 4096;
  while (T > 256 && rows * ((longest + T - 1) / T) < want_units) T /= 2;
  T = ((T + block_size - 1) / block_size) * block_size;
  return T;
}

static int32_t choose_partition_tokens(const int32_t* context_lens_host, int32_t n_seqs,
                                       int32_t max_q, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t dk, int32_t dv, int32_t block_size, int32_t dtype,
                                       int32_t latent, int32_t n_shards, int32_t interleave);

int32_t pa_choose_partition_tokens(const int32_t* context_lens_host, int32_t n_seqs,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                                   int32_t block_size, int32_t dtype, int32_t latent,
                                   int32_t n_shards, int32_t interleave) {
  return choose_partition_tokens(context_lens_host, n_seqs, 0, n_q_heads, n_kv_heads, dk, dv,
                                 block_size, dtype, latent, n_shards, interleave);
}

int32_t pa_choose_partition_tokens_multi(const int32_t* context_lens_host, int32_t n_seqs,
                                         int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t dk, int32_t dv, int32_t block_size, int32_t dtype,
                                         int32_t latent, int32_t n_shards, int32_t interleave) {
  if (max_q_len < 1) return -1;
  return choose_partition_tokens(context_lens_host, n_seqs, max_q_len, n_q_heads, n_kv_heads, dk,
                                 dv, block_size, dtype, latent, n_shards, interleave);
}

// max_q == 0: pa_decode's launch (one new token, no query_start); else pa_decode_multi's
static int32_t choose_partition_tokens(const int32_t* context_lens_host, int32_t n_seqs,
                                       int32_t max_q, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t dk, int32_t dv, int32_t block_size, int32_t dtype,
                                       int32_t latent, int32_t n_shards, int32_t interleave) {
  if (!context_lens_host || n_seqs < 1 || n_q_heads < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0 || block_size < 1 || block_size > PA_MAX_BLOCK_SIZE ||
      n_shards < 1 || interleave < 1 || int64_t(n_shards) * interleave > (int64_t(1) << 30) ||
      !valid_cache_dtype(dtype))
    return -1;
  pa::DecodeArgs a{};
  a.hq = n_q_heads;
  a.hkv = n_kv_heads;
  a.dk = dk;
  a.dv = dv;
  a.bs = block_size;
  a.dtype = dtype == PA_FP8_E4M3 ? PA_BF16 : dtype;  // E4M3 cache: bf16 queries
  a.kv_dtype = dtype;
  a.max_q = max_q > 0 ? max_q : 1;
  a.query_start = max_q > 0 ? &a.n_seqs : nullptr;  // only its NULL-ness matters
  a.v_cache = latent ? nullptr : static_cast<const void*>(&a);  // only its NULL-ness matters
  std::vector<int32_t> shard_len_v(size_t(n_seqs) * n_shards);
  int32_t longest = 0;
  for (int b = 0; b < n_seqs; ++b)
    for (int r = 0; r < n_shards; ++r) {
      const int32_t Lr = pa::shard_len(std::max(context_lens_host[b], 0), n_shards, interleave, r);
      shard_len_v[size_t(b) * n_shards + r] = Lr;
      longest = std::max(longest, Lr);
    }
  if (longest == 0) return block_size;
  // the kernel variant can depend on the partition size; partitions as long as the
  // longest shard stand for the sizes the scan below can pick (short contexts stay short)
  a.part_tokens = longest;
  const pa::KernelChoice kc = pa::choose_kernel(a);
  int cus = 0, xccs = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;  // MI355X
  }
  if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xccs <= 0 ||
      cus % xccs != 0) {
    (void)hipGetLastError();
    xccs = cus == 256 ? 8 : 1;
  }
  // Cost of a partition size T, in token-times.  Workgroups are dispatched to the XCDs
  // round-robin by their linear id (x fastest: the partition index), each XCD running
  // (its CUs x workgroups per CU) at a time; the busiest XCD sets the number of rounds,
  // each about T tokens plus a fixed per-unit cost (prologue, and writing then merging
  // the partition's output rows).
  const int64_t slots_per_xcd = int64_t(cus / xccs) * (kc.workgroups_per_cu > 0 ? kc.workgroups_per_cu : 2);
  const int64_t partial_bytes = int64_t(n_q_heads / n_kv_heads) * dv * 4 * 2;
  const int64_t token_bytes = int64_t(latent ? dk : dk + dv) * elem_bytes(dtype);
  const int64_t overhead = 128 + partial_bytes / (token_bytes > 0 ? token_bytes : 1);
  const int64_t Y = int64_t(n_seqs) * n_shards, Z = kc.units_per_partition;
  const int32_t max_m = (longest + block_size - 1) / block_size;
  // every multiple of the block size while the scan stays cheap, else a coarser grid
  const int64_t work = int64_t(max_m) * Y * Z;
  const int32_t step = work <= (int64_t(1) << 24) ? 1 : std::max<int32_t>(1, max_m / 512);
  int32_t best_T = block_size * max_m;
  double best_cost = 1e300;
  std::vector<int64_t> per_xcd(static_cast<size_t>(xccs), 0);
  std::vector<int64_t> load;
  for (int32_t m = 1; m <= max_m; m += (m < 16 ? 1 : step)) {
    const int64_t T = int64_t(block_size) * m;
    if (kc.persistent) {
      // resident grid: unit u (pairs in order, then partitions, KV head fastest) goes to
      // workgroup u mod G; the busiest workgroup's tokens plus per-unit costs decide
      int64_t units = 0;
      for (int64_t y = 0; y < Y; ++y) units += (shard_len_v[size_t(y)] + T - 1) / T * Z;
      if (units == 0) continue;
      const int64_t G = std::min<int64_t>(int64_t(cus) * (kc.workgroups_per_cu > 0 ? kc.workgroups_per_cu : 1), units);
      load.assign(size_t(G), 0);
      int64_t u = 0;
      for (int64_t y = 0; y < Y; ++y) {
        const int64_t Lr = shard_len_v[size_t(y)];
        for (int64_t t0 = 0; t0 < Lr; t0 += T)
          for (int64_t z = 0; z < Z; ++z, ++u) load[size_t(u % G)] += std::min<int64_t>(T, Lr - t0) + overhead;
      }
      const double cost = double(*std::max_element(load.begin(), load.end()));
      if (cost < best_cost * (1 - 1e-9)) {
        best_cost = cost;
        best_T = int32_t(T);
      }
      continue;
    }
    const int64_t parts = (longest + T - 1) / T;   // grid x
    std::fill(per_xcd.begin(), per_xcd.end(), 0);
    for (int64_t y = 0; y < Y; ++y) {
      const int64_t n_p = (shard_len_v[size_t(y)] + T - 1) / T;   // non-empty partitions
      if (n_p == 0) continue;
      for (int64_t z = 0; z < Z; ++z) {
        // ids parts*(y + Y z) + p for p < n_p, counted per residue mod xccs
        const int64_t base = (parts * (y + Y * z)) % xccs;
        for (int x = 0; x < xccs; ++x) {
          const int64_t first = ((x - base) % xccs + xccs) % xccs;   // smallest p with id % xccs == x
          if (first < n_p) per_xcd[size_t(x)] += (n_p - 1 - first) / xccs + 1;
        }
      }
    }
    int64_t rounds = 0;
    for (int x = 0; x < xccs; ++x) rounds = std::max(rounds, (per_xcd[size_t(x)] + slots_per_xcd - 1) / slots_per_xcd);
    const double cost = double(rounds) * double(std::min<int64_t>(T, longest) + overhead);
    if (cost < best_cost * (1 - 1e-9)) {
      best_cost = cost;
      best_T = int32_t(T);
    }
  }
  return best_T;
}

int pa_slot_mapping(const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                    int32_t n_shards, int32_t interleave, int32_t block_size,
                    int32_t max_blocks_per_shard, int64_t n_blocks, int64_t* slot_mapping,
                    int32_t* err_flag, void* stream) {
  REQUIRE(block_table && context_lens && slot_mapping, PA_ERR_NULL,
          "pa_slot_mapping: block_table, context_lens and slot_mapping must be non-NULL");
  REQUIRE(n_seqs >= 0, PA_ERR_SHAPE, "n_seqs=%d must be >= 0", n_seqs);
  if (int rc = check_placement(n_shards, interleave, block_size)) return rc;
  REQUIRE(max_blocks_per_shard >= 1 && n_blocks >= 1, PA_ERR_SHAPE,
          "max_blocks_per_shard=%d and n_blocks=%lld must be >= 1", max_blocks_per_shard,
          (long long)n_blocks);
  if (n_seqs == 0) return ok();
  return hip_status(pa::launch_slot_mapping(block_table, context_lens, n_seqs, n_shards, interleave,
                                            block_size, max_blocks_per_shard, n_blocks,
                                            slot_mapping, err_flag, (hipStream_t)stream),
                    "pa_slot_mapping launch");
}

int pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int64_t* slot_mapping, int32_t n_tokens, int32_t n_kv_heads, int32_t dk,
                 int32_t dv, int32_t block_size, int64_t n_blocks, int32_t dtype,
                 int32_t* err_flag, void* stream) {
  REQUIRE(k_new && k_cache && slot_mapping, PA_ERR_NULL,
          "pa_kv_append: k_new, k_cache and slot_mapping must be non-NULL");
  REQUIRE((v_new == nullptr) == (v_cache == nullptr), PA_ERR_NULL,
          "pa_kv_append: v_new and v_cache must both be NULL (latent cache) or both non-NULL");
  REQUIRE(valid_dtype(dtype), PA_ERR_UNSUPPORTED, "dtype=%d is not PA_F32 or PA_BF16", dtype);
  REQUIRE(n_tokens >= 0, PA_ERR_SHAPE, "n_tokens=%d must be >= 0", n_tokens);
  REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 65535, PA_ERR_SHAPE, "n_kv_heads=%d out of range", n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED, "dk=%d must be in [1, %d]", dk, PA_MAX_HEAD_DIM);
  REQUIRE(v_cache == nullptr || (dv >= 1 && dv <= PA_MAX_HEAD_DIM), PA_ERR_UNSUPPORTED,
          "dv=%d must be in [1, %d]", dv, PA_MAX_HEAD_DIM);
  REQUIRE(block_size >= 1 && block_size <= PA_MAX_BLOCK_SIZE, PA_ERR_UNSUPPORTED,
          "block_size=%d must be in [1, %d]", block_size, PA_MAX_BLOCK_SIZE);
  REQUIRE(n_blocks >= 1, PA_ERR_SHAPE, "n_blocks=%lld must be >= 1", (long long)n_blocks);
  if (n_tokens == 0) return ok();
  return hip_status(pa::launch_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, n_tokens,
                                         n_kv_heads, dk, dv, block_size, n_blocks, dtype, err_flag,
                                         (hipStream_t)stream),
                    "pa_kv_append launch");
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n_pairs,
                   int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size, int64_t n_blocks,
                   int32_t dtype, int32_t* err_flag, void* stream) {
  REQUIRE(k_cache && pairs, PA_ERR_NULL, "pa_copy_blocks: k_cache and pairs must be non-NULL");
  REQUIRE(valid_cache_dtype(dtype), PA_ERR_UNSUPPORTED,
          "dtype=%d is not PA_F32, PA_BF16 or PA_FP8_E4M3", dtype);
  REQUIRE(n_pairs >= 0 && n_pairs <= (1 << 22), PA_ERR_SHAPE, "n_pairs=%d must be in [0, 2^22]",
          n_pairs);
  REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 65535, PA_ERR_SHAPE, "n_kv_heads=%d out of range", n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED, "dk=%d must be in [1, %d]", dk, PA_MAX_HEAD_DIM);
  REQUIRE(v_cache == nullptr || (dv >= 1 && dv <= PA_MAX_HEAD_DIM), PA_ERR_UNSUPPORTED,
          "dv=%d must be in [1, %d]", dv, PA_MAX_HEAD_DIM);
  REQUIRE(block_size >= 1 && block_size <= PA_MAX_BLOCK_SIZE, PA_ERR_UNSUPPORTED,
          "block_size=%d must be in [1, %d]", block_size, PA_MAX_BLOCK_SIZE);
  REQUIRE(n_blocks >= 1, PA_ERR_SHAPE, "n_blocks=%lld must be >= 1", (long long)n_blocks);
  if (n_pairs == 0) return ok();
  const int64_t es = elem_bytes(dtype);
  const int64_t k_bytes = int64_t(n_kv_heads) * block_size * dk * es;
  const int64_t v_bytes = v_cache != nullptr ? int64_t(n_kv_heads) * block_size * dv * es : 0;
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, pairs, n_pairs, k_bytes, v_bytes,
                                           n_blocks, err_flag, (hipStream_t)stream),
                    "pa_copy_blocks launch");
}

int pa_kv_append_fp8(const void* k_new, const void* v_new, int32_t new_dtype, uint8_t* k_cache,
                     uint8_t* v_cache, const float* k_scale, const float* v_scale,
                     int32_t n_scales, const int64_t* slot_mapping, int32_t n_tokens,
                     int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
                     int64_t n_blocks, int32_t* err_flag, void* stream) {
  REQUIRE(k_new && k_cache && slot_mapping && k_scale, PA_ERR_NULL,
          "pa_kv_append_fp8: k_new, k_cache, k_scale and slot_mapping must be non-NULL");
  REQUIRE((v_new == nullptr) == (v_cache == nullptr), PA_ERR_NULL,
          "pa_kv_append_fp8: v_new and v_cache must both be NULL (latent cache) or both non-NULL");
  REQUIRE(v_cache == nullptr || v_scale != nullptr, PA_ERR_NULL,
          "pa_kv_append_fp8: v_scale must be non-NULL with a value cache");
  REQUIRE(valid_dtype(new_dtype), PA_ERR_UNSUPPORTED, "new_dtype=%d is not PA_F32 or PA_BF16",
          new_dtype);
  REQUIRE(n_tokens >= 0, PA_ERR_SHAPE, "n_tokens=%d must be >= 0", n_tokens);
  REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 65535, PA_ERR_SHAPE, "n_kv_heads=%d out of range", n_kv_heads);
  REQUIRE(n_scales == 1 || n_scales == n_kv_heads, PA_ERR_SHAPE,
          "n_scales=%d must be 1 or n_kv_heads=%d", n_scales, n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED, "dk=%d must be in [1, %d]", dk, PA_MAX_HEAD_DIM);
  REQUIRE(v_cache == nullptr || (dv >= 1 && dv <= PA_MAX_HEAD_DIM), PA_ERR_UNSUPPORTED,
          "dv=%d must be in [1, %d]", dv, PA_MAX_HEAD_DIM);
  REQUIRE(block_size >= 1 && block_size <= PA_MAX_BLOCK_SIZE, PA_ERR_UNSUPPORTED,
          "block_size=%d must be in [1, %d]", block_size, PA_MAX_BLOCK_SIZE);
  REQUIRE(n_blocks >= 1, PA_ERR_SHAPE, "n_blocks=%lld must be >= 1", (long long)n_blocks);
  if (n_tokens == 0) return ok();
  return hip_status(pa::launch_kv_append_fp8(k_new, v_new, new_dtype, k_cache, v_cache, k_scale,
                                             v_scale, n_scales, slot_mapping, n_tokens, n_kv_heads,
                                             dk, dv, block_size, n_blocks, err_flag,
                                             (hipStream_t)stream),
                    "pa_kv_append_fp8 launch");
}

int pa_kv_append_routed(const void* k_new, const void* v_new, int32_t new_dtype, void* k_cache,
                        void* v_cache, int32_t cache_dtype, const float* k_scale,
                        const float* v_scale, int32_t n_scales, const int32_t* block_table,
                        const int32_t* context_lens, int32_t n_seqs, int32_t n_kv_heads, int32_t dk,
                        int32_t dv, int32_t block_size, int64_t n_blocks,
                        int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
                        int64_t* slot_mapping, int32_t* err_flag, void* stream) {
  REQUIRE(k_new && k_cache && block_table && context_lens, PA_ERR_NULL,
          "pa_kv_append_routed: k_new, k_cache, block_table and context_lens must be non-NULL");
  REQUIRE((v_new == nullptr) == (v_cache == nullptr), PA_ERR_NULL,
          "pa_kv_append_routed: v_new and v_cache must both be NULL (latent cache) or both non-NULL");
  REQUIRE(valid_dtype(new_dtype), PA_ERR_UNSUPPORTED, "new_dtype=%d is not PA_F32 or PA_BF16",
          new_dtype);
  REQUIRE(valid_cache_dtype(cache_dtype), PA_ERR_UNSUPPORTED,
          "cache_dtype=%d is not PA_F32, PA_BF16 or PA_FP8_E4M3", cache_dtype);
  REQUIRE(cache_dtype == PA_FP8_E4M3 || cache_dtype == new_dtype, PA_ERR_UNSUPPORTED,
          "new_dtype=%d must equal cache_dtype=%d (or the cache be PA_FP8_E4M3)", new_dtype,
          cache_dtype);
  if (cache_dtype == PA_FP8_E4M3) {
    REQUIRE(k_scale && (v_cache == nullptr || v_scale), PA_ERR_NULL,
            "pa_kv_append_routed: an E4M3 cache needs k_scale (and v_scale with a value cache)");
    REQUIRE(n_scales == 1 || n_scales == n_kv_heads, PA_ERR_SHAPE,
            "n_scales=%d must be 1 or n_kv_heads=%d", n_scales, n_kv_heads);
  }
  REQUIRE(n_seqs >= 0 && n_seqs <= (1 << 30), PA_ERR_SHAPE, "n_seqs=%d out of range", n_seqs);
  REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 65535, PA_ERR_SHAPE, "n_kv_heads=%d out of range", n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED, "dk=%d must be in [1, %d]", dk, PA_MAX_HEAD_DIM);
  REQUIRE(v_cache == nullptr || (dv >= 1 && dv <= PA_MAX_HEAD_DIM), PA_ERR_UNSUPPORTED,
          "dv=%d must be in [1, %d]", dv, PA_MAX_HEAD_DIM);
  if (int rc = check_placement(n_shards, interleave, block_size)) return rc;
  REQUIRE(max_blocks_per_shard >= 1 && n_blocks >= 1, PA_ERR_SHAPE,
          "max_blocks_per_shard=%d and n_blocks=%lld must be >= 1", max_blocks_per_shard,
          (long long)n_blocks);
  if (n_seqs == 0) return ok();
  return hip_status(pa::launch_kv_append_routed(k_new, v_new, new_dtype, k_cache, v_cache,
                                                cache_dtype, k_scale, v_scale, n_scales, block_table,
                                                context_lens, n_seqs, n_shards, interleave,
                                                max_blocks_per_shard, n_kv_heads, dk, dv, block_size,
                                                n_blocks, slot_mapping, err_flag,
                                                (hipStream_t)stream),
                    "pa_kv_append_routed launch");
}

}  // extern "C"

namespace {

// Checks shared by pa_decode and pa_decode_fp8; fills the kernel arguments.
int check_decode(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                 int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
                 int64_t n_blocks, int32_t max_blocks_per_shard, int32_t n_shards,
                 int32_t interleave, int32_t partition_tokens, int32_t max_partitions, float scale,
                 int32_t dtype, float* part_out, float* part_lse, int32_t* err_flag,
                 pa::DecodeArgs* out) {
  REQUIRE(q && k_cache && block_table && context_lens && part_out && part_lse, PA_ERR_NULL,
          "%s: q, k_cache, block_table, context_lens, part_out and part_lse must be non-NULL", fn);
  REQUIRE(valid_dtype(dtype), PA_ERR_UNSUPPORTED, "dtype=%d is not PA_F32 or PA_BF16", dtype);
  REQUIRE(n_seqs >= 0, PA_ERR_SHAPE, "n_seqs=%d must be >= 0", n_seqs);
  REQUIRE(n_q_heads >= 1 && n_kv_heads >= 1 && n_q_heads % n_kv_heads == 0, PA_ERR_SHAPE,
          "n_q_heads=%d must be a positive multiple of n_kv_heads=%d", n_q_heads, n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED, "dk=%d must be in [1, %d]", dk, PA_MAX_HEAD_DIM);
  REQUIRE(dv >= 1 && dv <= 512, PA_ERR_UNSUPPORTED, "dv=%d must be in [1, 512]", dv);
  REQUIRE(v_cache != nullptr || dv <= dk, PA_ERR_SHAPE,
          "latent cache (v_cache NULL) needs dv=%d <= dk=%d", dv, dk);
  if (int rc = check_placement(n_shards, interleave, block_size)) return rc;
  REQUIRE(max_blocks_per_shard >= 1 && n_blocks >= 1, PA_ERR_SHAPE,
          "max_blocks_per_shard=%d and n_blocks=%lld must be >= 1", max_blocks_per_shard,
          (long long)n_blocks);
  REQUIRE(partition_tokens >= 1 && partition_tokens % block_size == 0, PA_ERR_SHAPE,
          "partition_tokens=%d must be a positive multiple of block_size=%d", partition_tokens,
          block_size);
  REQUIRE(max_partitions >= 1, PA_ERR_BUFFER, "max_partitions=%d must be >= 1", max_partitions);
  REQUIRE(int64_t(max_partitions) * n_seqs * n_shards <= 0x7fffffff, PA_ERR_SHAPE,
          "max_partitions*n_seqs*n_shards=%lld exceeds 2^31-1",
          (long long)max_partitions * n_seqs * n_shards);
  REQUIRE(n_kv_heads * ((n_q_heads / n_kv_heads + 15) / 16) <= 65535, PA_ERR_SHAPE,
          "too many heads");
  pa::DecodeArgs a{q,        k_cache,         v_cache,    block_table, context_lens, n_seqs,
                   n_q_heads, n_kv_heads,     dk,         dv,          block_size,   n_blocks,
                   max_blocks_per_shard, n_shards, interleave, partition_tokens, max_partitions,
                   scale,    dtype,           part_out,   part_lse,    err_flag};
  a.kv_dtype = dtype;
  a.k_scale = a.v_scale = nullptr;
  a.n_scales = 0;
  a.query_start = nullptr;
  a.max_q = 1;
  a.n_rows = n_seqs;
  a.k_new = a.v_new = nullptr;
  a.new_dtype = dtype;
  a.slots_out = nullptr;
  *out = a;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
              int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
              int64_t n_blocks, int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
              int32_t partition_tokens, int32_t max_partitions, float scale, int32_t dtype,
              float* part_out, float* part_lse, int32_t* err_flag, void* stream) {
  pa::DecodeArgs a;
  if (int rc = check_decode("pa_decode", q, k_cache, v_cache, block_table, context_lens, n_seqs,
                            n_q_heads, n_kv_heads, dk, dv, block_size, n_blocks,
                            max_blocks_per_shard, n_shards, interleave, partition_tokens,
                            max_partitions, scale, dtype, part_out, part_lse, err_flag, &a))
    return rc;
  if (n_seqs == 0) return ok();
  return hip_status(pa::dispatch_decode(a, (hipStream_t)stream), "pa_decode launch");
}

int pa_decode_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                  const float* k_scale, const float* v_scale, int32_t n_scales,
                  const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                  int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                  int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                  int32_t n_shards, int32_t interleave, int32_t partition_tokens,
                  int32_t max_partitions, float scale, int32_t q_dtype, float* part_out,
                  float* part_lse, int32_t* err_flag, void* stream) {
  pa::DecodeArgs a;
  if (int rc = check_decode("pa_decode_fp8", q, k_cache, v_cache, block_table, context_lens,
                            n_seqs, n_q_heads, n_kv_heads, dk, dv, block_size, n_blocks,
                            max_blocks_per_shard, n_shards, interleave, partition_tokens,
                            max_partitions, scale, q_dtype, part_out, part_lse, err_flag, &a))
    return rc;
  REQUIRE(k_scale && (v_cache == nullptr || v_scale), PA_ERR_NULL,
          "pa_decode_fp8: k_scale (and v_scale with a value cache) must be non-NULL");
  REQUIRE(n_scales == 1 || n_scales == n_kv_heads, PA_ERR_SHAPE,
          "n_scales=%d must be 1 or n_kv_heads=%d", n_scales, n_kv_heads);
  if (n_seqs == 0) return ok();
  a.kv_dtype = PA_FP8_E4M3;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.n_scales = n_scales;
  return hip_status(pa::dispatch_decode(a, (hipStream_t)stream), "pa_decode_fp8 launch");
}

int pa_decode_step(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                   void* k_cache, void* v_cache, int32_t cache_dtype, const float* k_scale,
                   const float* v_scale, int32_t n_scales, const int32_t* block_table,
                   const int32_t* context_lens, int32_t n_seqs, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size, int64_t n_blocks,
                   int32_t max_blocks_per_shard, int32_t n_shards, int32_t interleave,
                   int32_t partition_tokens, int32_t max_partitions, float scale, int32_t q_dtype,
                   int64_t* slot_mapping, float* part_out, float* part_lse, int32_t* err_flag,
                   void* stream) {
  pa::DecodeArgs a;
  if (int rc = check_decode("pa_decode_step", q, k_cache, v_cache, block_table, context_lens,
                            n_seqs, n_q_heads, n_kv_heads, dk, dv, block_size, n_blocks,
                            max_blocks_per_shard, n_shards, interleave, partition_tokens,
                            max_partitions, scale, q_dtype, part_out, part_lse, err_flag, &a))
    return rc;
  REQUIRE(k_new && (v_new == nullptr) == (v_cache == nullptr), PA_ERR_NULL,
          "pa_decode_step: k_new must be non-NULL, v_new NULL exactly when v_cache is");
  REQUIRE(valid_dtype(new_dtype), PA_ERR_UNSUPPORTED, "new_dtype=%d is not PA_F32 or PA_BF16",
          new_dtype);
  REQUIRE(valid_cache_dtype(cache_dtype), PA_ERR_UNSUPPORTED,
          "cache_dtype=%d is not PA_F32, PA_BF16 or PA_FP8_E4M3", cache_dtype);
  if (cache_dtype == PA_FP8_E4M3) {
    REQUIRE(k_scale && (v_cache == nullptr || v_scale), PA_ERR_NULL,
            "pa_decode_step: an E4M3 cache needs k_scale (and v_scale with a value cache)");
    REQUIRE(n_scales == 1 || n_scales == n_kv_heads, PA_ERR_SHAPE,
            "n_scales=%d must be 1 or n_kv_heads=%d", n_scales, n_kv_heads);
    a.kv_dtype = PA_FP8_E4M3;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.n_scales = n_scales;
  } else {
    REQUIRE(cache_dtype == q_dtype && new_dtype == q_dtype, PA_ERR_UNSUPPORTED,
            "new_dtype=%d and cache_dtype=%d must equal q_dtype=%d (or the cache be PA_FP8_E4M3)",
            new_dtype, cache_dtype, q_dtype);
  }
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  a.slots_out = slot_mapping;
  if (n_seqs == 0) return ok();
  return hip_status(pa::dispatch_decode(a, (hipStream_t)stream), "pa_decode_step launch");
}

int pa_decode_step_static(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                          void* k_cache, void* v_cache, int32_t cache_dtype, const float* k_scale,
                          const float* v_scale, int32_t n_scales, const int32_t* block_table,
                          const int32_t* context_lens, int32_t n_seqs, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t dk, int32_t dv, int32_t block_size,
                          int64_t n_blocks, int32_t max_blocks_per_shard, int32_t n_shards,
                          int32_t interleave, int32_t partition_tokens, int32_t max_partitions,
                          float scale, int32_t q_dtype, int64_t* slot_mapping, void* out,
                          int32_t out_dtype, float* lse, int32_t* err_flag, void* stream) {
  // the checks the two calls below would make after the first has launched, and the size
  REQUIRE(out && lse, PA_ERR_NULL, "pa_decode_step_static: out and lse must be non-NULL");
  REQUIRE(valid_dtype(out_dtype), PA_ERR_UNSUPPORTED, "out_dtype=%d is not PA_F32 or PA_BF16",
          out_dtype);
  REQUIRE(n_seqs >= 0 && n_q_heads >= 1 && n_shards >= 1 && max_partitions >= 1 && dv >= 1,
          PA_ERR_SHAPE, "n_seqs=%d, n_q_heads=%d, n_shards=%d, max_partitions=%d, dv=%d out of range",
          n_seqs, n_q_heads, n_shards, max_partitions, dv);
  REQUIRE(int64_t(n_seqs) * n_q_heads <= 0x7fffffff, PA_ERR_SHAPE, "n_seqs*n_q_heads too large");
  auto round256 = [](uint64_t x) { return (x + 255) / 256 * 256; };
  const uint64_t rows = uint64_t(n_seqs) * uint64_t(n_shards) * uint64_t(max_partitions) * uint64_t(n_q_heads);
  const uint64_t out_bytes = round256(rows * uint64_t(dv) * 4);
  const uint64_t lse_bytes = round256(rows * 4);
  REQUIRE(out_bytes + lse_bytes <= pa::kStaticScratchBytes, PA_ERR_BUFFER,
          "pa_decode_step_static: the partials need %llu bytes, more than the %llu of the "
          "library's array", (unsigned long long)(out_bytes + lse_bytes),
          (unsigned long long)pa::kStaticScratchBytes);
  const bool direct = n_shards == 1 && max_partitions == 1 && out_dtype == PA_F32;
  float* po = static_cast<float*>(out);
  float* pl = lse;
  if (!direct && n_seqs > 0) {
    char* base = nullptr;
    const hipError_t e = pa::static_scratch(&base);
    if (e != hipSuccess) return hip_status(e, "pa_decode_step_static: address of the partials array");
    po = reinterpret_cast<float*>(base);
    pl = reinterpret_cast<float*>(base + out_bytes);
  }
  const int rc = pa_decode_step(q, k_new, v_new, new_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                v_scale, n_scales, block_table, context_lens, n_seqs, n_q_heads,
                                n_kv_heads, dk, dv, block_size, n_blocks, max_blocks_per_shard,
                                n_shards, interleave, partition_tokens, max_partitions, scale,
                                q_dtype, slot_mapping, po, pl, err_flag, stream);
  if (rc != PA_OK || direct || n_seqs == 0) return rc;
  return pa_merge_lse(po, pl, n_seqs, n_shards * max_partitions, n_q_heads, dv, out, out_dtype, lse,
                      stream);
}

int pa_slot_mapping_multi(const int32_t* block_table, const int32_t* context_lens,
                          const int32_t* query_start, int32_t n_seqs, int32_t n_rows,
                          int32_t n_shards, int32_t interleave, int32_t block_size,
                          int32_t max_blocks_per_shard, int64_t n_blocks, int64_t* slot_mapping,
                          int32_t* err_flag, void* stream) {
  REQUIRE(block_table && context_lens && query_start && slot_mapping, PA_ERR_NULL,
          "pa_slot_mapping_multi: block_table, context_lens, query_start and slot_mapping must "
          "be non-NULL");
  REQUIRE(n_seqs >= 0 && n_rows >= 0, PA_ERR_SHAPE, "n_seqs=%d and n_rows=%d must be >= 0", n_seqs,
          n_rows);
  if (int rc = check_placement(n_shards, interleave, block_size)) return rc;
  REQUIRE(max_blocks_per_shard >= 1 && n_blocks >= 1, PA_ERR_SHAPE,
          "max_blocks_per_shard=%d and n_blocks=%lld must be >= 1", max_blocks_per_shard,
          (long long)n_blocks);
  if (n_seqs == 0) return ok();
  return hip_status(pa::launch_slot_mapping_multi(block_table, context_lens, query_start, n_seqs,
                                                  n_shards, interleave, block_size,
                                                  max_blocks_per_shard, n_blocks, n_rows,
                                                  slot_mapping, err_flag, (hipStream_t)stream),
                    "pa_slot_mapping_multi launch");
}

int pa_decode_multi(const void* q, int32_t q_dtype, const int32_t* query_start, int32_t n_rows,
                    int32_t max_q_len, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                    const float* k_scale, const float* v_scale, int32_t n_scales,
                    const int32_t* block_table, const int32_t* context_lens, int32_t n_seqs,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t dk, int32_t dv,
                    int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                    int32_t n_shards, int32_t interleave, int32_t partition_tokens,
                    int32_t max_partitions, float scale, float* part_out, float* part_lse,
                    int32_t* err_flag, void* stream) {
  pa::DecodeArgs a;
  if (int rc = check_decode("pa_decode_multi", q, k_cache, v_cache, block_table, context_lens,
                            n_seqs, n_q_heads, n_kv_heads, dk, dv, block_size, n_blocks,
                            max_blocks_per_shard, n_shards, interleave, partition_tokens,
                            max_partitions, scale, q_dtype, part_out, part_lse, err_flag, &a))
    return rc;
  REQUIRE(query_start != nullptr, PA_ERR_NULL, "pa_decode_multi: query_start must be non-NULL");
  REQUIRE(n_rows >= 0 && max_q_len >= 1, PA_ERR_SHAPE, "n_rows=%d must be >= 0 and max_q_len=%d >= 1",
          n_rows, max_q_len);
  REQUIRE(kv_dtype == q_dtype || kv_dtype == PA_FP8_E4M3, PA_ERR_UNSUPPORTED,
          "kv_dtype=%d must equal q_dtype=%d or be PA_FP8_E4M3", kv_dtype, q_dtype);
  if (kv_dtype == PA_FP8_E4M3) {
    REQUIRE(k_scale && (v_cache == nullptr || v_scale), PA_ERR_NULL,
            "pa_decode_multi: an E4M3 cache needs k_scale (and v_scale with a value cache)");
    REQUIRE(n_scales == 1 || n_scales == n_kv_heads, PA_ERR_SHAPE,
            "n_scales=%d must be 1 or n_kv_heads=%d", n_scales, n_kv_heads);
  }
  const int64_t g = n_q_heads / n_kv_heads;
  REQUIRE(int64_t(n_kv_heads) * ((int64_t(max_q_len) * g + 15) / 16) <= 65535, PA_ERR_SHAPE,
          "n_kv_heads * ceil(max_q_len * n_q_heads / n_kv_heads / 16) exceeds 65535");
  if (n_seqs == 0 || n_rows == 0) return ok();
  a.query_start = query_start;
  a.max_q = max_q_len;
  a.n_rows = n_rows;
  if (kv_dtype == PA_FP8_E4M3) {
    a.kv_dtype = PA_FP8_E4M3;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.n_scales = n_scales;
  }
  return hip_status(pa::dispatch_decode(a, (hipStream_t)stream), "pa_decode_multi launch");
}

int pa_merge_lse(const float* part_out, const float* part_lse, int32_t n_seqs, int32_t n_parts,
                 int32_t n_q_heads, int32_t dv, void* out, int32_t out_dtype, float* lse,
                 void* stream) {
  REQUIRE(part_out && part_lse && out, PA_ERR_NULL,
          "pa_merge_lse: part_out, part_lse and out must be non-NULL");
  REQUIRE(valid_dtype(out_dtype), PA_ERR_UNSUPPORTED, "out_dtype=%d is not PA_F32 or PA_BF16", out_dtype);
  REQUIRE(n_seqs >= 0 && n_parts >= 1 && n_q_heads >= 1, PA_ERR_SHAPE,
          "n_seqs=%d, n_parts=%d, n_q_heads=%d out of range", n_seqs, n_parts, n_q_heads);
  REQUIRE(dv >= 1 && dv <= 512, PA_ERR_UNSUPPORTED, "dv=%d must be in [1, 512]", dv);
  REQUIRE(int64_t(n_seqs) * n_q_heads <= 0x7fffffff, PA_ERR_SHAPE, "n_seqs*n_q_heads too large");
  if (n_seqs == 0) return ok();
  return hip_status(pa::launch_merge(part_out, part_lse, n_seqs, n_parts, n_q_heads, dv, out,
                                     out_dtype, lse, (hipStream_t)stream),
                    "pa_merge_lse launch");
}

int pa_gather_kv(const void* k_cache, const void* v_cache, const int32_t* block_table,
                 int32_t seq, int32_t shard, int32_t context_len, int32_t n_kv_heads, int32_t dk,
                 int32_t dv, int32_t block_size, int64_t n_blocks, int32_t max_blocks_per_shard,
                 int32_t n_shards, int32_t interleave, int32_t dtype, void* k_out, void* v_out,
                 int32_t* err_flag, void* stream) {
  REQUIRE(k_cache && block_table && k_out && v_out, PA_ERR_NULL,
          "pa_gather_kv: k_cache, block_table, k_out and v_out must be non-NULL");
  REQUIRE(valid_cache_dtype(dtype), PA_ERR_UNSUPPORTED,
          "dtype=%d is not PA_F32, PA_BF16 or PA_FP8_E4M3", dtype);
  if (int rc = check_placement(n_shards, interleave, block_size)) return rc;
  REQUIRE(seq >= 0 && shard >= 0 && shard < n_shards && context_len >= 0, PA_ERR_SHAPE,
          "seq=%d, shard=%d (n_shards=%d), context_len=%d out of range", seq, shard, n_shards,
          context_len);
  REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 65535, PA_ERR_SHAPE, "n_kv_heads=%d out of range", n_kv_heads);
  REQUIRE(dk >= 1 && dk <= PA_MAX_HEAD_DIM && dv >= 1 && dv <= PA_MAX_HEAD_DIM, PA_ERR_UNSUPPORTED,
          "dk=%d, dv=%d must be in [1, %d]", dk, dv, PA_MAX_HEAD_DIM);
  REQUIRE(v_cache != nullptr || dv <= dk, PA_ERR_SHAPE, "latent cache needs dv <= dk");
  REQUIRE(max_blocks_per_shard >= 1 && n_blocks >= 1, PA_ERR_SHAPE,
          "max_blocks_per_shard and n_blocks must be >= 1");
  const int L_r = pa::shard_len(context_len, n_shards, interleave, shard);
  if (L_r == 0) return ok();
  const int32_t* row = block_table + (int64_t(seq) * n_shards + shard) * max_blocks_per_shard;
  return hip_status(pa::launch_gather(k_cache, v_cache, row, L_r, n_kv_heads, dk, dv, block_size,
                                      n_blocks, max_blocks_per_shard, dtype, k_out, v_out,
                                      err_flag, (hipStream_t)stream),
                    "pa_gather_kv launch");
}

}  // extern "C"
