// block_pool.cpp -- host-side accounting of a pool of fixed-size KV blocks, the
// pa_pool_* entry points of include/pa.h.
//
// Follows the PagedAttention page (ai-compass.weeybrid.co.jp, "What is PagedAttention?"):
//  - block-table section: a sequence's tokens fill its last block while it has room; a
//    full (or missing) last block means a newly taken block appended to its table;
//  - "Reusing blocks freed when a request ends": a finished sequence hands its blocks
//    back; any sequence may take them next, nothing is moved or compacted;
//  - "Sharing common blocks and copy-on-write": a forked sequence points at its parent's
//    blocks; a per-block reference count keeps a block out of the free list while any
//    table lists it; a sequence about to write into a shared last block first takes a
//    new block, records (shared, new) as a block copy for the device, drops its
//    reference to the shared one and lists the new one instead;
//  - limits section: when the free blocks do not cover a request it has to wait, here
//    PA_ERR_EXHAUSTED with the pool unchanged.
// Free blocks are handed out oldest-freed first (a FIFO queue, initially 0..n-1).
#include <stdint.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "pa_error.h"

struct pa_block_pool {
  struct Seq {
    std::vector<int32_t> table;  // physical blocks in logical order
    int64_t length = 0;          // tokens stored
  };

  int32_t block_size = 0;
  std::deque<int32_t> free_blocks;
  std::vector<int32_t> refs;  // per physical block: tables that list it
  std::unordered_map<int64_t, Seq> seqs;

  void release(int32_t b) {
    if (--refs[b] == 0) free_blocks.push_back(b);
  }
  int32_t take() {
    const int32_t b = free_blocks.front();
    free_blocks.pop_front();
    refs[b] = 1;
    return b;
  }
};

namespace {

using pa::fail;
using pa::ok;

// Blocks an append of n tokens to `s` takes from the free list: one copy of a shared,
// partly filled last block, plus the new blocks for the tokens its room cannot hold.
struct AppendPlan {
  bool copy_last;
  int64_t new_blocks;
};

AppendPlan plan_append(const pa_block_pool& p, const pa_block_pool::Seq& s, int64_t n) {
  AppendPlan plan{false, 0};
  if (n == 0) return plan;
  const int64_t bs = p.block_size;
  const int64_t capacity = int64_t(s.table.size()) * bs;
  const int64_t room = capacity - s.length;
  if (room > 0 && p.refs[s.table.back()] > 1) plan.copy_last = true;
  const int64_t beyond = n - room;
  if (beyond > 0) plan.new_blocks = (beyond + bs - 1) / bs;
  return plan;
}

int do_append(pa_block_pool* p, pa_block_pool::Seq& s, int64_t n, int64_t* copies,
              int32_t max_copies, int32_t* n_copies) {
  const AppendPlan plan = plan_append(*p, s, n);
  const int64_t needed = plan.new_blocks + (plan.copy_last ? 1 : 0);
  if (needed > int64_t(p->free_blocks.size()))
    return fail(PA_ERR_EXHAUSTED, "pa_pool: %lld free blocks, the request needs %lld",
                (long long)p->free_blocks.size(), (long long)needed);
  if (plan.copy_last && (copies == nullptr || max_copies < 1))
    return fail(PA_ERR_BUFFER, "pa_pool_append: a copy-on-write copy needs room in `copies`");
  int32_t made = 0;
  if (plan.copy_last) {
    const int32_t shared = s.table.back();
    const int32_t mine = p->take();
    copies[0] = shared;
    copies[1] = mine;
    made = 1;
    p->release(shared);
    s.table.back() = mine;
  }
  for (int64_t i = 0; i < plan.new_blocks; ++i) s.table.push_back(p->take());
  s.length += n;
  if (n_copies != nullptr) *n_copies = made;
  return ok();
}

}  // namespace

extern "C" {

pa_block_pool* pa_pool_create(int64_t n_blocks, int32_t block_size) {
  if (n_blocks < 0 || n_blocks > INT32_MAX || block_size < 1) {
    fail(PA_ERR_SHAPE, "pa_pool_create: n_blocks=%lld must be in [0, 2^31-1], block_size=%d >= 1",
         (long long)n_blocks, block_size);
    return nullptr;
  }
  pa_block_pool* p = new (std::nothrow) pa_block_pool;
  if (p == nullptr) return nullptr;
  try {
    p->block_size = block_size;
    p->refs.assign(size_t(n_blocks), 0);
    for (int64_t b = 0; b < n_blocks; ++b) p->free_blocks.push_back(int32_t(b));
  } catch (const std::bad_alloc&) {
    delete p;
    fail(PA_ERR_SHAPE, "pa_pool_create: out of host memory");
    return nullptr;
  }
  ok();
  return p;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int pa_pool_add(pa_block_pool* pool, int64_t seq, int64_t n_tokens) {
  if (pool == nullptr) return fail(PA_ERR_NULL, "pa_pool_add: pool is NULL");
  if (n_tokens < 0) return fail(PA_ERR_SHAPE, "pa_pool_add: n_tokens=%lld < 0", (long long)n_tokens);
  if (pool->seqs.count(seq)) return fail(PA_ERR_SEQUENCE, "pa_pool_add: sequence %lld exists", (long long)seq);
  pa_block_pool::Seq s;
  // A new table shares nothing, so no copy can arise.
  const int rc = do_append(pool, s, n_tokens, nullptr, 0, nullptr);
  if (rc != PA_OK) return rc;
  pool->seqs.emplace(seq, std::move(s));
  return ok();
}

int pa_pool_append(pa_block_pool* pool, int64_t seq, int64_t n_tokens, int64_t* copies,
                   int32_t max_copies, int32_t* n_copies) {
  if (pool == nullptr) return fail(PA_ERR_NULL, "pa_pool_append: pool is NULL");
  if (n_tokens < 0) return fail(PA_ERR_SHAPE, "pa_pool_append: n_tokens=%lld < 0", (long long)n_tokens);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ERR_SEQUENCE, "pa_pool_append: no sequence %lld", (long long)seq);
  if (n_copies != nullptr) *n_copies = 0;
  return do_append(pool, it->second, n_tokens, copies, max_copies, n_copies);
}

int pa_pool_fork(pa_block_pool* pool, int64_t parent, int64_t child) {
  if (pool == nullptr) return fail(PA_ERR_NULL, "pa_pool_fork: pool is NULL");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return fail(PA_ERR_SEQUENCE, "pa_pool_fork: no sequence %lld", (long long)parent);
  if (pool->seqs.count(child)) return fail(PA_ERR_SEQUENCE, "pa_pool_fork: sequence %lld exists", (long long)child);
  pa_block_pool::Seq s = it->second;
  for (int32_t b : s.table) ++pool->refs[b];
  pool->seqs.emplace(child, std::move(s));
  return ok();
}

int pa_pool_finish(pa_block_pool* pool, int64_t seq) {
  if (pool == nullptr) return fail(PA_ERR_NULL, "pa_pool_finish: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ERR_SEQUENCE, "pa_pool_finish: no sequence %lld", (long long)seq);
  for (int32_t b : it->second.table) pool->release(b);
  pool->seqs.erase(it);
  return ok();
}

int64_t pa_pool_num_free(const pa_block_pool* pool) {
  return pool == nullptr ? -1 : int64_t(pool->free_blocks.size());
}

int64_t pa_pool_length(const pa_block_pool* pool, int64_t seq) {
  if (pool == nullptr) return -1;
  auto it = pool->seqs.find(seq);
  return it == pool->seqs.end() ? -1 : it->second.length;
}

int64_t pa_pool_num_blocks(const pa_block_pool* pool, int64_t seq) {
  if (pool == nullptr) return -1;
  auto it = pool->seqs.find(seq);
  return it == pool->seqs.end() ? -1 : int64_t(it->second.table.size());
}

int32_t pa_pool_refcount(const pa_block_pool* pool, int64_t block) {
  if (pool == nullptr || block < 0 || block >= int64_t(pool->refs.size())) return -1;
  return pool->refs[size_t(block)];
}

int64_t pa_pool_table(const pa_block_pool* pool, int64_t seq, int32_t* table, int64_t capacity) {
  if (pool == nullptr) return -1;
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return -1;
  const std::vector<int32_t>& t = it->second.table;
  if (int64_t(t.size()) > capacity || (table == nullptr && !t.empty())) return -1;
  for (size_t j = 0; j < t.size(); ++j) table[j] = t[j];
  return int64_t(t.size());
}

}  // extern "C"
