// Host-side KV block manager behind the pkv_pool / pkv_seq_* / pkv_block_*
// entry points of include/pagedkv.h.
//
// The pool is a flat set of fixed 16-token blocks; a sequence is a block table
// plus a length; a new block is taken only when the sequence's current block
// is full, and a finished sequence returns its blocks [KV Cache 工程学 §15.5].
// Blocks are shared between tables by reference count, which is how parallel
// samples and common prompts are stored once [新一代 KV Cache 管理 §8.1];
// writing into a shared block copies it first [KV Cache 与 PagedAttention,
// first article].  Batch appends are all-or-nothing: every mutation is logged
// and undone in reverse order when the free pool runs dry part-way.
//
// Plain C++17 with no HIP dependency, so it also builds with the host
// compiler and its sanitizers.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

int pkv_set_error(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

extern "C" const char *pkv_last_error(void) { return g_last_error.c_str(); }
extern "C" const char *pkv_version(void) { return "pagedkv 0.1 gfx950"; }

int pkv_check_layout(const pkv_layout *L) {
  if (!L) return pkv_set_error(PKV_ERR_INVALID, "layout is NULL");
  if (L->num_blocks <= 0) return pkv_set_error(PKV_ERR_INVALID, "num_blocks must be > 0 (got %d)", L->num_blocks);
  if (L->block_size != PKV_BLOCK_SIZE)
    return pkv_set_error(PKV_ERR_INVALID, "block_size must be 16 (got %d)", L->block_size);
  if (L->num_kv_heads <= 0) return pkv_set_error(PKV_ERR_INVALID, "num_kv_heads must be > 0");
  if (L->head_dim != 64 && L->head_dim != 128)
    return pkv_set_error(PKV_ERR_INVALID, "head_dim must be 64 or 128 (got %d)", L->head_dim);
  if (L->kv_dtype != PKV_F32 && L->kv_dtype != PKV_BF16 && L->kv_dtype != PKV_INT8 && L->kv_dtype != PKV_FP8)
    return pkv_set_error(PKV_ERR_INVALID, "kv_dtype must be PKV_F32, PKV_BF16, PKV_INT8 or PKV_FP8");
  return PKV_OK;
}

struct pkv_pool {
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  pkv_layout layout{};
  std::vector<int32_t> free_stack;  // top is back()
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;

  // Prefix cache [KV Cache 工程学 §15.6; 新一代 KV Cache 管理 §8.3]: a full
  // block is keyed by a hash of the whole prefix that ends with it, so the
  // same block content after a different prefix never matches.  A cached
  // block whose reference count drops to zero stays cached ("idle") in an LRU
  // list and is evicted only when the free stack is empty.
  struct CacheEntry {
    uint64_t key, parent;            // chain hash of this block and of the one before
    int32_t tok[PKV_BLOCK_SIZE];     // the block's token ids (checked on a hit)
  };
  bool pc_on = false;
  std::vector<CacheEntry> pc;        // per block, meaningful while cached[b]
  std::vector<uint8_t> cached;
  std::unordered_map<uint64_t, int32_t> pc_map;
  std::vector<int32_t> lru_prev, lru_next;  // idle cached blocks, oldest at lru_head
  int32_t lru_head = -1, lru_tail = -1, n_idle = 0;
  pkv_prefix_stats pst{};

  // Swap to host memory ("fine-grained eviction" [KV Cache 与
  // PagedAttention, summary]; Clock replacement [PagedAttention：大模型KV
  // Cache内存管理革新 §3.3]).  A table entry e < 0 names host slot -e-1.
  // refbit is the Clock reference bit of each device block: set when the
  // block is taken, written, or named in an exported table.
  mutable std::vector<uint8_t> refbit;
  int32_t hand = 0;
  int32_t num_host = 0;
  std::vector<int32_t> host_free;  // top is back()
  std::vector<int32_t> host_ref;
  int64_t swapped_out = 0, swapped_in = 0;

  // Undo log of one all-or-nothing operation.
  enum class Op { Alloc, AllocEvict, TablePush, CowSwap, Len, RefBit };
  struct Undo {
    Op op;
    int64_t seq;
    int32_t a, b;
  };
  std::vector<Undo> log;

  bool valid_block(int32_t b) const { return b >= 0 && b < layout.num_blocks; }
  static bool resident(const Seq &s) {
    for (int32_t e : s.table)
      if (e < 0) return false;
    return true;
  }

  int32_t available() const { return (int32_t)free_stack.size() + n_idle; }

  void lru_unlink(int32_t b) {
    const int32_t p = lru_prev[b], n = lru_next[b];
    (p >= 0 ? lru_next[p] : lru_head) = n;
    (n >= 0 ? lru_prev[n] : lru_tail) = p;
    lru_prev[b] = lru_next[b] = -1;
    --n_idle;
  }
  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    (lru_tail >= 0 ? lru_next[lru_tail] : lru_head) = b;
    lru_tail = b;
    ++n_idle;
  }
  void lru_push_front(int32_t b) {
    lru_next[b] = lru_head;
    lru_prev[b] = -1;
    (lru_head >= 0 ? lru_prev[lru_head] : lru_tail) = b;
    lru_head = b;
    ++n_idle;
  }

  // Take a block: the top of the free stack, else the least recently used
  // idle cached block, which leaves the cache.  *evicted tells which.
  int take(int32_t *out, bool *evicted) {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
      *evicted = false;
    } else if (lru_head >= 0) {
      b = lru_head;
      lru_unlink(b);
      pc_map.erase(pc[b].key);
      cached[b] = 0;
      ++pst.evictions;
      *evicted = true;
    } else {
      return pkv_set_error(PKV_ERR_NO_BLOCKS, "no free blocks (pool of %d)", layout.num_blocks);
    }
    ref[b] = 1;
    refbit[b] = 1;
    *out = b;
    return PKV_OK;
  }
  int alloc(int32_t *out) {
    bool ev;
    return take(out, &ev);
  }
  // Reference count reached zero: back to the free stack, or idle in the cache.
  void release(int32_t b) {
    if (cached[b])
      lru_push_back(b);
    else
      free_stack.push_back(b);
  }
  // Undo of an eviction by take(): the block is cached and the oldest idle again.
  void unevict(int32_t b) {
    ref[b] = 0;
    cached[b] = 1;
    pc_map[pc[b].key] = b;
    lru_push_front(b);
    --pst.evictions;
  }

  void rollback() {
    for (auto it = log.rbegin(); it != log.rend(); ++it) {
      switch (it->op) {
        case Op::Alloc:  // popped from the top: push back on top
          ref[it->a] = 0;
          free_stack.push_back(it->a);
          break;
        case Op::AllocEvict:
          unevict(it->a);
          break;
        case Op::TablePush:
          seqs[it->seq].table.pop_back();
          break;
        case Op::CowSwap:  // table tail went a -> b and a lost one reference
          seqs[it->seq].table.back() = it->a;
          ref[it->a] += 1;
          break;
        case Op::Len:
          seqs[it->seq].len = it->a;
          break;
        case Op::RefBit:
          refbit[it->a] = (uint8_t)it->b;
          break;
      }
    }
    log.clear();
  }

  // Append n tokens to one sequence, logging every change.
  int append_one(int64_t id, int32_t n, int64_t *slots, int32_t *cow, int32_t cow_cap, int32_t *n_cow) {
    Seq &s = seqs[id];
    for (int32_t k = 0; k < n; ++k) {
      int32_t pos = s.len;
      if (pos % PKV_BLOCK_SIZE == 0) {
        int32_t b;
        bool ev;
        if (int rc = take(&b, &ev)) return rc;
        log.push_back({ev ? Op::AllocEvict : Op::Alloc, id, b, 0});
        s.table.push_back(b);
        log.push_back({Op::TablePush, id, 0, 0});
      } else if (ref[s.table.back()] > 1) {
        if (*n_cow >= cow_cap)
          return pkv_set_error(PKV_ERR_CAPACITY, "copy-on-write pair buffer too small (cap %d)", cow_cap);
        int32_t old = s.table.back(), b;
        bool ev;
        if (int rc = take(&b, &ev)) return rc;
        log.push_back({ev ? Op::AllocEvict : Op::Alloc, id, b, 0});
        ref[old] -= 1;  // stays >= 1: another table still holds it
        s.table.back() = b;
        log.push_back({Op::CowSwap, id, old, b});
        cow[2 * *n_cow] = old;
        cow[2 * *n_cow + 1] = b;
        ++*n_cow;
      }
      const int32_t blk = s.table[pos / PKV_BLOCK_SIZE];
      log.push_back({Op::RefBit, id, blk, refbit[blk]});
      refbit[blk] = 1;
      slots[k] = (int64_t)blk * PKV_BLOCK_SIZE + pos % PKV_BLOCK_SIZE;
      log.push_back({Op::Len, id, pos, 0});
      s.len = pos + 1;
    }
    return PKV_OK;
  }
};

namespace {
int need_pool(const pkv_pool *p) { return p ? PKV_OK : pkv_set_error(PKV_ERR_INVALID, "pool is NULL"); }
}  // namespace

extern "C" int pkv_pool_create(const pkv_layout *layout, const int32_t *free_order, pkv_pool **out) {
  if (int rc = pkv_check_layout(layout)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  const int32_t n = layout->num_blocks;
  std::vector<int32_t> order(n);
  if (free_order) {
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= n || seen[b])
        return pkv_set_error(PKV_ERR_INVALID, "free_order is not a permutation of [0, %d)", n);
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < n; ++i) order[i] = i;
  }
  pkv_pool *p = new (std::nothrow) pkv_pool();
  if (!p) return pkv_set_error(PKV_ERR_INVALID, "out of host memory");
  p->layout = *layout;
  p->free_stack.assign(order.rbegin(), order.rend());  // first hand-out = order[0]
  p->ref.assign(n, 0);
  p->pc.resize(n);
  p->cached.assign(n, 0);
  p->lru_prev.assign(n, -1);
  p->lru_next.assign(n, -1);
  p->refbit.assign(n, 0);
  *out = p;
  return PKV_OK;
}

extern "C" int pkv_pool_destroy(pkv_pool *pool) {
  delete pool;
  return PKV_OK;
}

extern "C" int pkv_block_alloc(pkv_pool *pool, int32_t *block_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!block_out) return pkv_set_error(PKV_ERR_INVALID, "block_out is NULL");
  return pool->alloc(block_out);
}

extern "C" int pkv_block_incref(pkv_pool *pool, int32_t block) {
  if (int rc = need_pool(pool)) return rc;
  if (!pool->valid_block(block)) return pkv_set_error(PKV_ERR_BAD_BLOCK, "block %d out of range", block);
  if (pool->ref[block] <= 0) return pkv_set_error(PKV_ERR_REFCOUNT, "incref of free block %d", block);
  pool->ref[block] += 1;
  return PKV_OK;
}

extern "C" int pkv_block_free(pkv_pool *pool, int32_t block) {
  if (int rc = need_pool(pool)) return rc;
  if (!pool->valid_block(block)) return pkv_set_error(PKV_ERR_BAD_BLOCK, "block %d out of range", block);
  if (pool->ref[block] <= 0) return pkv_set_error(PKV_ERR_REFCOUNT, "free of free block %d", block);
  if (--pool->ref[block] == 0) pool->release(block);
  return PKV_OK;
}

extern "C" int pkv_block_refcount(const pkv_pool *pool, int32_t block, int32_t *out) {
  if (int rc = need_pool(pool)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  if (!pool->valid_block(block)) return pkv_set_error(PKV_ERR_BAD_BLOCK, "block %d out of range", block);
  *out = pool->ref[block];
  return PKV_OK;
}

extern "C" int pkv_pool_num_free(const pkv_pool *pool, int32_t *out) {
  if (int rc = need_pool(pool)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  *out = pool->available();
  return PKV_OK;
}

extern "C" int pkv_seq_create(pkv_pool *pool, int64_t *id_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!id_out) return pkv_set_error(PKV_ERR_INVALID, "id_out is NULL");
  int64_t id = pool->next_id++;
  pool->seqs.emplace(id, pkv_pool::Seq{});
  *id_out = id;
  return PKV_OK;
}

extern "C" int pkv_seq_fork(pkv_pool *pool, int64_t parent, int64_t *child_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!child_out) return pkv_set_error(PKV_ERR_INVALID, "child_out is NULL");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)parent);
  pkv_pool::Seq child = it->second;  // copy before inserting (rehash safety)
  for (int32_t b : child.table)
    if (b >= 0 && pool->ref[b] <= 0)
      return pkv_set_error(PKV_ERR_REFCOUNT, "fork of sequence %lld holding free block %d", (long long)parent, b);
  for (int32_t b : child.table) {
    if (b >= 0)
      pool->ref[b] += 1;
    else
      pool->host_ref[-b - 1] += 1;
  }
  int64_t id = pool->next_id++;
  pool->seqs.emplace(id, std::move(child));
  *child_out = id;
  return PKV_OK;
}

extern "C" int pkv_batch_append_slots(pkv_pool *pool, const int64_t *ids, int32_t num_seqs, int32_t n,
                                      int64_t *slots_out, int32_t *cow_pairs_out, int32_t cow_cap,
                                      int32_t *n_cow) {
  if (int rc = need_pool(pool)) return rc;
  if (num_seqs < 0 || n < 0) return pkv_set_error(PKV_ERR_INVALID, "negative count");
  if (num_seqs > 0 && !ids) return pkv_set_error(PKV_ERR_INVALID, "ids is NULL");
  if ((int64_t)num_seqs * n > 0 && !slots_out) return pkv_set_error(PKV_ERR_INVALID, "slots_out is NULL");
  if (cow_cap < 0 || (cow_cap > 0 && !cow_pairs_out)) return pkv_set_error(PKV_ERR_INVALID, "bad cow buffer");
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!pool->seqs.count(ids[i])) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)ids[i]);
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!pkv_pool::resident(pool->seqs[ids[i]]))
      return pkv_set_error(PKV_ERR_INVALID, "sequence %lld has blocks swapped out; swap it in first",
                           (long long)ids[i]);
  int32_t ncow = 0;
  pool->log.clear();
  for (int32_t i = 0; i < num_seqs; ++i) {
    int rc = pool->append_one(ids[i], n, slots_out + (int64_t)i * n, cow_pairs_out, cow_cap, &ncow);
    if (rc) {
      pool->rollback();
      return rc;
    }
  }
  pool->log.clear();
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
}

extern "C" int pkv_seq_append_slots(pkv_pool *pool, int64_t id, int32_t n, int64_t *slots_out,
                                    int32_t *cow_pairs_out, int32_t cow_cap, int32_t *n_cow) {
  return pkv_batch_append_slots(pool, &id, 1, n, slots_out, cow_pairs_out, cow_cap, n_cow);
}

extern "C" int pkv_seq_free(pkv_pool *pool, int64_t id) {
  if (int rc = need_pool(pool)) return rc;
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  // All or nothing: every block must have at least as many references as
  // the table holds it (a caller that freed a block the sequence still held
  // can make it appear twice).
  std::unordered_map<int32_t, int32_t> held;
  for (int32_t b : it->second.table)
    if (b >= 0) ++held[b];
  for (const auto &kv : held)
    if (pool->ref[kv.first] < kv.second)
      return pkv_set_error(PKV_ERR_REFCOUNT, "free of sequence %lld holding block %d %d times, refcount %d",
                           (long long)id, kv.first, kv.second, pool->ref[kv.first]);
  // Blocks reaching zero go back in table order; cached ones turn idle
  // deepest first, so that of a prefix released together the tail is
  // evicted before the head (a cached block is only reachable through its
  // prefix).
  std::vector<int32_t> idle;
  for (int32_t b : it->second.table) {
    if (b < 0) {  // a host entry
      if (--pool->host_ref[-b - 1] == 0) pool->host_free.push_back(-b - 1);
      continue;
    }
    if (--pool->ref[b] == 0) {
      if (pool->cached[b])
        idle.push_back(b);
      else
        pool->free_stack.push_back(b);
    }
  }
  for (auto r = idle.rbegin(); r != idle.rend(); ++r) pool->lru_push_back(*r);
  pool->seqs.erase(it);
  return PKV_OK;
}

extern "C" int pkv_seq_len(const pkv_pool *pool, int64_t id, int32_t *len_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!len_out) return pkv_set_error(PKV_ERR_INVALID, "len_out is NULL");
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  *len_out = it->second.len;
  return PKV_OK;
}

extern "C" int pkv_seq_block_table(const pkv_pool *pool, int64_t id, int32_t *out, int32_t cap, int32_t *n_out) {
  if (int rc = need_pool(pool)) return rc;
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  const auto &t = it->second.table;
  if (n_out) *n_out = (int32_t)t.size();
  if ((int32_t)t.size() > cap) return pkv_set_error(PKV_ERR_CAPACITY, "table of %zu entries, cap %d", t.size(), cap);
  if (!t.empty() && !out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  std::copy(t.begin(), t.end(), out);
  return PKV_OK;
}

extern "C" int pkv_batch_block_tables(const pkv_pool *pool, const int64_t *ids, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int32_t *tables_out, int32_t *context_lens_out) {
  if (int rc = need_pool(pool)) return rc;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return pkv_set_error(PKV_ERR_INVALID, "negative count");
  if (num_seqs > 0 && (!ids || !context_lens_out || (max_blocks_per_seq > 0 && !tables_out)))
    return pkv_set_error(PKV_ERR_INVALID, "NULL argument");
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = pool->seqs.find(ids[i]);
    if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)ids[i]);
    if ((int32_t)it->second.table.size() > max_blocks_per_seq)
      return pkv_set_error(PKV_ERR_CAPACITY, "sequence %lld holds %zu blocks > %d", (long long)ids[i],
                           it->second.table.size(), max_blocks_per_seq);
    if (!pkv_pool::resident(it->second))
      return pkv_set_error(PKV_ERR_INVALID, "sequence %lld has blocks swapped out; swap it in first",
                           (long long)ids[i]);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto &s = pool->seqs.find(ids[i])->second;
    int32_t *row = tables_out + (int64_t)i * max_blocks_per_seq;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks_per_seq, 0);
    context_lens_out[i] = s.len;
    for (int32_t b : s.table) pool->refbit[b] = 1;
  }
  return PKV_OK;
}

extern "C" int pkv_pool_stats(const pkv_pool *pool, pkv_stats *out) {
  if (int rc = need_pool(pool)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  const int32_t n = pool->layout.num_blocks;
  std::vector<int32_t> fill(n, 0);
  int64_t logical = 0;
  for (const auto &kv : pool->seqs) {
    const auto &s = kv.second;
    logical += s.len;
    for (size_t j = 0; j < s.table.size(); ++j) {
      if (s.table[j] < 0) continue;  // on the host
      int32_t f = std::min<int32_t>(PKV_BLOCK_SIZE, s.len - (int32_t)j * PKV_BLOCK_SIZE);
      fill[s.table[j]] = std::max(fill[s.table[j]], f);
    }
  }
  int64_t stored = 0;
  int32_t shared = 0;
  for (int32_t b = 0; b < n; ++b) {
    stored += fill[b];
    shared += pool->ref[b] > 1;
  }
  out->num_blocks = n;
  out->num_free = pool->available();
  out->num_used = n - out->num_free;
  out->num_shared = shared;
  out->num_seqs = (int64_t)pool->seqs.size();
  out->tokens_logical = logical;
  out->tokens_stored = stored;
  out->usage = (double)out->num_used / n;
  out->internal_fragmentation = out->num_used ? 1.0 - (double)stored / ((double)out->num_used * PKV_BLOCK_SIZE) : 0.0;
  return PKV_OK;
}

extern "C" int64_t pkv_kv_bytes_per_token(const pkv_layout *layout, int32_t num_layers) {
  if (pkv_check_layout(layout) || num_layers < 0) return 0;
  return (int64_t)num_layers * 2 * layout->num_kv_heads * pkv_row_bytes(layout);
}

extern "C" int64_t pkv_pool_bytes(const pkv_layout *layout) {
  if (pkv_check_layout(layout)) return 0;
  return (int64_t)layout->num_blocks * layout->num_kv_heads * pkv_tile_bytes(layout);
}

extern "C" int pkv_validate_tables(const pkv_layout *layout, const int32_t *tables, const int32_t *context_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq) {
  if (int rc = pkv_check_layout(layout)) return rc;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return pkv_set_error(PKV_ERR_INVALID, "negative count");
  if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !tables)))
    return pkv_set_error(PKV_ERR_INVALID, "NULL argument");
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t n = context_lens[i];
    if (n < 0 || (int64_t)n > (int64_t)PKV_BLOCK_SIZE * max_blocks_per_seq)
      return pkv_set_error(PKV_ERR_INVALID, "sequence %d: length %d outside [0, %d]", i, n,
                           PKV_BLOCK_SIZE * max_blocks_per_seq);
    int32_t nb = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    for (int32_t j = 0; j < nb; ++j) {
      int32_t b = tables[(int64_t)i * max_blocks_per_seq + j];
      if (b < 0 || b >= layout->num_blocks)
        return pkv_set_error(PKV_ERR_BAD_BLOCK, "sequence %d entry %d: block %d out of range", i, j, b);
    }
  }
  return PKV_OK;
}

// ------------------------------------------------------------- prefix cache
namespace {

// FNV-1a, 64-bit (offset basis 14695981039346656037, prime 1099511628211),
// over the little-endian bytes of the previous block's key followed by the
// block's 16 token ids: the key of block i covers tokens [0, 16 (i + 1)).
uint64_t fnv1a_block(uint64_t parent, const int32_t *tok) {
  uint64_t h = 14695981039346656037ull;
  auto feed = [&h](uint8_t byte) {
    h ^= byte;
    h *= 1099511628211ull;
  };
  for (int k = 0; k < 8; ++k) feed((uint8_t)(parent >> (8 * k)));
  for (int t = 0; t < PKV_BLOCK_SIZE; ++t)
    for (int k = 0; k < 4; ++k) feed((uint8_t)((uint32_t)tok[t] >> (8 * k)));
  return h;
}

// The cached block of (parent key, tokens), or -1.
int32_t lookup(const pkv_pool *p, uint64_t parent, const int32_t *tok, uint64_t *key_out) {
  const uint64_t key = fnv1a_block(parent, tok);
  *key_out = key;
  auto it = p->pc_map.find(key);
  if (it == p->pc_map.end()) return -1;
  const auto &e = p->pc[it->second];
  if (e.parent != parent || !std::equal(tok, tok + PKV_BLOCK_SIZE, e.tok)) return -1;
  return it->second;
}

}  // namespace

extern "C" int pkv_prefix_cache_enable(pkv_pool *pool, int32_t enable) {
  if (int rc = need_pool(pool)) return rc;
  if (!enable && pool->pc_on) {
    // Idle cached blocks return to the free stack (oldest first); blocks in
    // use simply stop being cached.
    while (pool->lru_head >= 0) {
      const int32_t b = pool->lru_head;
      pool->lru_unlink(b);
      pool->free_stack.push_back(b);
    }
    std::fill(pool->cached.begin(), pool->cached.end(), 0);
    pool->pc_map.clear();
  }
  pool->pc_on = enable != 0;
  return PKV_OK;
}

extern "C" int pkv_seq_create_from_prefix(pkv_pool *pool, const int32_t *token_ids, int32_t n, int64_t *id_out,
                                          int32_t *n_cached_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!id_out || !n_cached_out || n < 0 || (n > 0 && !token_ids))
    return pkv_set_error(PKV_ERR_INVALID, "bad arguments");
  pkv_pool::Seq s;
  if (pool->pc_on) {
    uint64_t parent = 0;
    for (int32_t i = 0; i + 1 <= n / PKV_BLOCK_SIZE; ++i) {
      uint64_t key;
      const int32_t b = lookup(pool, parent, token_ids + (int64_t)i * PKV_BLOCK_SIZE, &key);
      if (b < 0) break;
      if (pool->ref[b] == 0) pool->lru_unlink(b);
      ++pool->ref[b];
      s.table.push_back(b);
      s.len += PKV_BLOCK_SIZE;
      parent = key;
    }
    ++pool->pst.lookups;
    pool->pst.query_tokens += n / PKV_BLOCK_SIZE * PKV_BLOCK_SIZE;
    pool->pst.hit_tokens += s.len;
  }
  const int64_t id = pool->next_id++;
  *n_cached_out = s.len;
  pool->seqs.emplace(id, std::move(s));
  *id_out = id;
  return PKV_OK;
}

extern "C" int pkv_seq_register_prefix(pkv_pool *pool, int64_t id, const int32_t *token_ids, int32_t n,
                                       int32_t *n_registered) {
  if (int rc = need_pool(pool)) return rc;
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  if (n < 0 || (n > 0 && !token_ids)) return pkv_set_error(PKV_ERR_INVALID, "bad arguments");
  const auto &s = it->second;
  if (n > s.len) return pkv_set_error(PKV_ERR_INVALID, "register of %d tokens, sequence holds %d", n, s.len);
  int32_t added = 0;
  if (pool->pc_on) {
    uint64_t parent = 0;
    for (int32_t i = 0; i + 1 <= n / PKV_BLOCK_SIZE; ++i) {
      const int32_t *tok = token_ids + (int64_t)i * PKV_BLOCK_SIZE;
      uint64_t key;
      const int32_t b = s.table[i];
      if (b < 0) break;  // swapped out: the cache names device blocks only
      const int32_t hit = lookup(pool, parent, tok, &key);
      // Content already cached (maybe in another block), or this block
      // already cached under its own prefix: leave the cache as it is.
      if (hit < 0 && !pool->cached[b] && !pool->pc_map.count(key)) {
        auto &e = pool->pc[b];
        e.key = key;
        e.parent = parent;
        std::copy(tok, tok + PKV_BLOCK_SIZE, e.tok);
        pool->cached[b] = 1;
        pool->pc_map.emplace(key, b);
        ++added;
      }
      parent = key;
    }
    pool->pst.registered += added;
  }
  if (n_registered) *n_registered = added;
  return PKV_OK;
}

extern "C" int pkv_prefix_cache_stats(const pkv_pool *pool, pkv_prefix_stats *out) {
  if (int rc = need_pool(pool)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  *out = pool->pst;
  out->cached_blocks = (int32_t)pool->pc_map.size();
  out->idle_blocks = pool->n_idle;
  out->hit_rate = out->query_tokens ? (double)out->hit_tokens / (double)out->query_tokens : 0.0;
  return PKV_OK;
}

// ------------------------------------------------------------ host swap
extern "C" int pkv_swap_configure(pkv_pool *pool, int32_t num_host_blocks) {
  if (int rc = need_pool(pool)) return rc;
  if (num_host_blocks < 0) return pkv_set_error(PKV_ERR_INVALID, "num_host_blocks < 0");
  for (int32_t r : pool->host_ref)
    if (r > 0) return pkv_set_error(PKV_ERR_INVALID, "host slots still hold swapped-out blocks");
  pool->num_host = num_host_blocks;
  pool->host_ref.assign(num_host_blocks, 0);
  pool->host_free.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) pool->host_free[i] = num_host_blocks - 1 - i;  // slot 0 first
  return PKV_OK;
}

extern "C" int pkv_swap_out(pkv_pool *pool, int32_t want, const int64_t *protect_ids, int32_t n_protect,
                            int32_t *pairs_out, int32_t cap, int32_t *n_out) {
  if (int rc = need_pool(pool)) return rc;
  if (want < 0 || n_protect < 0 || cap < 0) return pkv_set_error(PKV_ERR_INVALID, "negative count");
  if ((n_protect > 0 && !protect_ids) || (want > 0 && !pairs_out) || !n_out)
    return pkv_set_error(PKV_ERR_INVALID, "NULL argument");
  if (want > cap) return pkv_set_error(PKV_ERR_CAPACITY, "want %d blocks, pair buffer holds %d", want, cap);
  std::vector<uint8_t> guarded(pool->layout.num_blocks, 0), named(pool->layout.num_blocks, 0);
  std::vector<int32_t> entries(pool->layout.num_blocks, 0);
  for (const auto &kv : pool->seqs)
    for (int32_t b : kv.second.table)
      if (b >= 0) ++entries[b];
  // Candidates: blocks named by some table whose every reference is a table
  // entry; a block the caller also holds (pkv_block_alloc / incref) stays,
  // so the caller's id keeps naming it.
  for (int32_t b = 0; b < pool->layout.num_blocks; ++b) named[b] = entries[b] > 0 && entries[b] == pool->ref[b];
  for (int32_t i = 0; i < n_protect; ++i) {
    auto it = pool->seqs.find(protect_ids[i]);
    if (it == pool->seqs.end())
      return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)protect_ids[i]);
    for (int32_t b : it->second.table)
      if (b >= 0) guarded[b] = 1;
  }
  // Clock: the hand passes over device blocks from where it last stopped; a
  // candidate with its reference bit set gets a second chance.
  const int32_t N = pool->layout.num_blocks;
  int32_t got = 0;
  std::vector<int32_t> remap;  // device block -> its host entry, for the victims
  for (int64_t examined = 0; got < want && !pool->host_free.empty() && examined < 2 * (int64_t)N; ++examined) {
    const int32_t b = pool->hand;
    pool->hand = (pool->hand + 1) % N;
    if (!named[b] || pool->cached[b] || guarded[b]) continue;
    if (pool->refbit[b]) {
      pool->refbit[b] = 0;
      continue;
    }
    const int32_t slot = pool->host_free.back();
    pool->host_free.pop_back();
    pool->host_ref[slot] = pool->ref[b];
    if (remap.empty()) remap.assign(N, 0);
    remap[b] = -slot - 1;
    named[b] = 0;  // free now: a second turn of the hand passes it over
    pool->ref[b] = 0;
    pool->free_stack.push_back(b);
    pairs_out[2 * got] = b;
    pairs_out[2 * got + 1] = slot;
    ++got;
  }
  if (got)  // every table entry naming a victim now names its host slot
    for (auto &kv : pool->seqs)
      for (int32_t &e : kv.second.table)
        if (e >= 0 && remap[e] < 0) e = remap[e];
  pool->swapped_out += got;
  *n_out = got;
  return PKV_OK;
}

extern "C" int pkv_seq_swap_in(pkv_pool *pool, int64_t id, int32_t *pairs_out, int32_t cap, int32_t *n_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!n_out || cap < 0 || (cap > 0 && !pairs_out)) return pkv_set_error(PKV_ERR_INVALID, "bad arguments");
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  std::vector<int32_t> slots;  // distinct host entries in table order
  for (int32_t e : it->second.table)
    if (e < 0 && std::find(slots.begin(), slots.end(), -e - 1) == slots.end()) slots.push_back(-e - 1);
  *n_out = (int32_t)slots.size();
  if ((int32_t)slots.size() > cap)
    return pkv_set_error(PKV_ERR_CAPACITY, "%zu blocks to swap in, pair buffer holds %d", slots.size(), cap);
  if ((int32_t)slots.size() > pool->available())
    return pkv_set_error(PKV_ERR_NO_BLOCKS, "%zu blocks to swap in, %d available", slots.size(), pool->available());
  std::unordered_map<int32_t, int32_t> back;  // host entry -> new device block
  for (size_t k = 0; k < slots.size(); ++k) {
    int32_t b;
    pool->alloc(&b);  // cannot fail: enough blocks were counted above
    const int32_t slot = slots[k];
    pool->ref[b] = pool->host_ref[slot];
    pool->host_ref[slot] = 0;
    pool->host_free.push_back(slot);
    back[-slot - 1] = b;
    pairs_out[2 * k] = slot;
    pairs_out[2 * k + 1] = b;
  }
  if (!back.empty())  // every sharer of a swapped-in block follows it
    for (auto &kv : pool->seqs)
      for (int32_t &e : kv.second.table)
        if (e < 0) {
          auto f = back.find(e);
          if (f != back.end()) e = f->second;
        }
  pool->swapped_in += (int64_t)slots.size();
  return PKV_OK;
}

extern "C" int pkv_seq_resident(const pkv_pool *pool, int64_t id, int32_t *resident_out) {
  if (int rc = need_pool(pool)) return rc;
  if (!resident_out) return pkv_set_error(PKV_ERR_INVALID, "resident_out is NULL");
  auto it = pool->seqs.find(id);
  if (it == pool->seqs.end()) return pkv_set_error(PKV_ERR_BAD_SEQ, "unknown sequence %lld", (long long)id);
  *resident_out = pkv_pool::resident(it->second) ? 1 : 0;
  return PKV_OK;
}

extern "C" int pkv_swap_space_stats(const pkv_pool *pool, pkv_swap_stats *out) {
  if (int rc = need_pool(pool)) return rc;
  if (!out) return pkv_set_error(PKV_ERR_INVALID, "out is NULL");
  int32_t used = 0;
  for (int32_t r : pool->host_ref) used += r > 0;
  out->host_blocks = pool->num_host;
  out->host_used = used;
  out->host_free = (int32_t)pool->host_free.size();
  out->clock_hand = pool->hand;
  out->swapped_out = pool->swapped_out;
  out->swapped_in = pool->swapped_in;
  return PKV_OK;
}
