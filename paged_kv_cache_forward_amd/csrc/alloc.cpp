// Host block allocator: block tables, refcounted sharing, copy-on-write.
//
// "Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
// (slavadubrov.com), section "Ungenutzten Platz in Blöcken berechnen": blocks
// are handed out as a sequence grows and given back when the request ends, and
// only a sequence's last block is partly filled.  Same page, section
// "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung", and "PagedAttention
// et vLLM" (aiunderstanding.org), FAQ on sharing: requests can point at the same
// block, and a copy is made only when one of them diverges.  "Внутреннее
// устройство vLLM" (artificials.ru), paragraph on paged attention: running out
// of blocks is the point where a scheduler preempts, so an append that cannot
// be satisfied fails without changing anything.
//
// Prefix caching: "Внутреннее устройство vLLM" (artificials.ru), paragraph on
// prefix caching: blocks of tokens are hashed and kept, and a request that
// begins with the same tokens reuses the matching blocks.
//
// The exact rules (free-list order, id assignment, copy trigger, block hash,
// registration and eviction) are stated in include/pagedattn.h.  Everything
// here is single-threaded per allocator and touches no GPU state.
#include <algorithm>
#include <cstdint>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedattn.h"
#include "status.h"

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // Free list (head = next block handed out); a prefix-cache hit can take a
  // block from the middle, hence a list with each member's position.
  std::list<int32_t> free_list;
  std::vector<std::list<int32_t>::iterator> free_pos;
  std::vector<char> is_free;
  std::vector<int32_t> refcount;
  // Prefix cache: hash -> registered block; per block its hash, parent hash, tokens.
  struct Reg {
    bool on = false;
    uint64_t hash = 0, parent = 0;
    std::vector<int32_t> tokens;
  };
  std::vector<Reg> reg;
  std::unordered_map<uint64_t, int32_t> cache;
  int64_t lookups = 0, hit_blocks = 0, evictions = 0;
  struct Seq {
    bool live = false;
    int32_t length = 0;
    std::vector<int32_t> table;
  };
  std::vector<Seq> seqs;  // indexed by id; ids never reused

  Seq* find(int32_t id) {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  const Seq* find(int32_t id) const {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
};

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void push_free(pa_alloc* a, int32_t b) {
  a->free_pos[b] = a->free_list.insert(a->free_list.end(), b);
  a->is_free[b] = 1;
}

static void unregister(pa_alloc* a, int32_t b) {
  pa_alloc::Reg& r = a->reg[b];
  if (!r.on) return;
  auto it = a->cache.find(r.hash);
  if (it != a->cache.end() && it->second == b) a->cache.erase(it);
  r.on = false;
  r.tokens.clear();
  a->evictions += 1;
}

// Head of the free list, for a write: a registered block is evicted first.
static int32_t pop_free(pa_alloc* a) {
  const int32_t b = a->free_list.front();
  a->free_list.pop_front();
  a->is_free[b] = 0;
  unregister(a, b);
  return b;
}

// FNV-1a 64 (offset basis 0xcbf29ce484222325, prime 0x100000001b3) of the
// parent hash's 8 little-endian bytes, then each token id's 4 little-endian bytes.
static uint64_t block_hash(uint64_t parent, const int32_t* tok, int32_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&](uint8_t byte) {
    h ^= byte;
    h *= 0x100000001b3ull;
  };
  for (int k = 0; k < 8; ++k) mix((uint8_t)(parent >> (8 * k)));
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t u = (uint32_t)tok[t];
    for (int k = 0; k < 4; ++k) mix((uint8_t)(u >> (8 * k)));
  }
  return h;
}
static constexpr uint64_t kHashRoot = 0xcbf29ce484222325ull;

extern "C" pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                                     const int32_t* free_order, pa_alloc** out) {
  if (out == nullptr) return pa::fail(PA_ERR_ARG, "pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_ARG, "pa_alloc_create: num_blocks=%d block_size=%d must be > 0",
                    num_blocks, block_size);
  pa_alloc* a = new (std::nothrow) pa_alloc();
  if (a == nullptr) return pa::fail(PA_ERR_ARG, "pa_alloc_create: host allocation failed");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  a->free_pos.resize(num_blocks);
  a->is_free.assign(num_blocks, 0);
  a->reg.resize(num_blocks);
  if (free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t k = 0; k < num_blocks; ++k) {
      int32_t b = free_order[k];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return pa::fail(PA_ERR_ARG, "pa_alloc_create: free_order is not a permutation (entry %d = %d)",
                        k, b);
      }
      seen[b] = 1;
      push_free(a, b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) push_free(a, b);
  }
  *out = a;
  return PA_OK;
}

extern "C" void pa_alloc_destroy(pa_alloc* a) { delete a; }

extern "C" pa_status pa_seq_create(pa_alloc* a, int32_t* seq_id) {
  if (a == nullptr || seq_id == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_create: NULL argument");
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq_id = (int32_t)a->seqs.size() - 1;
  return PA_OK;
}

extern "C" pa_status pa_seq_fork(pa_alloc* a, int32_t parent, int32_t share_tokens, int32_t* child) {
  if (a == nullptr || child == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_fork: NULL argument");
  const pa_alloc::Seq* p = a->find(parent);
  if (p == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_fork: unknown sequence %d", parent);
  if (share_tokens < 0 || share_tokens > p->length)
    return pa::fail(PA_ERR_ARG, "pa_seq_fork: share_tokens %d outside [0, %d]", share_tokens, p->length);
  const int64_t nshare = ceil_div(share_tokens, a->block_size);
  std::vector<int32_t> shared(p->table.begin(), p->table.begin() + nshare);
  for (int32_t b : shared) a->refcount[b] += 1;
  a->seqs.emplace_back();  // may move `p`; it is not used past this point
  pa_alloc::Seq& c = a->seqs.back();
  c.live = true;
  c.length = share_tokens;
  c.table = std::move(shared);
  *child = (int32_t)a->seqs.size() - 1;
  return PA_OK;
}

extern "C" pa_status pa_seq_append(pa_alloc* a, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                                   int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow) {
  if (a == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_append: NULL allocator");
  if (n_cow != nullptr) *n_cow = 0;
  pa_alloc::Seq* s = a->find(seq);
  if (s == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_append: unknown sequence %d", seq);
  if (n_tokens < 0) return pa::fail(PA_ERR_ARG, "pa_seq_append: n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return PA_OK;
  if (slots_out == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_append: slots_out is NULL");
  if ((int64_t)s->length + n_tokens > INT32_MAX)
    return pa::fail(PA_ERR_ARG, "pa_seq_append: sequence length overflows int32");
  const int32_t B = a->block_size;
  const int64_t start = s->length;
  const int64_t end = start + n_tokens;

  // Pass 1: count fresh blocks and copies without changing state.  Only the
  // block holding position `start` can be a partly written shared block; any
  // later position inside an existing block lies in that same block.
  int64_t fresh_needed = ceil_div(end, B) - ceil_div(start, B);
  int32_t copies = 0;
  if (start % B != 0) {
    int32_t b = s->table[start / B];
    if (a->refcount[b] > 1) copies = 1;
  }
  if (fresh_needed + copies > (int64_t)a->free_list.size())
    return pa::fail(PA_ERR_OOM, "pa_seq_append: needs %lld blocks, %zu free",
                    (long long)(fresh_needed + copies), a->free_list.size());
  if (copies > 0 && (cow_pairs_out == nullptr || cow_cap < copies || n_cow == nullptr))
    return pa::fail(PA_ERR_ARG, "pa_seq_append: a copy-on-write pair is due but cow_cap=%d", cow_cap);

  // Pass 2: apply, position by position.  A registered block written in place
  // (no copy due) leaves the prefix cache first.
  if (start % B != 0 && copies == 0) unregister(a, s->table[start / B]);
  int32_t ncow = 0;
  for (int64_t p = start; p < end; ++p) {
    const int64_t j = p / B;
    if (p % B == 0) {
      int32_t fresh = pop_free(a);
      a->refcount[fresh] = 1;
      s->table.push_back(fresh);
    } else if (p == start && copies > 0) {
      int32_t old = s->table[j];
      int32_t fresh = pop_free(a);
      a->refcount[fresh] = 1;
      a->refcount[old] -= 1;
      s->table[j] = fresh;
      cow_pairs_out[2 * ncow] = old;
      cow_pairs_out[2 * ncow + 1] = fresh;
      ++ncow;
    }
    slots_out[p - start] = (int64_t)s->table[j] * B + p % B;
  }
  s->length = (int32_t)end;
  if (n_cow != nullptr) *n_cow = ncow;
  return PA_OK;
}

extern "C" pa_status pa_seq_free(pa_alloc* a, int32_t seq) {
  if (a == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_free: NULL allocator");
  pa_alloc::Seq* s = a->find(seq);
  if (s == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_free: unknown sequence %d", seq);
  for (int32_t b : s->table) {
    if (--a->refcount[b] == 0) push_free(a, b);   // a registered block stays registered
  }
  s->table.clear();
  s->table.shrink_to_fit();
  s->length = 0;
  s->live = false;
  return PA_OK;
}

extern "C" pa_status pa_seq_block_table(const pa_alloc* a, int32_t seq, int32_t* out, int32_t cap,
                                        int32_t* n_blocks, int32_t* len) {
  if (a == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_block_table: NULL allocator");
  const pa_alloc::Seq* s = a->find(seq);
  if (s == nullptr) return pa::fail(PA_ERR_ARG, "pa_seq_block_table: unknown sequence %d", seq);
  const int32_t n = (int32_t)s->table.size();
  if (n_blocks != nullptr) *n_blocks = n;
  if (len != nullptr) *len = s->length;
  if (out == nullptr) return PA_OK;
  if (cap < n) return pa::fail(PA_ERR_ARG, "pa_seq_block_table: cap %d < %d blocks", cap, n);
  std::copy(s->table.begin(), s->table.end(), out);
  return PA_OK;
}

extern "C" pa_status pa_alloc_stats(const pa_alloc* a, pa_alloc_stats_t* st) {
  if (a == nullptr || st == nullptr) return pa::fail(PA_ERR_ARG, "pa_alloc_stats: NULL argument");
  int64_t used = 0, shared = 0;
  for (int32_t r : a->refcount) {
    used += r > 0;
    shared += r > 1;
  }
  int64_t tokens = 0, slots = 0;
  for (const auto& s : a->seqs) {
    if (!s.live) continue;
    tokens += s.length;
    slots += (int64_t)s.table.size() * a->block_size;
  }
  st->blocks_total = a->num_blocks;
  st->blocks_free = (int64_t)a->free_list.size();
  st->blocks_used = used;
  st->blocks_shared = shared;
  st->tokens_logical = tokens;
  st->slots_logical = slots;
  st->slots_physical = used * a->block_size;
  return PA_OK;
}

extern "C" pa_status pa_alloc_shared_blocks(const pa_alloc* a, const int32_t* seq_ids, int32_t n, int32_t* out) {
  if (a == nullptr || (n > 0 && (seq_ids == nullptr || out == nullptr)))
    return pa::fail(PA_ERR_ARG, "pa_alloc_shared_blocks: NULL argument");
  if (n < 0) return pa::fail(PA_ERR_ARG, "pa_alloc_shared_blocks: n %d < 0", n);
  for (int32_t i = 0; i < n; ++i)
    if (a->find(seq_ids[i]) == nullptr)
      return pa::fail(PA_ERR_ARG, "pa_alloc_shared_blocks: unknown sequence %d", seq_ids[i]);
  for (int32_t i = 0; i < n; ++i) {
    int32_t k = 0;
    if (i > 0) {
      const auto& t0 = a->find(seq_ids[i - 1])->table;
      const auto& t1 = a->find(seq_ids[i])->table;
      const size_t m = std::min(t0.size(), t1.size());
      while ((size_t)k < m && t0[k] == t1[k]) ++k;
    }
    out[i] = k;
  }
  return PA_OK;
}

extern "C" int32_t pa_block_refcount(const pa_alloc* a, int32_t block) {
  if (a == nullptr || block < 0 || block >= a->num_blocks) return -1;
  return a->refcount[block];
}

extern "C" pa_status pa_alloc_free_list(const pa_alloc* a, int32_t* out, int32_t cap, int32_t* n) {
  if (a == nullptr || n == nullptr) return pa::fail(PA_ERR_ARG, "pa_alloc_free_list: NULL argument");
  *n = (int32_t)a->free_list.size();
  if (out == nullptr) return PA_OK;
  int32_t k = 0;
  for (auto it = a->free_list.begin(); it != a->free_list.end() && k < cap; ++it) out[k++] = *it;
  return PA_OK;
}

extern "C" pa_status pa_prefix_register(pa_alloc* a, int32_t seq, const int32_t* tokens, int32_t n_tokens) {
  if (a == nullptr) return pa::fail(PA_ERR_ARG, "pa_prefix_register: NULL allocator");
  pa_alloc::Seq* s = a->find(seq);
  if (s == nullptr) return pa::fail(PA_ERR_ARG, "pa_prefix_register: unknown sequence %d", seq);
  if (n_tokens < 0 || n_tokens > s->length)
    return pa::fail(PA_ERR_ARG, "pa_prefix_register: n_tokens %d outside [0, %d]", n_tokens, s->length);
  if (n_tokens > 0 && tokens == nullptr) return pa::fail(PA_ERR_ARG, "pa_prefix_register: tokens is NULL");
  const int32_t B = a->block_size;
  uint64_t parent = kHashRoot;
  for (int32_t b = 0; b < n_tokens / B; ++b) {
    const uint64_t h = block_hash(parent, tokens + (int64_t)b * B, B);
    const int32_t blk = s->table[b];
    pa_alloc::Reg& r = a->reg[blk];
    if (!r.on && a->cache.find(h) == a->cache.end()) {
      r.on = true;
      r.hash = h;
      r.parent = parent;
      r.tokens.assign(tokens + (int64_t)b * B, tokens + (int64_t)(b + 1) * B);
      a->cache.emplace(h, blk);
    }
    parent = h;
  }
  return PA_OK;
}

extern "C" pa_status pa_prefix_lookup(pa_alloc* a, const int32_t* tokens, int32_t n_tokens, int32_t* seq_id,
                                      int32_t* n_cached) {
  if (a == nullptr || seq_id == nullptr || n_cached == nullptr)
    return pa::fail(PA_ERR_ARG, "pa_prefix_lookup: NULL argument");
  if (n_tokens < 0) return pa::fail(PA_ERR_ARG, "pa_prefix_lookup: n_tokens %d < 0", n_tokens);
  if (n_tokens > 0 && tokens == nullptr) return pa::fail(PA_ERR_ARG, "pa_prefix_lookup: tokens is NULL");
  const int32_t B = a->block_size;
  const int32_t max_blocks = n_tokens > 0 ? (n_tokens - 1) / B : 0;   // leave at least one token
  std::vector<int32_t> hits;
  uint64_t parent = kHashRoot;
  for (int32_t b = 0; b < max_blocks; ++b) {
    const int32_t* tk = tokens + (int64_t)b * B;
    const uint64_t h = block_hash(parent, tk, B);
    auto it = a->cache.find(h);
    if (it == a->cache.end()) break;
    const pa_alloc::Reg& r = a->reg[it->second];
    if (r.parent != parent || !std::equal(r.tokens.begin(), r.tokens.end(), tk)) break;
    hits.push_back(it->second);
    parent = h;
  }
  for (int32_t blk : hits) {
    if (a->refcount[blk] == 0 && a->is_free[blk]) {
      a->free_list.erase(a->free_pos[blk]);
      a->is_free[blk] = 0;
    }
    a->refcount[blk] += 1;
  }
  a->seqs.emplace_back();
  pa_alloc::Seq& c = a->seqs.back();
  c.live = true;
  c.length = (int32_t)hits.size() * B;
  c.table = std::move(hits);
  a->lookups += 1;
  a->hit_blocks += (int64_t)c.table.size();
  *seq_id = (int32_t)a->seqs.size() - 1;
  *n_cached = c.length;
  return PA_OK;
}

extern "C" pa_status pa_prefix_stats(const pa_alloc* a, pa_prefix_stats_t* st) {
  if (a == nullptr || st == nullptr) return pa::fail(PA_ERR_ARG, "pa_prefix_stats: NULL argument");
  int64_t reg = 0, reg_free = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b) {
    if (!a->reg[b].on) continue;
    reg += 1;
    reg_free += a->refcount[b] == 0;
  }
  st->blocks_registered = reg;
  st->registered_free = reg_free;
  st->lookups = a->lookups;
  st->hit_blocks = a->hit_blocks;
  st->evictions = a->evictions;
  return PA_OK;
}
