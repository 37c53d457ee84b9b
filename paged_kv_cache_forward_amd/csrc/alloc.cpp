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
// The exact rules (free-list order, id assignment, copy trigger) are stated in
// include/pagedattn.h.  Everything here is single-threaded per allocator and
// touches no GPU state.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "pagedattn.h"
#include "status.h"

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
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
      a->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) a->free_list.push_back(b);
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

  // Pass 2: apply, position by position.
  int32_t ncow = 0;
  for (int64_t p = start; p < end; ++p) {
    const int64_t j = p / B;
    if (p % B == 0) {
      int32_t fresh = a->free_list.front();
      a->free_list.pop_front();
      a->refcount[fresh] = 1;
      s->table.push_back(fresh);
    } else if (p == start && copies > 0) {
      int32_t old = s->table[j];
      int32_t fresh = a->free_list.front();
      a->free_list.pop_front();
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
    if (--a->refcount[b] == 0) a->free_list.push_back(b);
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
