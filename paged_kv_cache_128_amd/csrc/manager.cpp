// Host-side KV block manager behind the C ABI (declared in include/pkv.h).
//
// The manager is the CPU metadata plane of [MiniPaged-Qwen] §8: an ordered
// free list of physical block ids plus, per live sequence, its length and its
// block table.  Semantics follow [MiniPaged-Qwen] §9 (append_token) and
// [mini-vLLM BM] (allocate_for_prefill / append_slot_for_decode /
// free_sequence / can_allocate).  Every operation validates first and mutates
// only after all checks pass, so a failed call leaves the state unchanged.
//
// The free list is a ring buffer of capacity num_blocks: allocation pops the
// front, release pushes at the back, and the list can never hold more than
// num_blocks ids while the invariants hold.
//
// Prefix sharing and copy-on-write ([impl-detail] "Copy-on-Write共享"): each
// block has a reference count, the number of tables holding it; a block
// returns to the free list when its count drops to 0.  An append whose
// token lands in a block other tables also hold takes a free block for the
// sequence and queues a (source, destination) copy that the caller runs on
// the device before the step's write.
//
// Swap to host ([impl-detail] "异构内存支持"): swap-out releases a sequence's
// blocks and keeps its length; swap-in gives it fresh blocks, all or nothing.
// The caller copies the block contents out before the blocks are reused and
// back after swap-in.
#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Sequence {
  int32_t length = 0;            // tokens written == next write position
  std::vector<int32_t> table;    // logical block -> physical block id
  uint64_t mark = 0;             // batch-call epoch that last listed it (duplicate check)
};

// Room for one more table entry, grown geometrically, so that an append
// that opens a block cannot fail midway.
void reserve_one(std::vector<int32_t>& t) {
  if (t.size() == t.capacity()) t.reserve(t.size() < 8 ? 8 : 2 * t.size());
}

}  // namespace

struct pkv_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  bool sort_on_release = false;
  // ring buffer holding the free list, front at `head`
  std::vector<int32_t> ring;
  int64_t head = 0;
  int64_t count = 0;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<int32_t> ref;                            // tables holding each block
  std::vector<std::pair<int32_t, int32_t>> copies;     // queued (source, destination)
  std::unordered_map<int64_t, int32_t> swapped;        // swapped-out sequence -> length
  uint64_t epoch = 0;                                  // batch calls so far (Sequence::mark)

  int32_t free_at(int64_t i) const { return ring[(head + i) % num_blocks]; }
  int32_t pop_front() {
    int32_t v = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    return v;
  }
  void push_back(int32_t v) {
    ring[(head + count) % num_blocks] = v;
    ++count;
  }
  void sort_free() {
    std::vector<int32_t> tmp;
    tmp.reserve(count);
    for (int64_t i = 0; i < count; ++i) tmp.push_back(free_at(i));
    std::sort(tmp.begin(), tmp.end());
    head = 0;
    for (int64_t i = 0; i < count; ++i) ring[i] = tmp[i];
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

extern "C" {

pkv_manager* pkv_manager_create(int32_t num_blocks, int32_t block_size,
                                const int32_t* initial_free_order, uint32_t flags) {
  if (num_blocks <= 0 || block_size <= 0 || (flags & ~PKV_SORT_ON_RELEASE) != 0) return nullptr;
  pkv_manager* m = new (std::nothrow) pkv_manager();
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->sort_on_release = (flags & PKV_SORT_ON_RELEASE) != 0;
    m->ring.resize(num_blocks);
    m->ref.assign(num_blocks, 0);
    if (initial_free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t v = initial_free_order[i];
        if (v < 0 || v >= num_blocks || seen[v]) {
          delete m;
          return nullptr;
        }
        seen[v] = 1;
        m->ring[i] = v;
      }
    } else {
      for (int32_t i = 0; i < num_blocks; ++i) m->ring[i] = i;
    }
    m->head = 0;
    m->count = num_blocks;
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pkv_manager_destroy(pkv_manager* mgr) { delete mgr; }

int pkv_can_allocate(const pkv_manager* m, int32_t num_tokens) {
  if (!m || num_tokens < 0) return PKV_ERR_INVALID;
  return m->blocks_for(num_tokens) <= m->count ? 1 : 0;
}

int32_t pkv_num_free_blocks(const pkv_manager* m) {
  return m ? static_cast<int32_t>(m->count) : PKV_ERR_INVALID;
}

int32_t pkv_num_live_sequences(const pkv_manager* m) {
  return m ? static_cast<int32_t>(m->seqs.size()) : PKV_ERR_INVALID;
}

int pkv_allocate_for_prefill(pkv_manager* m, int64_t seq_id, int32_t num_tokens,
                             int64_t* slots_out) {
  if (!m || seq_id < 0 || num_tokens < 0) return PKV_ERR_INVALID;
  if (m->seqs.count(seq_id) || m->swapped.count(seq_id)) return PKV_ERR_ALREADY_PREFILLED;
  const int64_t need = m->blocks_for(num_tokens);
  if (need > m->count) return PKV_ERR_OOM;
  Sequence s;
  try {
    s.table.reserve(need);
    for (int64_t i = 0; i < need; ++i) s.table.push_back(m->free_at(i));
    s.length = num_tokens;
    m->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (int64_t i = 0; i < need; ++i) m->ref[m->pop_front()] = 1;
  if (slots_out) {
    const std::vector<int32_t>& t = m->seqs[seq_id].table;
    const int64_t bs = m->block_size;
    for (int64_t p = 0; p < num_tokens; ++p) slots_out[p] = t[p / bs] * bs + p % bs;
  }
  return PKV_OK;
}

int pkv_share_prefix(pkv_manager* m, int64_t donor_id, int64_t seq_id, int32_t num_tokens) {
  if (!m || seq_id < 0 || num_tokens < 0) return PKV_ERR_INVALID;
  auto d = m->seqs.find(donor_id);
  if (d == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  if (m->seqs.count(seq_id) || m->swapped.count(seq_id)) return PKV_ERR_ALREADY_PREFILLED;
  if (num_tokens > d->second.length) return PKV_ERR_INVALID;
  const int64_t n = m->blocks_for(num_tokens);
  Sequence s;
  try {
    s.table.assign(d->second.table.begin(), d->second.table.begin() + n);
    s.length = num_tokens;
    m->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (int32_t pb : m->seqs[seq_id].table) ++m->ref[pb];
  return PKV_OK;
}

// Does the next append of `s` take a block: one it opens, or a copy of a
// block other tables hold (`dropped` = references earlier appends of the
// same call release from that block)?
static bool append_takes_block(const pkv_manager* m, const Sequence& s, int32_t dropped) {
  const int64_t lb = s.length / m->block_size;
  if (lb == static_cast<int64_t>(s.table.size())) return true;
  return m->ref[s.table[lb]] - dropped > 1;
}

// One append on a live sequence already checked to have a block available
// when it needs one and room in the copy queue ([MiniPaged-Qwen] §9.1-§9.3;
// copy-on-write of [impl-detail] "Copy-on-Write机制").
static int64_t append_one(pkv_manager* m, Sequence& s, int32_t* new_block) {
  const int64_t bs = m->block_size;
  const int64_t L = s.length;
  const int64_t logical_block = L / bs;
  const int64_t block_offset = L % bs;
  *new_block = -1;
  if (logical_block == static_cast<int64_t>(s.table.size())) {
    int32_t pb = m->pop_front();
    m->ref[pb] = 1;
    s.table.push_back(pb);
    *new_block = pb;
  } else if (m->ref[s.table[logical_block]] > 1) {
    const int32_t old = s.table[logical_block];
    const int32_t pb = m->pop_front();
    --m->ref[old];
    m->ref[pb] = 1;
    s.table[logical_block] = pb;
    m->copies.emplace_back(old, pb);
    *new_block = pb;
  }
  s.length = static_cast<int32_t>(L + 1);
  return static_cast<int64_t>(s.table[logical_block]) * bs + block_offset;
}

int pkv_append_slot_for_decode(pkv_manager* m, int64_t seq_id, int64_t* slot_out) {
  if (!m || !slot_out) return PKV_ERR_INVALID;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  Sequence& s = it->second;
  if (s.length == INT32_MAX) return PKV_ERR_INVALID;
  const bool opens = (s.length / m->block_size) == static_cast<int64_t>(s.table.size());
  if (append_takes_block(m, s, 0) && m->count == 0) return PKV_ERR_OOM;
  try {
    if (opens) reserve_one(s.table);
    m->copies.reserve(m->copies.size() + 1);
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  int32_t nb;
  *slot_out = append_one(m, s, &nb);
  return PKV_OK;
}

int pkv_append_slots_for_decode(pkv_manager* m, const int64_t* seq_ids, int32_t n,
                                int64_t* slots_out, int32_t* lens_out, int32_t* new_block_out) {
  if (!m || n < 0 || (n > 0 && !seq_ids)) return PKV_ERR_INVALID;
  // The ids' sequences, with the duplicate check by epoch marks (no
  // allocation once the buffer has grown); when some id is not live, the
  // set-based check decides which error comes first (duplicates before
  // unknown ids).
  thread_local std::vector<Sequence*> seqs;
  bool all_live = true, dup = false;
  try {
    seqs.resize(static_cast<size_t>(n));
    const uint64_t ep = ++m->epoch;
    for (int32_t i = 0; i < n; ++i) {
      auto it = m->seqs.find(seq_ids[i]);
      if (it == m->seqs.end()) {
        all_live = false;
        continue;
      }
      Sequence& s = it->second;
      if (s.mark == ep) dup = true;
      s.mark = ep;
      seqs[i] = &s;
    }
    if (!all_live) {
      std::unordered_set<int64_t> seen;
      seen.reserve(static_cast<size_t>(n) * 2);
      for (int32_t i = 0; i < n; ++i)
        if (!seen.insert(seq_ids[i]).second) return PKV_ERR_INVALID;
      return PKV_ERR_NOT_LIVE;
    }
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  if (dup) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (seqs[i]->length == INT32_MAX) return PKV_ERR_INVALID;
  // blocks the call takes, in array order: opened blocks and copies on write
  // (a copy drops one reference from the shared block for later rows)
  int64_t need = 0;
  try {
    std::unordered_map<int32_t, int32_t> dropped;
    for (int32_t i = 0; i < n; ++i) {
      Sequence* s = seqs[i];
      const int64_t lb = s->length / m->block_size;
      const bool opens = lb == static_cast<int64_t>(s->table.size());
      const int32_t pb = opens ? -1 : s->table[lb];
      const int32_t d = opens ? 0 : (dropped.count(pb) ? dropped[pb] : 0);
      if (append_takes_block(m, *s, d)) {
        ++need;
        if (!opens) dropped[pb] = d + 1;
      }
    }
    if (need > m->count) return PKV_ERR_OOM;
    for (int32_t i = 0; i < n; ++i)
      if (seqs[i]->length / m->block_size == static_cast<int64_t>(seqs[i]->table.size()))
        reserve_one(seqs[i]->table);
    m->copies.reserve(m->copies.size() + need);
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t nb;
    int64_t slot = append_one(m, *seqs[i], &nb);
    if (slots_out) slots_out[i] = slot;
    if (lens_out) lens_out[i] = seqs[i]->length;
    if (new_block_out) new_block_out[i] = nb;
  }
  return PKV_OK;
}

int pkv_append_tokens(pkv_manager* m, int64_t seq_id, int32_t num_tokens, int64_t* slots_out) {
  if (!m || num_tokens < 0) return PKV_ERR_INVALID;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  Sequence& s = it->second;
  if (static_cast<int64_t>(s.length) + num_tokens > INT32_MAX) return PKV_ERR_INVALID;
  const int64_t bs = m->block_size;
  int64_t need = m->blocks_for(static_cast<int64_t>(s.length) + num_tokens) - static_cast<int64_t>(s.table.size());
  if (num_tokens > 0 && s.length / bs < static_cast<int64_t>(s.table.size()) &&
      m->ref[s.table[s.length / bs]] > 1)
    ++need;
  if (need > m->count) return PKV_ERR_OOM;
  try {
    s.table.reserve(m->blocks_for(static_cast<int64_t>(s.length) + num_tokens));
    m->copies.reserve(m->copies.size() + 1);
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < num_tokens; ++i) {
    int32_t nb;
    const int64_t slot = append_one(m, s, &nb);
    if (slots_out) slots_out[i] = slot;
  }
  return PKV_OK;
}

int pkv_admit_batch(pkv_manager* m, const int64_t* seq_ids, const int32_t* chunk_lens, int32_t n,
                    int32_t extend_live, int64_t* slots_out, int32_t* lens_out) {
  if (!m || n < 0 || (n > 0 && (!seq_ids || !chunk_lens))) return PKV_ERR_INVALID;
  const int64_t bs = m->block_size;
  int64_t need = 0;
  try {
    std::unordered_set<int64_t> seen;
    seen.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
      if (seq_ids[i] < 0 || chunk_lens[i] < 0) return PKV_ERR_INVALID;
      if (!seen.insert(seq_ids[i]).second) return PKV_ERR_INVALID;
    }
    // the blocks the whole batch takes, in array order: new tables, opened
    // blocks, and a copy of each shared tail block a chunk writes into (a
    // copy drops one reference from that block for later chunks)
    std::unordered_map<int32_t, int32_t> dropped;
    for (int32_t i = 0; i < n; ++i) {
      if (m->swapped.count(seq_ids[i])) return PKV_ERR_ALREADY_PREFILLED;
      auto it = m->seqs.find(seq_ids[i]);
      if (it == m->seqs.end()) {
        need += m->blocks_for(chunk_lens[i]);
        continue;
      }
      if (!extend_live) return PKV_ERR_ALREADY_PREFILLED;
      const Sequence& s = it->second;
      if (static_cast<int64_t>(s.length) + chunk_lens[i] > INT32_MAX) return PKV_ERR_INVALID;
      need += m->blocks_for(static_cast<int64_t>(s.length) + chunk_lens[i]) - static_cast<int64_t>(s.table.size());
      if (chunk_lens[i] > 0 && s.length / bs < static_cast<int64_t>(s.table.size())) {
        const int32_t tail = s.table[s.length / bs];
        const int32_t d = dropped.count(tail) ? dropped[tail] : 0;
        if (m->ref[tail] - d > 1) {
          ++need;
          dropped[tail] = d + 1;
        }
      }
    }
    if (need > m->count) return PKV_ERR_OOM;
    // room for every table entry and queued copy before anything changes
    for (int32_t i = 0; i < n; ++i) {
      auto it = m->seqs.find(seq_ids[i]);
      if (it != m->seqs.end())
        it->second.table.reserve(m->blocks_for(static_cast<int64_t>(it->second.length) + chunk_lens[i]));
    }
    m->seqs.reserve(m->seqs.size() + static_cast<size_t>(n));
    m->copies.reserve(m->copies.size() + static_cast<size_t>(n));
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  int64_t at = 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t* dst = slots_out ? slots_out + at : nullptr;
    const int r = m->seqs.count(seq_ids[i]) ? pkv_append_tokens(m, seq_ids[i], chunk_lens[i], dst)
                                            : pkv_allocate_for_prefill(m, seq_ids[i], chunk_lens[i], dst);
    if (r != PKV_OK) return PKV_ERR_INVARIANT;     // cannot happen: every check passed above
    if (lens_out) lens_out[i] = m->seqs[seq_ids[i]].length;
    at += chunk_lens[i];
  }
  return PKV_OK;
}

int pkv_swap_out(pkv_manager* m, int64_t seq_id, int32_t* ids_out, int32_t cap, int32_t* count_out) {
  if (!m || cap < 0 || !count_out || (cap > 0 && !ids_out)) return PKV_ERR_INVALID;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  const std::vector<int32_t>& t = it->second.table;
  if (static_cast<int64_t>(t.size()) > cap) return PKV_ERR_INVALID;
  for (int32_t pb : t)
    if (m->ref[pb] > 1) return PKV_ERR_INVALID;    // a shared block stays in other tables
  try {
    m->swapped.emplace(seq_id, it->second.length);
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (size_t i = 0; i < t.size(); ++i) {
    ids_out[i] = t[i];
    m->ref[t[i]] = 0;
    m->push_back(t[i]);
  }
  *count_out = static_cast<int32_t>(t.size());
  if (m->sort_on_release) m->sort_free();
  m->seqs.erase(it);
  return PKV_OK;
}

int pkv_swap_in(pkv_manager* m, int64_t seq_id, int32_t* ids_out, int32_t cap, int32_t* count_out) {
  if (!m || cap < 0 || !count_out || (cap > 0 && !ids_out)) return PKV_ERR_INVALID;
  if (m->seqs.count(seq_id)) return PKV_ERR_ALREADY_PREFILLED;
  auto it = m->swapped.find(seq_id);
  if (it == m->swapped.end()) return PKV_ERR_NOT_LIVE;
  const int64_t need = m->blocks_for(it->second);
  if (need > cap) return PKV_ERR_INVALID;
  if (need > m->count) return PKV_ERR_OOM;
  Sequence s;
  try {
    s.table.reserve(need);
    for (int64_t i = 0; i < need; ++i) s.table.push_back(m->free_at(i));
    s.length = it->second;
    m->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PKV_ERR_INVALID;
  }
  for (int64_t i = 0; i < need; ++i) {
    const int32_t pb = m->pop_front();
    m->ref[pb] = 1;
    ids_out[i] = pb;
  }
  *count_out = static_cast<int32_t>(need);
  m->swapped.erase(it);
  return PKV_OK;
}

int pkv_is_swapped(const pkv_manager* m, int64_t seq_id) {
  if (!m) return PKV_ERR_INVALID;
  return m->swapped.count(seq_id) ? 1 : 0;
}

int pkv_free_sequence(pkv_manager* m, int64_t seq_id) {
  if (!m) return PKV_ERR_INVALID;
  if (m->swapped.erase(seq_id)) return PKV_OK;     // a swapped-out sequence holds no blocks
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  for (int32_t pb : it->second.table)
    if (--m->ref[pb] == 0) m->push_back(pb);
  if (m->sort_on_release) m->sort_free();
  m->seqs.erase(it);
  return PKV_OK;
}

int32_t pkv_context_len(const pkv_manager* m, int64_t seq_id) {
  if (!m) return PKV_ERR_INVALID;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  return it->second.length;
}

int pkv_get_block_table(const pkv_manager* m, int64_t seq_id, int32_t* out, int32_t cap,
                        int32_t* len_out) {
  if (!m || cap < 0 || (cap > 0 && !out)) return PKV_ERR_INVALID;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
  const std::vector<int32_t>& t = it->second.table;
  if (static_cast<int64_t>(t.size()) > cap) return PKV_ERR_INVALID;
  std::copy(t.begin(), t.end(), out);
  if (len_out) *len_out = static_cast<int32_t>(t.size());
  return PKV_OK;
}

int pkv_get_block_tables(const pkv_manager* m, const int64_t* seq_ids, int32_t n, int32_t width,
                         int32_t pad, int32_t* out) {
  if (!m || n < 0 || width < 0 || (n > 0 && (!seq_ids || (width > 0 && !out))))
    return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return PKV_ERR_NOT_LIVE;
    if (static_cast<int64_t>(it->second.table.size()) > width) return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = m->seqs.find(seq_ids[i])->second.table;
    int32_t* row = out + static_cast<int64_t>(i) * width;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + width, pad);
  }
  return PKV_OK;
}

int pkv_get_context_lens(const pkv_manager* m, const int64_t* seq_ids, int32_t n, int32_t* out) {
  if (!m || n < 0 || (n > 0 && (!seq_ids || !out))) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (!m->seqs.count(seq_ids[i])) return PKV_ERR_NOT_LIVE;
  for (int32_t i = 0; i < n; ++i) out[i] = m->seqs.find(seq_ids[i])->second.length;
  return PKV_OK;
}

int pkv_get_free_list(const pkv_manager* m, int32_t* out, int32_t cap, int32_t* count_out) {
  if (!m || cap < 0 || (cap > 0 && !out)) return PKV_ERR_INVALID;
  if (m->count > cap) return PKV_ERR_INVALID;
  for (int64_t i = 0; i < m->count; ++i) out[i] = m->free_at(i);
  if (count_out) *count_out = static_cast<int32_t>(m->count);
  return PKV_OK;
}

int32_t pkv_block_ref_count(const pkv_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return PKV_ERR_INVALID;
  return m->ref[block];
}

int pkv_take_block_copies(pkv_manager* m, int32_t* src, int32_t* dst, int32_t cap,
                          int32_t* count_out) {
  if (!m || cap < 0 || !count_out || (cap > 0 && (!src || !dst))) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(m->copies.size()) > cap) return PKV_ERR_INVALID;
  for (size_t i = 0; i < m->copies.size(); ++i) {
    src[i] = m->copies[i].first;
    dst[i] = m->copies[i].second;
  }
  *count_out = static_cast<int32_t>(m->copies.size());
  m->copies.clear();
  return PKV_OK;
}

int pkv_check_invariants(const pkv_manager* m) {
  if (!m) return PKV_ERR_INVALID;
  const int64_t N = m->num_blocks;
  std::vector<int32_t> holders(N, 0);
  int64_t distinct = 0;
  for (const auto& kv : m->seqs) {
    const Sequence& s = kv.second;
    if (static_cast<int64_t>(s.table.size()) != m->blocks_for(s.length)) return PKV_ERR_INVARIANT;  // I5
    for (size_t i = 0; i < s.table.size(); ++i) {
      const int32_t pb = s.table[i];
      if (pb < 0 || pb >= N) return PKV_ERR_INVARIANT;           // I4
      for (size_t j = 0; j < i; ++j)
        if (s.table[j] == pb) return PKV_ERR_INVARIANT;          // I1: twice in one table
      if (holders[pb]++ == 0) ++distinct;
    }
  }
  for (int64_t pb = 0; pb < N; ++pb)
    if (holders[pb] > 0 && m->ref[pb] != holders[pb]) return PKV_ERR_INVARIANT;  // I1: counts
  std::vector<char> in_free(N, 0);
  for (int64_t i = 0; i < m->count; ++i) {
    int32_t pb = m->free_at(i);
    if (pb < 0 || pb >= N) return PKV_ERR_INVARIANT;             // I4
    if (in_free[pb]) return PKV_ERR_INVARIANT;                   // I6
    in_free[pb] = 1;
    if (holders[pb] || m->ref[pb] != 0) return PKV_ERR_INVARIANT;  // I2
  }
  if (distinct + m->count != N) return PKV_ERR_INVARIANT;        // I3
  return PKV_OK;
}

int pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t n, int64_t num_slots, int64_t* first_repeat) {
  if (first_repeat) *first_repeat = -1;
  if (n < 0 || num_slots < 0 || (n > 0 && !slot_mapping)) return PKV_ERR_INVALID;
  // (slot, index) pairs of the in-range entries; after sorting, equal slots
  // sit together in index order, and each one but the first is a repeat
  std::vector<std::pair<int64_t, int64_t>> v;
  v.reserve(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i)
    if (slot_mapping[i] >= 0 && slot_mapping[i] < num_slots) v.emplace_back(slot_mapping[i], i);
  std::sort(v.begin(), v.end());
  int64_t first = -1;
  for (size_t k = 1; k < v.size(); ++k)
    if (v[k].first == v[k - 1].first && (first < 0 || v[k].second < first)) first = v[k].second;
  if (first < 0) return PKV_OK;
  if (first_repeat) *first_repeat = first;
  return PKV_ERR_INVALID;
}

}  // extern "C"
