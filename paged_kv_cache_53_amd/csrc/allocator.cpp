// Host block allocator of libpagedkv: free list, reference counts, block tables.
//
// The block manager the pages describe -- fixed-size physical blocks in one
// pool, a per-sequence table from logical to physical block, blocks taken on
// demand when a sequence fills its last one ("PagedAttention -- Math + Memory
// Model", section "PagedAttention: blocks and the block table"), a free list
// served from its head and refilled at its tail (the simulator in
// "KV-Cache Optimization & PagedAttention for Long-Context Agents", section
// "Python Implementation: Paged KV-Cache Virtual Memory Simulator"), and
// shared blocks with reference counts and copy-on-write ("PagedAttention --
// Math + Memory Model", section "Copy-on-write: sharing blocks across
// samples").  Every operation is all-or-nothing.  Plain C++17, no HIP.
//
// Swapping to host memory ("Reserve for the worst case, or page", section
// "What this model leaves out": a preempted sequence's blocks can move to host
// memory instead of being recomputed): a fixed number of host slots with their
// own FIFO free list; swap-out moves every block of a sequence in logical order
// to the next host slots and drops the sequence's references as a free does;
// swap-in takes fresh device blocks in logical order and returns the host slots
// to the tail of their list.  Both return the copy pairs for the caller's
// block-copy kernel.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <limits>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"

namespace {

struct Sequence {
  std::vector<int32_t> blocks;  // logical block i -> physical block id
  int64_t len = 0;              // tokens
};

struct Swapped {
  std::vector<int32_t> host_slots;  // logical block i -> host slot
  int64_t len = 0;
};

}  // namespace

struct pkv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;  // front = next block handed out
  std::vector<int32_t> ref;       // sequences whose table holds the block
  std::unordered_map<int64_t, Sequence> seqs;
  int32_t shared_blocks = 0;      // blocks with ref > 1, kept current
  int32_t num_host = -1;          // host slots (-1: no swap space yet)
  std::deque<int32_t> host_free;  // front = next host slot handed out
  std::unordered_map<int64_t, Swapped> swapped;

  // Drops one reference of each block of s, in logical order; a block at zero rejoins the free list.
  void release(const Sequence& s) {
    for (int32_t b : s.blocks) {
      dec_ref(b);
      if (ref[b] == 0) free_list.push_back(b);
    }
  }

  void inc_ref(int32_t b) {
    if (++ref[b] == 2) ++shared_blocks;
  }
  void dec_ref(int32_t b) {
    if (ref[b]-- == 2) --shared_blocks;
  }

  // Blocks an append of n tokens to a sequence of length len / last block needs.
  int64_t blocks_needed(const Sequence* s, int64_t n) const {
    const int64_t L = s ? s->len : 0;
    if (n <= 0) return 0;
    const int64_t B = block_size;
    // positions p in [L, L+n) with p % B == 0
    const int64_t first = (L + B - 1) / B * B;
    int64_t fresh = first < L + n ? (L + n - 1 - first) / B + 1 : 0;
    const bool cow = s && (L % B) != 0 && ref[s->blocks.back()] > 1;
    return fresh + (cow ? 1 : 0);
  }

  // The append itself; the caller checked capacity.
  void append(Sequence& s, int32_t n, int64_t* slots, int32_t* cow_pair, int32_t* n_cow) {
    const int64_t B = block_size;
    const int64_t L = s.len;
    int32_t copies = 0;
    for (int64_t p = L; p < L + n; ++p) {
      if (p % B == 0) {
        const int32_t b = free_list.front();
        free_list.pop_front();
        ref[b] = 1;
        s.blocks.push_back(b);
      } else if (p == L && ref[s.blocks.back()] > 1) {
        const int32_t old_b = s.blocks.back();
        const int32_t new_b = free_list.front();
        free_list.pop_front();
        dec_ref(old_b);
        ref[new_b] = 1;
        s.blocks.back() = new_b;
        if (cow_pair) {
          cow_pair[0] = old_b;
          cow_pair[1] = new_b;
        }
        ++copies;
      }
      if (slots) slots[p - L] = static_cast<int64_t>(s.blocks[p / B]) * B + p % B;
    }
    s.len = L + n;
    if (n_cow) *n_cow = copies;
  }
};

extern "C" {

int pkv_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                         pkv_allocator** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID;
  *out = nullptr;
  if (initial_free_order) {
    std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PKV_ERR_INVALID;
      seen[b] = 1;
    }
  }
  pkv_allocator* a = new (std::nothrow) pkv_allocator();
  if (!a) return PKV_ERR_OOM;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(static_cast<size_t>(num_blocks), 0);
  for (int32_t i = 0; i < num_blocks; ++i)
    a->free_list.push_back(initial_free_order ? initial_free_order[i] : i);
  *out = a;
  return PKV_OK;
}

void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

int pkv_alloc(pkv_allocator* a, int64_t seq_id, int32_t n_new_tokens, int64_t* slots_out,
              int32_t* cow_pair_out, int32_t* n_cow) {
  if (!a || n_new_tokens < 0 || a->swapped.count(seq_id)) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq_id);
  Sequence* s = it == a->seqs.end() ? nullptr : &it->second;
  const int64_t len = s ? s->len : 0;
  if (len + n_new_tokens > std::numeric_limits<int32_t>::max()) return PKV_ERR_INVALID;
  if (a->blocks_needed(s, n_new_tokens) > static_cast<int64_t>(a->free_list.size()))
    return PKV_ERR_OOM;
  if (!s) s = &a->seqs[seq_id];
  a->append(*s, n_new_tokens, slots_out, cow_pair_out, n_cow);
  return PKV_OK;
}

int pkv_alloc_batch(pkv_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int32_t n_new_each,
                    int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow) {
  if (!a || n_seqs < 0 || n_new_each < 0 || (n_seqs > 0 && !seq_ids)) return PKV_ERR_INVALID;
  std::unordered_set<int64_t> ids;
  ids.reserve(static_cast<size_t>(n_seqs) * 2);
  int64_t need = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!ids.insert(seq_ids[i]).second || a->swapped.count(seq_ids[i])) return PKV_ERR_INVALID;
    auto it = a->seqs.find(seq_ids[i]);
    const Sequence* s = it == a->seqs.end() ? nullptr : &it->second;
    if ((s ? s->len : 0) + n_new_each > std::numeric_limits<int32_t>::max()) return PKV_ERR_INVALID;
    need += a->blocks_needed(s, n_new_each);
  }
  if (need > static_cast<int64_t>(a->free_list.size())) return PKV_ERR_OOM;
  int32_t copies = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    Sequence& s = a->seqs[seq_ids[i]];
    int32_t pair[2];
    int32_t c = 0;
    a->append(s, n_new_each, slots_out ? slots_out + static_cast<int64_t>(i) * n_new_each : nullptr,
              pair, &c);
    if (c) {
      if (cow_pairs_out) {
        cow_pairs_out[2 * copies] = pair[0];
        cow_pairs_out[2 * copies + 1] = pair[1];
      }
      ++copies;
    }
  }
  if (n_cow) *n_cow = copies;
  return PKV_OK;
}

int pkv_fork(pkv_allocator* a, int64_t parent, int64_t child, int32_t n_shared_tokens) {
  if (!a || n_shared_tokens < -1) return PKV_ERR_INVALID;
  auto pit = a->seqs.find(parent);
  if (pit == a->seqs.end()) return PKV_ERR_NOT_FOUND;
  if (a->seqs.count(child) || a->swapped.count(child)) return PKV_ERR_INVALID;
  const int64_t plen = pit->second.len;
  const int64_t n = n_shared_tokens < 0 ? plen : n_shared_tokens;
  if (n > plen) return PKV_ERR_INVALID;
  const int64_t nb = (n + a->block_size - 1) / a->block_size;
  Sequence c;
  c.blocks.assign(pit->second.blocks.begin(), pit->second.blocks.begin() + nb);
  c.len = n;
  for (int32_t b : c.blocks) a->inc_ref(b);
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_free(pkv_allocator* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID;
  auto sw = a->swapped.find(seq_id);
  if (sw != a->swapped.end()) {   // a swapped-out sequence gives back its host slots
    for (int32_t h : sw->second.host_slots) a->host_free.push_back(h);
    a->swapped.erase(sw);
    return PKV_OK;
  }
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_NOT_FOUND;
  a->release(it->second);
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_allocator_set_swap_space(pkv_allocator* a, int32_t host_blocks) {
  if (!a || host_blocks < 0 || a->num_host >= 0) return PKV_ERR_INVALID;
  a->num_host = host_blocks;
  for (int32_t h = 0; h < host_blocks; ++h) a->host_free.push_back(h);
  return PKV_OK;
}

int pkv_swap_out(pkv_allocator* a, int64_t seq_id, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!a || cap < 0 || a->num_host < 0) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_NOT_FOUND;
  const Sequence& s = it->second;
  const int32_t nb = static_cast<int32_t>(s.blocks.size());
  if (n_pairs) *n_pairs = nb;
  if (!pairs_out || cap < nb) return PKV_ERR_INVALID;
  if (nb > static_cast<int32_t>(a->host_free.size())) return PKV_ERR_OOM;
  Swapped w;
  w.len = s.len;
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t h = a->host_free.front();
    a->host_free.pop_front();
    pairs_out[2 * i] = s.blocks[i];
    pairs_out[2 * i + 1] = h;
    w.host_slots.push_back(h);
  }
  a->release(s);
  a->seqs.erase(it);
  a->swapped.emplace(seq_id, std::move(w));
  return PKV_OK;
}

int pkv_swap_in(pkv_allocator* a, int64_t seq_id, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!a || cap < 0) return PKV_ERR_INVALID;
  auto it = a->swapped.find(seq_id);
  if (it == a->swapped.end()) return PKV_ERR_NOT_FOUND;
  const Swapped& w = it->second;
  const int32_t nb = static_cast<int32_t>(w.host_slots.size());
  if (n_pairs) *n_pairs = nb;
  if (!pairs_out || cap < nb) return PKV_ERR_INVALID;
  if (nb > static_cast<int32_t>(a->free_list.size())) return PKV_ERR_OOM;
  Sequence s;
  s.len = w.len;
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t b = a->free_list.front();
    a->free_list.pop_front();
    a->ref[b] = 1;
    s.blocks.push_back(b);
    pairs_out[2 * i] = w.host_slots[i];
    pairs_out[2 * i + 1] = b;
  }
  for (int32_t h : w.host_slots) a->host_free.push_back(h);
  a->swapped.erase(it);
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_swap_stats(const pkv_allocator* a, int32_t* host_blocks, int32_t* host_free, int64_t* swapped_seqs) {
  if (!a) return PKV_ERR_INVALID;
  if (host_blocks) *host_blocks = a->num_host < 0 ? 0 : a->num_host;
  if (host_free) *host_free = static_cast<int32_t>(a->host_free.size());
  if (swapped_seqs) *swapped_seqs = static_cast<int64_t>(a->swapped.size());
  return PKV_OK;
}

int pkv_get_block_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                        int32_t* n_blocks, int32_t* seq_len) {
  if (!a || cap < 0) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_NOT_FOUND;
  const auto& t = it->second.blocks;
  if (out) {
    const size_t n = std::min(t.size(), static_cast<size_t>(cap));
    std::copy(t.begin(), t.begin() + n, out);
  }
  if (n_blocks) *n_blocks = static_cast<int32_t>(t.size());
  if (seq_len) *seq_len = static_cast<int32_t>(it->second.len);
  return PKV_OK;
}

int pkv_fill_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t n_seqs,
                          int32_t* tables, int32_t stride, int32_t pad_value, int32_t* seq_lens) {
  if (!a || n_seqs < 0 || stride < 0 || (n_seqs > 0 && (!seq_ids || !tables))) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_NOT_FOUND;
    if (it->second.blocks.size() > static_cast<size_t>(stride)) return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Sequence& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + static_cast<int64_t>(i) * stride;
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + s.blocks.size(), row + stride, pad_value);
    if (seq_lens) seq_lens[i] = static_cast<int32_t>(s.len);
  }
  return PKV_OK;
}

int pkv_allocator_stats(const pkv_allocator* a, pkv_stats* out) {
  if (!a || !out) return PKV_ERR_INVALID;
  std::memset(out, 0, sizeof(*out));
  out->num_blocks = a->num_blocks;
  out->block_size = a->block_size;
  out->free_blocks = static_cast<int32_t>(a->free_list.size());
  out->allocated_blocks = a->num_blocks - out->free_blocks;
  out->shared_blocks = a->shared_blocks;
  out->num_seqs = static_cast<int64_t>(a->seqs.size());
  int64_t live = 0;
  for (const auto& kv : a->seqs) live += kv.second.len;
  out->live_tokens = live;
  out->allocated_slots = static_cast<int64_t>(out->allocated_blocks) * a->block_size;
  return PKV_OK;
}

int32_t pkv_block_ref_count(const pkv_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

int pkv_free_list(const pkv_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || cap < 0) return PKV_ERR_INVALID;
  if (out) {
    const size_t m = std::min(a->free_list.size(), static_cast<size_t>(cap));
    std::copy(a->free_list.begin(), a->free_list.begin() + m, out);
  }
  if (n) *n = static_cast<int32_t>(a->free_list.size());
  return PKV_OK;
}

}  // extern "C"
