// Host block allocator for the paged KV cache.
//
// Policy ("Stop Wasting GPU Memory" page, Technical Details: "Core Architecture",
// "Single Sequence Generation", "Copy-on-Write for Parallel Sampling", "Beam Search
// Optimization"; the ml-canon page's block-table sketch):
//   * each sequence owns a block table of physical block ids and a token count;
//   * a token opens a new block only when the last one is full, so waste stays in the
//     last block;
//   * forks share blocks through per-block reference counts;
//   * the first write into a shared partial block moves the writer onto a private copy
//     of that one block (a copy pair for the device), the old count drops by one; the
//     last holder writes in place;
//   * freeing drops one reference per table entry and returns blocks at zero to the
//     pool immediately.
// The pool is a LIFO stack seeded with the caller's hand-out order.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedattn.h"

struct pa_allocator {
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
    // Dry-run state of a batched append (valid while stamp equals the allocator's gen).
    uint64_t stamp = 0;
    int64_t len_after = 0;
    int32_t last_after = -1;  // current last block after earlier copy-on-write, -1 = private fresh block
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcnt;
  std::unordered_map<int64_t, Seq> seqs;
  // Scratch of batched appends: a generation counter, per-block count changes of the dry run
  // (valid while delta_stamp equals gen) and the batch's sequences.
  uint64_t gen = 0;
  std::vector<int32_t> delta;
  std::vector<uint64_t> delta_stamp;
  std::vector<Seq*> batch;

  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refcnt[b] = 1;
    return b;
  }

  static int64_t blocks_of(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

  // Blocks an append of n tokens needs, given the sequence's state and the current
  // count of its last block.
  int64_t need(const Seq& s, int32_t n, int32_t last_count) const {
    int64_t fresh = blocks_of(s.len + n, block_size) - blocks_of(s.len, block_size);
    int64_t cow = (n > 0 && s.len % block_size != 0 && last_count > 1) ? 1 : 0;
    return fresh + cow;
  }

  // Performs the append; the caller has checked capacity.  Emits at most one pair.
  void do_append(Seq& s, int32_t n, int32_t* slots, int32_t* pairs, int32_t* n_pairs) {
    for (int32_t i = 0; i < n; ++i) {
      const int64_t pos = s.len;
      if (static_cast<int64_t>(s.table.size()) * block_size <= pos) {
        s.table.push_back(take());
      } else if (refcnt[s.table.back()] > 1) {
        const int32_t old = s.table.back();
        const int32_t fresh = take();
        refcnt[old] -= 1;
        s.table.back() = fresh;
        pairs[2 * *n_pairs] = old;
        pairs[2 * *n_pairs + 1] = fresh;
        *n_pairs += 1;
      }
      slots[i] = s.table.back() * block_size + static_cast<int32_t>(pos % block_size);
      s.len = pos + 1;
    }
  }
};

extern "C" {

int32_t pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pa_allocator** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return PA_ERR_INVALID_ARG;
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return PA_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcnt.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PA_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      a->free_stack[num_blocks - 1 - i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[num_blocks - 1 - i] = i;
  }
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_seq_add(pa_allocator* a, int64_t id) {
  if (!a) return PA_ERR_INVALID_ARG;
  if (a->seqs.count(id)) return PA_ERR_INVALID_ARG;
  a->seqs.emplace(id, pa_allocator::Seq{});
  return PA_OK;
}

int32_t pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
  if (!a) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end() || a->seqs.count(child)) return PA_ERR_INVALID_ARG;
  pa_allocator::Seq copy = it->second;
  for (int32_t b : copy.table) a->refcnt[b] += 1;
  a->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

int32_t pa_seq_append(pa_allocator* a, int64_t id, int32_t n, int32_t* slots_out, int32_t* pairs_out,
                      int32_t pairs_cap, int32_t* n_pairs) {
  if (!a || n < 0 || !n_pairs || (n > 0 && !slots_out) || pairs_cap < 0) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return PA_ERR_INVALID_ARG;
  pa_allocator::Seq& s = it->second;
  const int32_t last_count = s.table.empty() ? 0 : a->refcnt[s.table.back()];
  const int64_t need = a->need(s, n, last_count);
  const bool cow = need > a->blocks_of(s.len + n, a->block_size) - a->blocks_of(s.len, a->block_size);
  if (cow && (pairs_cap < 1 || !pairs_out)) return PA_ERR_INVALID_ARG;
  if (need > static_cast<int64_t>(a->free_stack.size())) return PA_ERR_OUT_OF_BLOCKS;
  if (s.len + n > static_cast<int64_t>(INT32_MAX)) return PA_ERR_INVALID_ARG;
  *n_pairs = 0;
  a->do_append(s, n, slots_out, pairs_out, n_pairs);
  return PA_OK;
}

int32_t pa_seq_append_batch(pa_allocator* a, const int64_t* ids, int32_t n_seqs, const int32_t* counts,
                            int32_t* slots_out, int32_t* pairs_out, int32_t pairs_cap, int32_t* n_pairs) {
  if (!a || n_seqs < 0 || !n_pairs || pairs_cap < 0 || (n_seqs > 0 && (!ids || !counts)))
    return PA_ERR_INVALID_ARG;
  // Dry run: replay the batch on lengths and last-block counts only, so the whole
  // batch is admitted or refused before any state changes.  Sequences that appear
  // more than once, and siblings sharing a last block, are replayed in order.  The
  // replay state lives in the sequences and a per-block array, stamped with this call's
  // generation, so nothing is allocated per call once the scratch has grown.
  const uint64_t gen = ++a->gen;
  if (a->delta.size() != static_cast<size_t>(a->num_blocks)) {
    a->delta.assign(a->num_blocks, 0);
    a->delta_stamp.assign(a->num_blocks, 0);
  }
  if (a->batch.size() < static_cast<size_t>(n_seqs)) a->batch.resize(n_seqs);
  int64_t need_total = 0, pairs_total = 0, tokens_total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = a->seqs.find(ids[i]);
    if (it == a->seqs.end() || counts[i] < 0) return PA_ERR_INVALID_ARG;
    pa_allocator::Seq& s = it->second;
    a->batch[i] = &s;
    if (s.stamp != gen) {
      s.stamp = gen;
      s.len_after = s.len;
      s.last_after = s.table.empty() ? -1 : s.table.back();
    }
    const int64_t len = s.len_after;
    const int32_t n = counts[i];
    tokens_total += n;
    if (n == 0) continue;
    const int64_t fresh = a->blocks_of(len + n, a->block_size) - a->blocks_of(len, a->block_size);
    need_total += fresh;
    if (len % a->block_size != 0) {
      const int32_t last = s.last_after;
      if (last >= 0) {
        const int32_t cnt = a->refcnt[last] + (a->delta_stamp[last] == gen ? a->delta[last] : 0);
        if (cnt > 1) {
          need_total += 1;
          pairs_total += 1;
          if (a->delta_stamp[last] != gen) {
            a->delta_stamp[last] = gen;
            a->delta[last] = 0;
          }
          a->delta[last] -= 1;
          s.last_after = -1;  // now a private fresh block (count 1)
        }
      }
    }
    if (len + n > static_cast<int64_t>(INT32_MAX)) return PA_ERR_INVALID_ARG;
    s.len_after = len + n;
    if (fresh > 0) s.last_after = -1;  // the last block is freshly taken
  }
  if (tokens_total > 0 && !slots_out) return PA_ERR_INVALID_ARG;
  if (pairs_total > pairs_cap || (pairs_total > 0 && !pairs_out)) return PA_ERR_INVALID_ARG;
  if (need_total > static_cast<int64_t>(a->free_stack.size())) return PA_ERR_OUT_OF_BLOCKS;
  *n_pairs = 0;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    a->do_append(*a->batch[i], counts[i], slots_out + off, pairs_out, n_pairs);
    off += counts[i];
  }
  return PA_OK;
}

int32_t pa_seq_free(pa_allocator* a, int64_t id) {
  if (!a) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return PA_ERR_INVALID_ARG;
  for (int32_t b : it->second.table) {
    a->refcnt[b] -= 1;
    if (a->refcnt[b] == 0) a->free_stack.push_back(b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

int32_t pa_seq_table(const pa_allocator* a, int64_t id, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return PA_ERR_INVALID_ARG;
  const auto& t = it->second.table;
  *n = static_cast<int32_t>(t.size());
  if (static_cast<int64_t>(t.size()) > cap || (!t.empty() && !out)) return PA_ERR_INVALID_ARG;
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PA_OK;
}

int64_t pa_seq_len(const pa_allocator* a, int64_t id) {
  if (!a) return -1;
  auto it = a->seqs.find(id);
  return it == a->seqs.end() ? -1 : it->second.len;
}

int32_t pa_num_free(const pa_allocator* a) { return a ? static_cast<int32_t>(a->free_stack.size()) : -1; }

int32_t pa_refcount(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refcnt[block];
}

int32_t pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0) return PA_ERR_INVALID_ARG;
  *n = static_cast<int32_t>(a->free_stack.size());
  if (*n > cap || (*n > 0 && !out)) return PA_ERR_INVALID_ARG;
  if (*n > 0) std::memcpy(out, a->free_stack.data(), a->free_stack.size() * sizeof(int32_t));
  return PA_OK;
}

int32_t pa_build_batch(const pa_allocator* a, const int64_t* ids, int32_t n, int32_t max_blocks,
                       int32_t* tables_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks < 0) return PA_ERR_INVALID_ARG;
  if (n > 0 && (!ids || !lens_out || (max_blocks > 0 && !tables_out))) return PA_ERR_INVALID_ARG;
  std::vector<const pa_allocator::Seq*> rows(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(ids[i]);
    if (it == a->seqs.end()) return PA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks) return PA_ERR_INVALID_ARG;
    if (it->second.len > INT32_MAX) return PA_ERR_INVALID_ARG;
    rows[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = *rows[i];
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    const size_t used = s.table.size();
    if (used) std::memcpy(row, s.table.data(), used * sizeof(int32_t));
    std::fill(row + used, row + max_blocks, -1);
    lens_out[i] = static_cast<int32_t>(s.len);
  }
  return PA_OK;
}

// Groups of forked sequences for the decode: runs of consecutive sequences whose block tables name
// the same physical blocks for their first full blocks, every other sequence alone.  Forks keep the
// blocks they inherit until they write into one, so samples and beams of one prompt form such runs.
int32_t pa_shared_prefixes(const int32_t* tables, const int32_t* lens, int32_t num_seqs, int32_t max_blocks,
                           int32_t block_size, int32_t max_members, int32_t min_blocks, int32_t* groups,
                           int32_t groups_cap, int32_t* num_groups) {
  if (num_seqs < 0 || max_blocks < 1 || block_size < 1 || max_members < 1 || min_blocks < 1 || !num_groups)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!tables || !lens || !groups || groups_cap < num_seqs)) return PA_ERR_INVALID_ARG;
  auto full = [&](int32_t s) {
    const int32_t n = lens[s];
    return n <= 0 ? 0 : std::min(n / block_size, max_blocks);
  };
  int32_t ng = 0;
  int32_t i = 0;
  while (i < num_seqs) {
    const int32_t* row_i = tables + static_cast<int64_t>(i) * max_blocks;
    int32_t k = full(i);
    int32_t j = i + 1;
    while (j < num_seqs && j - i < max_members) {
      const int32_t* row_j = tables + static_cast<int64_t>(j) * max_blocks;
      const int32_t lim = std::min(k, full(j));
      int32_t common = lim;
      if (std::memcmp(row_i, row_j, static_cast<size_t>(lim) * sizeof(int32_t)) != 0)
        common = static_cast<int32_t>(std::mismatch(row_i, row_i + lim, row_j).first - row_i);
      if (common < min_blocks) break;
      k = common;
      ++j;
    }
    if (j - i < 2) {  // nobody to share with
      j = i + 1;
      k = 0;
    }
    groups[3 * ng + 0] = i;
    groups[3 * ng + 1] = j - i;
    groups[3 * ng + 2] = k;
    ++ng;
    i = j;
  }
  *num_groups = ng;
  return PA_OK;
}

// Prefill scheduling order: sequences by descending work, the (row, token) pairs of their chunk (a row at
// position p sees p + 1 tokens), ties in batch order.  Started first, the longest workgroups no longer
// make the launch's tail.
int32_t pa_prefill_order(const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs, int32_t* order) {
  if (num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!context_lens || !query_start || !order) return PA_ERR_INVALID_ARG;
  std::vector<int64_t> work(static_cast<size_t>(num_seqs));
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = std::max<int32_t>(0, context_lens[s]);
    const int64_t c = std::max<int64_t>(0, int64_t{query_start[s + 1]} - query_start[s]);
    // rows i = 0 .. c - 1 at positions n - c + i; those at position >= 0 see n - c + i + 1 tokens
    const int64_t first = std::max<int64_t>(0, c - n);  // rows before it have no position
    const int64_t lo = n - c + first + 1, hi = n;     // tokens seen by the first and last such row
    work[static_cast<size_t>(s)] = c > first ? (lo + hi) * (c - first) / 2 : 0;
    order[s] = s;
  }
  std::stable_sort(order, order + num_seqs,
                   [&](int32_t a, int32_t b) { return work[static_cast<size_t>(a)] > work[static_cast<size_t>(b)]; });
  return PA_OK;
}

}  // extern "C"
