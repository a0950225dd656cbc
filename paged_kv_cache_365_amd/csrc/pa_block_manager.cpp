// Host-side block manager of the paged KV pool (include/pa_block_manager.h).
//
// Block scheduling, copy-on-write and prefix sharing as §2.2-§2.3 of the page
// "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space) describe
// them; the policy that makes every choice unique is stated in the header.
//
// Every operation is O(blocks it touches): the free list is a stack, the LRU
// list of cached blocks is intrusive (prev/next arrays over block ids), and
// registered prefixes live in a hash map keyed by (chain of the previous
// block, the block's 16 token ids).  Nothing here touches the GPU.
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pa_block_manager.h"

namespace {

constexpr int kMaxBs = 16;  // tokens per block: 16, or 8
constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

// FNV-1a over the 8 little-endian bytes of prev, then the block's bs int32
// token ids as 4 little-endian bytes each.
uint64_t chain_hash(uint64_t prev, const int32_t* tok, int bs) {
  uint64_t h = kFnvOffset;
  for (int i = 0; i < 8; ++i) {
    h ^= (prev >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  for (int t = 0; t < bs; ++t) {
    const uint32_t u = static_cast<uint32_t>(tok[t]);
    for (int i = 0; i < 4; ++i) {
      h ^= (u >> (8 * i)) & 0xffu;
      h *= kFnvPrime;
    }
  }
  return h;
}

struct Key {
  uint64_t prev;          // chain of the prefix before this block
  int32_t tok[kMaxBs];    // the block's token ids (entries past the block size are 0)
  int32_t bs;
  bool operator==(const Key& o) const {
    return prev == o.prev && memcmp(tok, o.tok, sizeof(tok)) == 0;
  }
};
struct KeyHash {
  size_t operator()(const Key& k) const {
    return static_cast<size_t>(chain_hash(k.prev, k.tok, k.bs));
  }
};

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
  bool hashing = false;
  uint64_t chain = 0;         // chain of the last full block (0 = empty prefix)
  int32_t cur[kMaxBs] = {0};  // token ids of the current partial block
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks;
  int32_t bs;  // tokens per block
  std::vector<int32_t> ref;
  std::vector<int32_t> free_stack;
  // LRU list of cached (unreferenced, registered) blocks: head = oldest
  std::vector<int32_t> lru_prev, lru_next;
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1, lru_count = 0;
  // registration
  std::vector<uint8_t> registered;
  std::vector<Key> key_of;
  std::unordered_map<Key, int32_t, KeyHash> block_of;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, Seq> swapped;  // table empty while swapped out
  int64_t prefix_hits = 0, cow_copies = 0, evictions = 0;

  pa_block_manager(int32_t n, int32_t block_size)
      : num_blocks(n), bs(block_size), ref(n, 0), lru_prev(n, -1), lru_next(n, -1), in_lru(n, 0),
        registered(n, 0), key_of(n) {
    free_stack.reserve(n);
    for (int32_t b = n - 1; b >= 0; --b) free_stack.push_back(b);
  }

  int32_t available() const { return static_cast<int32_t>(free_stack.size()) + lru_count; }

  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++lru_count;
  }
  void lru_remove(int32_t b) {
    const int32_t p = lru_prev[b], nx = lru_next[b];
    if (p >= 0) lru_next[p] = nx; else lru_head = nx;
    if (nx >= 0) lru_prev[nx] = p; else lru_tail = p;
    lru_prev[b] = lru_next[b] = -1;
    in_lru[b] = 0;
    --lru_count;
  }

  // a block for a new owner (caller checked availability)
  int32_t take() {
    if (!free_stack.empty()) {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      return b;
    }
    const int32_t b = lru_head;
    lru_remove(b);
    block_of.erase(key_of[b]);
    registered[b] = 0;
    ++evictions;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (registered[b]) lru_push_back(b);
      else free_stack.push_back(b);
    }
  }

  int32_t div_up(int64_t x) const { return static_cast<int32_t>((x + bs - 1) / bs); }

  int32_t blocks_needed(const Seq& s, int32_t n) const {
    if (n <= 0) return 0;
    const int64_t L = s.len;
    int32_t need = div_up(L + n) - div_up(L);
    if (L % bs != 0 && ref[s.table.back()] > 1) need += 1;  // copy-on-write
    return need;
  }

  Key make_key(uint64_t prev, const int32_t* tok) const {
    Key k;
    k.prev = prev;
    k.bs = bs;
    memset(k.tok, 0, sizeof(k.tok));
    memcpy(k.tok, tok, sizeof(int32_t) * bs);
    return k;
  }

  // append n tokens (availability already checked)
  void append(Seq& s, const int32_t* tokens, int32_t n, int64_t* slots, int32_t* cp) {
    cp[0] = cp[1] = -1;
    if (!tokens) s.hashing = false;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t t = s.len;
      const int32_t off = t % bs;
      if (off == 0) {
        const int32_t b = take();
        ref[b] = 1;
        s.table.push_back(b);
      } else if (i == 0 && ref[s.table.back()] > 1) {
        const int32_t src = s.table.back();
        const int32_t dst = take();
        ref[dst] = 1;
        --ref[src];  // still referenced by another table
        s.table.back() = dst;
        cp[0] = src;
        cp[1] = dst;
        ++cow_copies;
      }
      const int32_t b = s.table[t / bs];
      slots[i] = static_cast<int64_t>(b) * bs + off;
      s.len = t + 1;
      if (s.hashing) {
        s.cur[off] = tokens[i];
        if (off == bs - 1) {
          const Key k = make_key(s.chain, s.cur);
          s.chain = chain_hash(k.prev, k.tok, bs);
          if (!registered[b] && block_of.find(k) == block_of.end()) {
            block_of.emplace(k, b);
            key_of[b] = k;
            registered[b] = 1;
          }
        }
      }
    }
  }

  void release_table(Seq& s) {
    for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) release(*it);
    s.table.clear();
  }
};

namespace {

bool valid_bm(const pa_block_manager* bm) { return bm != nullptr; }

}  // namespace

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (block_size != 8 && block_size != 16) return PA_ERR_UNSUPPORTED;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager(num_blocks, block_size);
  if (!bm) return PA_ERR_NO_SPACE;
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_block_manager* bm, int64_t seq_id, int32_t hashing) {
  if (!valid_bm(bm)) return PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id) || bm->swapped.count(seq_id)) return PA_ERR_INVALID_ARG;
  Seq s;
  s.hashing = hashing != 0;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_bm_match_prefix(pa_block_manager* bm, int64_t seq_id, const int32_t* prompt,
                             int32_t n, int32_t* cached_tokens) {
  if (!valid_bm(bm) || !cached_tokens || n < 0 || (n > 0 && !prompt)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  if (s.len != 0 || !s.hashing) return PA_ERR_INVALID_ARG;
  const int32_t bs = bm->bs;
  const int32_t max_blocks = n > 0 ? (n - 1) / bs : 0;
  uint64_t prev = 0;
  for (int32_t i = 0; i < max_blocks; ++i) {
    const Key k = bm->make_key(prev, prompt + static_cast<size_t>(i) * bs);
    auto f = bm->block_of.find(k);
    if (f == bm->block_of.end()) break;
    const int32_t b = f->second;
    if (bm->ref[b] == 0) bm->lru_remove(b);
    ++bm->ref[b];
    s.table.push_back(b);
    s.len += bs;
    ++bm->prefix_hits;
    prev = chain_hash(prev, k.tok, bs);
  }
  s.chain = prev;
  *cached_tokens = s.len;
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids, int32_t n,
                       int64_t* slots, int32_t* copy_src_dst) {
  if (!valid_bm(bm) || n < 0 || !copy_src_dst || (n > 0 && !slots)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  if (static_cast<int64_t>(s.len) + n > INT32_MAX - kMaxBs) return PA_ERR_INVALID_ARG;
  if (bm->blocks_needed(s, n) > bm->available()) return PA_ERR_NO_SPACE;
  bm->append(s, token_ids, n, slots, copy_src_dst);
  return PA_OK;
}

pa_status pa_bm_append_step(pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            const int32_t* token_ids, int64_t* slots, int32_t* copies,
                            int32_t* num_copies) {
  if (!valid_bm(bm) || n < 0 || !num_copies || (n > 0 && (!seq_ids || !slots || !copies)))
    return PA_ERR_INVALID_ARG;
  std::vector<Seq*> ss(static_cast<size_t>(n));
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || !seen.insert(seq_ids[i]).second) return PA_ERR_INVALID_ARG;
    if (it->second.len > INT32_MAX - 2 * kMaxBs) return PA_ERR_INVALID_ARG;
    ss[i] = &it->second;
    need += bm->blocks_needed(it->second, 1);
  }
  if (need > bm->available()) return PA_ERR_NO_SPACE;
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t cp[2];
    bm->append(*ss[i], token_ids ? token_ids + i : nullptr, 1, slots + i, cp);
    if (cp[0] >= 0) {
      copies[2 * nc] = cp[0];
      copies[2 * nc + 1] = cp[1];
      ++nc;
    }
  }
  *num_copies = nc;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!valid_bm(bm)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child) || bm->swapped.count(child))
    return PA_ERR_INVALID_ARG;
  Seq c = it->second;  // table, length, hashing state
  for (int32_t b : c.table) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_block_manager* bm, int64_t seq_id) {
  if (!valid_bm(bm)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) {
    // a swapped-out sequence holds no blocks: forget it
    return bm->swapped.erase(seq_id) ? PA_OK : PA_ERR_INVALID_ARG;
  }
  bm->release_table(it->second);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                         int32_t* num_blocks, int32_t* context_len) {
  if (!valid_bm(bm) || !num_blocks || !context_len || capacity < 0) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (nb > capacity || (nb > 0 && !table)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < nb; ++i) table[i] = s.table[i];
  *num_blocks = nb;
  *context_len = s.len;
  bm->release_table(s);
  bm->swapped.emplace(seq_id, std::move(s));
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                        int32_t* num_blocks) {
  if (!valid_bm(bm) || !num_blocks || capacity < 0) return PA_ERR_INVALID_ARG;
  auto it = bm->swapped.find(seq_id);
  if (it == bm->swapped.end()) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int32_t need = bm->div_up(s.len);
  if (need > capacity || (need > 0 && !table)) return PA_ERR_INVALID_ARG;
  if (need > bm->available()) return PA_ERR_NO_SPACE;
  s.table.reserve(static_cast<size_t>(need));
  for (int32_t i = 0; i < need; ++i) {
    const int32_t b = bm->take();
    bm->ref[b] = 1;
    s.table.push_back(b);
    table[i] = b;
  }
  *num_blocks = need;
  bm->seqs.emplace(seq_id, std::move(s));
  bm->swapped.erase(it);
  return PA_OK;
}

pa_status pa_bm_get_table(const pa_block_manager* bm, int64_t seq_id, int32_t* row,
                          int32_t capacity, int32_t* num_blocks, int32_t* context_len) {
  if (!valid_bm(bm) || !num_blocks || !context_len || capacity < 0) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  const Seq& s = it->second;
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (nb > capacity || (nb > 0 && !row)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < nb; ++i) row[i] = s.table[i];
  *num_blocks = nb;
  *context_len = s.len;
  return PA_OK;
}

pa_status pa_bm_fill_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            int32_t* tables, int32_t max_blocks_per_seq, int32_t* context_lens) {
  if (!valid_bm(bm) || n < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !tables || !context_lens)) return PA_ERR_INVALID_ARG;
  std::vector<const Seq*> ss(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {  // validate everything before writing
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    if (static_cast<int32_t>(it->second.table.size()) > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
    ss[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t* row = tables + static_cast<size_t>(i) * max_blocks_per_seq;
    const int32_t nb = static_cast<int32_t>(ss[i]->table.size());
    for (int32_t j = 0; j < nb; ++j) row[j] = ss[i]->table[j];
    for (int32_t j = nb; j < max_blocks_per_seq; ++j) row[j] = -1;
    context_lens[i] = ss[i]->len;
  }
  return PA_OK;
}

pa_status pa_bm_sort_longest_first(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                   int64_t* out_ids) {
  if (!valid_bm(bm) || n < 0 || (n > 0 && (!seq_ids || !out_ids))) return PA_ERR_INVALID_ARG;
  std::vector<std::pair<int32_t, int64_t>> v(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    v[i] = {it->second.len, seq_ids[i]};
  }
  std::stable_sort(v.begin(), v.end(),
                   [](const std::pair<int32_t, int64_t>& x, const std::pair<int32_t, int64_t>& y) {
                     return x.first > y.first;
                   });
  for (int32_t i = 0; i < n; ++i) out_ids[i] = v[i].second;
  return PA_OK;
}

pa_status pa_bm_common_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                              int32_t* prefix_blocks) {
  if (!valid_bm(bm) || n < 0 || !prefix_blocks || (n > 0 && !seq_ids)) return PA_ERR_INVALID_ARG;
  std::vector<const Seq*> ss(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    ss[i] = &it->second;
  }
  int32_t k = 0;
  if (n > 0) {
    int32_t min_len = ss[0]->len;
    for (const Seq* q : ss) min_len = std::min(min_len, q->len);
    k = std::min(static_cast<int32_t>(ss[0]->table.size()), min_len / bm->bs);
    for (int32_t i = 1; i < n && k > 0; ++i) {
      const std::vector<int32_t>& t = ss[i]->table;
      int32_t j = 0;
      while (j < k && j < static_cast<int32_t>(t.size()) && t[j] == ss[0]->table[j]) ++j;
      k = j;
    }
  }
  *prefix_blocks = k;
  return PA_OK;
}

pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* st) {
  if (!valid_bm(bm) || !st) return PA_ERR_INVALID_ARG;
  int32_t used = 0;
  for (int32_t r : bm->ref) used += r > 0;
  st->num_blocks = bm->num_blocks;
  st->free_blocks = static_cast<int32_t>(bm->free_stack.size());
  st->cached_blocks = bm->lru_count;
  st->used_blocks = used;
  st->num_seqs = static_cast<int32_t>(bm->seqs.size());
  st->swapped_seqs = static_cast<int32_t>(bm->swapped.size());
  st->prefix_hit_blocks = bm->prefix_hits;
  st->cow_copies = bm->cow_copies;
  st->evictions = bm->evictions;
  return PA_OK;
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block) {
  if (!valid_bm(bm) || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pa_bm_blocks_needed(const pa_block_manager* bm, int64_t seq_id, int32_t n) {
  if (!valid_bm(bm) || n < 0) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return -1;
  return bm->blocks_needed(it->second, n);
}

}  // extern "C"
