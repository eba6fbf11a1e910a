// Host block manager: FIFO free pool, per-block reference counts,
// append-slot allocation with copy-on-write of a shared partial last block.
//
// Blocks are allocated only when a sequence needs one and are returned as
// soon as their last user goes away (ybb.press, "vLLM PagedAttention
// 大模型推理架构深度实战", §2.2); every decode iteration checks whether the
// sequence needs a new block (§6); shared blocks are reference counted and
// a sequence about to modify a shared block copies it first (§2.3).
//
// Swapping: when device memory runs short, the KV of low-priority sequences
// moves to CPU memory and comes back later (§3.2; the scheduler swaps
// sequences out and in under memory pressure, §6; swapped-out KV stays in
// host memory, §9 item 5).  A second FIFO pool of host blocks holds them:
// swap_out of a set of sequences gives every distinct device block they
// reference one host block, in walk order (sequences as listed, tables in
// logical order), and emits the (device, host) copy pairs; each device
// block loses the set's references and returns to the device pool, in the
// same walk order, when its count reaches zero.  swap_in is the mirror.
//
// Prefix caching: requests that share a prompt reuse its cached KV blocks
// instead of recomputing them (explore.n1n.ai, "vLLM 深度解析", section
// "vLLM 生态的核心功能亮点"; ybb.press §7.3; gheillcoat.github.io, "概念-vLLM",
// section 3).  A full block written with token ids is keyed by FNV-1a 64 over
// its parent's key (8 bytes, little-endian; 0 for a first block) and its 16
// ids (4 bytes each, little-endian); a prompt reuses the longest run of its
// leading full blocks whose key, parent key and ids all match.  A registered
// block whose count drops to zero becomes evictable (least recently released
// first) instead of free; allocation takes free blocks first, then evicts.
//
// The queue discipline, the choice of which sharer copies (the one that
// appends, while the block is still shared) and the all-or-nothing rule make
// the tables reproducible; they are readings, the pages fix none of them.
#include <array>
#include <algorithm>
#include <cstdint>
#include <deque>
#include <iterator>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pagedkv::fail;

namespace {

constexpr int32_t kMaxBlock = 64;        // largest block size accepted

struct Seq {
  std::vector<int32_t> table;  // logical -> physical block (host block if on_host)
  int32_t len = 0;             // tokens appended so far
  bool on_host = false;        // swapped out
  bool track = false;          // token ids known (prefix caching)
  std::vector<int32_t> toks;   // token ids, when tracked
  uint64_t last_key = 0;       // key of the last full block
};

uint64_t fnv1a64_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

// Key of a full block of n tokens: FNV-1a 64 over the parent key then the ids.
uint64_t block_key(uint64_t parent, const int32_t* toks, int n) {
  unsigned char buf[8 + 4 * kMaxBlock];
  for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(parent >> (8 * i));
  for (int t = 0; t < n; ++t) {
    const uint32_t v = static_cast<uint32_t>(toks[t]);
    for (int i = 0; i < 4; ++i) buf[8 + 4 * t + i] = static_cast<unsigned char>(v >> (8 * i));
  }
  return fnv1a64_bytes(0xCBF29CE484222325ull, buf, 8 + 4 * static_cast<size_t>(n));
}

// A FIFO free pool with reference counts.
struct Pool {
  std::deque<int32_t> free_q;
  std::vector<int32_t> ref;

  bool init(int32_t n, const int32_t* order) {
    ref.assign(n, 0);
    free_q.clear();
    if (!order) {
      for (int32_t i = 0; i < n; ++i) free_q.push_back(i);
      return true;
    }
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= n || seen[b]) return false;
      seen[b] = 1;
      free_q.push_back(b);
    }
    return true;
  }
};

}  // namespace

struct pa_bm {
  int32_t bs = PA_BLOCK_SIZE;                    // tokens per block
  int32_t num_blocks = 0;
  int32_t num_host_blocks = 0;
  Pool dev;
  Pool host;
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache (device blocks)
  bool caching = false;
  std::unordered_map<uint64_t, int32_t> cache;   // key -> block
  std::vector<char> registered;                  // per block
  std::vector<uint64_t> bkey, bparent;
  std::vector<int32_t> btok;                     // [block][bs] ids of registered blocks
  std::list<int32_t> lru;                        // evictable, oldest release first
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<char> in_lru;
  int64_t queried = 0, hits = 0;

  void init_cache_state() {
    registered.assign(num_blocks, 0);
    bkey.assign(num_blocks, 0);
    bparent.assign(num_blocks, 0);
    btok.assign(static_cast<size_t>(num_blocks) * bs, 0);
    lru_pos.assign(num_blocks, lru.end());
    in_lru.assign(num_blocks, 0);
  }

  // Blocks an allocation can take: free plus evictable.
  int64_t available() const {
    return static_cast<int64_t>(dev.free_q.size()) + static_cast<int64_t>(lru.size());
  }

  // Blocks an append of n tokens to `s` takes from the pool.
  int64_t blocks_needed(const Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    const int64_t p = s.len;
    int64_t fresh = (p + n + bs - 1) / bs - (p + bs - 1) / bs;
    int64_t cow = (p % bs != 0 && dev.ref[s.table.back()] > 1) ? 1 : 0;
    return fresh + cow;
  }

  // A device block for a new use (count 1): free first, else evict.
  int32_t pop() {
    int32_t b;
    if (!dev.free_q.empty()) {
      b = dev.free_q.front();
      dev.free_q.pop_front();
    } else {
      b = lru.front();
      lru.pop_front();
      in_lru[b] = 0;
      cache.erase(bkey[b]);
      registered[b] = 0;
    }
    dev.ref[b] = 1;
    return b;
  }

  // A device block's count reached zero.
  void release(int32_t b) {
    if (registered[b]) {
      lru.push_back(b);
      lru_pos[b] = std::prev(lru.end());
      in_lru[b] = 1;
    } else {
      dev.free_q.push_back(b);
    }
  }

  void revive(int32_t b) {
    lru.erase(lru_pos[b]);
    in_lru[b] = 0;
  }

  // Records a token id; registers the block it completes.
  void note_token(Seq& s, int32_t tok) {
    if (!s.track) return;
    s.toks.push_back(tok);
    if (s.toks.size() % bs != 0) return;
    const int32_t* blk = s.toks.data() + s.toks.size() - bs;
    const uint64_t key = block_key(s.last_key, blk, bs);
    const int32_t b = s.table[s.toks.size() / bs - 1];
    if (!cache.count(key) && !registered[b]) {
      cache.emplace(key, b);
      registered[b] = 1;
      bkey[b] = key;
      bparent[b] = s.last_key;
      for (int i = 0; i < bs; ++i) btok[static_cast<size_t>(b) * bs + i] = blk[i];
    }
    s.last_key = key;
  }

  // Appends one token; the caller has checked that blocks are available.
  int64_t append_one(Seq& s, int32_t* cow_src, int32_t* cow_dst) {
    const int32_t p = s.len;
    if (p % bs == 0) {
      s.table.push_back(pop());
    } else if (dev.ref[s.table.back()] > 1) {
      const int32_t old = s.table.back();
      const int32_t b = pop();
      dev.ref[old] -= 1;
      s.table.back() = b;
      *cow_src = old;
      *cow_dst = b;
    }
    s.len = p + 1;
    return static_cast<int64_t>(s.table[p / bs]) * bs + p % bs;
  }
};

extern "C" {

pa_bm* pa_bm_create_ex(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       int32_t num_host_blocks, const int32_t* host_free_order) {
  if (num_blocks < 0 || num_host_blocks < 0) {
    fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks %d, num_host_blocks %d", num_blocks,
         num_host_blocks);
    return nullptr;
  }
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) {
    fail(PA_ERR_UNSUPPORTED, "pa_bm_create: block_size %d (8, 16, 32 or 64)", block_size);
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm;
  if (!bm) {
    fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
    return nullptr;
  }
  bm->bs = block_size;
  bm->num_blocks = num_blocks;
  bm->num_host_blocks = num_host_blocks;
  if (!bm->dev.init(num_blocks, free_order)) {
    delete bm;
    fail(PA_ERR_INVALID_ARG, "pa_bm_create: free_order is not a permutation of 0..%d",
         num_blocks - 1);
    return nullptr;
  }
  if (!bm->host.init(num_host_blocks, host_free_order)) {
    delete bm;
    fail(PA_ERR_INVALID_ARG, "pa_bm_create: host_free_order is not a permutation of 0..%d",
         num_host_blocks - 1);
    return nullptr;
  }
  bm->init_cache_state();
  return bm;
}

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size,
                    const int32_t* free_order) {
  return pa_bm_create_ex(num_blocks, block_size, free_order, 0, nullptr);
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: null manager");
  if (bm->seqs.count(seq_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_add_seq: sequence %lld exists",
                (long long)seq_id);
  Seq s;
  s.track = bm->caching;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: null manager");
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_fork: unknown parent %lld",
                (long long)parent_id);
  if (bm->seqs.count(child_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_fork: child %lld exists",
                (long long)child_id);
  if (it->second.on_host)
    return fail(PA_ERR_SWAPPED, "pa_bm_fork: parent %lld is swapped out",
                (long long)parent_id);
  Seq child = it->second;  // copy before emplace may rehash
  for (int32_t b : child.table) bm->dev.ref[b] += 1;
  bm->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

}  // extern "C"

namespace {

// Appends n tokens (ids: their token ids, or null when unknown); all or nothing.
pa_status append_n(pa_bm* bm, int64_t seq_id, int32_t n, const int32_t* ids, int64_t* slots,
                   int32_t* cow_src, int32_t* cow_dst, const char* fn) {
  if (!bm || !cow_src || !cow_dst || (n > 0 && !slots))
    return fail(PA_ERR_INVALID_ARG, "%s: null argument", fn);
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "%s: n = %d < 0", fn, n);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "%s: unknown sequence %lld", fn, (long long)seq_id);
  Seq& s = it->second;
  if (s.on_host)
    return fail(PA_ERR_SWAPPED, "%s: sequence %lld is swapped out", fn, (long long)seq_id);
  if (static_cast<int64_t>(s.len) + n > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: length overflow", fn);
  const int64_t need = bm->blocks_needed(s, n);
  if (need > bm->available())
    return fail(PA_ERR_NO_BLOCKS, "%s: sequence %lld needs %lld blocks, %lld available", fn,
                (long long)seq_id, (long long)need, (long long)bm->available());
  if (!ids && n > 0) {
    s.track = false;
    s.toks.clear();
  }
  *cow_src = -1;
  *cow_dst = -1;
  for (int32_t i = 0; i < n; ++i) {
    slots[i] = bm->append_one(s, cow_src, cow_dst);
    if (ids) bm->note_token(s, ids[i]);
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_bm_append_tokens(pa_bm* bm, int64_t seq_id, int32_t n,
                              int64_t* slots, int32_t* cow_src,
                              int32_t* cow_dst) {
  return append_n(bm, seq_id, n, nullptr, slots, cow_src, cow_dst, "pa_bm_append_tokens");
}

pa_status pa_bm_append_token_ids(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                                 int64_t* slots, int32_t* cow_src, int32_t* cow_dst) {
  if (n > 0 && !tokens)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_append_token_ids: null tokens");
  return append_n(bm, seq_id, n, tokens, slots, cow_src, cow_dst, "pa_bm_append_token_ids");
}

pa_status pa_bm_enable_prefix_caching(pa_bm* bm) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_enable_prefix_caching: null manager");
  bm->caching = true;
  return PA_OK;
}

pa_status pa_bm_add_seq_prompt(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                               int64_t* slots, int32_t* num_cached) {
  if (!bm || !num_cached || n < 0 || (n > 0 && (!tokens || !slots)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_prompt: bad argument");
  if (bm->seqs.count(seq_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_add_seq_prompt: sequence %lld exists",
                (long long)seq_id);
  // the longest run of leading full blocks found in the cache
  std::vector<int32_t> hit;
  uint64_t parent = 0;
  if (bm->caching) {
    for (int32_t k = 0; k < n / bm->bs; ++k) {
      const int32_t* blk = tokens + static_cast<int64_t>(k) * bm->bs;
      const uint64_t key = block_key(parent, blk, bm->bs);
      auto c = bm->cache.find(key);
      if (c == bm->cache.end()) break;
      const int32_t b = c->second;
      bool same = bm->bparent[b] == parent;
      for (int i = 0; i < bm->bs && same; ++i) same = bm->btok[static_cast<size_t>(b) * bm->bs + i] == blk[i];
      if (!same) break;
      hit.push_back(b);
      parent = key;
    }
  }
  int64_t revived = 0;
  for (int32_t b : hit) revived += bm->dev.ref[b] == 0 ? 1 : 0;
  const int64_t need = (static_cast<int64_t>(n) + bm->bs - 1) / bm->bs - static_cast<int64_t>(hit.size());
  if (need > bm->available() - revived)
    return fail(PA_ERR_NO_BLOCKS, "pa_bm_add_seq_prompt: prompt needs %lld new blocks, %lld available",
                (long long)need, (long long)(bm->available() - revived));
  Seq s;
  s.track = bm->caching;
  if (bm->caching) {
    bm->queried += n / bm->bs;
    bm->hits += static_cast<int64_t>(hit.size());
  }
  for (int32_t b : hit) {
    if (bm->dev.ref[b] == 0) bm->revive(b);
    bm->dev.ref[b] += 1;
    s.table.push_back(b);
  }
  const int32_t nc = bm->bs * static_cast<int32_t>(hit.size());
  s.len = nc;
  if (s.track) s.toks.assign(tokens, tokens + nc);
  s.last_key = parent;
  for (int32_t p = 0; p < nc; ++p)
    slots[p] = static_cast<int64_t>(s.table[p / bm->bs]) * bm->bs + p % bm->bs;
  Seq& stored = bm->seqs.emplace(seq_id, std::move(s)).first->second;
  int32_t cs = -1, cd = -1;
  for (int32_t p = nc; p < n; ++p) {
    slots[p] = bm->append_one(stored, &cs, &cd);
    bm->note_token(stored, tokens[p]);
  }
  *num_cached = nc;
  return PA_OK;
}

pa_status pa_bm_shared_prefix_groups(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                     int32_t* groups, int32_t cap, int32_t* num_groups) {
  if (!bm || !num_groups || n < 0 || cap < 0 || (n > 0 && !seq_ids) || (cap > 0 && !groups))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_shared_prefix_groups: bad argument");
  std::vector<const Seq*> ss(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_shared_prefix_groups: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (it->second.on_host)
      return fail(PA_ERR_SWAPPED, "pa_bm_shared_prefix_groups: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    ss[i] = &it->second;
  }
  int32_t k = 0;
  for (int32_t i = 0; i < n;) {
    const std::vector<int32_t>& t0 = ss[i]->table;
    int32_t j = i + 1;
    while (j < n && !t0.empty() && !ss[j]->table.empty() && ss[j]->table[0] == t0[0]) ++j;
    if (j - i >= 2) {
      int32_t m = INT32_MAX;
      for (int32_t r = i; r < j; ++r) m = std::min(m, (ss[r]->len - 1) / bm->bs);
      for (int32_t r = i + 1; r < j; ++r) {
        const std::vector<int32_t>& t = ss[r]->table;
        int32_t c = 0;
        const int32_t lim = static_cast<int32_t>(std::min(t.size(), t0.size()));
        while (c < lim && t[c] == t0[c]) ++c;
        m = std::min(m, c);
      }
      if (m >= 1) {
        if (k >= cap)
          return fail(PA_ERR_INVALID_ARG, "pa_bm_shared_prefix_groups: more than %d groups", cap);
        groups[3 * k] = i;
        groups[3 * k + 1] = j - i;
        groups[3 * k + 2] = m;
        ++k;
      }
    }
    i = j;
  }
  *num_groups = k;
  return PA_OK;
}

pa_status pa_bm_cache_stats(const pa_bm* bm, int64_t* queried_blocks, int64_t* hit_blocks,
                            int32_t* registered_blocks, int32_t* evictable_blocks) {
  if (!bm || !queried_blocks || !hit_blocks || !registered_blocks || !evictable_blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_stats: null argument");
  *queried_blocks = bm->queried;
  *hit_blocks = bm->hits;
  *registered_blocks = static_cast<int32_t>(bm->cache.size());
  *evictable_blocks = static_cast<int32_t>(bm->lru.size());
  return PA_OK;
}

pa_status pa_bm_append_slot(pa_bm* bm, int64_t seq_id, int64_t* slot,
                            int32_t* cow_src, int32_t* cow_dst) {
  if (!slot) return fail(PA_ERR_INVALID_ARG, "pa_bm_append_slot: null slot");
  return pa_bm_append_tokens(bm, seq_id, 1, slot, cow_src, cow_dst);
}

pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seq_ids, int32_t n,
                             int64_t* slots, int32_t* cow_pairs,
                             int32_t* num_pairs) {
  if (!bm || !num_pairs || (n > 0 && (!seq_ids || !slots || !cow_pairs)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: null argument");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: n < 0");
  // Validate everything and count blocks first: all or nothing.
  std::vector<Seq*> ss(n);
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_append_batch: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (!seen.insert(seq_ids[i]).second)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: sequence %lld listed twice",
                  (long long)seq_ids[i]);
    ss[i] = &it->second;
    if (ss[i]->on_host)
      return fail(PA_ERR_SWAPPED, "pa_bm_append_batch: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    if (ss[i]->len == INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: length overflow");
  }
  // Copies caused by earlier members of the batch lower the counts later
  // members see, so count in order on a scratch copy of the touched counts.
  std::unordered_map<int32_t, int32_t> ref_delta;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *ss[i];
    if (s.len % bm->bs == 0) {
      need += 1;
    } else {
      const int32_t last = s.table.back();
      const int32_t r = bm->dev.ref[last] + ref_delta[last];
      if (r > 1) {
        need += 1;
        ref_delta[last] -= 1;
      }
    }
  }
  if (need > bm->available())
    return fail(PA_ERR_NO_BLOCKS, "pa_bm_append_batch: batch needs %lld blocks, %lld available",
                (long long)need, (long long)bm->available());
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src = -1, dst = -1;
    ss[i]->track = false;                // token ids unknown
    ss[i]->toks.clear();
    slots[i] = bm->append_one(*ss[i], &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * np] = src;
      cow_pairs[2 * np + 1] = dst;
      ++np;
    }
  }
  *num_pairs = np;
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_free_seq: null manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_free_seq: unknown sequence %lld",
                (long long)seq_id);
  for (int32_t b : it->second.table) {
    if (it->second.on_host) {
      if (--bm->host.ref[b] == 0) bm->host.free_q.push_back(b);
    } else if (--bm->dev.ref[b] == 0) {
      bm->release(b);
    }
  }
  bm->seqs.erase(it);
  return PA_OK;
}

}  // extern "C"

namespace {

// swap_out (to_host) / swap_in of a set of sequences; all or nothing.
pa_status move_seqs(pa_bm* bm, const int64_t* seq_ids, int32_t n, bool to_host,
                    int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs, const char* fn) {
  if (!bm || !num_pairs || n < 0 || pairs_cap < 0 || (n > 0 && !seq_ids) ||
      (pairs_cap > 0 && !pairs))
    return fail(PA_ERR_INVALID_ARG, "%s: bad argument", fn);
  std::vector<Seq*> ss(n);
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < n; ++i)      // a repeated id is reported before anything else
    if (!seen.insert(seq_ids[i]).second)
      return fail(PA_ERR_INVALID_ARG, "%s: sequence %lld listed twice", fn,
                  (long long)seq_ids[i]);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "%s: unknown sequence %lld", fn, (long long)seq_ids[i]);
    if (it->second.on_host == to_host)
      return fail(PA_ERR_SWAPPED, "%s: sequence %lld is already %s", fn, (long long)seq_ids[i],
                  to_host ? "swapped out" : "on the device");
    ss[i] = &it->second;
  }
  Pool& src = to_host ? bm->dev : bm->host;
  Pool& dst = to_host ? bm->host : bm->dev;
  std::vector<int32_t> order;
  std::unordered_map<int32_t, int32_t> mapping;
  for (Seq* s : ss)
    for (int32_t b : s->table)
      if (mapping.emplace(b, -1).second) order.push_back(b);
  const int64_t room = to_host ? static_cast<int64_t>(bm->host.free_q.size()) : bm->available();
  if (static_cast<int64_t>(order.size()) > room)
    return fail(PA_ERR_NO_BLOCKS, "%s: %zu blocks to move, %lld available", fn, order.size(),
                (long long)room);
  if (static_cast<int64_t>(order.size()) > pairs_cap)
    return fail(PA_ERR_INVALID_ARG, "%s: pairs buffer holds %d pairs, %zu needed", fn,
                pairs_cap, order.size());
  for (size_t k = 0; k < order.size(); ++k) {
    int32_t d;
    if (to_host) {
      d = dst.free_q.front();
      dst.free_q.pop_front();
    } else {
      d = bm->pop();
    }
    dst.ref[d] = 0;
    mapping[order[k]] = d;
    pairs[2 * k] = order[k];
    pairs[2 * k + 1] = d;
  }
  for (Seq* s : ss) {
    for (int32_t& b : s->table) {
      const int32_t d = mapping[b];
      dst.ref[d] += 1;
      if (--src.ref[b] == 0) {
        if (to_host) bm->release(b);
        else src.free_q.push_back(b);
      }
      b = d;
    }
    s->on_host = to_host;
  }
  *num_pairs = static_cast<int32_t>(order.size());
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_bm_swap_out(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs,
                         int32_t pairs_cap, int32_t* num_pairs) {
  return move_seqs(bm, seq_ids, n, true, pairs, pairs_cap, num_pairs, "pa_bm_swap_out");
}

pa_status pa_bm_swap_in(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs,
                        int32_t pairs_cap, int32_t* num_pairs) {
  return move_seqs(bm, seq_ids, n, false, pairs, pairs_cap, num_pairs, "pa_bm_swap_in");
}

int32_t pa_bm_num_free_host(const pa_bm* bm) {
  return bm ? static_cast<int32_t>(bm->host.free_q.size()) : -1;
}

int32_t pa_bm_host_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_host_blocks) return -1;
  return bm->host.ref[block];
}

pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq_id, int32_t* swapped) {
  if (!bm || !swapped) return fail(PA_ERR_INVALID_ARG, "pa_bm_is_swapped: null argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_is_swapped: unknown sequence %lld",
                (long long)seq_id);
  *swapped = it->second.on_host ? 1 : 0;
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_bm* bm) {
  return bm ? static_cast<int32_t>(bm->available()) : -1;
}

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->dev.ref[block];
}

pa_status pa_bm_length(const pa_bm* bm, int64_t seq_id, int32_t* len) {
  if (!bm || !len) return fail(PA_ERR_INVALID_ARG, "pa_bm_length: null argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_length: unknown sequence %lld",
                (long long)seq_id);
  *len = it->second.len;
  return PA_OK;
}

pa_status pa_bm_pack(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                     int32_t* block_tables, int32_t cap, int32_t* context_lens) {
  if (!bm || (n > 0 && (!seq_ids || !block_tables || !context_lens)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_pack: null argument");
  if (n < 0 || cap < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_pack: negative size");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_pack: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (it->second.on_host)
      return fail(PA_ERR_SWAPPED, "pa_bm_pack: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    if (static_cast<int64_t>(it->second.table.size()) > cap)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_pack: sequence %lld has %zu blocks > cap %d",
                  (long long)seq_ids[i], it->second.table.size(), cap);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + static_cast<int64_t>(i) * cap;
    const int32_t m = static_cast<int32_t>(s.table.size());
    for (int32_t j = 0; j < m; ++j) row[j] = s.table[j];
    for (int32_t j = m; j < cap; ++j) row[j] = -1;
    context_lens[i] = s.len;
  }
  return PA_OK;
}

}  // extern "C"
