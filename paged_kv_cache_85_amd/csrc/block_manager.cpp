// Host block manager: the bookkeeping that turns sequences of token IDs into
// the paged-attention kernels' inputs (block tables, slot mapping, cached
// prefix lengths).
//
// The engines keep this state on the CPU ("nano-vLLM Part 4", section 1: the
// block manager holds block IDs, reference counts and prefix-hash metadata,
// none of it in GPU memory).  The pool is a fixed set of equal blocks handed
// out and returned in constant time ("mini-vLLM", features list); full blocks are
// registered under a hash of their tokens chained with the previous block's
// hash, so a new sequence that starts with the same full blocks reuses them
// with a reference count (smzdm Nano-vLLM walk-through, scheduling and memory:
// a shared system prompt is computed once; "nano-vLLM Part 4", comparison
// table: an exact full-block prefix cache).  The key of block i is a 64-bit
// hash chained over all the sequence's tokens up to the end of block i (a
// block's K/V depends on every earlier token), and a lookup also compares the
// block's own tokens: the reuse is exact up to a collision of that 64-bit
// chain hash, as in the engines the pages describe.  Freed blocks keep
// their registration until the free list hands them out again, so a
// sequence preempted and recomputed finds its computed blocks (smzdm
// walk-through, scheduling and memory; "mini-vLLM": preemption must hand
// back every block).
//
// Free list: an intrusive doubly linked list over block IDs (push at the
// tail, pop at the head, unlink from the middle when a cached free block is
// reused), so every operation on it is O(1).
#include <stdint.h>

#include <algorithm>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Block {
  int32_t ref = 0;
  bool hashed = false;  // registered under `hash` in the prefix map
  uint64_t hash = 0;
  int32_t prev = -1, next = -1;  // free-list links
  bool free = true;
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // chain hash of each full block
  int32_t num_cached = 0;  // leading tokens whose K/V the cache already held
};

// 64-bit key of a block's tokens chained with the previous block's hash.
// Tokens go round-robin into four lanes, each a (xor, multiply, xor-shift)
// chain, so the four multiplies of consecutive tokens overlap instead of
// forming one serial dependence; the lanes are then folded in order through
// the splitmix64 finaliser.  Only a lookup key: hits also compare the block's
// own tokens.
uint64_t mix(uint64_t h) {
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ULL;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebULL;
  h ^= h >> 31;
  return h;
}

inline uint64_t lane_step(uint64_t x, int32_t t) {
  x = (x ^ (uint64_t)(uint32_t)t) * 0xff51afd7ed558ccdULL;
  return x ^ (x >> 32);
}

uint64_t block_hash(uint64_t prev, const int32_t* t, int n) {
  uint64_t l0 = prev ^ 0x243f6a8885a308d3ULL, l1 = prev ^ 0x13198a2e03707344ULL,
           l2 = prev ^ 0xa4093822299f31d0ULL, l3 = prev ^ 0x082efa98ec4e6c89ULL;
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    l0 = lane_step(l0, t[i]);
    l1 = lane_step(l1, t[i + 1]);
    l2 = lane_step(l2, t[i + 2]);
    l3 = lane_step(l3, t[i + 3]);
  }
  if (i < n) l0 = lane_step(l0, t[i++]);
  if (i < n) l1 = lane_step(l1, t[i++]);
  if (i < n) l2 = lane_step(l2, t[i++]);
  uint64_t h = mix((uint64_t)n ^ 0x9e3779b97f4a7c15ULL);
  h = mix(h ^ l0);
  h = mix(h ^ l1);
  h = mix(h ^ l2);
  return mix(h ^ l3);
}

}  // namespace

struct pa_block_manager {
  int32_t bs;
  std::vector<Block> blocks;
  std::vector<int32_t> content;  // tokens of each block (bs per block), valid when hashed
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Seq> seqs;

  void push_free(int32_t b) {
    Block& k = blocks[b];
    k.free = true;
    k.prev = tail;
    k.next = -1;
    if (tail >= 0) blocks[tail].next = b; else head = b;
    tail = b;
    ++nfree;
  }
  void unlink(int32_t b) {
    Block& k = blocks[b];
    if (k.prev >= 0) blocks[k.prev].next = k.next; else head = k.next;
    if (k.next >= 0) blocks[k.next].prev = k.prev; else tail = k.prev;
    k.prev = k.next = -1;
    k.free = false;
    --nfree;
  }
  // A block for new content: the head of the free list, dropping any old
  // registration (its tokens are about to be overwritten).
  int32_t take_fresh() {
    const int32_t b = head;
    unlink(b);
    Block& k = blocks[b];
    if (k.hashed) {
      auto it = by_hash.find(k.hash);
      if (it != by_hash.end() && it->second == b) by_hash.erase(it);
      k.hashed = false;
    }
    k.ref = 1;
    return b;
  }
  void register_full(int32_t b, uint64_t h, const int32_t* t) {
    Block& k = blocks[b];
    k.hashed = true;
    k.hash = h;
    std::copy(t, t + bs, content.begin() + (size_t)b * bs);
    by_hash[h] = b;
  }
  // Cached block registered under chain hash h whose own tokens are t; or -1.
  int32_t lookup(uint64_t h, const int32_t* t) const {
    auto it = by_hash.find(h);
    if (it == by_hash.end()) return -1;
    const int32_t b = it->second;
    const int32_t* c = content.data() + (size_t)b * bs;
    for (int i = 0; i < bs; ++i)
      if (c[i] != t[i]) return -1;
    return b;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1 || (long long)num_blocks * block_size > INT32_MAX)
    return nullptr;
  pa_block_manager* m = new pa_block_manager();
  m->bs = block_size;
  m->blocks.resize(num_blocks);
  m->content.assign((size_t)num_blocks * block_size, 0);
  for (int32_t b = 0; b < num_blocks; ++b) m->push_free(b);
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_num_free(const pa_block_manager* m) { return m ? m->nfree : -1; }

int pa_bm_allocate(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                   int32_t num_tokens, int32_t* num_cached_tokens) {
  if (!m || num_tokens < 1 || !tokens) return PA_E_INVAL;
  if (m->seqs.count(seq_id)) return PA_E_INVAL;
  const int bs = m->bs;
  const int nblocks = (num_tokens + bs - 1) / bs;
  // Plan first (no state change), so that a shortage leaves everything as it
  // was.  Each full block is hashed once; the partial last block never is.
  const int nfull = num_tokens / bs;
  std::vector<uint64_t> h((size_t)nfull);
  for (int i = 0; i < nfull; ++i)
    h[i] = block_hash(i ? h[i - 1] : 0, tokens + (size_t)i * bs, bs);
  std::vector<int32_t> hit;
  for (int i = 0; i < nfull; ++i) {
    const int32_t b = m->lookup(h[i], tokens + (size_t)i * bs);
    if (b < 0) break;
    hit.push_back(b);
  }
  int need_fresh = nblocks - (int)hit.size();
  int free_after = m->nfree;
  for (int32_t b : hit)
    if (m->blocks[b].free) --free_after;  // a cached free block leaves the list
  if (need_fresh > free_after) return PA_E_NOMEM;

  Seq s;
  s.tokens.assign(tokens, tokens + num_tokens);
  s.blocks.reserve(nblocks);
  s.hashes = h;
  for (int i = 0; i < nblocks; ++i) {
    if (i < (int)hit.size()) {
      const int32_t b = hit[i];
      Block& k = m->blocks[b];
      if (k.free) {
        m->unlink(b);
        k.ref = 1;
      } else {
        ++k.ref;
      }
      s.blocks.push_back(b);
      s.num_cached += bs;
    } else {
      const int32_t b = m->take_fresh();
      if (i < nfull) m->register_full(b, h[i], tokens + (size_t)i * bs);
      s.blocks.push_back(b);
    }
  }
  // A fully cached prompt still recomputes its last token (a step needs at
  // least one query row).
  if (s.num_cached == num_tokens) s.num_cached = num_tokens - 1;
  if (num_cached_tokens) *num_cached_tokens = s.num_cached;
  m->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_append(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot) {
  if (!m) return PA_E_INVAL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_E_INVAL;
  Seq& s = it->second;
  const int bs = m->bs;
  const int n = (int)s.tokens.size();  // position of the new token
  if (n % bs == 0) {                    // it opens a new block
    if (m->nfree == 0) return PA_E_NOMEM;
    s.blocks.push_back(m->take_fresh());
  }
  s.tokens.push_back(token);
  const int32_t b = s.blocks[n / bs];
  if ((n + 1) % bs == 0) {  // the block is now full: register it
    const int i = n / bs;  // index of the block just filled
    const uint64_t h = block_hash(i ? s.hashes[i - 1] : 0, s.tokens.data() + (size_t)i * bs, bs);
    s.hashes.push_back(h);
    m->register_full(b, h, s.tokens.data() + (size_t)i * bs);
  }
  if (slot) *slot = b * bs + n % bs;
  return PA_OK;
}

int pa_bm_free(pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_E_INVAL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_E_INVAL;
  const std::vector<int32_t>& bl = it->second.blocks;
  for (auto r = bl.rbegin(); r != bl.rend(); ++r) {  // last blocks freed first
    Block& k = m->blocks[*r];
    if (--k.ref == 0) m->push_free(*r);
  }
  m->seqs.erase(it);
  return PA_OK;
}

int pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* out, int32_t capacity,
                      int32_t* num_blocks) {
  if (!m) return PA_E_INVAL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_E_INVAL;
  const std::vector<int32_t>& bl = it->second.blocks;
  if (num_blocks) *num_blocks = (int32_t)bl.size();
  if ((int32_t)bl.size() > capacity) return PA_E_INVAL;
  if (out)
    for (size_t i = 0; i < bl.size(); ++i) out[i] = bl[i];
  return PA_OK;
}

int pa_bm_seq_info(const pa_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                   int32_t* num_cached_tokens) {
  if (!m) return PA_E_INVAL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_E_INVAL;
  if (num_tokens) *num_tokens = (int32_t)it->second.tokens.size();
  if (num_cached_tokens) *num_cached_tokens = it->second.num_cached;
  return PA_OK;
}

int pa_bm_slots(const pa_block_manager* m, int64_t seq_id, int32_t first, int32_t count,
                int32_t* slots) {
  if (!m || count < 0 || first < 0) return PA_E_INVAL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_E_INVAL;
  const Seq& s = it->second;
  if ((long long)first + count > (long long)s.blocks.size() * m->bs) return PA_E_INVAL;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t j = first + i;
    slots[i] = s.blocks[j / m->bs] * m->bs + j % m->bs;
  }
  return PA_OK;
}

int pa_bm_append_batch(pa_block_manager* m, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t num_seqs, int32_t* slots, int32_t* num_done) {
  if (num_done) *num_done = 0;
  if (!m || num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !tokens || !slots))) return PA_E_INVAL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int rc = pa_bm_append(m, seq_ids[i], tokens[i], slots + i);
    if (rc != PA_OK) return rc;
    if (num_done) *num_done = i + 1;
  }
  return PA_OK;
}

int pa_bm_plan_decode(const pa_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                      int32_t table_width, int32_t* block_tables, int32_t* context_lens,
                      int32_t* max_context_len) {
  if (!m || num_seqs < 0 || table_width < 1) return PA_E_INVAL;
  if (num_seqs > 0 && (!seq_ids || !block_tables || !context_lens)) return PA_E_INVAL;
  std::vector<const Seq*> ss((size_t)num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {  // validate everything before writing
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || (int64_t)it->second.blocks.size() > table_width) return PA_E_INVAL;
    ss[i] = &it->second;
  }
  int32_t mx = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const std::vector<int32_t>& bl = ss[i]->blocks;
    int32_t* row = block_tables + (size_t)i * table_width;
    std::copy(bl.begin(), bl.end(), row);
    std::fill(row + bl.size(), row + table_width, 0);
    context_lens[i] = (int32_t)ss[i]->tokens.size();
    mx = std::max(mx, context_lens[i]);
  }
  if (max_context_len) *max_context_len = mx;
  return PA_OK;
}

int pa_bm_plan_prefill(const pa_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t table_width, int32_t* block_tables, int32_t* cu_seqlens_q,
                       int32_t* cu_seqlens_k, int32_t* slot_mapping, int32_t slot_capacity,
                       int32_t* max_seqlen_q, int32_t* max_seqlen_k) {
  if (!m || num_seqs < 0 || table_width < 1 || slot_capacity < 0) return PA_E_INVAL;
  if (!cu_seqlens_q || !cu_seqlens_k) return PA_E_INVAL;
  if (num_seqs > 0 && (!seq_ids || !block_tables)) return PA_E_INVAL;
  std::vector<const Seq*> ss((size_t)num_seqs);
  long long rows = 0, keys = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || (int64_t)it->second.blocks.size() > table_width) return PA_E_INVAL;
    ss[i] = &it->second;
    rows += (long long)it->second.tokens.size() - it->second.num_cached;
    keys += (long long)it->second.tokens.size();
  }
  if (rows > slot_capacity || keys > INT32_MAX || (rows > 0 && !slot_mapping)) return PA_E_INVAL;
  const int bs = m->bs;
  int32_t mq = 0, mk = 0, q = 0, k = 0;
  cu_seqlens_q[0] = cu_seqlens_k[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *ss[i];
    const int32_t n = (int32_t)s.tokens.size(), lq = n - s.num_cached;
    int32_t* row = block_tables + (size_t)i * table_width;
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + s.blocks.size(), row + table_width, 0);
    for (int32_t j = s.num_cached; j < n; ++j) slot_mapping[q++] = s.blocks[j / bs] * bs + j % bs;
    k += n;
    cu_seqlens_q[i + 1] = q;
    cu_seqlens_k[i + 1] = k;
    mq = std::max(mq, lq);
    mk = std::max(mk, n);
  }
  if (max_seqlen_q) *max_seqlen_q = mq;
  if (max_seqlen_k) *max_seqlen_k = mk;
  return PA_OK;
}

}  // extern "C"
