// Host-side prefix index: chain-hash prefix cache over a paged block pool and
// a radix tree (C ABI in include/pkv_prefix.h). Plain C++17, no GPU calls.
//
// Chain hashing follows "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화"
// (aitrends.kr) §05 (a block's hash covers its parent's hash, its token IDs and
// extra keys; reuse up to the first miss) and §06 (tenant salt in the
// identifier); the block pool follows §02 and "KV Cache 완전 정리" (cell-devlog)
// "PagedAttention" (blocks on demand, unused blocks reused). The radix tree
// follows §03-§04 of the first page (longest-prefix match, insert after a
// request, leaf-first LRU eviction sparing shared prefixes) and the second
// page's "RadixAttention" section.
#include "../../include/pkv_prefix.h"
#include "pkv_status.hpp"

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

int fail(int code, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b);
  return pkv::record_status(code, buf);
}
int ok() { return pkv::record_status(PKV_OK, nullptr); }

// splitmix64 finaliser (Steele, Lea, Flood; the mixing step of Vigna's
// splitmix64 generator): a bijective 64-bit mix
uint64_t mix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// chain hash of one block from its parent's hash, its tokens and the extra key
uint64_t chain_hash(uint64_t parent, const int32_t* tok, int B, uint64_t extra) {
  uint64_t h = mix64(parent ^ 0x5bd1e9955bd1e995ull);
  for (int i = 0; i < B; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tok[i]);
  return mix64(h ^ mix64(extra));
}
uint64_t root_hash(uint64_t salt) { return mix64(salt ^ 0x2545f4914f6cdd1dull); }

}  // namespace

// ============================================================================
// chain-hash prefix cache
// ============================================================================
struct pkv_prefix_cache {
  struct Request {
    std::vector<int32_t> blocks, tokens;
    std::vector<uint64_t> hashes;  // chain hash of each full block
    uint64_t salt = 0, extra = 0;
    int64_t published = 0;         // leading full blocks already handled by commit/hits
  };
  int64_t nb = 0;
  int B = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  // published blocks: chain hash, parent chain hash, token IDs
  std::vector<uint8_t> pub;
  std::vector<uint64_t> hash, parent;
  std::vector<int32_t> tok;  // nb * B
  std::unordered_map<uint64_t, int32_t> cached;
  // LRU list of evictable blocks (published, ref 0): front = least recent
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_lru;
  int32_t head = -1, tail = -1;
  int64_t n_lru = 0;
  std::unordered_map<int64_t, Request> req;
  int64_t next_rid = 0;

  void lru_push(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    in_lru[b] = 1;
    ++n_lru;
  }
  void lru_remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    in_lru[b] = 0;
    --n_lru;
  }
  // a published block whose chain hash, parent hash and tokens all agree
  int32_t lookup(uint64_t h, uint64_t par, const int32_t* t) const {
    auto it = cached.find(h);
    if (it == cached.end()) return -1;
    const int32_t b = it->second;
    if (parent[b] != par || std::memcmp(&tok[(size_t)b * B], t, sizeof(int32_t) * B) != 0) return -1;
    return b;
  }
  int32_t take() {  // caller has checked that a block is available
    if (!free_list.empty()) {
      const int32_t b = free_list.front();
      free_list.pop_front();
      return b;
    }
    const int32_t b = head;
    lru_remove(b);
    cached.erase(hash[b]);
    pub[b] = 0;
    return b;
  }
  std::vector<uint64_t> chain(const int32_t* t, int64_t n, uint64_t salt, uint64_t extra) const {
    std::vector<uint64_t> out;
    uint64_t h = root_hash(salt);
    for (int64_t i = 0; i + B <= n; i += B) {
      h = chain_hash(h, t + i, B, extra);
      out.push_back(h);
    }
    return out;
  }
};

extern "C" {

int pkv_pc_create(int64_t num_blocks, int32_t block_size, pkv_prefix_cache** out) {
  if (!out) return fail(PKV_ERR_NULL, "pkv_pc_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || num_blocks >= (1ll << 31))
    return fail(PKV_ERR_SHAPE, "pkv_pc_create: num_blocks %lld outside [1, 2^31)", num_blocks);
  if (block_size < 1 || block_size > 4096)
    return fail(PKV_ERR_SHAPE, "pkv_pc_create: block_size %lld outside [1, 4096]", block_size);
  pkv_prefix_cache* pc = new (std::nothrow) pkv_prefix_cache();
  if (!pc) return fail(PKV_ERR_SHAPE, "pkv_pc_create: out of host memory");
  try {
    pc->nb = num_blocks;
    pc->B = block_size;
    for (int64_t b = 0; b < num_blocks; ++b) pc->free_list.push_back((int32_t)b);
    pc->ref.assign(num_blocks, 0);
    pc->pub.assign(num_blocks, 0);
    pc->hash.assign(num_blocks, 0);
    pc->parent.assign(num_blocks, 0);
    pc->tok.assign((size_t)num_blocks * block_size, 0);
    pc->prev.assign(num_blocks, -1);
    pc->next.assign(num_blocks, -1);
    pc->in_lru.assign(num_blocks, 0);
  } catch (...) {
    delete pc;
    return fail(PKV_ERR_SHAPE, "pkv_pc_create: out of host memory for %lld blocks", num_blocks);
  }
  *out = pc;
  return ok();
}

void pkv_pc_destroy(pkv_prefix_cache* pc) { delete pc; }

int pkv_pc_admit(pkv_prefix_cache* pc, const int32_t* tokens, int64_t n, uint64_t salt, uint64_t extra,
                 int32_t* block_table, int64_t max_blocks, int64_t* slot_mapping, int64_t* prefix_len,
                 int64_t* request_id) {
  if (!pc || !tokens || !block_table || !slot_mapping || !prefix_len || !request_id)
    return fail(PKV_ERR_NULL, "pkv_pc_admit: a required pointer is NULL");
  if (n < 1) return fail(PKV_ERR_SHAPE, "pkv_pc_admit: a request has at least one token (n = %lld)", n);
  const int B = pc->B;
  const int64_t nblk = (n + B - 1) / B;
  if (max_blocks < nblk)
    return fail(PKV_ERR_SHAPE, "pkv_pc_admit: block_table holds %lld entries, %lld needed", max_blocks, nblk);
  std::vector<uint64_t> ch = pc->chain(tokens, n, salt, extra);
  // sequential matching up to the first miss
  std::vector<int32_t> hit_blocks;
  uint64_t par = root_hash(salt);
  for (size_t i = 0; i < ch.size(); ++i) {
    const int32_t b = pc->lookup(ch[i], par, tokens + i * B);
    if (b < 0) break;
    hit_blocks.push_back(b);
    par = ch[i];
  }
  int64_t hits = (int64_t)hit_blocks.size();
  if (hits * B == n) {  // everything cached: still compute the last block
    --hits;
    hit_blocks.pop_back();
  }
  const int64_t need = nblk - hits;
  int64_t reclaimable = pc->n_lru;
  for (int32_t b : hit_blocks) reclaimable -= pc->in_lru[b] ? 1 : 0;
  if (need > (int64_t)pc->free_list.size() + reclaimable)
    return fail(PKV_ERR_NO_BLOCKS, "pkv_pc_admit: %lld blocks needed, %lld free or evictable", need,
                (long long)pc->free_list.size() + reclaimable);
  for (int32_t b : hit_blocks) {
    if (pc->ref[b] == 0) pc->lru_remove(b);
    ++pc->ref[b];
  }
  pkv_prefix_cache::Request r;
  r.blocks = hit_blocks;
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = pc->take();
    pc->ref[b] = 1;
    r.blocks.push_back(b);
  }
  r.tokens.assign(tokens, tokens + n);
  r.hashes = std::move(ch);
  r.salt = salt;
  r.extra = extra;
  r.published = hits;
  const int64_t prefix = hits * B;
  for (int64_t i = 0; i < nblk; ++i) block_table[i] = r.blocks[i];
  for (int64_t t = prefix; t < n; ++t) slot_mapping[t - prefix] = (int64_t)r.blocks[t / B] * B + t % B;
  *prefix_len = prefix;
  *request_id = pc->next_rid;
  pc->req.emplace(pc->next_rid++, std::move(r));
  return ok();
}

int pkv_pc_append(pkv_prefix_cache* pc, int64_t request_id, int32_t token, int64_t* slot) {
  if (!pc || !slot) return fail(PKV_ERR_NULL, "pkv_pc_append: a required pointer is NULL");
  auto it = pc->req.find(request_id);
  if (it == pc->req.end()) return fail(PKV_ERR_NOT_FOUND, "pkv_pc_append: unknown request %lld", request_id);
  auto& r = it->second;
  const int B = pc->B;
  const int64_t t = (int64_t)r.tokens.size();
  if (t / B == (int64_t)r.blocks.size()) {
    if (pc->free_list.empty() && pc->n_lru == 0)
      return fail(PKV_ERR_NO_BLOCKS, "pkv_pc_append: no block for token %lld of request %lld", t, request_id);
    const int32_t b = pc->take();
    pc->ref[b] = 1;
    r.blocks.push_back(b);
  }
  r.tokens.push_back(token);
  if ((int64_t)r.tokens.size() % B == 0) {  // a block just filled up: its chain hash
    const uint64_t par = r.hashes.empty() ? root_hash(r.salt) : r.hashes.back();
    r.hashes.push_back(chain_hash(par, r.tokens.data() + r.tokens.size() - B, B, r.extra));
  }
  *slot = (int64_t)r.blocks[t / B] * B + t % B;
  return ok();
}

int pkv_pc_commit(pkv_prefix_cache* pc, int64_t request_id, int64_t* published) {
  if (!pc) return fail(PKV_ERR_NULL, "pkv_pc_commit: cache is NULL");
  auto it = pc->req.find(request_id);
  if (it == pc->req.end()) return fail(PKV_ERR_NOT_FOUND, "pkv_pc_commit: unknown request %lld", request_id);
  auto& r = it->second;
  const int B = pc->B;
  int64_t count = 0;
  for (int64_t i = r.published; i < (int64_t)r.hashes.size(); ++i) {
    const int32_t b = r.blocks[i];
    if (pc->cached.count(r.hashes[i]) || pc->pub[b]) continue;  // already cached elsewhere: stays private
    pc->cached.emplace(r.hashes[i], b);
    pc->pub[b] = 1;
    pc->hash[b] = r.hashes[i];
    pc->parent[b] = i == 0 ? root_hash(r.salt) : r.hashes[i - 1];
    std::memcpy(&pc->tok[(size_t)b * B], r.tokens.data() + i * B, sizeof(int32_t) * B);
    ++count;
  }
  r.published = (int64_t)r.hashes.size();
  if (published) *published = count;
  return ok();
}

int pkv_pc_release(pkv_prefix_cache* pc, int64_t request_id) {
  if (!pc) return fail(PKV_ERR_NULL, "pkv_pc_release: cache is NULL");
  auto it = pc->req.find(request_id);
  if (it == pc->req.end()) return fail(PKV_ERR_NOT_FOUND, "pkv_pc_release: unknown request %lld", request_id);
  const auto& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
    if (--pc->ref[*b] == 0) {
      if (pc->pub[*b]) pc->lru_push(*b);
      else pc->free_list.push_back(*b);
    }
  }
  pc->req.erase(it);
  return ok();
}

int pkv_pc_block_table(const pkv_prefix_cache* pc, int64_t request_id, int32_t* block_table, int64_t max_blocks,
                       int64_t* num_blocks) {
  if (!pc || !num_blocks || (max_blocks > 0 && !block_table))
    return fail(PKV_ERR_NULL, "pkv_pc_block_table: a required pointer is NULL");
  auto it = pc->req.find(request_id);
  if (it == pc->req.end())
    return fail(PKV_ERR_NOT_FOUND, "pkv_pc_block_table: unknown request %lld", request_id);
  const auto& blocks = it->second.blocks;
  const int64_t n = (int64_t)blocks.size();
  for (int64_t i = 0; i < std::min(n, max_blocks); ++i) block_table[i] = blocks[i];
  *num_blocks = n;
  return ok();
}

int pkv_pc_stats(const pkv_prefix_cache* pc, int64_t* free_blocks, int64_t* evictable, int64_t* cached) {
  if (!pc) return fail(PKV_ERR_NULL, "pkv_pc_stats: cache is NULL");
  if (free_blocks) *free_blocks = (int64_t)pc->free_list.size();
  if (evictable) *evictable = pc->n_lru;
  if (cached) *cached = (int64_t)pc->cached.size();
  return ok();
}

}  // extern "C"

// ============================================================================
// radix tree
// ============================================================================
struct pkv_radix {
  struct Node {
    std::vector<int32_t> key;     // tokens on the edge from the parent
    std::vector<int64_t> values;  // one per token of the edge
    std::map<std::vector<int32_t>, int32_t> children;  // keyed by their first page
    int32_t parent = -1;
    int64_t lock = 0, access = 0, nid = 0;
    bool alive = true;
  };
  int page = 1;
  std::vector<Node> nodes;  // node 0 is the root; removed nodes stay, not alive
  std::vector<int32_t> spare;
  int64_t clock = 0, next_nid = 0, total = 0;

  int32_t make(std::vector<int32_t> key, std::vector<int64_t> values, int32_t par) {
    int32_t id;
    if (!spare.empty()) {
      id = spare.back();
      spare.pop_back();
      nodes[id] = Node();
    } else {
      id = (int32_t)nodes.size();
      nodes.emplace_back();
    }
    Node& x = nodes[id];
    x.key = std::move(key);
    x.values = std::move(values);
    x.parent = par;
    x.nid = next_nid++;
    return id;
  }
  std::vector<int32_t> first_page(const std::vector<int32_t>& k) const {
    return std::vector<int32_t>(k.begin(), k.begin() + page);
  }
  std::vector<int32_t> page_at(const int32_t* t, int64_t pos) const { return std::vector<int32_t>(t + pos, t + pos + page); }
  // whole pages of a (edge) and b (rest of the query) that agree
  int64_t common_pages(const std::vector<int32_t>& a, const int32_t* b, int64_t blen) const {
    int64_t n = 0;
    while (n + page <= (int64_t)a.size() && n + page <= blen &&
           std::memcmp(a.data() + n, b + n, sizeof(int32_t) * page) == 0)
      n += page;
    return n;
  }
  // cut node's edge after `at` tokens; returns the new upper node
  int32_t split(int32_t node, int64_t at) {
    const int32_t par = nodes[node].parent;
    std::vector<int32_t> ukey(nodes[node].key.begin(), nodes[node].key.begin() + at);
    std::vector<int64_t> uval(nodes[node].values.begin(), nodes[node].values.begin() + at);
    const int32_t up = make(std::move(ukey), std::move(uval), par);  // may reallocate `nodes`
    Node& x = nodes[node];
    Node& u = nodes[up];
    u.lock = x.lock;
    u.access = x.access;
    nodes[par].children[first_page(u.key)] = up;
    x.key.erase(x.key.begin(), x.key.begin() + at);
    x.values.erase(x.values.begin(), x.values.begin() + at);
    x.parent = up;
    u.children[first_page(x.key)] = node;
    return up;
  }
  // deepest node whose path is a prefix of t[0..n), splitting a part-matched
  // edge; returns the node and the matched length
  std::pair<int32_t, int64_t> walk(const int32_t* t, int64_t n) {
    int32_t node = 0;
    int64_t pos = 0;
    while (pos + page <= n) {
      auto it = nodes[node].children.find(page_at(t, pos));
      if (it == nodes[node].children.end()) break;
      const int32_t child = it->second;
      const int64_t c = common_pages(nodes[child].key, t + pos, n - pos);
      if (c < (int64_t)nodes[child].key.size()) return {split(child, c), pos + c};
      node = child;
      pos += c;
    }
    return {node, pos};
  }
};

extern "C" {

int pkv_radix_create(int32_t page, pkv_radix** out) {
  if (!out) return fail(PKV_ERR_NULL, "pkv_radix_create: out is NULL");
  *out = nullptr;
  if (page < 1 || page > 4096) return fail(PKV_ERR_SHAPE, "pkv_radix_create: page %lld outside [1, 4096]", page);
  pkv_radix* t = new (std::nothrow) pkv_radix();
  if (!t) return fail(PKV_ERR_SHAPE, "pkv_radix_create: out of host memory");
  t->page = page;
  t->make({}, {}, -1);  // root
  *out = t;
  return ok();
}

void pkv_radix_destroy(pkv_radix* t) { delete t; }

int pkv_radix_match(pkv_radix* t, const int32_t* tokens, int64_t n, int64_t* values, int64_t* matched) {
  if (!t || !matched || (n > 0 && (!tokens || !values)))
    return fail(PKV_ERR_NULL, "pkv_radix_match: a required pointer is NULL");
  if (n < 0) return fail(PKV_ERR_SHAPE, "pkv_radix_match: negative length %lld", n);
  const int64_t now = ++t->clock;
  int32_t node = 0;
  int64_t pos = 0;
  while (pos + t->page <= n) {
    auto it = t->nodes[node].children.find(t->page_at(tokens, pos));
    if (it == t->nodes[node].children.end()) break;
    pkv_radix::Node& c = t->nodes[it->second];
    const int64_t m = t->common_pages(c.key, tokens + pos, n - pos);
    c.access = now;
    std::copy(c.values.begin(), c.values.begin() + m, values + pos);
    pos += m;
    if (m < (int64_t)c.key.size()) break;
    node = it->second;
  }
  *matched = pos;
  return ok();
}

int pkv_radix_insert(pkv_radix* t, const int32_t* tokens, int64_t n, const int64_t* values, int64_t* existing) {
  if (!t || (n > 0 && (!tokens || !values))) return fail(PKV_ERR_NULL, "pkv_radix_insert: a required pointer is NULL");
  if (n < 0) return fail(PKV_ERR_SHAPE, "pkv_radix_insert: negative length %lld", n);
  n -= n % t->page;
  const int64_t now = ++t->clock;
  auto [node, pos] = t->walk(tokens, n);
  for (int32_t x = node; x >= 0; x = t->nodes[x].parent) t->nodes[x].access = now;
  if (pos < n) {
    const int32_t leaf = t->make(std::vector<int32_t>(tokens + pos, tokens + n),
                                 std::vector<int64_t>(values + pos, values + n), node);
    t->nodes[leaf].access = now;
    t->nodes[node].children[t->first_page(t->nodes[leaf].key)] = leaf;
    t->total += n - pos;
  }
  if (existing) *existing = pos;
  return ok();
}

static int radix_lock_path(pkv_radix* t, const int32_t* tokens, int64_t length, int delta, const char* null_msg) {
  if (!t || (length > 0 && !tokens)) return pkv::record_status(PKV_ERR_NULL, null_msg);
  if (length < 0 || length % t->page)
    return fail(PKV_ERR_SHAPE, "lock length %lld is not a whole number of %lld-token pages", length, t->page);
  auto [node, pos] = t->walk(tokens, length);
  if (pos != length) return fail(PKV_ERR_NOT_FOUND, "the first %lld tokens are not stored (%lld are)", length, pos);
  if (delta < 0)
    for (int32_t x = node; x > 0; x = t->nodes[x].parent)
      if (t->nodes[x].lock <= 0) return fail(PKV_ERR_NOT_FOUND, "unlock of %lld tokens without a lock", length);
  for (int32_t x = node; x > 0; x = t->nodes[x].parent) t->nodes[x].lock += delta;
  return ok();
}

int pkv_radix_lock(pkv_radix* t, const int32_t* tokens, int64_t length) {
  return radix_lock_path(t, tokens, length, +1, "pkv_radix_lock: a required pointer is NULL");
}

int pkv_radix_unlock(pkv_radix* t, const int32_t* tokens, int64_t length) {
  return radix_lock_path(t, tokens, length, -1, "pkv_radix_unlock: a required pointer is NULL");
}

int pkv_radix_evict(pkv_radix* t, int64_t num_tokens, int64_t* values, int64_t capacity, int64_t* evicted) {
  if (!t || !evicted || (capacity > 0 && !values)) return fail(PKV_ERR_NULL, "pkv_radix_evict: a required pointer is NULL");
  int64_t freed = 0;
  while (freed < num_tokens) {
    int32_t victim = -1;
    for (int32_t i = 1; i < (int32_t)t->nodes.size(); ++i) {
      const pkv_radix::Node& x = t->nodes[i];
      if (!x.alive || !x.children.empty() || x.lock != 0) continue;
      if (victim < 0 || x.access < t->nodes[victim].access ||
          (x.access == t->nodes[victim].access && x.nid < t->nodes[victim].nid))
        victim = i;
    }
    if (victim < 0) break;
    pkv_radix::Node& v = t->nodes[victim];
    if (freed + (int64_t)v.values.size() > capacity) break;
    std::copy(v.values.begin(), v.values.end(), values + freed);
    freed += (int64_t)v.values.size();
    t->total -= (int64_t)v.key.size();
    t->nodes[v.parent].children.erase(t->first_page(v.key));
    v.alive = false;
    v.key.clear();
    v.values.clear();
    t->spare.push_back(victim);
  }
  *evicted = freed;
  return ok();
}

int pkv_radix_total_tokens(const pkv_radix* t, int64_t* total) {
  if (!t || !total) return fail(PKV_ERR_NULL, "pkv_radix_total_tokens: a required pointer is NULL");
  *total = t->total;
  return ok();
}

}  // extern "C"
