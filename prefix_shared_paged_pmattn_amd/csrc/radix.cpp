// Host radix-tree KV cache manager (declared in pmattn_radix.h).
//
// The tree is keyed by token ids (RadixAttention, SGLang review "Core claim").
// A node holds the tokens of positions [start, start + tokens.size()) on its
// path and, for every block index those positions touch, the physical block
// holding them. When a path diverges inside a block, the diverging child names
// its own copy of that block (copy-on-write, XY-Serve review Figure 7), so the
// block a path uses for index j is the one named by the deepest node on the
// path that touches j; that block holds every slot of the path up to there.
//
// Ownership is by reference counts on blocks (tree nodes and live sequences),
// so evicting a tree leaf never frees a block a live sequence still uses.
#include <algorithm>
#include <cstdint>
#include <map>
#include <memory>
#include <new>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "pmattn_radix.h"
#include "plan_internal.h"

namespace pmattn {
namespace {

constexpr int kB = kBlock;

struct Node {
  int32_t start = 0;
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;  // blocks[i] holds block index start/16 + i
  Node* parent = nullptr;
  std::map<int32_t, std::unique_ptr<Node>> children;  // by first token
  uint64_t last_use = 0;
  int32_t end() const { return start + (int32_t)tokens.size(); }
  int32_t first_block() const { return start / kB; }
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  // source block of the copy-on-write order admit gave out (-1: none). The
  // sequence holds a reference on it until its next extend, publish or
  // release, by which time the copy has run: otherwise an eviction during the
  // admit could free it, and a later admit of the same batch could receive it
  // as a fresh block (or copy destination) while the copy still reads it.
  int32_t cow_src = -1;
};

struct Match {
  int32_t len = 0;
  std::vector<Node*> path;  // nodes touched, root excluded, in order
};

}  // namespace
}  // namespace pmattn

struct pmattn_radix_s {
  int32_t num_blocks = 0;
  std::vector<int32_t> refs;
  std::vector<int32_t> free_list;
  pmattn::Node root;
  std::unordered_map<int32_t, pmattn::Seq> seqs;
  int32_t next_seq = 1;
  uint64_t clock = 0;
  int32_t nodes = 0;
  int64_t tree_tokens = 0;
  int64_t evicted = 0;
  std::set<std::pair<uint64_t, pmattn::Node*>> leaves;  // evictable: by last use
};

namespace pmattn {
namespace {

using Cache = pmattn_radix_s;

void ref(Cache& c, int32_t b) { ++c.refs[b]; }
void unref(Cache& c, int32_t b) {
  if (--c.refs[b] == 0) c.free_list.push_back(b);
}
void drop_cow_src(Cache& c, Seq& s) {
  if (s.cow_src >= 0) unref(c, s.cow_src);
  s.cow_src = -1;
}

bool is_leaf(const Node* n) { return n->parent && n->children.empty(); }
void leaf_out(Cache& c, Node* n) { c.leaves.erase({n->last_use, n}); }
void leaf_in(Cache& c, Node* n) {
  if (is_leaf(n)) c.leaves.insert({n->last_use, n});
}
void touch(Cache& c, Node* n, uint64_t t) {
  const bool leaf = is_leaf(n);
  if (leaf) leaf_out(c, n);
  n->last_use = t;
  if (leaf) leaf_in(c, n);
}

// Longest prefix of tokens[0, n) along the tree; path = nodes touched.
Match match(Cache& c, const int32_t* tokens, int32_t n) {
  Match m;
  Node* cur = &c.root;
  while (m.len < n) {
    auto it = cur->children.find(tokens[m.len]);
    if (it == cur->children.end()) break;
    Node* ch = it->second.get();
    int32_t k = 0;
    const int32_t lim = std::min<int32_t>((int32_t)ch->tokens.size(), n - m.len);
    while (k < lim && ch->tokens[k] == tokens[m.len + k]) ++k;
    m.path.push_back(ch);
    m.len += k;
    if (k < (int32_t)ch->tokens.size()) break;
    cur = ch;
  }
  return m;
}

// Block holding block index j on a matched path: the deepest node touching j
// at a position below `limit` (the match length).
int32_t path_block(const Match& m, int32_t j) {
  for (auto it = m.path.rbegin(); it != m.path.rend(); ++it) {
    const Node* nd = *it;
    if (nd->start >= m.len) continue;
    if (nd->first_block() <= j && j * kB < std::min(nd->end(), m.len)) return nd->blocks[j - nd->first_block()];
  }
  return -1;
}

// Drop leaf n from the tree (its block references go).
void evict_leaf(Cache& c, Node* n) {
  leaf_out(c, n);
  for (int32_t b : n->blocks) unref(c, b);
  c.tree_tokens -= (int64_t)n->tokens.size();
  --c.nodes;
  ++c.evicted;
  Node* par = n->parent;
  par->children.erase(n->tokens[0]);  // destroys n
  leaf_in(c, par);
}

// Take k free blocks, evicting least-recently-used leaves as needed. On
// failure nothing is taken (evictions already made stay: they only dropped
// cache entries).
bool take_blocks(Cache& c, int32_t k, std::vector<int32_t>& out) {
  while ((int32_t)c.free_list.size() < k && !c.leaves.empty()) evict_leaf(c, c.leaves.begin()->second);
  if ((int32_t)c.free_list.size() < k) return false;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t b = c.free_list.back();
    c.free_list.pop_back();
    c.refs[b] = 1;
    out.push_back(b);
  }
  return true;
}

// Split node n at position p (n->start < p < n->end()): n keeps [start, p),
// a new child takes [p, end) with n's children.
Node* split(Cache& c, Node* n, int32_t p) {
  const bool leaf = is_leaf(n);
  if (leaf) leaf_out(c, n);
  auto tail = std::make_unique<Node>();
  const int32_t cut = p - n->start;
  tail->start = p;
  tail->tokens.assign(n->tokens.begin() + cut, n->tokens.end());
  const int32_t fb = n->first_block(), tb = p / kB;
  tail->blocks.assign(n->blocks.begin() + (tb - fb), n->blocks.end());
  tail->last_use = n->last_use;
  tail->children = std::move(n->children);
  n->children.clear();
  for (auto& kv : tail->children) kv.second->parent = tail.get();
  tail->parent = n;
  n->tokens.resize(cut);
  const int32_t keep = (p - 1) / kB - fb + 1;  // block indices n still touches
  // references of the indices only the tail touches move to the tail; the
  // index both halves touch (a split inside a block) gains one
  for (int32_t j = tb; j < fb + keep; ++j) ref(c, n->blocks[j - fb]);
  n->blocks.resize(keep);
  Node* t = tail.get();
  n->children[t->tokens[0]] = std::move(tail);
  ++c.nodes;
  leaf_in(c, t);
  (void)leaf;
  return t;
}

}  // namespace
}  // namespace pmattn

using namespace pmattn;

extern "C" {

pmattn_status pmattn_radix_create(int32_t num_blocks, pmattn_radix_t* out) {
  clear_error();
  if (!out) return fail(PMATTN_E_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1) return fail(PMATTN_E_INVALID, "num_blocks must be >= 1");
  try {
    auto* c = new pmattn_radix_s();
    c->num_blocks = num_blocks;
    c->refs.assign(num_blocks, 0);
    c->free_list.reserve(num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b) c->free_list.push_back(b);
    *out = c;
  } catch (const std::bad_alloc&) {
    return fail(PMATTN_E_NOMEM, "host allocation failed");
  }
  return PMATTN_OK;
}

void pmattn_radix_destroy(pmattn_radix_t c) { delete c; }

pmattn_status pmattn_radix_admit(pmattn_radix_t c, const int32_t* tokens, int32_t n,
                                 int32_t* seq_id, int32_t* cached_len, int32_t* block_table,
                                 int32_t capacity, pmattn_block_copy* copy, int32_t* num_copies) {
  clear_error();
  if (!c || !seq_id || !cached_len || !num_copies || (n > 0 && (!tokens || !block_table || !copy)))
    return fail(PMATTN_E_INVALID, "NULL argument");
  if (n < 0) return fail(PMATTN_E_INVALID, "n < 0");
  const int32_t nb = (n + kB - 1) / kB;
  if (capacity < nb) return fail(PMATTN_E_INVALID, "block_table capacity < ceil(n/16)");
  try {
    Match m = match(*c, tokens, n);
    const int32_t full = m.len / kB, partial = m.len % kB;
    std::vector<int32_t> shared;
    for (int32_t j = 0; j < full; ++j) shared.push_back(path_block(m, j));
    const int32_t src = partial ? path_block(m, full) : -1;
    // mark the matched nodes recently used and pin their blocks before any
    // eviction; the path is not used after take_blocks (it may evict nodes)
    const uint64_t t = ++c->clock;
    for (Node* nd : m.path) touch(*c, nd, t);
    for (int32_t b : shared) ref(*c, b);
    if (src >= 0) ref(*c, src);
    std::vector<int32_t> fresh;
    if (!take_blocks(*c, nb - full, fresh)) {
      for (int32_t b : shared) unref(*c, b);
      if (src >= 0) unref(*c, src);
      return fail(PMATTN_E_CAPACITY, "block pool exhausted");
    }
    Seq s;
    s.cow_src = src;  // the reference taken above stays with the sequence
    s.tokens.assign(tokens, tokens + n);
    s.blocks = shared;
    s.blocks.insert(s.blocks.end(), fresh.begin(), fresh.end());
    const int32_t id = c->next_seq++;
    c->seqs.emplace(id, std::move(s));
    std::copy(c->seqs[id].blocks.begin(), c->seqs[id].blocks.end(), block_table);
    *num_copies = 0;
    if (src >= 0) {
      copy->src = src;
      copy->dst = c->seqs[id].blocks[full];
      copy->slots = partial;
      *num_copies = 1;
    }
    *seq_id = id;
    *cached_len = m.len;
  } catch (const std::bad_alloc&) {
    return fail(PMATTN_E_NOMEM, "host allocation failed");
  }
  return PMATTN_OK;
}

pmattn_status pmattn_radix_extend(pmattn_radix_t c, int32_t seq_id, const int32_t* tokens,
                                  int32_t n, int32_t* block_table, int32_t capacity) {
  clear_error();
  if (!c || !block_table || (n > 0 && !tokens)) return fail(PMATTN_E_INVALID, "NULL argument");
  if (n < 0) return fail(PMATTN_E_INVALID, "n < 0");
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(PMATTN_E_INVALID, "unknown seq_id");
  Seq& s = it->second;
  drop_cow_src(*c, s);
  const int32_t total = (int32_t)s.tokens.size() + n;
  const int32_t nb = (total + kB - 1) / kB;
  if (capacity < nb) return fail(PMATTN_E_INVALID, "block_table capacity too small");
  try {
    std::vector<int32_t> fresh;
    if (!take_blocks(*c, nb - (int32_t)s.blocks.size(), fresh))
      return fail(PMATTN_E_CAPACITY, "block pool exhausted");
    s.tokens.insert(s.tokens.end(), tokens, tokens + n);
    s.blocks.insert(s.blocks.end(), fresh.begin(), fresh.end());
    std::copy(s.blocks.begin(), s.blocks.end(), block_table);
  } catch (const std::bad_alloc&) {
    return fail(PMATTN_E_NOMEM, "host allocation failed");
  }
  return PMATTN_OK;
}

pmattn_status pmattn_radix_publish(pmattn_radix_t c, int32_t seq_id) {
  clear_error();
  if (!c) return fail(PMATTN_E_INVALID, "NULL cache");
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(PMATTN_E_INVALID, "unknown seq_id");
  Seq& s = it->second;
  drop_cow_src(*c, s);
  const int32_t n = (int32_t)s.tokens.size();
  try {
    Match m = match(*c, s.tokens.data(), n);
    const uint64_t t = ++c->clock;
    for (Node* nd : m.path) touch(*c, nd, t);
    if (m.len == n) return PMATTN_OK;  // already cached
    Node* parent = &c->root;
    if (!m.path.empty()) {
      parent = m.path.back();
      if (m.len < parent->end()) split(*c, parent, m.len);  // parent keeps [start, m.len)
    }
    const bool was_leaf = is_leaf(parent);
    if (was_leaf) leaf_out(*c, parent);
    auto leaf = std::make_unique<Node>();
    leaf->start = m.len;
    leaf->tokens.assign(s.tokens.begin() + m.len, s.tokens.end());
    for (int32_t j = m.len / kB; j <= (n - 1) / kB; ++j) {
      leaf->blocks.push_back(s.blocks[j]);
      ref(*c, s.blocks[j]);
    }
    leaf->parent = parent;
    leaf->last_use = t;
    Node* lp = leaf.get();
    parent->children[lp->tokens[0]] = std::move(leaf);
    ++c->nodes;
    c->tree_tokens += (int64_t)lp->tokens.size();
    leaf_in(*c, lp);
  } catch (const std::bad_alloc&) {
    return fail(PMATTN_E_NOMEM, "host allocation failed");
  }
  return PMATTN_OK;
}

pmattn_status pmattn_radix_release(pmattn_radix_t c, int32_t seq_id) {
  clear_error();
  if (!c) return fail(PMATTN_E_INVALID, "NULL cache");
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(PMATTN_E_INVALID, "unknown seq_id");
  drop_cow_src(*c, it->second);
  for (int32_t b : it->second.blocks) unref(*c, b);
  c->seqs.erase(it);
  return PMATTN_OK;
}

pmattn_status pmattn_radix_match(pmattn_radix_t c, const int32_t* tokens, int32_t n, int32_t* matched) {
  clear_error();
  if (!c || !matched || (n > 0 && !tokens)) return fail(PMATTN_E_INVALID, "NULL argument");
  if (n < 0) return fail(PMATTN_E_INVALID, "n < 0");
  *matched = match(*c, tokens, n).len;
  return PMATTN_OK;
}

pmattn_status pmattn_radix_stats_get(pmattn_radix_t c, pmattn_radix_stats* out) {
  clear_error();
  if (!c || !out) return fail(PMATTN_E_INVALID, "NULL argument");
  out->num_blocks = c->num_blocks;
  out->free_blocks = (int32_t)c->free_list.size();
  out->tree_nodes = c->nodes;
  out->tree_tokens = (int32_t)c->tree_tokens;
  out->live_seqs = (int32_t)c->seqs.size();
  out->evicted_nodes = c->evicted;
  return PMATTN_OK;
}

pmattn_status pmattn_radix_block_refs(pmattn_radix_t c, int32_t block, int32_t* refs) {
  clear_error();
  if (!c || !refs || block < 0 || block >= c->num_blocks) return fail(PMATTN_E_INVALID, "bad argument");
  *refs = c->refs[block];
  return PMATTN_OK;
}

}  // extern "C"
