// Host radix tree and slot allocator (see radix_tree.h for the cited semantics).
#include "radix_tree.h"

#include <algorithm>
#include <cstring>

namespace rax {

// ------------------------------------------------------------------ allocator
SlotAllocator::SlotAllocator(int64_t num_slots)
    : num_slots_(num_slots), num_free_(num_slots), hint_(0), words_((num_slots + 63) / 64, ~0ull) {
  const int64_t tail = num_slots & 63;
  if (tail) words_.back() = (1ull << tail) - 1;
}

bool SlotAllocator::alloc(int64_t n, int32_t* out) {
  if (n > num_free_) return false;
  int64_t got = 0;
  int64_t w = hint_;
  const int64_t nw = static_cast<int64_t>(words_.size());
  while (got < n && w < nw) {
    uint64_t bits = words_[w];
    while (bits && got < n) {
      const int b = __builtin_ctzll(bits);
      bits &= bits - 1;
      out[got++] = static_cast<int32_t>(w * 64 + b);
    }
    words_[w] = bits;
    if (bits == 0) ++w;
  }
  hint_ = w;
  num_free_ -= n;
  return true;
}

void SlotAllocator::release_one(int32_t s) {
  words_[s >> 6] |= 1ull << (s & 63);
  ++num_free_;
  if ((s >> 6) < hint_) hint_ = s >> 6;
}

void SlotAllocator::release(const int32_t* slots, int64_t n) {
  for (int64_t i = 0; i < n; ++i) release_one(slots[i]);
}

// ----------------------------------------------------------------------- tree
RadixTree::RadixTree(int64_t num_slots) : alloc_(num_slots) {
  root_ = new Node();
  root_->id = 0;
  nodes_[0] = root_;
}

RadixTree::~RadixTree() {
  for (auto& kv : nodes_) delete kv.second;
}

Node* RadixTree::new_node() {
  Node* n = new Node();
  n->id = next_id_++;
  nodes_[n->id] = n;
  return n;
}

const Node* RadixTree::find(int64_t id) const {
  auto it = nodes_.find(id);
  return it == nodes_.end() ? nullptr : it->second;
}

void RadixTree::lru_remove(Node* n) {
  if (n->in_lru) {
    lru_.erase({n->tick, n->id});
    n->in_lru = false;
  }
}

void RadixTree::lru_update(Node* n) {
  const bool want = n != root_ && !n->host && n->ndev == 0 && n->ref == 0;
  if (want && !n->in_lru) {
    lru_.insert({n->tick, n->id});
    n->in_lru = true;
  } else if (!want && n->in_lru) {
    lru_remove(n);
  }
}

void RadixTree::hlru_remove(Node* n) {
  if (n->in_hlru) {
    hlru_.erase({n->tick, n->id});
    n->in_hlru = false;
  }
}

void RadixTree::hlru_update(Node* n) {
  const bool want = n->host && n->children.empty() && n->ref == 0;
  if (want && !n->in_hlru) {
    hlru_.insert({n->tick, n->id});
    n->in_hlru = true;
  } else if (!want && n->in_hlru) {
    hlru_remove(n);
  }
}

bool RadixTree::set_host_tier(int64_t host_slots) {
  if (host_slots < 0 || host_tokens > 0) return false;
  host_alloc_ = SlotAllocator(host_slots);
  return true;
}

void RadixTree::erase_node(Node* n) {
  lru_remove(n);
  hlru_remove(n);
  Node* p = n->parent;
  p->children.erase(n->tokens[0]);
  if (!n->host) --p->ndev;
  nodes_.erase(n->id);
  delete n;
  lru_update(p);
  hlru_update(p);
}

Node* RadixTree::split(Node* child, int64_t k) {
  Node* up = new_node();
  Node* parent = child->parent;
  up->parent = parent;
  up->tokens.assign(child->tokens.begin(), child->tokens.begin() + k);
  up->slots.assign(child->slots.begin(), child->slots.begin() + k);
  up->ref = child->ref;
  up->tick = child->tick;
  up->host = child->host;
  up->ndev = child->host ? 0 : 1;
  up->depth_end = parent->depth_end + k;
  child->tokens.erase(child->tokens.begin(), child->tokens.begin() + k);
  child->slots.erase(child->slots.begin(), child->slots.begin() + k);
  child->parent = up;
  up->children[child->tokens[0]] = child;
  parent->children[up->tokens[0]] = up;
  return up;  // not a leaf; child keeps its LRU key (tick, id)
}

Node* RadixTree::walk(const int32_t* tokens, int64_t n, int64_t* matched, int32_t* out) {
  return walk_from(root_, 0, tokens, n, matched, out);
}

Node* RadixTree::walk_from(Node* node, int64_t i0, const int32_t* tokens, int64_t n, int64_t* matched,
                           int32_t* out) {
  int64_t i = i0;
  while (i < n) {
    auto it = node->children.find(tokens[i]);
    if (it == node->children.end() || it->second->host) break;  // the device part only
    Node* c = it->second;
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    const int64_t lim = std::min(len, n - i);
    int64_t k = 1;  // first token matches by construction
    while (k < lim && c->tokens[k] == tokens[i + k]) ++k;
    if (out) std::memcpy(out + i, c->slots.data(), sizeof(int32_t) * k);
    i += k;
    if (k < len) {
      node = split(c, k);
      break;
    }
    node = c;
  }
  *matched = i;
  return node;
}

void RadixTree::tick_path(Node* n) {
  for (; n != root_; n = n->parent) {
    if (n->in_lru) {
      lru_.erase({n->tick, n->id});
      n->tick = clock_;
      lru_.insert({n->tick, n->id});
    } else {
      n->tick = clock_;
    }
  }
}

int64_t RadixTree::prefix_len(const int32_t* tokens, int64_t n) const {
  const Node* node = root_;
  int64_t i = 0;
  while (i < n) {
    auto it = node->children.find(tokens[i]);
    if (it == node->children.end() || it->second->host) break;
    const Node* c = it->second;
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    const int64_t lim = std::min(len, n - i);
    int64_t k = 1;
    while (k < lim && c->tokens[k] == tokens[i + k]) ++k;
    i += k;
    if (k < len) break;
    node = c;
  }
  return i;
}

int64_t RadixTree::match(const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* out_node) {
  ++clock_;
  int64_t m = 0;
  Node* node = walk(tokens, n, &m, out_slots);
  tick_path(node);
  matched_total += m;
  *out_node = node->id;
  return m;
}

bool RadixTree::insert(const int32_t* tokens, const int32_t* slots, int64_t n, int32_t* out_slots,
                       int64_t* out_existing, int64_t* out_node) {
  return insert_at(root_, 0, tokens, slots, n, out_slots, out_existing, out_node);
}

int RadixTree::insert_from(int64_t start, int64_t trusted, const int32_t* tokens, const int32_t* slots, int64_t n,
                           int32_t* out_slots, int64_t* out_existing, int64_t* out_node) {
  auto it = nodes_.find(start);
  if (it == nodes_.end() || trusted < 0) return 1;
  Node* s = it->second;
  if (s->host || s->depth_end > n) return 1;
  while (s != root_ && s->depth_end > trusted) s = s->parent;
  const int64_t d = s->depth_end;
  // the start's own label must end the first d tokens (its ancestors are the caller's word)
  const int64_t len = static_cast<int64_t>(s->tokens.size());
  if (s != root_ && !std::equal(s->tokens.begin(), s->tokens.end(), tokens + d - len)) return 1;
  return insert_at(s, d, tokens, slots, n, out_slots, out_existing, out_node) ? 0 : 2;
}

bool RadixTree::insert_at(Node* start, int64_t d, const int32_t* tokens, const int32_t* slots, int64_t n,
                          int32_t* out_slots, int64_t* out_existing, int64_t* out_node) {
  // positions before d hold the tree's own slots (insert_from's contract): checked from d
  for (int64_t i = d; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= alloc_.num_slots() || alloc_.is_free(slots[i])) return false;
  }
  ++clock_;
  int64_t m = d;
  std::vector<int32_t> tree_slots(static_cast<size_t>(n));
  if (d) std::memcpy(tree_slots.data(), slots, sizeof(int32_t) * d);
  Node* node = walk_from(start, d, tokens, n, &m, tree_slots.data());
  for (int64_t i = d; i < m; ++i) {
    if (slots[i] != tree_slots[i]) alloc_.release_one(slots[i]);
  }
  const int64_t m_dev = m;
  // host nodes on the path take the caller's (device) slots: the KV is fresh on the device
  while (m < n) {
    auto it = node->children.find(tokens[m]);
    if (it == node->children.end()) break;
    Node* c = it->second;  // a host node (the device walk stopped at it)
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    const int64_t lim = std::min(len, n - m);
    int64_t k = 1;
    while (k < lim && c->tokens[k] == tokens[m + k]) ++k;
    Node* u = k < len ? split(c, k) : c;
    hlru_remove(u);
    host_alloc_.release(u->slots.data(), static_cast<int64_t>(u->slots.size()));
    host_tokens -= k;
    u->slots.assign(slots + m, slots + m + k);
    u->host = false;
    ++node->ndev;
    std::memcpy(tree_slots.data() + m, slots + m, sizeof(int32_t) * k);
    lru_update(node);
    lru_update(u);
    m += k;
    node = u;
    if (k < len) break;
  }
  if (m < n) {
    Node* leaf = new_node();
    leaf->parent = node;
    leaf->tokens.assign(tokens + m, tokens + n);
    leaf->slots.assign(slots + m, slots + n);
    leaf->depth_end = node->depth_end + (n - m);
    leaf->tick = clock_;
    node->children[tokens[m]] = leaf;
    ++node->ndev;
    lru_update(node);  // no longer a leaf
    lru_update(leaf);
    std::memcpy(tree_slots.data() + m, slots + m, sizeof(int32_t) * (n - m));
    node = leaf;
  }
  inserted_total += n - m_dev;
  tick_path(node);
  if (out_slots && n) std::memcpy(out_slots, tree_slots.data(), sizeof(int32_t) * n);
  *out_existing = m_dev;
  *out_node = node->id;
  return true;
}

int RadixTree::lock_ref(int64_t id, int32_t delta) {
  auto it = nodes_.find(id);
  if (it == nodes_.end()) return 1;
  Node* start = it->second;
  if (start->host) return 3;  // only device KV can be pinned for a running request
  if (delta < 0) {
    for (Node* n = start; n != root_; n = n->parent)
      if (n->ref + delta < 0) return 2;
  }
  for (Node* n = start; n != root_; n = n->parent) {
    n->ref += delta;
    lru_update(n);
  }
  return 0;
}

void RadixTree::drop_host_leaves(int64_t need) {
  while (host_alloc_.num_free() < need && !hlru_.empty()) {
    Node* h = nodes_[hlru_.begin()->second];
    host_alloc_.release(h->slots.data(), static_cast<int64_t>(h->slots.size()));
    host_tokens -= static_cast<int64_t>(h->slots.size());
    erase_node(h);
  }
}

void RadixTree::drop_subtree(Node* n, int32_t* out_freed, int64_t cap, int64_t* freed) {
  while (!n->children.empty()) drop_subtree(n->children.begin()->second, out_freed, cap, freed);
  if (n->host) {
    host_alloc_.release(n->slots.data(), static_cast<int64_t>(n->slots.size()));
    host_tokens -= static_cast<int64_t>(n->slots.size());
  } else {
    for (int32_t s : n->slots) {
      if (out_freed && *freed < cap) out_freed[*freed] = s;
      alloc_.release_one(s);
      ++*freed;
    }
  }
  erase_node(n);
}

int64_t RadixTree::evict(int64_t num_tokens, int32_t* out_freed, int64_t cap) {
  int64_t freed = 0;
  while (freed < num_tokens && !lru_.empty()) {
    Node* n = nodes_[lru_.begin()->second];
    lru_remove(n);
    const int64_t len = static_cast<int64_t>(n->slots.size());
    if (host_alloc_.num_slots() > 0) drop_host_leaves(len);
    std::vector<int32_t> hs(static_cast<size_t>(len));
    if (host_alloc_.num_slots() > 0 && host_alloc_.alloc(len, hs.data())) {
      // demote: the KV moves to the host tier, the node stays in the tree
      for (int64_t i = 0; i < len; ++i) {
        const int32_t s = n->slots[i];
        pending_.push(0, s, hs[i]);
        if (out_freed && freed < cap) out_freed[freed] = s;
        alloc_.release_one(s);
        ++freed;
      }
      n->slots = hs;
      n->host = true;
      host_tokens += len;
      demoted_total += len;
      --n->parent->ndev;
      lru_update(n);  // drop_host_leaves may have made it a candidate again
      lru_update(n->parent);
      hlru_update(n);
    } else {
      drop_subtree(n, out_freed, cap, &freed);
    }
  }
  evicted_total += freed;
  return freed;
}

int64_t RadixTree::promote(const int32_t* tokens, int64_t n, std::vector<int32_t>* freed) {
  // device part (read only, no split), then the host continuation node by node
  Node* node = root_;
  int64_t i = 0;
  while (i < n) {
    auto it = node->children.find(tokens[i]);
    if (it == node->children.end() || it->second->host) break;
    Node* c = it->second;
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    if (n - i < len) return 0;
    for (int64_t k = 1; k < len; ++k)
      if (c->tokens[k] != tokens[i + k]) return 0;  // diverges inside a device node
    i += len;
    node = c;
  }
  int64_t done = 0;
  Node* locked = node == root_ ? nullptr : node;
  if (locked) lock_ref(locked->id, +1);  // keep the device path while allocating
  while (i < n) {
    auto it = node->children.find(tokens[i]);
    if (it == node->children.end()) break;
    Node* c = it->second;  // host
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    const int64_t lim = std::min(len, n - i);
    int64_t k = 1;
    while (k < lim && c->tokens[k] == tokens[i + k]) ++k;
    Node* u = k < len ? split(c, k) : c;
    ++u->ref;  // not droppable while its device slots are taken
    hlru_remove(u);
    std::vector<int32_t> ds(static_cast<size_t>(k));
    const int64_t short_by = k - alloc_.num_free();
    if (short_by > 0) {
      std::vector<int32_t> f(static_cast<size_t>(alloc_.num_slots()));
      const int64_t got = evict(short_by, f.data(), static_cast<int64_t>(f.size()));
      freed->insert(freed->end(), f.begin(), f.begin() + got);
    }
    --u->ref;
    if (!alloc_.alloc(k, ds.data())) {
      hlru_update(u);
      break;
    }
    for (int64_t j = 0; j < k; ++j) pending_.push(1, u->slots[j], ds[j]);
    host_alloc_.release(u->slots.data(), k);
    u->slots = ds;
    u->host = false;
    host_tokens -= k;
    promoted_total += k;
    ++node->ndev;
    lru_update(node);
    lru_update(u);
    lock_ref(u->id, +1);
    if (locked) lock_ref(locked->id, -1);
    locked = u;
    done += k;
    i += k;
    node = u;
    if (k < len) break;
  }
  if (locked) lock_ref(locked->id, -1);
  return done;
}

// Token depth of the deepest common ancestor of two nodes: bring both to the same depth,
// then climb together.
static int64_t lca_of(const Node* na, const Node* nb) {
  while (na->depth_end > nb->depth_end) na = na->parent;
  while (nb->depth_end > na->depth_end) nb = nb->parent;
  while (na != nb) {
    if (na->depth_end >= nb->depth_end) na = na->parent;
    else nb = nb->parent;
  }
  return na->depth_end;
}

bool RadixTree::lca_depth(int64_t a, int64_t b, int64_t* out) const {
  const Node* na = find(a);
  const Node* nb = find(b);
  if (!na || !nb) return false;
  *out = lca_of(na, nb);
  return true;
}

bool RadixTree::lca_depths(const int64_t* ids, int32_t n, int32_t* out) const {
  const Node* prev = nullptr;
  for (int32_t i = 0; i < n; ++i) {  // each id looked up once
    const Node* cur = find(ids[i]);
    if (!cur) return false;
    out[i] = i == 0 ? 0 : static_cast<int32_t>(lca_of(prev, cur));
    prev = cur;
  }
  return true;
}

void RadixTree::totals(int64_t* cached, int64_t* locked) const {
  int64_t c = 0, l = 0;
  for (auto& kv : nodes_) {
    if (kv.second->host) continue;  // counted in host_tokens
    const int64_t len = static_cast<int64_t>(kv.second->tokens.size());
    c += len;
    if (kv.second->ref > 0) l += len;
  }
  *cached = c;
  *locked = l;
}

int64_t RadixTree::dump(int64_t* buf, int64_t cap) const {
  int64_t pos = 0;
  std::vector<const Node*> stack;
  auto push_children = [&](const Node* n) {
    std::vector<const Node*> kids;
    kids.reserve(n->children.size());
    for (auto& kv : n->children) kids.push_back(kv.second);
    std::sort(kids.begin(), kids.end(),
              [](const Node* x, const Node* y) { return x->tokens[0] > y->tokens[0]; });
    for (const Node* k : kids) stack.push_back(k);  // smallest first token popped first
  };
  auto put = [&](int64_t v) {
    if (buf && pos < cap) buf[pos] = v;
    ++pos;
  };
  push_children(root_);
  while (!stack.empty()) {
    const Node* n = stack.back();
    stack.pop_back();
    put(n->id);
    put(n->parent->id);
    put(static_cast<int64_t>(n->tokens.size()));
    put(n->ref);
    put(n->tick);
    for (int32_t t : n->tokens) put(t);
    for (int32_t s : n->slots) put(n->host ? -1 - int64_t(s) : s);  // host slots as -1 - id
    push_children(n);
  }
  return pos;
}

}  // namespace rax
