// Host radix tree over a token-granular KV pool, with the pool's slot allocator.
//
// Operations follow the pages: longest-prefix match ("traverse"), insert of a
// finished or prefilled request as new edges / leaves, node split at a divergence
// point, ref counts that pin nodes used by running requests, and LRU eviction of
// leaves, with cached and running KV sharing one pool
// (2312.07104_SGLang notes, §3 and Figure 3; bowenzhou SGLang review, "Work loop";
// hustzhy SGLang post, §2.3). The reproducibility rules where the pages are silent
// (split on match, one logical tick per call, whole-leaf eviction, lowest-slot-first
// allocation, duplicate slots returned on insert) are stated in include/rax.h.
#pragma once

#include <cstdint>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

namespace rax {

// Free set of pool slots; hands out the lowest ids first.
class SlotAllocator {
 public:
  explicit SlotAllocator(int64_t num_slots);
  int64_t num_slots() const { return num_slots_; }
  int64_t num_free() const { return num_free_; }
  bool is_free(int32_t s) const { return (words_[s >> 6] >> (s & 63)) & 1ull; }
  // Takes n lowest free slots into out (ascending). False (nothing taken) if short.
  bool alloc(int64_t n, int32_t* out);
  // Returns slots; the caller has checked they are in range and not free.
  void release(const int32_t* slots, int64_t n);
  void release_one(int32_t s);

 private:
  int64_t num_slots_;
  int64_t num_free_;
  int64_t hint_;                 // no free bit below word hint_
  std::vector<uint64_t> words_;  // bit set = slot free
};

struct Node {
  int64_t id = 0;
  Node* parent = nullptr;
  std::vector<int32_t> tokens;  // edge label
  std::vector<int32_t> slots;   // one pool slot per label token
  std::unordered_map<int32_t, Node*> children;  // keyed by the child's first token
  int64_t depth_end = 0;        // tokens from the root to the end of this node
  int32_t ref = 0;
  int64_t tick = 0;
  bool in_lru = false;
  // host tier: the node's KV lives in host slots (slots holds host slot ids); host nodes
  // only ever have host descendants
  bool host = false;
  bool in_hlru = false;
  int32_t ndev = 0;             // children that are device nodes
};

// KV moves between the device pool and the host tier, in the order the tree decided
// them: kind 0 = demotion (device slot src -> host slot dst), 1 = promotion (host slot
// src -> device slot dst). Run in this order they are correct even when a slot freed by
// one move is taken by a later one.
struct Moves {
  std::vector<int32_t> kind, src, dst;
  void push(int32_t k, int32_t s, int32_t d) { kind.push_back(k); src.push_back(s); dst.push_back(d); }
  void clear() { kind.clear(); src.clear(); dst.clear(); }
};

class RadixTree {
 public:
  explicit RadixTree(int64_t num_slots);
  ~RadixTree();
  RadixTree(const RadixTree&) = delete;
  RadixTree& operator=(const RadixTree&) = delete;

  SlotAllocator& alloc() { return alloc_; }
  const SlotAllocator& alloc() const { return alloc_; }
  SlotAllocator& host_alloc() { return host_alloc_; }
  const SlotAllocator& host_alloc() const { return host_alloc_; }
  // Host tier of host_slots token slots (0 = none). Only while no node is on the host.
  bool set_host_tier(int64_t host_slots);
  // Moves recorded by evictions and promotions since the last take (see Moves).
  Moves& pending() { return pending_; }
  const Moves& pending() const { return pending_; }
  // Promote the host-resident continuation of tokens' cached device prefix to the device,
  // node by node: device slots for it (evicting, hence demoting, when short); stops at
  // the first node that does not fit. Returns the tokens promoted; freed device slots
  // append to freed.
  int64_t promote(const int32_t* tokens, int64_t n, std::vector<int32_t>* freed);

  int64_t match(const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* out_node);
  // Length of the longest cached prefix of tokens, without splitting or ticking anything.
  int64_t prefix_len(const int32_t* tokens, int64_t n) const;
  // Returns false (nothing changed) if a caller slot is out of range or free.
  bool insert(const int32_t* tokens, const int32_t* slots, int64_t n, int32_t* out_slots,
              int64_t* out_existing, int64_t* out_node);
  // The same insert, walking from a node on the sequence's path instead of the root:
  // `start` must be a device node whose root path spells the first tokens of the
  // sequence (a node matched for these tokens and still locked qualifies), and the
  // caller's slots for positions [0, trusted) must be the tree's. The walk starts at the
  // deepest of start and its ancestors that ends at or before `trusted`. Returns 1 for a
  // bad start (nothing changed), 2 for a bad slot (nothing changed), 0 when done.
  int insert_from(int64_t start, int64_t trusted, const int32_t* tokens, const int32_t* slots, int64_t n,
                  int32_t* out_slots, int64_t* out_existing, int64_t* out_node);
  // 0 ok, 1 unknown node, 2 would go below zero, 3 host node.
  int lock_ref(int64_t node, int32_t delta);
  int64_t evict(int64_t num_tokens, int32_t* out_freed, int64_t cap);
  bool lca_depth(int64_t a, int64_t b, int64_t* out) const;
  // out[0] = 0, out[i] = lca_depth(ids[i - 1], ids[i]); false if an id is unknown
  bool lca_depths(const int64_t* ids, int32_t n, int32_t* out) const;
  const Node* find(int64_t id) const;
  int64_t dump(int64_t* buf, int64_t cap) const;  // returns words needed

  int64_t num_nodes() const { return static_cast<int64_t>(nodes_.size()) - 1; }
  int64_t clock() const { return clock_; }
  void totals(int64_t* cached, int64_t* locked) const;
  int64_t matched_total = 0, inserted_total = 0, evicted_total = 0;
  int64_t demoted_total = 0, promoted_total = 0, host_tokens = 0;

 private:
  Node* new_node();
  Node* split(Node* child, int64_t k);  // upper part gets the first k tokens
  // Walks the longest cached prefix, splitting at its end. Returns the end node and
  // the matched length; appends the slots if out != nullptr.
  Node* walk(const int32_t* tokens, int64_t n, int64_t* matched, int32_t* out);
  // walk from `node`, tokens [i0, n) left to match (out indexed from position 0)
  Node* walk_from(Node* node, int64_t i0, const int32_t* tokens, int64_t n, int64_t* matched, int32_t* out);
  // insert with the walk starting at `start`, which ends at position d
  bool insert_at(Node* start, int64_t d, const int32_t* tokens, const int32_t* slots, int64_t n,
                 int32_t* out_slots, int64_t* out_existing, int64_t* out_node);
  void tick_path(Node* n);
  void lru_update(Node* n);  // re-evaluate device-candidate membership
  void lru_remove(Node* n);
  void hlru_update(Node* n);  // re-evaluate host-leaf membership
  void hlru_remove(Node* n);
  void erase_node(Node* n);   // unlink a node with no children
  void drop_host_leaves(int64_t need);
  void drop_subtree(Node* n, int32_t* out_freed, int64_t cap, int64_t* freed);

  SlotAllocator alloc_;
  Node* root_;
  int64_t next_id_ = 1;
  int64_t clock_ = 0;
  std::unordered_map<int64_t, Node*> nodes_;
  std::set<std::pair<int64_t, int64_t>> lru_;  // (tick, id): device nodes, ref 0, no device child
  std::set<std::pair<int64_t, int64_t>> hlru_;  // (tick, id): host nodes, no children, ref 0
  SlotAllocator host_alloc_{0};
  Moves pending_;
};

}  // namespace rax
