// Prefix-tree chunk manager and DFS plan builder (host only).  The readings it
// implements are listed in manager.h.
#include "manager.h"

#include <algorithm>
#include <functional>

namespace chunkattn {

namespace {
constexpr int kInvalidArg = -1;
constexpr int kNoCapacity = -3;
constexpr int kDupSeq = -4;
constexpr int kUnknownSeq = -5;
constexpr int kState = -10;
constexpr int kInternal = -11;
}  // namespace

Manager::Manager(int chunk, bool share) : C_(chunk), share_(share) {
  nodes_.emplace_back();  // root: no tokens, no slot
  nodes_[0].alive = true;
}

void Manager::set_capacity(int64_t capacity) {
  if (!live_.empty()) throw Error(kState, "pool can only change while no sequence is live");
  if (capacity < 0 || capacity > INT32_MAX) throw Error(kInvalidArg, "capacity out of range");
  capacity_ = capacity;
  free_.reset(capacity);
}

int32_t Manager::alloc_slot() { return free_.take(); }

int32_t Manager::new_node(int32_t parent, int32_t start) {
  int32_t idx;
  if (!free_nodes_.empty()) {
    // a freed node: its lists are empty and keep their room
    idx = free_nodes_.back();
    free_nodes_.pop_back();
    Node& r = nodes_[idx];
    r.ref = 0;
    r.row = false;
  } else {
    idx = static_cast<int32_t>(nodes_.size());
    nodes_.emplace_back();
    Node& f = nodes_[idx];
    if (!spare_tokens_.empty()) {
      f.tokens.swap(spare_tokens_.back());
      spare_tokens_.pop_back();
    }
    if (!spare_ended_.empty()) {
      f.ended.swap(spare_ended_.back());
      spare_ended_.pop_back();
    }
  }
  Node& n = nodes_[idx];
  n.id = next_id_++;
  n.parent = parent;
  n.slot = alloc_slot();
  n.start = start;
  n.alive = true;
  ++n_nodes_;
  return idx;
}

void Manager::free_node(int32_t idx) {
  Node& n = nodes_[idx];
  free_.give(n.slot);
  n.alive = false;
  n.tokens.clear();
  n.children.clear();
  n.ended.clear();
  free_nodes_.push_back(idx);
  --n_nodes_;
}

void Manager::walk_insert(int64_t seq, const int32_t* tokens, int32_t n, InsertWalk* w) const {
  if (n < 1 || tokens == nullptr) throw Error(kInvalidArg, "insert needs at least one token");
  if (live_.count(seq)) throw Error(kDupSeq, "sequence id already live");
  // Walk from the root without touching anything.
  int32_t cur = 0, pos = 0, split_node = -1, split_at = 0;
  w->path.clear();  // matched chunks (the split one included)
  while (share_ && pos < n) {
    int32_t next = -1;
    for (int32_t c : nodes_[cur].children) {
      if (nodes_[c].tokens[0] == tokens[pos]) { next = c; break; }
    }
    if (next < 0) break;
    const std::vector<int32_t>& t = nodes_[next].tokens;
    int32_t lim = std::min<int32_t>(static_cast<int32_t>(t.size()), n - pos), k = 0;
    while (k < lim && t[k] == tokens[pos + k]) ++k;
    pos += k;
    w->path.push_back(next);
    if (k < static_cast<int32_t>(t.size())) { split_node = next; split_at = k; break; }
    cur = next;
  }
  const int64_t need = (split_node >= 0 ? 1 : 0) + chunks_for(n - pos, C_);
  if (need > free_slots())
    throw Error(kNoCapacity, "need " + std::to_string(need) + " chunk slots, " +
                                 std::to_string(free_slots()) + " free");
  w->cur = cur;
  w->pos = pos;
  w->split_node = split_node;
  w->split_at = split_at;
}

int32_t Manager::insert_ops(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops) const {
  InsertWalk w;
  walk_insert(seq, tokens, n, &w);
  for (int32_t x : w.path)
    if (nodes_[x].row)
      ops->push_back(KvOp{nodes_[x].slot, 0, static_cast<int32_t>(nodes_[x].tokens.size()), 0, -1, 0, x, kOpConvert});
  // the new chunks take the lowest free slots, the split's tail first
  FreeSlots::Walk slots(free_);
  int32_t pos = w.pos;
  if (w.split_node >= 0) {
    const Node& head = nodes_[w.split_node];
    ops->push_back(KvOp{slots.next(), 0, static_cast<int32_t>(head.tokens.size()) - w.split_at, w.split_at,
                        head.slot, 1});
  }
  while (pos < n) {
    const int32_t take = std::min<int32_t>(C_, n - pos);
    ops->push_back(KvOp{slots.next(), 0, take, pos, -1, 0});
    pos += take;
  }
  return w.pos;
}

void Manager::mark_tiles(const std::vector<KvOp>& converts) {
  for (const KvOp& o : converts)
    if (o.mode == kOpConvert && o.node >= 0) nodes_[o.node].row = false;
  structural_ = true;
}

int32_t Manager::insert(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops) {
  InsertWalk w;
  walk_insert(seq, tokens, n, &w);
  const std::vector<int32_t>& path = w.path;
  int32_t cur = w.cur, pos = w.pos;
  const int32_t split_node = w.split_node, split_at = w.split_at;
  const int32_t matched = pos;

  // Matched chunks become shared (or are split): the chunk-first path and
  // pool-to-pool copies read tiles, so row-major ones are converted first.
  for (int32_t x : path) {
    Node& nd = nodes_[x];
    if (!nd.row) continue;
    if (ops) ops->push_back(KvOp{nd.slot, 0, static_cast<int32_t>(nd.tokens.size()), 0, -1, 0, x, kOpConvert});
    nd.row = false;
  }

  if (split_node >= 0) {
    int32_t tail = new_node(split_node, nodes_[split_node].start + split_at);
    Node& head = nodes_[split_node];
    Node& t = nodes_[tail];
    t.tokens.assign(head.tokens.begin() + split_at, head.tokens.end());
    head.tokens.resize(split_at);
    t.children.swap(head.children);
    for (int32_t c : t.children) nodes_[c].parent = tail;
    head.children.push_back(tail);
    t.ended.swap(head.ended);
    for (int64_t s : t.ended) live_.find(s)->second.end = tail;
    t.ref = head.ref;
    if (ops)
      ops->push_back(KvOp{t.slot, 0, static_cast<int32_t>(t.tokens.size()), split_at, head.slot, 1});
    cur = split_node;
  }
  while (pos < n) {
    int32_t take = std::min<int32_t>(C_, n - pos);
    int32_t idx = new_node(cur, pos);
    Node& nd = nodes_[idx];
    nd.tokens.assign(tokens + pos, tokens + pos + take);
    nodes_[cur].children.push_back(idx);
    if (ops) ops->push_back(KvOp{nd.slot, 0, take, pos, -1, 0});
    cur = idx;
    pos += take;
  }
  nodes_[cur].ended.push_back(seq);
  live_.emplace(seq, Live{cur, n});
  for (int32_t x = cur; x != 0; x = nodes_[x].parent) nodes_[x].ref += 1;
  structural_ = true;
  return matched;
}

void Manager::append(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops, int32_t src_base) {
  auto it = live_.find(seq);
  if (it == live_.end()) throw Error(kUnknownSeq, "sequence id not live");
  if (n < 1 || tokens == nullptr) throw Error(kInvalidArg, "append needs at least one token");
  append_to(it, tokens, n, ops, src_base);
}

void Manager::append_to(std::map<int64_t, Live>::iterator it, const int32_t* tokens, int32_t n,
                        std::vector<KvOp>* ops, int32_t src_base) {
  const int64_t seq = it->first;
  int32_t e = it->second.end;
  const int32_t fill = static_cast<int32_t>(nodes_[e].tokens.size());
  const int32_t room = nodes_[e].ref == 1 ? C_ - fill : 0;
  const int32_t take = std::min(room, n);
  const int64_t need = chunks_for(n - take, C_);
  if (need > free_slots())
    throw Error(kNoCapacity, "need " + std::to_string(need) + " chunk slots, " +
                                 std::to_string(free_slots()) + " free");
  if (take > 0) {
    Node& nd = nodes_[e];
    nd.tokens.insert(nd.tokens.end(), tokens, tokens + take);
    if (ops) ops->push_back(KvOp{nd.slot, fill, take, src_base, -1, 0, e, nd.row ? kOpRows : kOpTiles});
    // growing into another 64-key tile adds a tile ref to the plan
    if (tiles_of(fill + take) != tiles_of(fill)) structural_ = true;
  }
  it->second.len += n;
  if (take == n) return;
  std::vector<int64_t>& ended = nodes_[e].ended;
  ended.erase(std::find(ended.begin(), ended.end(), seq));
  int32_t cur = e, i = take;
  int32_t pos = nodes_[e].start + static_cast<int32_t>(nodes_[e].tokens.size());
  while (i < n) {
    int32_t piece = std::min<int32_t>(C_, n - i);
    int32_t idx = new_node(cur, pos);
    Node& nd = nodes_[idx];
    nd.tokens.assign(tokens + i, tokens + i + piece);
    nd.ref = 1;
    nd.row = row_appends_;
    nodes_[cur].children.push_back(idx);
    if (ops) ops->push_back(KvOp{nd.slot, 0, piece, src_base + i, -1, 0, idx, nd.row ? kOpRows : kOpTiles});
    cur = idx;
    pos += piece;
    i += piece;
  }
  nodes_[cur].ended.push_back(seq);
  it->second.end = cur;
  structural_ = true;
}

void Manager::append_batch(const int64_t* seqs, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops) {
  if (n < 1 || seqs == nullptr || tokens == nullptr) throw Error(kInvalidArg, "append batch needs n >= 1");
  // The first offending entry decides the error (an unknown id before a
  // repeat at the same position); repeats are found by sorting (id, position).
  std::vector<std::pair<int64_t, int32_t>> order(static_cast<size_t>(n));
  for (int32_t j = 0; j < n; ++j) order[j] = {seqs[j], j};
  std::sort(order.begin(), order.end());
  int32_t first_repeat = n;
  for (int32_t j = 1; j < n; ++j)
    if (order[j].first == order[j - 1].first) first_repeat = std::min(first_repeat, order[j].second);
  int64_t need = 0;
  std::vector<std::map<int64_t, Live>::iterator> at(static_cast<size_t>(n));
  for (int32_t j = 0; j < n; ++j) {
    auto it = live_.find(seqs[j]);
    if (it == live_.end()) throw Error(kUnknownSeq, "sequence id not live: " + std::to_string(seqs[j]));
    if (j == first_repeat) throw Error(kInvalidArg, "sequence id repeated in a batch");
    const Node& e = nodes_[it->second.end];
    if (!(e.ref == 1 && static_cast<int32_t>(e.tokens.size()) < C_)) ++need;
    at[j] = it;
  }
  if (need > free_slots())
    throw Error(kNoCapacity, "need " + std::to_string(need) + " chunk slots, " +
                                 std::to_string(free_slots()) + " free");
  for (int32_t j = 0; j < n; ++j) append_to(at[j], tokens + j, 1, ops, j);
}

int64_t Manager::row_chunks() const {
  int64_t n = 0;
  for (size_t i = 1; i < nodes_.size(); ++i) n += nodes_[i].alive && nodes_[i].row ? 1 : 0;
  return n;
}

bool Manager::next_append_structural() const {
  for (const auto& kv : live_) {
    const Node& nd = nodes_[kv.second.end];
    const int32_t fill = static_cast<int32_t>(nd.tokens.size());
    if (nd.ref != 1 || fill >= C_ || tiles_of(fill + 1) != tiles_of(fill)) return true;
  }
  return false;
}

void Manager::stock_for_append(const NextAppend& next) {
  size_t fresh = 0;
  for (const NextAppend::Add& a : next.add) {
    if (static_cast<size_t>(a.idx) >= nodes_.size()) ++fresh;
    std::vector<int32_t>& ch = nodes_[a.parent].children;
    ch.reserve(ch.size() + 1);
  }
  // geometric growth: an exact reserve would move every node at every call
  if (nodes_.capacity() < next.n_nodes) nodes_.reserve(std::max(next.n_nodes, 2 * nodes_.capacity()));
  while (spare_tokens_.size() < fresh) {
    spare_tokens_.emplace_back();
    spare_tokens_.back().reserve(C_);
  }
  while (spare_ended_.size() < fresh) {
    spare_ended_.emplace_back();
    spare_ended_.back().reserve(1);
  }
}

bool Manager::predict_append_batch(const int64_t* seqs, int32_t n, NextAppend* out) const {
  NextAppend& x = *out;
  x.grow.clear();
  x.add.clear();
  x.structural = false;
  x.n_nodes = nodes_.size();
  if (n < 1 || seqs == nullptr) return false;
  std::vector<int64_t> sorted(seqs, seqs + n);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return false;
  // new chunks take node indices from the reuse list (last first), then the
  // end of the node array, and the lowest free slots in increasing order
  size_t reuse = free_nodes_.size();
  FreeSlots::Walk slots(free_);
  for (int32_t j = 0; j < n; ++j) {
    auto it = live_.find(seqs[j]);
    if (it == live_.end()) return false;
    const int32_t e = it->second.end;
    const Node& nd = nodes_[e];
    const int32_t fill = static_cast<int32_t>(nd.tokens.size());
    if (nd.ref == 1 && fill < C_) {
      x.grow.push_back(e);
      if (tiles_of(fill + 1) != tiles_of(fill)) x.structural = true;
      continue;
    }
    const int32_t slot = slots.next();
    if (slot < 0) return false;  // out of slots
    int32_t idx;
    if (reuse > 0) {
      idx = free_nodes_[--reuse];
    } else {
      idx = static_cast<int32_t>(x.n_nodes++);
    }
    x.add.push_back({e, idx, next_id_ + static_cast<int32_t>(x.add.size()), slot, nd.start + fill, seqs[j]});
    x.structural = true;
  }
  return true;
}

void Manager::remove(int64_t seq) {
  auto it = live_.find(seq);
  if (it == live_.end()) throw Error(kUnknownSeq, "sequence id not live");
  structural_ = true;
  int32_t e = it->second.end;
  live_.erase(it);
  std::vector<int64_t>& ended = nodes_[e].ended;
  ended.erase(std::find(ended.begin(), ended.end(), seq));
  for (int32_t x = e; x != 0;) {
    int32_t p = nodes_[x].parent;
    if (--nodes_[x].ref == 0) {
      std::vector<int32_t>& sib = nodes_[p].children;
      sib.erase(std::find(sib.begin(), sib.end(), x));
      free_node(x);
    }
    x = p;
  }
}

std::vector<int64_t> Manager::sequences() const {
  std::vector<int64_t> out;
  out.reserve(live_.size());
  for (const auto& kv : live_) out.push_back(kv.first);
  return out;
}

int32_t Manager::seq_len(int64_t seq) const {
  auto it = live_.find(seq);
  if (it == live_.end()) throw Error(kUnknownSeq, "sequence id not live");
  return it->second.len;
}

void Plan::clear() {
  rows.clear();
  dfs_seq.clear();
  dfs_qrow.clear();
  cf_units.clear();
  sf_tasks.clear();
  chunk_refs.clear();
  row_node.clear();
  ref_node.clear();
  ref_sub.clear();
  ref_task.clear();
  ref_pos.clear();
  private_ref.clear();
  seq_parts.clear();
  part_list.clear();
  cf_tasks = 0;
  sf_group = 0;
  n_parts = 0;
  dense_parts = 0;
  part_stride = 1;
  cf_chunk_reads = sf_chunk_reads = shared_chunks = shared_tokens = unique_tokens = attended_tokens = 0;
  row_refs = 0;
}

void Manager::build_plan(int cf_group, int sf_group, bool two_phase, Plan* plan, int64_t sf_min_tasks,
                         const NextAppend* next) const {
  Plan& P = *plan;
  P.clear();

  // The nodes as the plan sees them: the tree as it is, or with `next`'s
  // tokens appended (a grown chunk holds one token more; a new chunk, one
  // token, is its parent's last child and holds the sequence that moved to it).
  const size_t n_nodes = next ? next->n_nodes : nodes_.size();
  std::vector<int32_t> grown, virt, vchild_head, vchild_next;
  if (next) {
    grown.assign(n_nodes, 0);
    for (int32_t g : next->grow) grown[g] = 1;
    virt.assign(n_nodes, -1);
    vchild_head.assign(n_nodes, -1);
    vchild_next.assign(next->add.size(), -1);
    std::vector<int32_t> tail(n_nodes, -1);
    for (size_t k = 0; k < next->add.size(); ++k) {
      const NextAppend::Add& a = next->add[k];
      virt[a.idx] = static_cast<int32_t>(k);
      if (tail[a.parent] < 0)
        vchild_head[a.parent] = static_cast<int32_t>(k);
      else
        vchild_next[tail[a.parent]] = static_cast<int32_t>(k);
      tail[a.parent] = static_cast<int32_t>(k);
    }
  }
  auto added = [&](int32_t n) -> const NextAppend::Add* {
    return next && virt[n] >= 0 ? &next->add[virt[n]] : nullptr;
  };
  auto fill_of = [&](int32_t n) -> int32_t {
    if (added(n)) return 1;
    return static_cast<int32_t>(nodes_[n].tokens.size()) + (next ? grown[n] : 0);
  };
  auto ref_of = [&](int32_t n) -> int32_t { return added(n) ? 1 : nodes_[n].ref; };
  auto row_of = [&](int32_t n) -> bool { return added(n) ? row_appends_ : nodes_[n].row; };
  std::vector<int32_t> kids;
  auto children_of = [&](int32_t n) -> const std::vector<int32_t>& {
    if (!next) return nodes_[n].children;
    kids.clear();
    if (!added(n)) kids = nodes_[n].children;
    for (int32_t k = vchild_head[n]; k >= 0; k = vchild_next[k]) kids.push_back(next->add[k].idx);
    return kids;
  };
  std::vector<int64_t> ends;
  auto ended_of = [&](int32_t n) -> const std::vector<int64_t>& {
    if (!next) return nodes_[n].ended;
    ends.clear();
    if (const NextAppend::Add* a = added(n)) {
      ends.push_back(a->seq);
      return ends;
    }
    for (int64_t s : nodes_[n].ended) {
      bool moved = false;
      for (int32_t k = vchild_head[n]; k >= 0 && !moved; k = vchild_next[k]) moved = next->add[k].seq == s;
      if (!moved) ends.push_back(s);
    }
    return ends;
  };

  // Caller row of each sequence: rank in ascending id order.
  std::vector<int64_t> ids;
  ids.reserve(live_.size());
  for (const auto& kv : live_) ids.push_back(kv.first);
  auto qrow_of = [&](int64_t s) {
    return static_cast<int32_t>(std::lower_bound(ids.begin(), ids.end(), s) - ids.begin());
  };

  // Pass 1: DFS pre-order -> canonical rows, DFS order, row of each node,
  // the row where each DFS position's sequence ends.
  std::vector<int32_t> row_node;          // node index of each row
  std::vector<int32_t> end_row;           // per DFS position
  struct Frame { int32_t node, parent_row; bool closing; int32_t row; };
  std::vector<Frame> stack;
  {
    const std::vector<int32_t>& rc = children_of(0);
    for (auto it = rc.rbegin(); it != rc.rend(); ++it) stack.push_back({*it, -1, false, -1});
  }
  while (!stack.empty()) {
    Frame f = stack.back();
    stack.pop_back();
    if (f.closing) {
      P.rows[static_cast<size_t>(f.row) * 7 + 5] = static_cast<int32_t>(P.dfs_seq.size());
      continue;
    }
    const NextAppend::Add* a = added(f.node);
    int32_t r = static_cast<int32_t>(row_node.size());
    row_node.push_back(f.node);
    if (a)
      P.rows.insert(P.rows.end(), {a->id, f.parent_row, a->start, 1, static_cast<int32_t>(P.dfs_seq.size()), -1,
                                   a->slot});
    else
      P.rows.insert(P.rows.end(), {nodes_[f.node].id, f.parent_row, nodes_[f.node].start, fill_of(f.node),
                                   static_cast<int32_t>(P.dfs_seq.size()), -1, nodes_[f.node].slot});
    P.row_node.push_back(f.node);
    for (int64_t s : ended_of(f.node)) {
      P.dfs_seq.push_back(s);
      P.dfs_qrow.push_back(qrow_of(s));
      end_row.push_back(r);
    }
    stack.push_back({f.node, f.parent_row, true, r});
    const std::vector<int32_t>& ch = children_of(f.node);
    for (auto it = ch.rbegin(); it != ch.rend(); ++it) stack.push_back({*it, r, false, -1});
  }
  const int32_t n_rows = static_cast<int32_t>(row_node.size());
  const int32_t n_seq = static_cast<int32_t>(P.dfs_seq.size());
  auto R = [&](int32_t r, int c) { return P.rows[static_cast<size_t>(r) * 7 + c]; };

  // Pass 2: runs of shared chunks (range >= 2).  A child with the same range
  // as its parent continues the parent's run (a chain: one child, nobody
  // ends at the parent); a run holds at most cf_group chunks, and a chain
  // longer than that is cut into as few runs as the limit allows, of equal
  // length to within one row: no run is left with a stub of a chain, whose
  // units would hold block slots for little work (2,112 shared + 512
  // private tokens, 32 sequences: runs of 11 + 11 + 11 chunks instead of
  // 16 + 16 + 1, 53.0-53.1 against 53.8 us).
  std::vector<int32_t> task_of_row(n_rows, -1);
  struct Task { int32_t b, e, chunk_begin, n_chunks, last_row; };
  std::vector<Task> tasks;
  for (int32_t r = 0; r < n_rows; ++r) {
    int32_t b = R(r, 4), e = R(r, 5), p = R(r, 1);
    P.unique_tokens += R(r, 3);
    P.attended_tokens += static_cast<int64_t>(R(r, 3)) * (e - b);
    if (e - b < 2) continue;
    ++P.shared_chunks;
    P.shared_tokens += R(r, 3);
    if (!two_phase) continue;
    int32_t t = p >= 0 ? task_of_row[p] : -1;
    // n_chunks counts the tile refs of the run (one per chunk of 64)
    const int32_t nt = tiles_of(R(r, 3));
    if (t >= 0 && tasks[t].b == b && tasks[t].e == e && tasks[t].last_row == p) {
      tasks[t].n_chunks += nt;
      tasks[t].last_row = r;
    } else {
      t = static_cast<int32_t>(tasks.size());
      tasks.push_back({b, e, -1, nt, r});
    }
    task_of_row[r] = t;
  }
  {
    // cut the chains: each run takes rows up to ceil(left / runs left) tiles
    std::vector<std::vector<int32_t>> chain_rows(tasks.size());
    for (int32_t r = 0; r < n_rows; ++r)
      if (task_of_row[r] >= 0) chain_rows[task_of_row[r]].push_back(r);
    std::vector<Task> cut;
    const int32_t g = std::max(1, cf_group);
    for (size_t t = 0; t < tasks.size(); ++t) {
      int32_t left = tasks[t].n_chunks;
      const std::vector<int32_t>& rows = chain_rows[t];
      for (size_t i = 0; i < rows.size();) {
        const int32_t runs_left = (left + g - 1) / g, cap = (left + runs_left - 1) / runs_left;
        const int32_t id = static_cast<int32_t>(cut.size());
        cut.push_back({tasks[t].b, tasks[t].e, -1, 0, -1});
        do {
          cut[id].n_chunks += tiles_of(R(rows[i], 3));
          cut[id].last_row = rows[i];
          task_of_row[rows[i]] = id;
          ++i;
        } while (i < rows.size() && cut[id].n_chunks + tiles_of(R(rows[i], 3)) <= cap);
        left -= cut[id].n_chunks;
      }
    }
    tasks.swap(cut);
  }
  // chunk refs of each run, in row order; its 32-row units (partial ids later)
  std::vector<int32_t> unit_task;
  {
    std::vector<std::vector<int32_t>> task_rows(tasks.size());
    for (int32_t r = 0; r < n_rows; ++r)
      if (task_of_row[r] >= 0) task_rows[task_of_row[r]].push_back(r);
    for (size_t t = 0; t < tasks.size(); ++t) {
      tasks[t].chunk_begin = static_cast<int32_t>(P.chunk_refs.size() / 2);
      for (int32_t r : task_rows[t])
        for (int32_t k = 0; k < tiles_of(R(r, 3)); ++k) {
          if (row_of(row_node[r])) throw Error(kInternal, "plan: a shared chunk is stored row-major");
          P.chunk_refs.push_back(tile_slot(R(r, 6), k));
          P.chunk_refs.push_back(tile_fill(R(r, 3), k));
          P.ref_node.push_back(row_node[r]);
          P.ref_sub.push_back(k);
        }
      P.cf_chunk_reads += tasks[t].n_chunks * ((tasks[t].e - tasks[t].b + 31) / 32);
      for (int32_t rb = 0; rb * 32 < tasks[t].e - tasks[t].b; ++rb) {
        CfUnit u{};
        u.chunk_begin = tasks[t].chunk_begin;
        u.n_chunks = tasks[t].n_chunks;
        u.row_begin = tasks[t].b + rb * 32;
        u.n_rows = std::min(32, tasks[t].e - tasks[t].b - rb * 32);
        u.reuse = tasks[t].e - tasks[t].b > 32 ? 1 : 0;
        u.qrow_base = P.dfs_qrow[u.row_begin];
        for (int r = 1; r < u.n_rows; ++r)
          if (P.dfs_qrow[u.row_begin + r] != u.qrow_base + r) u.qrow_base = -1;
        for (int c = 0; c < kCfInline && c < u.n_chunks; ++c) {
          u.slot[c] = P.chunk_refs[2 * (u.chunk_begin + c)];
          u.n_valid[c] = P.chunk_refs[2 * (u.chunk_begin + c) + 1];
        }
        P.cf_units.push_back(u);
        unit_task.push_back(static_cast<int32_t>(t));
      }
    }
    P.cf_tasks = static_cast<int64_t>(tasks.size());
  }

  // Pass 3: per sequence, the shared runs on its path (root first) and its
  // private chunk refs; then the refs cut into sequence-first tasks.
  // entries[ent_first[i] + j] is the j-th partial of sequence i in merge
  // order: a run t (t >= 0) or a sequence-first task k (-1 - k).
  std::vector<int32_t> run_first(static_cast<size_t>(n_seq) + 1, 0), runs;
  std::vector<int32_t> priv_first(static_cast<size_t>(n_seq) + 1, 0);
  std::vector<std::pair<int32_t, int32_t>> priv;  // (row, tile of the row's chunk)
  std::vector<int32_t> path;
  for (int32_t i = 0; i < n_seq; ++i) {
    path.clear();
    for (int32_t r = end_row[i]; r >= 0; r = R(r, 1)) path.push_back(r);
    std::reverse(path.begin(), path.end());
    run_first[i] = static_cast<int32_t>(runs.size());
    priv_first[i] = static_cast<int32_t>(priv.size());
    int32_t last_task = -1;
    for (int32_t r : path) {
      int32_t t = task_of_row[r];
      if (t >= 0) {
        if (t != last_task) runs.push_back(t);
        last_task = t;
      } else {
        for (int32_t k = 0; k < tiles_of(R(r, 3)); ++k) priv.push_back({r, k});
      }
    }
  }
  run_first[n_seq] = static_cast<int32_t>(runs.size());
  priv_first[n_seq] = static_cast<int32_t>(priv.size());
  if (sf_group <= 0) {
    // Left open: the largest of 16, 8 and 4 (or 3, below) refs per task
    // that still makes at least sf_min_tasks tasks, so that the last round of
    // blocks on the chip stays well filled; longer tasks mean fewer partials
    // to write and merge.  Where chunk-first units share the launch the bar is 8/5 of
    // that: their long blocks hold slots through the first rounds, and the
    // sequence-first tail needs more, shorter blocks to even out behind them
    // (1024 shared + 1024 private tokens at 64 and 72 sequences, 32 heads:
    // group 8 in 170.4 and 190.1 us where 16 took 174.2 and 193.4).
    sf_group = 4;
    const int64_t target = P.cf_units.empty() ? sf_min_tasks : (sf_min_tasks * 8 + 4) / 5;
    for (int g : {16, 8}) {
      int64_t tasks = 0;
      for (int32_t i = 0; i < n_seq; ++i) tasks += (priv_first[i + 1] - priv_first[i] + g - 1) / g;
      if (tasks >= target) {
        sf_group = g;
        break;
      }
    }
    // Falling back to 4 behind chunk-first units: 3 when that makes more
    // tasks and no sequence is left a one-chunk remainder (8 private chunks
    // become 3 + 3 + 2).  4,096 shared + 512 private tokens, 32 sequences:
    // 57.9-58.2 us against 58.9; 2,048 + 512 at 48 sequences 72.5 against
    // 73.1-73.3 us.  4 chunks (3 + 1) measured slower with 3 and stay at 4.
    if (sf_group == 4 && !P.cf_units.empty()) {
      bool no_single = true;
      int64_t t3 = 0, t4 = 0;
      for (int32_t i = 0; i < n_seq; ++i) {
        const int32_t n = priv_first[i + 1] - priv_first[i];
        if (n > 1 && n % 3 == 1) no_single = false;
        t3 += (n + 2) / 3;
        t4 += (n + 3) / 4;
      }
      if (no_single && t3 > t4) sf_group = 3;
    }
  }
  P.sf_group = sf_group;
  std::vector<int32_t> ent_first(static_cast<size_t>(n_seq) + 1, 0), entries;
  int32_t max_parts = 0;
  for (int32_t i = 0; i < n_seq; ++i) {
    ent_first[i] = static_cast<int32_t>(entries.size());
    entries.insert(entries.end(), runs.begin() + run_first[i], runs.begin() + run_first[i + 1]);
    const int32_t p0 = priv_first[i], p1 = priv_first[i + 1];
    for (int32_t j = p0; j < p1; j += sf_group) {
      const int32_t stop = std::min(p1, j + sf_group);
      SfTask st{};
      st.chunk_begin = static_cast<int32_t>(P.chunk_refs.size() / 2);
      st.n_chunks = stop - j;
      st.dfs_pos = i;
      st.part_id = -1;
      st.qrow = P.dfs_qrow[i];
      st.append_at = -1;
      for (int32_t q = j; q < stop; ++q) {
        const int c = q - j;
        const int32_t r = priv[q].first, k = priv[q].second;
        const bool row = row_of(row_node[r]);
        const int32_t slot = tile_slot(R(r, 6), k), fill = tile_fill(R(r, 3), k) | (row ? kRowBit : 0);
        P.row_refs += row ? 1 : 0;
        // the last tile of the chunk where the sequence ends takes its next
        // decoded token
        if (r == end_row[i] && k + 1 == tiles_of(R(r, 3))) st.append_at = c;
        if (c < kSfInline) {
          st.slot[c] = slot;
          st.n_valid[c] = fill;
        }
        if (R(r, 5) - R(r, 4) >= 2) st.reuse = 1;
        P.chunk_refs.push_back(slot);
        P.chunk_refs.push_back(fill);
        P.ref_node.push_back(row_node[r]);
        P.ref_sub.push_back(k);
      }
      P.sf_chunk_reads += st.n_chunks;
      entries.push_back(-1 - static_cast<int32_t>(P.sf_tasks.size()));
      P.sf_tasks.push_back(st);
    }
    max_parts = std::max(max_parts, static_cast<int32_t>(entries.size()) - ent_first[i]);
  }
  ent_first[n_seq] = static_cast<int32_t>(entries.size());

  // Partial ids.  Dense (a sequence's j-th partial is i * max_parts + j) when
  // no sequence has more than kDenseParts partials and the dense slots cost
  // at most about twice the partials themselves: the merge then computes
  // every address from the sequence's position and fetches all of them in
  // one round trip.  Otherwise compact ids: a run's rows take consecutive
  // ids, then the sequence-first tasks.
  const int64_t n_entries = static_cast<int64_t>(entries.size());
  const bool dense = max_parts <= kDenseParts && static_cast<int64_t>(n_seq) * max_parts <= 2 * n_entries + 64;
  P.dense_parts = dense ? max_parts : 0;
  std::vector<int32_t> task_part(tasks.size(), -1);  // dense: slot j; compact: base id
  if (P.dense_parts) {
    P.part_stride = max_parts;
    for (int32_t i = 0; i < n_seq; ++i)
      for (int32_t j = 0; ent_first[i] + j < ent_first[i + 1]; ++j) {
        const int32_t e = entries[ent_first[i] + j];
        if (e >= 0) {
          if (task_part[e] >= 0 && task_part[e] != j) throw Error(kInternal, "plan: run at two list positions");
          task_part[e] = j;
        } else {
          P.sf_tasks[-1 - e].part_id = i * max_parts + j;
        }
      }
    P.n_parts = n_seq * max_parts;
  } else {
    P.part_stride = 1;
    int32_t parts = 0;
    for (size_t t = 0; t < tasks.size(); ++t) {
      task_part[t] = parts;
      parts += tasks[t].e - tasks[t].b;
    }
    for (SfTask& st : P.sf_tasks) st.part_id = parts++;
    P.n_parts = parts;
  }
  for (size_t k = 0; k < P.cf_units.size(); ++k) {
    CfUnit& u = P.cf_units[k];
    const Task& tk = tasks[unit_task[k]];
    u.part_base = P.dense_parts ? u.row_begin * P.part_stride + task_part[unit_task[k]]
                                : task_part[unit_task[k]] + (u.row_begin - tk.b);
  }
  P.seq_parts.assign(static_cast<size_t>(n_seq) * 2, 0);
  for (int32_t i = 0; i < n_seq; ++i) {
    P.seq_parts[2 * i] = static_cast<int32_t>(P.part_list.size());
    for (int32_t q = ent_first[i]; q < ent_first[i + 1]; ++q) {
      const int32_t e = entries[q];
      P.part_list.push_back(e >= 0 ? (P.dense_parts ? i * P.part_stride + task_part[e] : task_part[e] + (i - tasks[e].b))
                                   : P.sf_tasks[-1 - e].part_id);
    }
    P.seq_parts[2 * i + 1] = ent_first[i + 1] - ent_first[i];
  }
  // Longest sequence-first tasks first: they start earliest, and the four
  // waves of a block get tasks of about the same length.  Among tasks of one
  // length, in the order of their first chunk's slot: blocks that run at the
  // same time then read slots close together also where decoding has
  // interleaved the sequences' chunks in the pool (one new chunk per
  // sequence per round); measured on MI355X, 32 sequences with 2,048 shared
  // and 496 private tokens grown that way take 55.1 us per step in sequence
  // order, 54.0 us in slot order, 52.7 us when inserted whole.
  std::stable_sort(P.sf_tasks.begin(), P.sf_tasks.end(), [&P](const SfTask& x, const SfTask& y) {
    if (x.n_chunks != y.n_chunks) return x.n_chunks > y.n_chunks;
    return P.chunk_refs[2 * x.chunk_begin] < P.chunk_refs[2 * y.chunk_begin];
  });
  // where each chunk ref lives, so a fill change can be patched in place
  P.ref_task.assign(P.ref_node.size(), -1);
  P.ref_pos.assign(P.ref_node.size(), -1);
  P.private_ref.assign(n_nodes, -1);
  for (size_t t = 0; t < P.sf_tasks.size(); ++t)
    for (int c = 0; c < P.sf_tasks[t].n_chunks; ++c) {
      const int32_t k = P.sf_tasks[t].chunk_begin + c;
      P.ref_task[k] = static_cast<int32_t>(t);
      P.ref_pos[k] = c;
      const int32_t node = P.ref_node[k];
      // a private chunk's appends go to its last tile
      if (ref_of(node) == 1 && P.ref_sub[k] + 1 == tiles_of(fill_of(node))) P.private_ref[node] = k;
    }
}

void Manager::refresh_fills(Plan* plan) const {
  Plan& P = *plan;
  P.unique_tokens = P.attended_tokens = P.shared_tokens = 0;
  const size_t n_rows = P.row_node.size();
  for (size_t r = 0; r < n_rows; ++r) {
    const int32_t fill = static_cast<int32_t>(nodes_[P.row_node[r]].tokens.size());
    int32_t* row = &P.rows[r * 7];
    row[3] = fill;
    P.unique_tokens += fill;
    P.attended_tokens += static_cast<int64_t>(fill) * (row[5] - row[4]);
    if (row[5] - row[4] >= 2) P.shared_tokens += fill;
  }
  for (size_t k = 0; k < P.ref_node.size(); ++k) {
    const Node& nd = nodes_[P.ref_node[k]];
    P.chunk_refs[2 * k + 1] =
        tile_fill(static_cast<int32_t>(nd.tokens.size()), P.ref_sub[k]) | (nd.row ? kRowBit : 0);
  }
  for (CfUnit& u : P.cf_units)
    for (int c = 0; c < kCfInline && c < u.n_chunks; ++c) u.n_valid[c] = P.chunk_refs[2 * (u.chunk_begin + c) + 1];
  for (SfTask& t : P.sf_tasks)
    for (int c = 0; c < kSfInline && c < t.n_chunks; ++c) t.n_valid[c] = P.chunk_refs[2 * (t.chunk_begin + c) + 1];
}

}  // namespace chunkattn
