// Host-side prefix-tree chunk manager: the trie of chunk nodes, the slot
// allocator, and the DFS flattening into the per-step work plan.
//
// Prefix-aware KV cache (paperlayer.ai summary of arXiv 2402.15220v4, section
// 3.1 and Figure 1; explainer 0h-n0.github.io/posts/paper-2402-15220,
// "Prefix-Aware KV Cache" and "dynamic prefix detection"): K/V are cut into
// chunks that are the nodes of a prefix tree; a path from the root is a token
// prefix and each live sequence is one path; a shared prefix is stored once;
// references are counted and an unreferenced chunk returns its slot.
//
// Readings for what the pages leave open (each one decides a bit of the
// exported table):
//  * a node holds at most C tokens; new paths are cut into full chunks;
//  * a divergence inside a node splits it -- the head keeps its slot, the tail
//    gets a new slot, becomes the only child, and inherits the node's
//    children and the sequences that ended in it;
//  * children stay in creation order; matching takes the first child whose
//    first token is the next token;
//  * sequences that end at a node precede its children in DFS order, in
//    arrival order;
//  * append writes in place only into a private (one reference) chunk that is
//    not full, otherwise grows new private chunks; appends never deduplicate;
//  * slots: lowest free index first; a split's tail slot before new tokens'
//    slots, which follow token order;
//  * a failing call changes nothing.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <functional>
#include <map>
#include <stdexcept>
#include <string>
#include <vector>

#include "kernels.h"

namespace chunkattn {

// Status codes mirror the CA_E_* values of the C header.
struct Error : std::runtime_error {
  int code;
  Error(int c, const std::string& m) : std::runtime_error(m), code(c) {}
};

// A device-side copy the host asks for after a tree mutation.  Either rows
// from the caller's K/V ([row][head][dim], fp16) or rows of another slot are
// written to key positions [dst_key0, dst_key0 + n_rows) of dst_slot.  A
// write that starts at key 0 is the chunk's first since its slot was
// allocated (keys are written in order), so the chunk's other keys are
// cleared with it.
// mode: how the chunk is stored.  kOpTiles writes into the tile layout;
// kOpRows writes rows of a chunk kept row-major (a chunk grown by appends);
// kOpConvert rewrites such a chunk's first n_rows keys into the tile layout
// (it is about to be shared or split), and must run before the other copies
// of the same mutation.
enum KvOpMode : int32_t { kOpTiles = 0, kOpRows = 1, kOpConvert = 2 };
struct KvOp {
  int32_t dst_slot;
  int32_t dst_key0;
  int32_t n_rows;
  int32_t src_row0;   // caller row (from_pool == 0) or source key (from_pool == 1)
  int32_t src_slot;   // only for from_pool
  int32_t from_pool;
  int32_t node = -1;  // manager node written (host bookkeeping only)
  int32_t mode = kOpTiles;
};

// Per-step work plan built from the DFS order.  All ids are int32 so the
// arrays go to the device as they are.
// Records are read by a block (a wave) with one scalar load; the first chunk
// refs of the task ride along (kCfInline, kSfInline in kernels.h), so it can
// start its tile loads after a single round trip to memory.

struct CfUnit {        // chunk-first: one 32-row block of one run of shared chunks
  int32_t chunk_begin; // into chunk_refs (pairs); refs past kCfInline are read there
  int32_t n_chunks;
  int32_t row_begin;   // DFS position of the block's first row
  int32_t n_rows;      // 1..32
  int32_t part_base;   // partial id of the block's first row; row r's is part_base + r * part_stride
  int32_t qrow_base;   // caller row of the first row if the rows' caller rows are consecutive, else -1
  int32_t reuse;       // 1: other units read these chunks too (run of more than 32 rows)
  int32_t pad;
  int32_t slot[kCfInline];
  int32_t n_valid[kCfInline];
  int32_t pad2[8];     // 128 bytes
};
struct SfTask {        // sequence-first: some private chunks of one sequence
  int32_t chunk_begin; // into chunk_refs; refs past kSfInline are read there
  int32_t n_chunks;
  int32_t dfs_pos;
  int32_t part_id;
  int32_t qrow;        // caller row of the sequence
  int32_t reuse;       // 1: some chunk is shared (read by other tasks; only without chunk-first)
  int32_t append_at;   // index (in this task) of the chunk where the sequence ends, or -1
  int32_t pad;
  int32_t slot[kSfInline];
  int32_t n_valid[kSfInline];  // 64 bytes
};

static_assert(sizeof(CfUnit) == 128 && sizeof(SfTask) == 64, "record layouts are read by the kernels");
static_assert(offsetof(CfUnit, reuse) == kCfReuseField * 4 && offsetof(SfTask, reuse) == kSfReuseField * 4 &&
                  offsetof(SfTask, append_at) == kSfAppendField * 4,
              "record fields sit where the kernels read them");

struct Plan {
  std::vector<int32_t> rows;        // canonical table, 7 ints per row
  std::vector<int64_t> dfs_seq;     // seq ids in DFS order
  std::vector<int32_t> dfs_qrow;    // caller row of each DFS position
  std::vector<CfUnit> cf_units;
  int64_t cf_tasks = 0;
  int32_t sf_group = 0;             // private chunk refs per sequence-first task
  std::vector<SfTask> sf_tasks;
  std::vector<int32_t> chunk_refs;  // (slot, n_valid) pairs
  std::vector<int32_t> row_node;    // manager node index of each table row
  std::vector<int32_t> ref_node;    // manager node index of each chunk ref
  std::vector<int32_t> ref_sub;     // 64-key tile of the chunk the ref covers (chunks of 128 span two)
  std::vector<int32_t> ref_task;    // sequence-first task holding the ref (-1: chunk-first)
  std::vector<int32_t> ref_pos;     // position of the ref within that task
  std::vector<int32_t> private_ref; // per manager node: its ref if the chunk has one sequence, else -1
  std::vector<int32_t> seq_parts;   // (first, count) into part_list, per DFS position
  std::vector<int32_t> part_list;   // partial ids, per sequence in merge order
  int32_t n_parts = 0;              // partial slots (dense: n_seq * dense_parts)
  int32_t dense_parts = 0;          // > 0: sequence i's j-th partial has id i * dense_parts + j
  int32_t part_stride = 1;          // id step between consecutive rows of a chunk-first unit
  int64_t cf_chunk_reads = 0;       // per head
  int64_t sf_chunk_reads = 0;       // per head
  int64_t shared_chunks = 0;
  int64_t shared_tokens = 0;
  int64_t unique_tokens = 0;
  int64_t attended_tokens = 0;
  int64_t row_refs = 0;             // chunk refs of row-major chunks (kRowBit set)

  // Empty every list but keep its storage (plans are rebuilt often while
  // decoding, at about the same size).
  void clear();
};

// The tree after one more token for each of a batch of sequences, as a plan
// sees it, without changing the tree: which chunks grow in place and which
// new chunks would be made (node index, id, slot, position, in the order
// append_batch allocates them).  Token values play no part in a plan.
struct NextAppend {
  struct Add {
    int32_t parent, idx, id, slot, start;
    int64_t seq;
  };
  std::vector<int32_t> grow;  // nodes that take their sequence's token in place
  std::vector<Add> add;       // new chunks
  size_t n_nodes = 0;         // size of the node array afterwards
  bool structural = false;    // the appends change the plan's shape
};

class Manager {
 public:
  Manager(int chunk, bool share);

  void set_capacity(int64_t capacity);   // only while empty
  int64_t capacity() const { return capacity_; }
  int64_t free_slots() const { return static_cast<int64_t>(free_.size()); }
  int chunk() const { return C_; }
  // Chunks made by appends from now on are stored row-major (default), or
  // in the tile layout like inserted ones.
  void set_row_appends(bool on) { row_appends_ = on; }
  bool row_appends() const { return row_appends_; }
  // Whether a live chunk node is stored row-major.
  bool row(int32_t node) const { return nodes_[node].row; }
  int64_t row_chunks() const;
  // The kernels read 64-key tiles: a chunk of C > 64 tokens is C / 64 tiles
  // (slot s owns tiles s * C / 64 ...), of which the plan lists those that
  // hold tokens; a chunk of 32 is half of tile s / 2 and its ref carries s
  // itself (the kernels find the tile and the half).
  int32_t tiles_of(int32_t fill) const { return C_ > kTileKeys ? std::max(1, (fill + kTileKeys - 1) / kTileKeys) : 1; }
  int32_t tile_slot(int32_t slot, int32_t t) const { return C_ > kTileKeys ? slot * (C_ / kTileKeys) + t : slot; }
  int32_t tile_fill(int32_t fill, int32_t t) const {
    return C_ > kTileKeys ? std::min(kTileKeys, fill - t * kTileKeys) : fill;
  }
  size_t live() const { return live_.size(); }
  int64_t nodes() const { return n_nodes_; }

  // Mutations return the device copies they need (possibly none).
  int32_t insert(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops);
  // The copies insert(seq, tokens, n) would return, in the same order and to
  // the same slots, without changing anything (same errors as insert): the
  // caller can enqueue them first and change the tree only once they are.
  int32_t insert_ops(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops) const;
  // After conversions to tiles (kOpConvert ops) went to the device but the
  // insert that needed them did not happen: the tree records the new layout.
  void mark_tiles(const std::vector<KvOp>& converts);
  // src_base: row of the caller's K/V that holds the first appended token.
  void append(int64_t seq, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops, int32_t src_base = 0);
  // One token for each of n sequences (token j, K/V row j).  All checks run
  // before anything changes (unknown or repeated id, too few free slots).
  void append_batch(const int64_t* seqs, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops);

  // What append_batch(seqs, n) would do, one token each (see NextAppend);
  // false if it would fail.
  bool predict_append_batch(const int64_t* seqs, int32_t n, NextAppend* out) const;
  // Whether one more token for every live sequence would change the plan's
  // shape (a last chunk full or shared, or a chunk opening another tile).
  bool next_append_structural() const;
  // Memory for the chunks a predicted append will open (node array room,
  // token and sequence lists, the parents' child lists), allocated now so
  // that the append itself allocates nothing: the host can do this while
  // the GPU still runs the previous step.
  void stock_for_append(const NextAppend& next);

  // True when the last mutations only grew chunks in place (no chunk created
  // or freed, no sequence joined or left) since the last clear_structural().
  bool fills_only() const { return !structural_; }
  void clear_structural() { structural_ = false; }
  void remove(int64_t seq);

  std::vector<int64_t> sequences() const;  // ascending
  int32_t seq_len(int64_t seq) const;

  // Build the canonical table and the work plan.  cf_group / sf_group: chunks
  // per chunk-first task and per sequence-first task.  Without two_phase every
  // chunk on a sequence's path, shared or not, goes to that sequence's
  // sequence-first tasks (physically shared pages, no chunk-first phase).
  // sf_group <= 0: chosen per plan, the largest of 16, 8, 4 that gives at
  // least sf_min_tasks sequence-first tasks, 8/5 of that when the plan has
  // chunk-first units, where 3 replaces 4 if it makes more tasks and leaves
  // no sequence a one-chunk remainder (Plan::sf_group says which).
  // With `next`, the plan of the tree after those appends (the same plan
  // that build_plan gives once they are made).
  void build_plan(int cf_group, int sf_group, bool two_phase, Plan* plan, int64_t sf_min_tasks = 0,
                  const NextAppend* next = nullptr) const;
  // Bring a plan built for the current structure up to date with chunk fills
  // that grew since: fill counts in the table, the chunk refs and the refs
  // carried inline by task records, and the token totals.
  void refresh_fills(Plan* plan) const;

 private:
  struct Node {
    int32_t id = -1;
    int32_t parent = -1;   // index into nodes_
    int32_t slot = -1;
    int32_t start = 0;     // position of the first token in the sequence
    int32_t ref = 0;       // live sequences through or ending at this node
    bool alive = false;
    bool row = false;      // stored row-major (made by an append, never shared since)
    std::vector<int32_t> tokens;
    std::vector<int32_t> children;  // indices, creation order
    std::vector<int64_t> ended;     // sequences ending here, arrival order
  };

  // An insert's walk from the root: the matched chunks, where the match
  // ends (the node and token position), and the chunk it splits, if any.
  struct InsertWalk {
    std::vector<int32_t> path;
    int32_t cur = 0, pos = 0, split_node = -1, split_at = 0;
  };
  void walk_insert(int64_t seq, const int32_t* tokens, int32_t n, InsertWalk* w) const;
  struct Live {
    int32_t end;  // node index where the sequence ends
    int32_t len;  // its length in tokens
  };
  // append() once its sequence is found
  void append_to(std::map<int64_t, Live>::iterator it, const int32_t* tokens, int32_t n, std::vector<KvOp>* ops,
                 int32_t src_base);
  int32_t new_node(int32_t parent, int32_t start);
  void free_node(int32_t idx);
  int32_t alloc_slot();
  static int64_t chunks_for(int64_t n, int C) { return (n + C - 1) / C; }

  int C_;
  bool share_;
  bool structural_ = true;
  bool row_appends_ = true;
  int64_t capacity_ = 0;
  int32_t next_id_ = 0;
  int64_t n_nodes_ = 0;
  std::vector<Node> nodes_;                 // nodes_[0] is the root
  std::vector<int32_t> free_nodes_;         // reusable indices in nodes_
  // empty lists with room reserved, taken by new nodes (stock_for_append)
  std::vector<std::vector<int32_t>> spare_tokens_;
  std::vector<std::vector<int64_t>> spare_ended_;
  // Free chunk slots, lowest first: one bit per slot (set = free) and the
  // index of the first word that may hold a free slot (every word below it
  // is all taken), so taking the lowest free slot costs a few word reads.
  class FreeSlots {
   public:
    void reset(int64_t capacity) {
      bits_.assign(static_cast<size_t>((capacity + 63) / 64), ~uint64_t{0});
      if (capacity % 64) bits_.back() = (uint64_t{1} << (capacity % 64)) - 1;
      n_ = capacity;
      first_ = 0;
    }
    int64_t size() const { return n_; }
    // the lowest free slot (there must be one)
    int32_t take() {
      while (bits_[first_] == 0) ++first_;
      uint64_t& w = bits_[first_];
      const int32_t s = static_cast<int32_t>(first_ * 64 + static_cast<size_t>(__builtin_ctzll(w)));
      w &= w - 1;
      --n_;
      return s;
    }
    void give(int32_t s) {
      bits_[static_cast<size_t>(s) >> 6] |= uint64_t{1} << (s & 63);
      ++n_;
      first_ = std::min(first_, static_cast<size_t>(s) >> 6);
    }
    // The free slots in increasing order, without taking them.
    class Walk {
     public:
      explicit Walk(const FreeSlots& f) : f_(f), word_(f.first_), left_(word_ < f.bits_.size() ? f.bits_[word_] : 0) {}
      // the next free slot, or -1 when none is left
      int32_t next() {
        while (left_ == 0) {
          if (++word_ >= f_.bits_.size()) return -1;
          left_ = f_.bits_[word_];
        }
        const int32_t s = static_cast<int32_t>(word_ * 64 + static_cast<size_t>(__builtin_ctzll(left_)));
        left_ &= left_ - 1;
        return s;
      }
     private:
      const FreeSlots& f_;
      size_t word_;
      uint64_t left_;
    };

   private:
    std::vector<uint64_t> bits_;
    int64_t n_ = 0;
    size_t first_ = 0;
  };
  FreeSlots free_;
  std::map<int64_t, Live> live_;           // live sequences by id
};

}  // namespace chunkattn
