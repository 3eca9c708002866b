// Random insert / append / batched append / remove sequences and plan builds
// on the host prefix-tree manager, for a sanitizer build (AddressSanitizer
// and UndefinedBehaviorSanitizer): every call either succeeds or throws the
// manager's own error (never an internal one), at chunk sizes 2 to 128, with
// chunks made by appends stored row-major or not.  Before every batched
// append over all live sequences, the plan predicted for the tree after it
// must equal the plan built once it is made (with or without the new chunks'
// memory reserved ahead), and the prediction must fail exactly when the
// append does.  Before every insert, the copies announced for it
// (insert_ops) must be the ones it returns, and fail exactly when it does.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include "manager.h"
using namespace chunkattn;

template <typename T>
static bool same(const std::vector<T>& a, const std::vector<T>& b) {
  return a.size() == b.size() && (a.empty() || std::memcmp(a.data(), b.data(), a.size() * sizeof(T)) == 0);
}

static bool same_ops(const std::vector<KvOp>& a, const std::vector<KvOp>& b) {
  if (a.size() != b.size()) return false;
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i].dst_slot != b[i].dst_slot || a[i].dst_key0 != b[i].dst_key0 || a[i].n_rows != b[i].n_rows ||
        a[i].src_row0 != b[i].src_row0 || a[i].src_slot != b[i].src_slot || a[i].from_pool != b[i].from_pool ||
        a[i].mode != b[i].mode || a[i].node != b[i].node)
      return false;
  return true;
}

static bool same_plan(const Plan& a, const Plan& b) {
  return same(a.rows, b.rows) && same(a.dfs_seq, b.dfs_seq) && same(a.dfs_qrow, b.dfs_qrow) &&
         same(a.cf_units, b.cf_units) && same(a.sf_tasks, b.sf_tasks) && same(a.chunk_refs, b.chunk_refs) &&
         same(a.row_node, b.row_node) && same(a.ref_node, b.ref_node) && same(a.ref_sub, b.ref_sub) &&
         same(a.ref_task, b.ref_task) && same(a.ref_pos, b.ref_pos) && same(a.private_ref, b.private_ref) &&
         same(a.seq_parts, b.seq_parts) && same(a.part_list, b.part_list) && a.n_parts == b.n_parts &&
         a.dense_parts == b.dense_parts && a.part_stride == b.part_stride && a.cf_tasks == b.cf_tasks &&
         a.sf_group == b.sf_group && a.row_refs == b.row_refs && a.unique_tokens == b.unique_tokens &&
         a.attended_tokens == b.attended_tokens && a.shared_tokens == b.shared_tokens;
}
int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 300;
  std::mt19937 rng(7);
  long ops_done = 0, errors = 0, predicted = 0;
  for (int t = 0; t < trials; ++t) {
    const int C = std::vector<int>{2, 3, 4, 32, 64, 128}[rng() % 6];
    const bool share = rng() % 10 != 0;
    Manager m(C, share);
    m.set_capacity(5 + rng() % 200);
    m.set_row_appends(rng() % 4 != 0);
    Plan plan;
    std::vector<int64_t> live;
    for (int s = 0; s < 200; ++s) {
      const int r = rng() % 100;
      std::vector<KvOp> ops;
      try {
        if (r < 40 || live.empty()) {
          int64_t id = rng() % 60;
          std::vector<int32_t> toks(1 + rng() % (C < 8 ? 20 : 400));
          for (auto& x : toks) x = rng() % 3;
          // the copies announced ahead are the ones the insert returns, and
          // announcing fails exactly when the insert does
          std::vector<KvOp> ahead;
          bool ahead_ok = true;
          try {
            m.insert_ops(id, toks.data(), (int32_t)toks.size(), &ahead);
          } catch (const Error& e) {
            if (e.code == -11) throw;
            ahead_ok = false;
          }
          bool done = false;
          try {
            m.insert(id, toks.data(), (int32_t)toks.size(), &ops);
            done = true;
          } catch (const Error& e) {
            if (ahead_ok || e.code == -11) throw;
          }
          if (done != ahead_ok || (done && !same_ops(ahead, ops))) {
            printf("FAIL: copies announced ahead differ from the insert's (trial %d step %d, C %d)\n", t, s, C);
            return 1;
          }
          live.push_back(id);
        } else if (r < 60) {
          int64_t id = live[rng() % live.size()];
          std::vector<int32_t> toks(1 + rng() % 5);
          for (auto& x : toks) x = rng() % 3;
          m.append(id, toks.data(), (int32_t)toks.size(), &ops);
        } else if (r < 80) {
          std::vector<int64_t> ids = m.sequences();
          std::vector<int32_t> toks(ids.size());
          for (auto& x : toks) x = rng() % 3;
          const int cfg = rng() % 3 ? 0 : 1 + rng() % 16, sfg = rng() % 2 ? 0 : 1 + rng() % 8;
          const bool two_phase = rng() % 5 != 0;
          const int64_t min_tasks = rng() % 100;
          NextAppend next;
          Plan pred, fresh;
          const bool can = m.predict_append_batch(ids.data(), (int32_t)ids.size(), &next);
          // memory for the new chunks reserved ahead changes nothing else
          if (can && rng() % 2) m.stock_for_append(next);
          if (can) m.build_plan(cfg, sfg, two_phase, &pred, min_tasks, &next);
          bool done = false;
          try {
            m.append_batch(ids.data(), toks.data(), (int32_t)ids.size(), &ops);
            done = true;
          } catch (const Error& e) {
            if (can || e.code == -11) throw;
          }
          if (done != can) {
            printf("FAIL: prediction %d, append %d (trial %d step %d)\n", can, done, t, s);
            return 1;
          }
          if (done) {
            m.build_plan(cfg, sfg, two_phase, &fresh, min_tasks);
            if (!same_plan(pred, fresh)) {
              printf("FAIL: predicted plan differs (trial %d step %d, C %d)\n", t, s, C);
              return 1;
            }
            ++predicted;
          }
        } else {
          int64_t id = live[rng() % live.size()];
          m.remove(id);
        }
      } catch (const Error& e) {
        if (e.code == -11) {
          printf("FAIL: internal error: %s (trial %d step %d)\n", e.what(), t, s);
          return 1;
        }
        ++errors;
      }
      live = m.sequences();
      if (rng() % 3 == 0) {
        try {
          m.build_plan(rng() % 3 ? 0 : 1 + rng() % 16, rng() % 2 ? 0 : 1 + rng() % 8, rng() % 5 != 0, &plan,
                       rng() % 100);
        } catch (const Error& e) {
          printf("FAIL: plan build: %s (trial %d step %d)\n", e.what(), t, s);
          return 1;
        }
        m.clear_structural();
        if (rng() % 2) m.refresh_fills(&plan);
      }
      ++ops_done;
    }
  }
  if (predicted < 100) {
    printf("FAIL: only %ld predicted appends\n", predicted);
    return 1;
  }
  printf("ok: %ld ops, %ld expected errors, %ld predicted plans equal to built ones\n", ops_done, errors, predicted);
  return 0;
}
