// Random insert / append / batched append / remove sequences and plan builds
// on the host prefix-tree manager, for a sanitizer build (AddressSanitizer
// and UndefinedBehaviorSanitizer): every call either succeeds or throws the
// manager's own error, at chunk sizes 2 to 128.
#include <cstdio>
#include <random>
#include <vector>
#include "manager.h"
using namespace chunkattn;
int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 300;
  std::mt19937 rng(7);
  long ops_done = 0, errors = 0;
  for (int t = 0; t < trials; ++t) {
    const int C = std::vector<int>{2, 3, 4, 32, 64, 128}[rng() % 6];
    const bool share = rng() % 10 != 0;
    Manager m(C, share);
    m.set_capacity(5 + rng() % 200);
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
          m.insert(id, toks.data(), (int32_t)toks.size(), &ops);
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
          m.append_batch(ids.data(), toks.data(), (int32_t)ids.size(), &ops);
        } else {
          int64_t id = live[rng() % live.size()];
          m.remove(id);
        }
      } catch (const Error&) {
        ++errors;
      }
      live = m.sequences();
      if (rng() % 3 == 0) {
        m.build_plan(rng() % 3 ? 0 : 1 + rng() % 16, rng() % 2 ? 0 : 1 + rng() % 8, rng() % 5 != 0, &plan, rng() % 100);
        m.clear_structural();
        if (rng() % 2) m.refresh_fills(&plan);
      }
      ++ops_done;
    }
  }
  printf("ok: %ld ops, %ld expected errors\n", ops_done, errors);
  return 0;
}
