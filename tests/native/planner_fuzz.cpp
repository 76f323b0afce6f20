// Planner fuzz for sanitizer builds (AddressSanitizer with libstdc++'s vector
// annotations, UndefinedBehaviorSanitizer): many random batches planned on one
// thread, so the planner's reused per-thread buffers meet every shape in turn.
// Built and run by tests/test_planner_sanitized.py; host code only.
#include <cstdio>
#include <random>
#include <vector>
#include "pkv_internal.hpp"
// the library's error-message sink, outside this translation unit's scope
namespace pkv { int set_error(int status, const char*, ...) { return status; } }
int main() {
  std::mt19937 rng(1234);
  std::vector<char> host(1 << 22);
  long n_ok = 0, n_items = 0;
  for (int it = 0; it < 20000; ++it) {   // about a second with the sanitizers
    const int hkv = std::vector<int>{1, 2, 4, 8, 3}[rng() % 5];
    const int G = std::vector<int>{1, 2, 4, 8, 16}[rng() % 5];
    pkv_shape s{};
    s.num_q_heads = hkv * G; s.num_kv_heads = hkv; s.head_dim = (rng() % 2) ? 128 : 64;
    s.page_size = std::vector<int>{1, 16, 64}[rng() % 3]; s.num_pages = 1 << 20; s.dtype = (rng() % 8) ? PKV_DTYPE_BF16 : PKV_DTYPE_FP32;
    const int B = 1 + rng() % 5;
    std::vector<int32_t> P(B), L(B);
    for (int b = 0; b < B; ++b) {
      P[b] = (rng() % 3 == 0) ? 0 : int32_t(rng() % 9000);
      L[b] = std::vector<int>{0, 1, 7, 64, 128, 300, 512, 2048}[rng() % 8];
    }
    if (L[0] == 0) L[0] = 5;
    const int window = (rng() % 4 == 0) ? int(1 + rng() % 5000) : 0;
    const int flags = (!window && rng() % 6 == 0) ? PKV_FLAG_NON_CAUSAL : 0;
    const int splits = (rng() % 4 == 0) ? int(rng() % 9) : 0;
    const int cus = std::vector<int>{0, 256, 80, 32, 1, 1024}[rng() % 6];
    pkv_plan plan; size_t bytes = 0;
    const bool meta = rng() % 3 != 0;
    int st = pkv::plan_extend(B, P.data(), L.data(), &s, window, flags, splits, cus ? cus : 256,
                              meta ? host.data() : nullptr, host.size(), &plan, &bytes);
    if (st == 0) {
      ++n_ok;
      n_items += plan.n_items;
    }
  }
  printf("ok %ld items %ld\n", n_ok, n_items);
}
