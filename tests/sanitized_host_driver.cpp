// Host-code driver for a build of the library's host side under AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_sanitized_host.py compiles and runs it;
// no GPU is used). Every GPU entry point is called only with arguments its host
// checks reject, so no HIP call is made; the pure host functions (sizes, fan-out,
// step reward, the draft selector) run for real. Prints one line per check and
// the selector's picks; exits with the number of failed checks.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "specverify.h"

static int failed = 0;

static void expect(const char* what, long long got, long long want) {
  const bool ok = got == want;
  std::printf("%s %s got %lld want %lld\n", ok ? "ok" : "FAIL", what, got, want);
  if (!ok) ++failed;
}

// A reward in [0, 1] that both this driver and the Python oracle compute exactly.
static double reward_of(int step, int arm) { return double((step * 7 + arm * 13) % 17) / 16.0; }

int main(int argc, char** argv) {
  (void)argc;
  (void)argv;
  // Fake device pointers: never dereferenced, every call below is refused first.
  alignas(256) static char fake[1024];
  void* p = fake;
  int32_t* ip = reinterpret_cast<int32_t*>(fake);
  float* fp = reinterpret_cast<float*>(fake);
  double* dp = reinterpret_cast<double*>(fake);

  // sizes
  expect("workspace C3 > 0", specverify_workspace_size(64, 1, 8, 128256, SV_BF16) > 0, 1);
  expect("workspace B=0", (long long)specverify_workspace_size(0, 1, 8, 100, SV_BF16), 0);
  expect("workspace gamma=33", (long long)specverify_workspace_size(4, 1, 33, 100, SV_BF16), 0);
  expect("workspace V=2^31", (long long)specverify_workspace_size(4, 1, 8, int64_t(1) << 31, SV_F32), 0);
  expect("workspace dtype", (long long)specverify_workspace_size(4, 1, 8, 100, 7), 0);
  expect("accept_prob workspace > 0", specverify_accept_prob_workspace_size(64, 1, 8, 128256, SV_BF16) > 0, 1);
  expect("accept_prob workspace K*gamma>64",
         (long long)specverify_accept_prob_workspace_size(4, 3, 22, 100, SV_BF16), 0);

  // the step: null pointers, bad sizes, strides, dtype, workspace
  auto step = [&](const void* t, int dtype, int64_t B, int64_t K, int64_t g, int64_t V, int64_t tsb,
                  void* ws, size_t wsb) {
    return specverify_step(t, p, dtype, ip, B, K, g, V, tsb, V, 4 * V, 4 * V, V, fp, 1, nullptr, ip,
                           ip, nullptr, nullptr, nullptr, nullptr, nullptr, ws, wsb, nullptr);
  };
  expect("step null target", step(nullptr, SV_BF16, 2, 1, 4, 1000, 5000, p, 1 << 20), SV_EINVAL);
  expect("step B=0", step(p, SV_BF16, 0, 1, 4, 1000, 5000, p, 1 << 20), SV_EINVAL);
  expect("step gamma=0", step(p, SV_BF16, 2, 1, 0, 1000, 5000, p, 1 << 20), SV_EINVAL);
  expect("step K*gamma>64", step(p, SV_BF16, 2, 3, 22, 1000, 5000, p, 1 << 20), SV_EINVAL);
  expect("step negative stride", step(p, SV_BF16, 2, 1, 4, 1000, -1, p, 1 << 20), SV_EINVAL);
  expect("step dtype", step(p, 9, 2, 1, 4, 1000, 5000, p, 1 << 20), SV_EDTYPE);
  expect("step no workspace", step(p, SV_BF16, 2, 1, 4, 1000, 5000, nullptr, 0), SV_EWORKSPACE);
  expect("step small workspace", step(p, SV_BF16, 2, 1, 4, 1000, 5000, p, 16), SV_EWORKSPACE);
  expect("step_noalloc null tokens",
         specverify_step_noalloc(p, p, SV_BF16, nullptr, 2, 1, 4, 1000, 5000, 1000, 4000, 4000,
                                 1000, fp, 1, nullptr, ip, ip, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr),
         SV_EINVAL);
  expect("step_noalloc too large",
         specverify_step_noalloc(p, p, SV_BF16, ip, 4096, 4, 16, 151936, 16 * 151936, 151936,
                                 64 * 151936, 16 * 151936, 151936, fp, 1, nullptr, ip, ip, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr),
         SV_ESCRATCH);

  // the other GPU entry points
  expect("normalize null lnZ",
         specverify_normalize(p, SV_BF16, 2, 3, 100, 300, 100, fp, nullptr, nullptr, p, 1 << 20, nullptr),
         SV_EINVAL);
  expect("normalize P=0",
         specverify_normalize(p, SV_BF16, 2, 0, 100, 300, 100, fp, dp, nullptr, p, 1 << 20, nullptr),
         SV_EINVAL);
  expect("accept gamma=33",
         specverify_accept(fp, fp, 2, 1, 33, 1, nullptr, ip, nullptr, nullptr), SV_EINVAL);
  expect("accept null logq",
         specverify_accept(fp, nullptr, 2, 1, 4, 1, nullptr, ip, nullptr, nullptr), SV_EINVAL);
  expect("residual_sample null n",
         specverify_residual_sample(p, p, SV_BF16, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, fp,
                                    dp, dp, ip, nullptr, 1, nullptr, ip, p, 1 << 20, nullptr),
         SV_EINVAL);
  expect("accept_prob null alpha",
         specverify_accept_prob(p, p, SV_BF16, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, fp, dp,
                                dp, nullptr, nullptr, p, 1 << 20, nullptr),
         SV_EINVAL);
  int32_t badfan[5] = {1, 2, -1, 0, 0};
  expect("topf negative fan-out",
         specverify_residual_topf(p, p, SV_BF16, 2, 1, 4, 1000, 5000, 1000, 4000, 4000, 1000, fp,
                                  dp, dp, badfan, ip, nullptr, nullptr),
         SV_EINVAL);
  int32_t bigfan[5] = {1, 2, SV_MAX_FANOUT + 1, 0, 0};
  expect("cache_lookup fan-out too large",
         specverify_cache_lookup(ip, bigfan, 2, 1, 4, ip, ip, ip, nullptr), SV_EINVAL);
  expect("branch_prune NaN tau",
         specverify_branch_prune(fp, 2, 2, 4, std::nan(""), 1, ip, nullptr, nullptr, nullptr),
         SV_EINVAL);
  expect("timing hook half", specverify_time_next_stream_kernel(p, nullptr), SV_EINVAL);
  expect("timing hook clear", specverify_time_next_stream_kernel(nullptr, nullptr), SV_OK);

  // pure host functions
  int32_t fan[33];
  expect("fanout ok", specverify_geometric_fanout(8, 72, 0.6, fan), SV_OK);
  long long sum = 0;
  for (int i = 0; i <= 8; ++i) sum += fan[i];
  expect("fanout total", sum, 72);
  expect("fanout ratio 0", specverify_geometric_fanout(8, 72, 0.0, fan), SV_EINVAL);
  expect("fanout gamma 33", specverify_geometric_fanout(33, 72, 0.5, fan), SV_EINVAL);
  const int32_t n[6] = {3, 0, 8, 8, -1, 5};
  double r = -1.0;
  expect("step_reward ok", specverify_step_reward(n, 6, 8, &r), SV_OK);
  // accepted drafts over chains x gamma (an error chain, n = -1, counts none)
  expect("step_reward value x gamma x chains", (long long)std::llround(r * 8 * 6), 3 + 0 + 8 + 8 + 0 + 5);
  for (int code = -8; code <= 1; ++code) expect("status string", specverify_status_string(code) != nullptr, 1);
  expect("version", specverify_version() >= 100, 1);

  // the draft selector: a fixed reward function; picks printed for the oracle
  struct Case { int policy, arms; uint64_t seed; };
  const Case cases[] = {{SV_BANDIT_UCB1, 3, 0}, {SV_BANDIT_UCB1, 7, 5},
                        {SV_BANDIT_THOMPSON, 3, 11}, {SV_BANDIT_THOMPSON, 5, (uint64_t(1) << 63) + 5}};
  for (const Case& c : cases) {
    const size_t bytes = specverify_bandit_state_size(c.arms);
    std::vector<unsigned char> state(bytes);
    expect("bandit init", specverify_bandit_init(state.data(), bytes, c.arms, c.policy, c.seed, 2.0), SV_OK);
    std::printf("picks %d %d %llu:", c.policy, c.arms, (unsigned long long)c.seed);
    for (int s = 0; s < 200; ++s) {
      int32_t arm = -1;
      if (specverify_bandit_select(state.data(), &arm) != SV_OK) ++failed;
      std::printf(" %d", arm);
      if (specverify_bandit_update(state.data(), arm, reward_of(s, arm)) != SV_OK) ++failed;
    }
    std::printf("\n");
    expect("bandit update bad arm", specverify_bandit_update(state.data(), c.arms, 0.5), SV_EINVAL);
    expect("bandit update reward > 1", specverify_bandit_update(state.data(), 0, 1.5), SV_EINVAL);
    int64_t pulls = 0;
    double rs = 0.0;
    expect("bandit stats", specverify_bandit_stats(state.data(), 0, &pulls, &rs), SV_OK);
  }
  expect("bandit size 0 arms", (long long)specverify_bandit_state_size(0), 0);
  std::printf("failed %d\n", failed);
  return failed;
}
