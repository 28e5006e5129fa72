// bandit.cpp -- host-side draft selection for the verification loop (C ABI).
//
// FlashSpec (technical summary, section 2 "Online bandit draft selection")
// picks the draft model of each decoding step as the arm of a K-armed bandit
// whose reward is the accepted fraction of the step's draft tokens, with UCB1
// or Thompson sampling. This runs on the host between steps: it reads the
// accept lengths a step produced (after the caller's copy to host memory) and
// returns the arm for the next step. Nothing here touches the GPU.
//
//   UCB1     Auer, Cesa-Bianchi and Fischer (2002): every arm once (lowest index
//            first), then argmax mean_i + sqrt(c ln t / n_i); ties to the lowest.
//   Thompson argmax theta_i ~ Beta(1 + S_i, 1 + n_i - S_i) (S_i: reward sum; a
//            fractional reward is a fractional pseudo-count). Beta = X / (X + Y)
//            with Gamma variates by Marsaglia and Tsang (2000; shapes >= 1),
//            normals by Box-Muller, uniforms of 53 bits from two words of a
//            Philox4x32-10 block (Salmon et al., SC'11) keyed by the seed with
//            counter (draw, arm, (variate << 16) | attempt, 2).
//
// Floating-point contraction is off in this file so that every expression
// rounds as written.

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "specverify.h"

#pragma clang fp contract(off)

namespace {

constexpr uint32_t kMagic = 0x53564244u;  // "SVBD"
constexpr uint32_t kPurposeBandit = 2;
constexpr int kMaxAttempts = 1000;

struct Header {
  uint32_t magic;
  int32_t arms;
  int32_t policy;
  int32_t pad;
  uint64_t seed;
  double c;
  int64_t t;      // rewards received so far
  int64_t draws;  // Thompson selections so far
};

struct Arm {
  int64_t pulls;
  double sum;
};

Header* header(void* s) { return static_cast<Header*>(s); }
const Header* header(const void* s) { return static_cast<const Header*>(s); }
Arm* arms_of(void* s) { return reinterpret_cast<Arm*>(static_cast<char*>(s) + sizeof(Header)); }
const Arm* arms_of(const void* s) {
  return reinterpret_cast<const Arm*>(static_cast<const char*>(s) + sizeof(Header));
}

bool valid(const void* s) { return s != nullptr && header(s)->magic == kMagic; }

// Philox4x32-10: ten rounds of two 32x32 -> 64-bit products mixed with the other
// words and the round key, the key advancing by two Weyl constants.
void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = uint64_t(0xD2511F53u) * c[0];
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c[2];
    const uint32_t n0 = uint32_t(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = uint32_t(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = uint32_t(p1);
    c[2] = n2;
    c[3] = uint32_t(p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

void block(uint64_t seed, int64_t t, int32_t arm, int g, int attempt, uint32_t w[4]) {
  w[0] = uint32_t(t);
  w[1] = uint32_t(arm);
  w[2] = uint32_t((g << 16) | attempt);
  w[3] = kPurposeBandit;
  philox(w, uint32_t(seed), uint32_t(seed >> 32));
}

// (floor(w0 / 2^5) 2^26 + floor(w1 / 2^6) + 1/2) 2^-53, strictly inside (0, 1)
double uniform53(uint32_t w0, uint32_t w1) {
  return (double(w0 >> 5) * 67108864.0 + double(w1 >> 6) + 0.5) * (1.0 / 9007199254740992.0);
}

double gamma_variate(double shape, uint64_t seed, int64_t t, int32_t arm, int g) {
  const double d = shape - 1.0 / 3.0;
  const double c = 1.0 / std::sqrt(9.0 * d);
  const double two_pi = 2.0 * 3.141592653589793;
  for (int attempt = 0; attempt < kMaxAttempts; ++attempt) {
    uint32_t w[4];
    block(seed, t, arm, g, attempt, w);
    const double u1 = uniform53(w[0], w[1]);
    const double u2 = uniform53(w[2], w[3]);
    const double x = std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2);
    double v = 1.0 + c * x;
    if (v <= 0.0) continue;
    v = v * v * v;
    uint32_t wa[4];
    block(seed, t, arm, g, attempt + kMaxAttempts, wa);
    const double u = uniform53(wa[0], wa[1]);
    const double x2 = x * x;
    if (u < 1.0 - 0.0331 * x2 * x2) return d * v;
    if (std::log(u) < 0.5 * x2 + d * (1.0 - v + std::log(v))) return d * v;
  }
  return d;
}

}  // namespace

extern "C" {

size_t specverify_bandit_state_size(int32_t arms) {
  if (arms < 1 || arms > SV_MAX_ARMS) return 0;
  return sizeof(Header) + size_t(arms) * sizeof(Arm);
}

int specverify_bandit_init(void* state, size_t state_bytes, int32_t arms, int32_t policy,
                           uint64_t seed, double c) {
  if (!state || arms < 1 || arms > SV_MAX_ARMS ||
      (policy != SV_BANDIT_UCB1 && policy != SV_BANDIT_THOMPSON) || !(c > 0.0) ||
      !std::isfinite(c))
    return SV_EINVAL;
  if (state_bytes < specverify_bandit_state_size(arms)) return SV_EWORKSPACE;
  std::memset(state, 0, specverify_bandit_state_size(arms));
  Header* h = header(state);
  h->magic = kMagic;
  h->arms = arms;
  h->policy = policy;
  h->seed = seed;
  h->c = c;
  return SV_OK;
}

int specverify_bandit_select(void* state, int32_t* arm) {
  if (!valid(state) || !arm) return SV_EINVAL;
  Header* h = header(state);
  const Arm* a = arms_of(state);
  int32_t best_i = 0;
  double best = -INFINITY;
  if (h->policy == SV_BANDIT_UCB1) {
    for (int32_t i = 0; i < h->arms; ++i)
      if (a[i].pulls == 0) {
        *arm = i;
        return SV_OK;
      }
    for (int32_t i = 0; i < h->arms; ++i) {
      const double n = double(a[i].pulls);
      const double idx = a[i].sum / n + std::sqrt(h->c * std::log(double(h->t)) / n);
      if (idx > best) {
        best = idx;
        best_i = i;
      }
    }
  } else {
    for (int32_t i = 0; i < h->arms; ++i) {
      const double x = gamma_variate(1.0 + a[i].sum, h->seed, h->draws, i, 0);
      const double y = gamma_variate(1.0 + double(a[i].pulls) - a[i].sum, h->seed, h->draws, i, 1);
      const double theta = x / (x + y);
      if (theta > best) {
        best = theta;
        best_i = i;
      }
    }
    h->draws += 1;
  }
  *arm = best_i;
  return SV_OK;
}

int specverify_bandit_update(void* state, int32_t arm, double reward) {
  if (!valid(state)) return SV_EINVAL;
  Header* h = header(state);
  if (arm < 0 || arm >= h->arms || !(reward >= 0.0 && reward <= 1.0)) return SV_EINVAL;
  Arm* a = arms_of(state);
  a[arm].pulls += 1;
  a[arm].sum += reward;
  h->t += 1;
  return SV_OK;
}

int specverify_bandit_stats(const void* state, int32_t arm, int64_t* pulls, double* reward_sum) {
  if (!valid(state)) return SV_EINVAL;
  const Header* h = header(state);
  if (arm < 0 || arm >= h->arms) return SV_EINVAL;
  if (pulls) *pulls = arms_of(state)[arm].pulls;
  if (reward_sum) *reward_sum = arms_of(state)[arm].sum;
  return SV_OK;
}

int specverify_step_reward(const int32_t* accept_len, int64_t chains, int64_t gamma,
                           double* reward) {
  if (!accept_len || !reward || chains < 1 || gamma < 1 || gamma > SV_MAX_GAMMA)
    return SV_EINVAL;
  int64_t total = 0;
  for (int64_t i = 0; i < chains; ++i) {
    const int32_t n = accept_len[i];
    total += n < 0 ? 0 : (n > gamma ? gamma : n);
  }
  *reward = double(total) / (double(chains) * double(gamma));
  return SV_OK;
}

}  // extern "C"
