// specverify.hip -- HIP kernels (gfx950 / CDNA4) and the C ABI of libspecverify.
//
// Batched speculative-sampling verification. The pieces, in the order a step
// runs them:
//   rowstats_kernel   streams every needed logit row once (128-bit loads),
//                     one wavefront per (row, chunk) unit: chunk maximum, lowest
//                     argmax and sum of exp2((z - max) * log2e / T), reduced
//                     across the wavefront with cross-lane shuffles.
//   accept_kernel     one workgroup per batch row: merges the chunk partials of
//                     the row's gamma+1 target and K*gamma draft rows into
//                     ln Z (double), gathers ln p / ln q at the draft tokens,
//                     draws the Philox accept uniforms and finds each chain's
//                     first rejection with one wavefront ballot.
//   sample_kernel     per (chain, vocabulary split): a second pass over the one
//                     row pair the chain needs (target/draft row n for the
//                     residual, target row gamma for the bonus), Gumbel-max by
//                     exponential race argmin_v E_v / w_v with E_v = -ln u_v
//                     (equivalent to argmax_v ln w_v + G_v), keeping the best
//                     two candidates; the last workgroup of a chain merges the
//                     splits and re-scores the two candidates in float64.
//   accept_scalar_kernel  the accept test alone from caller-supplied ln p/ln q.
//
// No matrix cores: nothing on this path is a dense contraction. No
// floating-point atomics: partials are merged in a fixed order, so results are
// bit-deterministic.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "specverify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kGroup = 8;                                    // consecutive vocabulary ids per lane group
constexpr int kRowGroups = 8;                                // groups per lane per normaliser unit
constexpr int64_t kUnit = int64_t(kWave) * kGroup * kRowGroups;  // 4096 logits per wavefront unit
constexpr int kSampleIters = 4;                              // groups per thread per sampling split
constexpr int64_t kSplit = int64_t(kBlock) * kGroup * kSampleIters;  // 8192 ids per workgroup
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;
constexpr uint32_t kPurposeAccept = 0;
constexpr uint32_t kPurposeSample = 1;

// Statistics of one (row, chunk) unit.
struct alignas(16) RowPartial {
  float m;      // largest raw logit in the chunk (-inf if none)
  int32_t idx;  // lowest id holding it (INT_MAX if none)
  double s;     // sum of exp2((z - m) * log2e / T) over the chunk (sampled rows)
};

// Best two sampling candidates of one split, ordered by (key, id).
struct alignas(16) Top2 {
  float k1;
  int32_t i1;
  float k2;
  int32_t i2;
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies whose halves are mixed with the other words and the round key; the
// key advances by two Weyl constants between rounds.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = uint64_t(kPhiloxM0) * c0;
    const uint64_t p1 = uint64_t(kPhiloxM1) * c2;
    const uint32_t n0 = uint32_t(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = uint32_t(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = uint32_t(p1);
    c2 = n2;
    c3 = uint32_t(p0);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// u = (floor(w / 2^9) + 1/2) * 2^-23: exact in float and double.
__device__ __forceinline__ float unit_uniform(uint32_t w) {
  return (float(w >> 9) + 0.5f) * 0x1p-23f;
}
__device__ __forceinline__ double unit_uniform_d(uint32_t w) {
  return (double(w >> 9) + 0.5) * 0x1p-23;
}
// ln u in double; for u >= 1/2, u - 1 is exact and log1p keeps full accuracy.
__device__ __forceinline__ double log_uniform_d(double u) {
  return u >= 0.5 ? log1p(u - 1.0) : log(u);
}

// ---------------------------------------------------------------------------
// Loading 8 consecutive logits (ids e0 .. e0+7) as float; ids >= end read -inf.
template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t e) {
  if constexpr (DT == SV_BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[e];
    return __uint_as_float(uint32_t(h) << 16);
  } else {
    return reinterpret_cast<const float*>(row)[e];
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void load8(const void* row, int64_t e0, int64_t end, float (&x)[kGroup]) {
  if (VEC && e0 + kGroup <= end) {
    if constexpr (DT == SV_BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(row) + e0);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xFFFF0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xFFFF0000u);
      x[4] = __uint_as_float(w.z << 16);
      x[5] = __uint_as_float(w.z & 0xFFFF0000u);
      x[6] = __uint_as_float(w.w << 16);
      x[7] = __uint_as_float(w.w & 0xFFFF0000u);
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row) + e0);
      const float4 a = p[0];
      const float4 b = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
  } else {
#pragma unroll
    for (int t = 0; t < kGroup; ++t) x[t] = (e0 + t < end) ? load_one<DT>(row, e0 + t) : -INFINITY;
  }
}

__device__ __forceinline__ const void* row_ptr(const void* base, int esz, int64_t off_elems) {
  return reinterpret_cast<const char*>(base) + off_elems * esz;
}

// ---------------------------------------------------------------------------
// Rows to normalise. Target rows: rho in [0, B*P): b = rho / P, j = rho % P.
// Draft rows: rho in [B*P, B*P + B*K*G): the rest in [b][k][j] order.
struct RowSet {
  const void* t;
  int64_t tsb, tsj;
  const void* d;
  int64_t dsb, dsk, dsj;
  int64_t B, P, K, G;
  const float* temp;
};

__device__ __forceinline__ void locate_row(const RowSet& rs, int64_t rho, int esz, const void*& ptr,
                                           int64_t& b, bool& is_draft) {
  const int64_t nt = rs.B * rs.P;
  if (rho < nt) {
    b = rho / rs.P;
    const int64_t j = rho - b * rs.P;
    ptr = row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj);
    is_draft = false;
  } else {
    const int64_t r = rho - nt;
    const int64_t kg = rs.K * rs.G;
    b = r / kg;
    const int64_t rem = r - b * kg;
    const int64_t k = rem / rs.G;
    const int64_t j = rem - k * rs.G;
    ptr = row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj);
    is_draft = true;
  }
}

__device__ __forceinline__ void better_max(float& m, int32_t& i, float om, int32_t oi) {
  if (om > m || (om == m && oi < i)) {
    m = om;
    i = oi;
  }
}

// One wavefront per (row, chunk) unit, grid-stride over units.
template <int DT, bool VEC, bool ARGMAX_ALL>
__global__ __launch_bounds__(kBlock) void rowstats_kernel(RowSet rs, int64_t V, int64_t nch,
                                                          int64_t clen, int64_t nunits,
                                                          RowPartial* __restrict__ part) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nwaves = int64_t(gridDim.x) * kWavesPerBlock;
  for (int64_t u = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6); u < nunits;
       u += nwaves) {
    const int64_t rho = u / nch;
    const int64_t c = u - rho * nch;
    const void* row;
    int64_t b;
    bool is_draft;
    locate_row(rs, rho, esz, row, b, is_draft);
    const float T = rs.temp[b];
    const bool sampled = T > 0.0f;
    if (is_draft && !sampled) continue;  // greedy chains never read their draft rows
    const int64_t start = c * clen;
    const int64_t end = start + clen < V ? start + clen : V;

    float x[kRowGroups][kGroup];
#pragma unroll
    for (int g = 0; g < kRowGroups; ++g) {
      const int64_t e0 = start + int64_t(kGroup) * (lane + kWave * g);
      if (e0 < end) {
        load8<DT, VEC>(row, e0, end, x[g]);
      } else {
#pragma unroll
        for (int t = 0; t < kGroup; ++t) x[g][t] = -INFINITY;
      }
    }

    float m = -INFINITY;
    int32_t idx = INT_MAX;
    if (!sampled || ARGMAX_ALL) {
#pragma unroll
      for (int g = 0; g < kRowGroups; ++g) {
        const int64_t e0 = start + int64_t(kGroup) * (lane + kWave * g);
#pragma unroll
        for (int t = 0; t < kGroup; ++t) {
          if (x[g][t] > m) {
            m = x[g][t];
            idx = int32_t(e0 + t);
          }
        }
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        const float om = __shfl_xor(m, off, kWave);
        const int32_t oi = __shfl_xor(idx, off, kWave);
        better_max(m, idx, om, oi);
      }
    } else {
#pragma unroll
      for (int g = 0; g < kRowGroups; ++g)
#pragma unroll
        for (int t = 0; t < kGroup; ++t) m = fmaxf(m, x[g][t]);
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    }

    double s = 0.0;
    if (sampled) {
      const float k2 = kLog2e / T;
      const float m0 = (m == -INFINITY) ? 0.0f : m;
#pragma unroll
      for (int g = 0; g < kRowGroups; ++g) {
        float sg = 0.0f;
#pragma unroll
        for (int t = 0; t < kGroup; ++t) sg += __builtin_amdgcn_exp2f((x[g][t] - m0) * k2);
        s += double(sg);
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    }
    if (lane == 0) part[u] = RowPartial{m, idx, s};
  }
}

// Merge the chunk partials of one row in chunk order: (max, lowest argmax, ln Z).
struct RowStat {
  double lnz;
  float m;
  int32_t idx;
};

__device__ RowStat merge_row(const RowPartial* __restrict__ p, int64_t nch, float T) {
  float m = -INFINITY;
  int32_t idx = INT_MAX;
  for (int64_t c = 0; c < nch; ++c) better_max(m, idx, p[c].m, p[c].idx);
  RowStat r;
  r.m = m;
  r.idx = idx;
  if (T > 0.0f) {
    if (!(m > -INFINITY)) {
      r.lnz = double(m);  // -inf (all masked) or NaN
    } else {
      const double k2 = kLog2eD / double(T);
      double s = 0.0;
      for (int64_t c = 0; c < nch; ++c) {
        if (p[c].m == -INFINITY) continue;
        s += p[c].s * exp2(double(p[c].m - m) * k2);
      }
      r.lnz = double(m) / double(T) + log(s);
    }
  } else if (T == 0.0f) {
    r.lnz = double(m);
  } else {
    r.lnz = NAN;
  }
  return r;
}

// ln Z and argmax of every row (specverify_normalize).
__global__ __launch_bounds__(kBlock) void finalize_rows_kernel(const RowPartial* __restrict__ part,
                                                               int64_t nrows, int64_t P, int64_t nch,
                                                               const float* __restrict__ temp,
                                                               double* __restrict__ lnz,
                                                               int32_t* __restrict__ amax) {
  const int64_t rho = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (rho >= nrows) return;
  const RowStat r = merge_row(part + rho * nch, nch, temp[rho / P]);
  lnz[rho] = r.lnz;
  if (amax) amax[rho] = r.idx == INT_MAX ? 0 : r.idx;
}

// ---------------------------------------------------------------------------
struct AcceptArgs {
  RowSet rs;
  int64_t V, nch;
  const RowPartial* part;
  const int32_t* tokens;
  uint64_t seed;
  const int64_t* pos0;
  int32_t* accept_len;
  int32_t* out_token;
  float* logp;
  float* logq;
  double* lnz_t_out;
  double* lnz_d_out;
  int32_t* dev_err;
  double* ws_lnz;    // [B*P + B*K*G] normalisers of every row
  uint32_t* ws_cnt;  // [B*K] sampling counters, zeroed here
};

// One workgroup per batch row: normalisers, gathers, accept tests, first rejections.
template <int DT>
__global__ __launch_bounds__(kBlock) void accept_kernel(AcceptArgs a) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  __shared__ double s_lnz[SV_MAX_GAMMA + 1 + SV_MAX_CHAIN_DECISIONS];
  __shared__ int32_t s_amax[SV_MAX_GAMMA + 1];
  __shared__ int32_t s_bad[SV_MAX_GAMMA + 1 + SV_MAX_CHAIN_DECISIONS];
  const RowSet& rs = a.rs;
  const int64_t b = blockIdx.x;
  const int P = int(rs.P);
  const int G = int(rs.G);
  const int K = int(rs.K);
  const int KG = K * G;
  const int t = threadIdx.x;
  const float T = rs.temp[b];
  const bool sampled = T > 0.0f;
  const bool greedy = T == 0.0f;

  if (t < P + KG) {
    const bool is_draft = t >= P;
    const int64_t rho = is_draft ? rs.B * P + b * KG + (t - P) : b * P + t;
    double lnz = NAN;
    int32_t bad = 0;
    if (!is_draft || sampled) {
      const RowStat r = merge_row(a.part + rho * a.nch, a.nch, T);
      lnz = r.lnz;
      bad = !(r.m > -INFINITY);
      if (!is_draft) s_amax[t] = r.idx == INT_MAX ? 0 : r.idx;
    }
    s_lnz[t] = lnz;
    s_bad[t] = bad;
    a.ws_lnz[rho] = lnz;
    if (!is_draft && a.lnz_t_out) a.lnz_t_out[b * P + t] = lnz;
    if (is_draft && sampled && a.lnz_d_out) a.lnz_d_out[b * KG + (t - P)] = lnz;
  }
  if (t < K) a.ws_cnt[b * K + t] = 0u;
  __syncthreads();

  if (t < kWave) {  // wavefront 0 decides every (branch, position) of this batch row
    bool acc = false;
    bool tok_bad = false;
    if (t < KG) {
      const int k = t / G;
      const int j = t - k * G;
      const int64_t chain = b * K + k;
      const int32_t x = a.tokens[chain * G + j];
      tok_bad = x < 0 || int64_t(x) >= a.V;
      double lp = 0.0, lq = 0.0;
      if (!tok_bad) {
        if (sampled) {
          const float zt = load_one<DT>(row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj), x);
          const float zd =
              load_one<DT>(row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj), x);
          lp = double(zt) / double(T) - s_lnz[j];
          lq = double(zd) / double(T) - s_lnz[P + t];
          const uint64_t pos = uint64_t(a.pos0 ? a.pos0[b] : 0) + uint64_t(j);
          const Philox4 r = philox4x32_10(0u, uint32_t(pos), uint32_t(chain), kPurposeAccept,
                                          uint32_t(a.seed), uint32_t(a.seed >> 32));
          acc = log_uniform_d(unit_uniform_d(r.w[0])) < lp - lq;
        } else if (greedy) {
          acc = x == s_amax[j];
          lp = acc ? 0.0 : -INFINITY;
          lq = 0.0;
        }
      }
      if (a.logp) a.logp[chain * G + j] = float(lp);
      if (a.logq) a.logq[chain * G + j] = float(lq);
    }
    const uint64_t acc_mask = __ballot(acc);
    const uint64_t bad_mask = __ballot(tok_bad);
    if (t < K) {
      const uint64_t low = (G == 64) ? ~0ull : ((1ull << G) - 1ull);
      const uint64_t bits = (acc_mask >> (t * G)) & low;
      const int n = __builtin_ctzll(~bits);  // leading accepts; <= G since bit G of ~bits is set
      int32_t err = 0;
      if ((bad_mask >> (t * G)) & low) err |= SV_ERR_TOKEN;
      if (!(sampled || greedy)) err |= SV_ERR_TEMP;
      for (int j = 0; j < P; ++j) err |= s_bad[j] ? SV_ERR_ROW : 0;
      if (sampled)
        for (int j = 0; j < G; ++j) err |= s_bad[P + t * G + j] ? SV_ERR_ROW : 0;
      const int64_t chain = b * K + t;
      if (err) {
        a.accept_len[chain] = -1;
        a.out_token[chain] = -1;
        if (a.dev_err) atomicOr(a.dev_err, err);
      } else {
        a.accept_len[chain] = n;
        if (greedy) a.out_token[chain] = s_amax[n];
      }
    }
  }
}

// ---------------------------------------------------------------------------
struct SampleArgs {
  const void* t;
  int64_t tsb, tsj;
  const void* d;
  int64_t dsb, dsk, dsj;
  int64_t B, K, G, V;
  const float* temp;
  const double* lnz_t;  // [B, G+1]
  const double* lnz_d;  // [B, K, G]
  const int32_t* amax_t;  // [B, G+1] or NULL (then greedy chains are left alone)
  const int32_t* accept_len;
  uint64_t seed;
  const int64_t* pos0;
  int32_t* out_token;
  int64_t nsplit;
  Top2* part;
  uint32_t* cnt;
};

__device__ __forceinline__ bool cand_less(float ka, int32_t ia, float kb, int32_t ib) {
  return ka < kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ void top2_insert(Top2& s, float key, int32_t id) {
  if (cand_less(key, id, s.k2, s.i2)) {
    if (cand_less(key, id, s.k1, s.i1)) {
      s.k2 = s.k1;
      s.i2 = s.i1;
      s.k1 = key;
      s.i1 = id;
    } else {
      s.k2 = key;
      s.i2 = id;
    }
  }
}

__device__ __forceinline__ Top2 top2_merge(const Top2& a, const Top2& b) {
  Top2 r;
  if (cand_less(b.k1, b.i1, a.k1, a.i1)) {
    r.k1 = b.k1;
    r.i1 = b.i1;
    const bool second_a = cand_less(a.k1, a.i1, b.k2, b.i2);
    r.k2 = second_a ? a.k1 : b.k2;
    r.i2 = second_a ? a.i1 : b.i2;
  } else {
    r.k1 = a.k1;
    r.i1 = a.i1;
    const bool second_b = cand_less(b.k1, b.i1, a.k2, a.i2);
    r.k2 = second_b ? b.k1 : a.k2;
    r.i2 = second_b ? b.i1 : a.i2;
  }
  return r;
}

__device__ __forceinline__ Top2 top2_empty() { return Top2{INFINITY, INT_MAX, INFINITY, INT_MAX}; }

// Workgroup-wide top-2 (every thread returns the result).
__device__ Top2 block_top2(Top2 v, Top2* sh) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    Top2 o;
    o.k1 = __shfl_xor(v.k1, off, kWave);
    o.i1 = __shfl_xor(v.i1, off, kWave);
    o.k2 = __shfl_xor(v.k2, off, kWave);
    o.i2 = __shfl_xor(v.i2, off, kWave);
    v = top2_merge(v, o);
  }
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  Top2 r = sh[0];
  for (int w = 1; w < kWavesPerBlock; ++w) r = top2_merge(r, sh[w]);
  __syncthreads();
  return r;
}

// Exponential-race keys of 8 ids: E_v / w_v with E_v = -log2 u_v (a constant
// factor ln 2 does not change the argmin) and w_v the unnormalised weight.
// residual: w = p - q with p = 2^(z_t*k2 - L2t), q = p * 2^((z_d - z_t)*k2 + D2)
// bonus (or empty-residual fallback): w = p.
template <int DT, bool VEC>
__device__ __forceinline__ void scan_group(const void* row_t, const void* row_d, bool residual,
                                           int64_t e0, int64_t end, float k2, float L2t, float D2,
                                           uint32_t pos, uint32_t r, uint32_t s0, uint32_t s1,
                                           Top2& best) {
  float zt[kGroup], zd[kGroup];
  load8<DT, VEC>(row_t, e0, end, zt);
  if (residual) load8<DT, VEC>(row_d, e0, end, zd);
  const uint32_t c0 = uint32_t(e0 >> 2);
  const Philox4 lo = philox4x32_10(c0, pos, r, kPurposeSample, s0, s1);
  const Philox4 hi = philox4x32_10(c0 + 1u, pos, r, kPurposeSample, s0, s1);
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    const float a2 = fmaf(zt[t], k2, -L2t);
    const float p = __builtin_amdgcn_exp2f(a2);
    float w = p;
    if (residual) w = p - __builtin_amdgcn_exp2f(a2 + fmaf(zd[t] - zt[t], k2, D2));
    const uint32_t word = t < 4 ? lo.w[t] : hi.w[t - 4];
    const float e2 = -__builtin_amdgcn_logf(unit_uniform(word));
    const float key = (w > 0.0f) ? e2 * __builtin_amdgcn_rcpf(w) : INFINITY;
    if (e0 + t < end) top2_insert(best, key, int32_t(e0 + t));
  }
}

// float64 score of candidate v: ln w_v + G_v with G_v = -ln(-ln u_v).
template <int DT>
__device__ double rescore(const void* row_t, const void* row_d, bool residual, int32_t v, double T,
                          double lzt, double lzd, uint32_t pos, uint32_t r, uint32_t s0,
                          uint32_t s1) {
  if (v < 0 || v == INT_MAX) return -INFINITY;
  const Philox4 blk = philox4x32_10(uint32_t(v) >> 2, pos, r, kPurposeSample, s0, s1);
  const double u = unit_uniform_d(blk.w[v & 3]);
  const double g = -log(-log_uniform_d(u));
  const double lp = double(load_one<DT>(row_t, v)) / T - lzt;
  if (!residual) return lp + g;
  const double lq = double(load_one<DT>(row_d, v)) / T - lzd;
  const double dd = lq - lp;
  if (!(dd < 0.0)) return -INFINITY;
  return lp + log(-expm1(dd)) + g;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void sample_kernel(SampleArgs a) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  __shared__ Top2 sh[kWavesPerBlock];
  __shared__ int s_last;
  const int64_t chain = blockIdx.x / a.nsplit;
  const int64_t split = blockIdx.x - chain * a.nsplit;
  const int64_t b = chain / a.K;
  const int64_t k = chain - b * a.K;
  const int G = int(a.G);
  const int n = a.accept_len[chain];
  const float T = a.temp[b];
  if (n < 0 || n > G) return;
  if (!(T > 0.0f)) {
    if (T == 0.0f && a.amax_t && split == 0 && threadIdx.x == 0)
      a.out_token[chain] = a.amax_t[b * (G + 1) + n];
    return;
  }
  const bool residual = n < G;
  const void* row_t = row_ptr(a.t, esz, b * a.tsb + int64_t(n) * a.tsj);
  const void* row_d = residual ? row_ptr(a.d, esz, b * a.dsb + k * a.dsk + int64_t(n) * a.dsj)
                               : nullptr;
  const double lzt = a.lnz_t[b * (G + 1) + n];
  const double lzd = residual ? a.lnz_d[(b * a.K + k) * G + n] : 0.0;
  const float k2 = kLog2e / T;
  const float L2t = float(lzt * kLog2eD);
  const float D2 = residual ? float((lzt - lzd) * kLog2eD) : 0.0f;
  const uint32_t pos = uint32_t(uint64_t(a.pos0 ? a.pos0[b] : 0) + uint64_t(n));
  const uint32_t r = uint32_t(chain);
  const uint32_t s0 = uint32_t(a.seed), s1 = uint32_t(a.seed >> 32);

  const int64_t start = split * kSplit;
  const int64_t end = start + kSplit < a.V ? start + kSplit : a.V;
  Top2 best = top2_empty();
#pragma unroll
  for (int it = 0; it < kSampleIters; ++it) {
    const int64_t e0 = start + int64_t(kGroup) * (threadIdx.x + int64_t(kBlock) * it);
    if (e0 < end)
      scan_group<DT, VEC>(row_t, row_d, residual, e0, end, k2, L2t, D2, pos, r, s0, s1, best);
  }
  best = block_top2(best, sh);

  if (threadIdx.x == 0) {
    a.part[chain * a.nsplit + split] = best;
    __threadfence();
    const uint32_t prev = atomicAdd(a.cnt + chain, 1u);
    s_last = prev == uint32_t(a.nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Last workgroup of the chain: merge the splits in order.
  Top2 all = top2_empty();
  if (threadIdx.x == 0) {
    for (int64_t s = 0; s < a.nsplit; ++s) {
      const Top2 p = a.part[chain * a.nsplit + s];
      all = top2_merge(all, p);
    }
    a.cnt[chain] = 0u;
    sh[0] = all;
  }
  __syncthreads();
  all = sh[0];
  __syncthreads();
  bool use_residual = residual;
  if (all.k1 == INFINITY && residual) {
    // Empty residual support (rounding only): draw from p_n with the same noise.
    use_residual = false;
    Top2 fb = top2_empty();
    for (int64_t e0 = int64_t(kGroup) * threadIdx.x; e0 < a.V; e0 += int64_t(kGroup) * kBlock)
      scan_group<DT, VEC>(row_t, row_d, false, e0, a.V, k2, L2t, D2, pos, r, s0, s1, fb);
    all = block_top2(fb, sh);
  }
  if (threadIdx.x == 0) {
    const double s1d = rescore<DT>(row_t, row_d, use_residual, all.i1, double(T), lzt, lzd, pos,
                                   r, s0, s1);
    const double s2d = rescore<DT>(row_t, row_d, use_residual, all.i2, double(T), lzt, lzd, pos,
                                   r, s0, s1);
    int32_t win = all.i1;
    if (s2d > s1d || (s2d == s1d && all.i2 < all.i1)) win = all.i2;
    if (win == INT_MAX) win = -1;
    a.out_token[chain] = win;
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// The accept test alone: one thread per chain.
__global__ __launch_bounds__(kBlock) void accept_scalar_kernel(const float* __restrict__ lp,
                                                               const float* __restrict__ lq,
                                                               int64_t nchains, int64_t K, int G,
                                                               uint64_t seed,
                                                               const int64_t* __restrict__ pos0,
                                                               int32_t* __restrict__ accept_len,
                                                               uint32_t* __restrict__ bits) {
  const int64_t c = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (c >= nchains) return;
  const int64_t b = c / K;
  const uint64_t p0 = uint64_t(pos0 ? pos0[b] : 0);
  uint64_t mask = 0;
  for (int j = 0; j < G; ++j) {
    const Philox4 r = philox4x32_10(0u, uint32_t(p0 + uint64_t(j)), uint32_t(c), kPurposeAccept,
                                    uint32_t(seed), uint32_t(seed >> 32));
    const double lu = log_uniform_d(unit_uniform_d(r.w[0]));
    const double diff = double(lp[c * G + j]) - double(lq[c * G + j]);
    if (lu < diff) mask |= 1ull << j;
  }
  accept_len[c] = __builtin_ctzll(~mask);
  if (bits) bits[c] = uint32_t(mask);
}

// ---------------------------------------------------------------------------
// Host side.

struct Layout {
  int64_t nch, clen, rows, chains, nsplit;
  size_t off_part, off_lnz, off_top, off_cnt, total;
};

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t chunks_per_row(int64_t V) { return (V + kUnit - 1) / kUnit; }
int64_t chunk_len(int64_t V) {
  const int64_t n = chunks_per_row(V);
  const int64_t l = (V + n - 1) / n;
  return (l + kGroup - 1) / kGroup * kGroup;
}

Layout make_layout(int64_t rows, int64_t chains, int64_t V) {
  Layout L;
  L.nch = chunks_per_row(V);
  L.clen = chunk_len(V);
  L.rows = rows;
  L.chains = chains;
  L.nsplit = (V + kSplit - 1) / kSplit;
  L.off_part = 0;
  L.off_lnz = align256(L.off_part + size_t(rows) * size_t(L.nch) * sizeof(RowPartial));
  L.off_top = align256(L.off_lnz + size_t(rows) * sizeof(double));
  L.off_cnt = align256(L.off_top + size_t(chains) * size_t(L.nsplit) * sizeof(Top2));
  L.total = align256(L.off_cnt + size_t(chains) * sizeof(uint32_t));
  return L;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s, int esz) { return (s * esz) % 16 == 0; }

int check_dtype(int dtype) { return (dtype == SV_F32 || dtype == SV_BF16) ? SV_OK : SV_EDTYPE; }
int esize(int dtype) { return dtype == SV_BF16 ? 2 : 4; }

int launch_status() { return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP; }

template <int DT, bool VEC>
void launch_rowstats_t(const RowSet& rs, int64_t V, const Layout& L, RowPartial* part,
                       bool argmax_all, hipStream_t st) {
  const int64_t units = L.rows * L.nch;
  int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = int64_t(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  if (argmax_all)
    hipLaunchKernelGGL((rowstats_kernel<DT, VEC, true>), dim3(unsigned(blocks)), dim3(kBlock), 0,
                       st, rs, V, L.nch, L.clen, units, part);
  else
    hipLaunchKernelGGL((rowstats_kernel<DT, VEC, false>), dim3(unsigned(blocks)), dim3(kBlock), 0,
                       st, rs, V, L.nch, L.clen, units, part);
}

void launch_rowstats(int dtype, bool vec, const RowSet& rs, int64_t V, const Layout& L,
                     RowPartial* part, bool argmax_all, hipStream_t st) {
  if (dtype == SV_BF16) {
    if (vec) launch_rowstats_t<SV_BF16, true>(rs, V, L, part, argmax_all, st);
    else launch_rowstats_t<SV_BF16, false>(rs, V, L, part, argmax_all, st);
  } else {
    if (vec) launch_rowstats_t<SV_F32, true>(rs, V, L, part, argmax_all, st);
    else launch_rowstats_t<SV_F32, false>(rs, V, L, part, argmax_all, st);
  }
}

void launch_sample(int dtype, bool vec, const SampleArgs& sa, hipStream_t st) {
  const int64_t blocks = sa.B * sa.K * sa.nsplit;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  if (dtype == SV_BF16) {
    if (vec) hipLaunchKernelGGL((sample_kernel<SV_BF16, true>), grid, dim3(kBlock), 0, st, sa);
    else hipLaunchKernelGGL((sample_kernel<SV_BF16, false>), grid, dim3(kBlock), 0, st, sa);
  } else {
    if (vec) hipLaunchKernelGGL((sample_kernel<SV_F32, true>), grid, dim3(kBlock), 0, st, sa);
    else hipLaunchKernelGGL((sample_kernel<SV_F32, false>), grid, dim3(kBlock), 0, st, sa);
  }
}

bool sizes_ok(int64_t B, int64_t K, int64_t G, int64_t V) {
  return B >= 1 && K >= 1 && G >= 1 && G <= SV_MAX_GAMMA && K * G <= SV_MAX_CHAIN_DECISIONS &&
         V >= 1 && V < (int64_t(1) << 31) && B * K < (int64_t(1) << 31) &&
         B <= (int64_t(1) << 31) / (G + 1);
}

bool workspace_ok(void* ws, size_t have, size_t need, int* status) {
  if (need > 0 && (ws == nullptr || have < need)) {
    *status = SV_EWORKSPACE;
    return false;
  }
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    *status = SV_EALIGN;
    return false;
  }
  return true;
}

size_t step_workspace(int64_t B, int64_t K, int64_t G, int64_t V) {
  return make_layout(B * (G + 1) + B * K * G, B * K, V).total;
}

}  // namespace

extern "C" {

size_t specverify_workspace_size(int64_t B, int64_t K, int64_t gamma, int64_t V, int dtype) {
  if (check_dtype(dtype) != SV_OK) return 0;
  if (K == 0) {  // specverify_normalize: P = gamma + 1 rows per batch row
    if (B < 1 || gamma < 0 || V < 1 || V >= (int64_t(1) << 31)) return 0;
    return make_layout(B * (gamma + 1), 0, V).total;
  }
  if (!sizes_ok(B, K, gamma, V)) return 0;
  return step_workspace(B, K, gamma, V);
}

int specverify_normalize(const void* logits, int dtype, int64_t B, int64_t P, int64_t V,
                         int64_t stride_b, int64_t stride_p, const float* temperature,
                         double* lnZ, int32_t* argmax, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!logits || !temperature || !lnZ) return SV_EINVAL;
  if (B < 1 || P < 1 || V < 1 || V >= (int64_t(1) << 31) || stride_b < 0 || stride_p < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  const Layout L = make_layout(B * P, 0, V);
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  const int esz = esize(dtype);
  const bool vec = aligned16(logits) && stride_ok(stride_b, esz) && stride_ok(stride_p, esz);
  RowSet rs{logits, stride_b, stride_p, nullptr, 0, 0, 0, B, P, 0, 1, temperature};
  auto* base = reinterpret_cast<char*>(workspace);
  auto* part = reinterpret_cast<RowPartial*>(base + L.off_part);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  launch_rowstats(dtype, vec, rs, V, L, part, argmax != nullptr, st);
  const int64_t rows = B * P;
  hipLaunchKernelGGL(finalize_rows_kernel, dim3(unsigned((rows + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, st, part, rows, P, L.nch, temperature, lnZ, argmax);
  return launch_status();
}

int specverify_accept(const float* logp, const float* logq, int64_t B, int64_t K, int64_t gamma,
                      uint64_t seed, const int64_t* pos0, int32_t* accept_len,
                      uint32_t* accept_bits, void* stream) {
  if (!logp || !logq || !accept_len) return SV_EINVAL;
  if (B < 1 || K < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || B * K >= (int64_t(1) << 31))
    return SV_EINVAL;
  const int64_t n = B * K;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(accept_scalar_kernel, dim3(unsigned((n + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, st, logp, logq, n, K, int(gamma), seed, pos0, accept_len, accept_bits);
  return launch_status();
}

int specverify_residual_sample(const void* target_logits, const void* draft_logits, int dtype,
                               int64_t B, int64_t K, int64_t gamma, int64_t V,
                               int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b,
                               int64_t d_stride_k, int64_t d_stride_j, const float* temperature,
                               const double* lnZ_target, const double* lnZ_draft,
                               const int32_t* argmax_target, const int32_t* accept_len,
                               uint64_t seed, const int64_t* pos0, int32_t* out_token,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !temperature || !lnZ_target || !lnZ_draft ||
      !argmax_target || !accept_len || !out_token)
    return SV_EINVAL;
  if (!sizes_ok(B, K, gamma, V)) return SV_EINVAL;
  if (t_stride_b < 0 || t_stride_j < 0 || d_stride_b < 0 || d_stride_k < 0 || d_stride_j < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  const Layout L = make_layout(B * (gamma + 1) + B * K * gamma, B * K, V);
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  const int esz = esize(dtype);
  const bool vec = aligned16(target_logits) && aligned16(draft_logits) &&
                   stride_ok(t_stride_b, esz) && stride_ok(t_stride_j, esz) &&
                   stride_ok(d_stride_b, esz) && stride_ok(d_stride_k, esz) &&
                   stride_ok(d_stride_j, esz);
  auto* base = reinterpret_cast<char*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto* cnt = reinterpret_cast<uint32_t*>(base + L.off_cnt);
  const int64_t chains = B * K;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(unsigned((chains + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, st, cnt, chains);
  SampleArgs sa{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                d_stride_j, B, K, gamma, V, temperature, lnZ_target, lnZ_draft, argmax_target,
                accept_len, seed, pos0, out_token, L.nsplit,
                reinterpret_cast<Top2*>(base + L.off_top), cnt};
  launch_sample(dtype, vec, sa, st);
  return launch_status();
}

int specverify_step(const void* target_logits, const void* draft_logits, int dtype,
                    const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                    int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b,
                    int64_t d_stride_k, int64_t d_stride_j, const float* temperature,
                    uint64_t seed, const int64_t* pos0, int32_t* accept_len, int32_t* out_token,
                    float* logp, float* logq, double* lnZ_target, double* lnZ_draft,
                    int32_t* device_error, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !accept_len ||
      !out_token)
    return SV_EINVAL;
  if (!sizes_ok(B, K, gamma, V)) return SV_EINVAL;
  if (t_stride_b < 0 || t_stride_j < 0 || d_stride_b < 0 || d_stride_k < 0 || d_stride_j < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  const Layout L = make_layout(B * (gamma + 1) + B * K * gamma, B * K, V);
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  const int esz = esize(dtype);
  const bool vec = aligned16(target_logits) && aligned16(draft_logits) &&
                   stride_ok(t_stride_b, esz) && stride_ok(t_stride_j, esz) &&
                   stride_ok(d_stride_b, esz) && stride_ok(d_stride_k, esz) &&
                   stride_ok(d_stride_j, esz);
  auto* base = reinterpret_cast<char*>(workspace);
  auto* part = reinterpret_cast<RowPartial*>(base + L.off_part);
  auto* ws_lnz = reinterpret_cast<double*>(base + L.off_lnz);
  auto* cnt = reinterpret_cast<uint32_t*>(base + L.off_cnt);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  RowSet rs{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
            d_stride_j, B, gamma + 1, K, gamma, temperature};
  launch_rowstats(dtype, vec, rs, V, L, part, false, st);

  AcceptArgs aa{rs, V, L.nch, part, draft_tokens, seed, pos0, accept_len, out_token, logp, logq,
                lnZ_target, lnZ_draft, device_error, ws_lnz, cnt};
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(accept_kernel<SV_BF16>, dim3(unsigned(B)), dim3(kBlock), 0, st, aa);
  else
    hipLaunchKernelGGL(accept_kernel<SV_F32>, dim3(unsigned(B)), dim3(kBlock), 0, st, aa);

  SampleArgs sa{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                d_stride_j, B, K, gamma, V, temperature, ws_lnz, ws_lnz + B * (gamma + 1),
                nullptr, accept_len, seed, pos0, out_token, L.nsplit,
                reinterpret_cast<Top2*>(base + L.off_top), cnt};
  launch_sample(dtype, vec, sa, st);
  return launch_status();
}

const char* specverify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (null pointer, size or stride out of range)";
    case SV_EDTYPE: return "unknown logit dtype";
    case SV_EWORKSPACE: return "workspace missing or too small";
    case SV_EALIGN: return "workspace not 256-byte aligned";
    case SV_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int specverify_version(void) { return 100; }

}  // extern "C"
