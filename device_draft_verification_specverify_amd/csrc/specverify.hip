// specverify.hip -- HIP kernels (gfx950 / CDNA4) and the C ABI of libspecverify.
//
// Batched speculative-sampling verification in two launches when the draw grid
// is resident at once, otherwise three (accept_kernel derives n per chain
// before the draws), and one more past 65536 chains:
//
//   stream_kernel   every needed logit row is read exactly once. Persistent
//                   workgroups (one per CU) walk 8 KB chunks of the flattened
//                   rows round robin, their wavefronts claiming chunks from an
//                   LDS counter; draft rows of greedy batch rows are left out.
//                   Each lane reduces its logits to (max, sum of exp2) with one
//                   fma + one exp per logit; each chunk ends in one cross-lane
//                   reduction and one 16-byte partial.
//   draw_kernel     one workgroup per (chain, vocabulary split). Each first
//                   derives its chain's n (or reads it from accept_kernel,
//                   which does the same per chain): ln Z of the chain's rows from the
//                   partials (8 lanes per row), ln p / ln q at the draft tokens,
//                   the accept uniforms and the first rejection by one ballot
//                   (split 0 writes the chain's outputs). Then it scans its split
//                   of the one row pair the chain needs -- target/draft row n for
//                   the residual, target row gamma for the bonus -- drawing
//                   Gumbel noise by exponential race, argmin_v E_v / w_v with
//                   E_v = -ln u_v (the same argmax as ln w_v + G_v), keeps its
//                   best two candidates and re-scores them in float64. The last
//                   split of a chain to finish (a per-chain counter) keeps the
//                   best score over the splits (ties to the lowest id).
//   finish_kernel   that last step, one wavefront per chain, when there are too
//                   many chains for the counters.
//
// The other entry points (normalise, accept test, residual sample, acceptance
// probability, top-F candidates, cache lookup, branch pruning) reuse these
// pieces; each kernel below says which.
//
// Hand-offs inside a launch (the per-chain counters) use relaxed agent-scope
// atomics after the publishing wavefront's stores have completed.
// No matrix cores (nothing here is a dense contraction) and no floating-point
// atomics: results are bit-deterministic.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "specverify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
// The streaming kernel runs one 1024-thread workgroup per CU whose wavefronts
// claim chunks from an LDS counter. A SIMD issues the memory instructions of
// its older wavefronts first, so with a fixed share per wavefront the youngest
// read at less than half the rate of the oldest and finish ~20 us later
// (measured: six 256-thread workgroups per CU, round-robin chunks).
constexpr int kStreamBlock = 1024;
constexpr int kStreamWaves = kStreamBlock / kWave;
constexpr int kVec = 8;                    // logits per vector (16 B of bf16, 32 B of f32)
constexpr int kSampleIters = 4;            // vectors per thread per sampling split
constexpr int64_t kSplit = int64_t(kBlock) * kVec * kSampleIters;  // 8192 ids per split
constexpr int64_t kMaxCompactB = 16384;    // batch rows whose greedy drafts are compacted out
constexpr int kMaxRowsPerChain = SV_MAX_GAMMA + 1 + SV_MAX_GAMMA;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;
constexpr uint32_t kPurposeAccept = 0;
constexpr uint32_t kPurposeSample = 1;

// Statistics of one row segment: s = sum over the segment of 2^((z - m) * k),
// k = float(log2(e) / T); m is the raw maximum and idx its lowest id.
struct alignas(16) RowPartial {
  float m;
  int32_t idx;
  double s;
};

// Best two sampling candidates of a wavefront or a split, ordered by (key, id),
// with the target and draft logits at each (for the float64 re-score).
struct Top2 {
  float k1;
  int32_t i1;
  float t1, d1;
  float k2;
  int32_t i2;
  float t2, d2;
};

// A split's draw result: the float64 score ln w_v + G_v of its best candidate.
struct alignas(16) Cand {
  double score;  // -inf when the split holds no candidate
  int32_t id;    // INT_MAX when none
  int32_t pad;
};

// What the accept test needs of one draft position of one chain, gathered
// during the stream by its grid's last workgroup: the target and draft logits
// at the draft token (0 for greedy rows and invalid tokens) and ln u of the
// accept uniform.
struct alignas(16) TokenAux {
  float zt, zd;
  double log_u;
};

// What the draw and finish kernels need of a chain (written by split 0 of the
// step's draw kernel, or by given_kernel).
struct alignas(16) ChainInfo {
  double lzt;  // ln Z of the target row the token is drawn from (row n, or gamma)
  double lzd;  // ln Z of draft row n (residual draws)
  int32_t n;   // accept length; -1 when no draw is needed (greedy, error)
  int32_t pad[3];
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies whose halves are mixed with the other words and the round key; the
// key advances by two Weyl constants between rounds.
struct Philox4 {
  uint32_t w[4];
};

// a ^ b ^ c in one instruction: gfx950's three-input bitwise operation with
// the truth table of odd parity (0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = uint64_t(kPhiloxM0) * c0;
    const uint64_t p1 = uint64_t(kPhiloxM1) * c2;
    const uint32_t n0 = xor3(uint32_t(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3(uint32_t(p0 >> 32), c3, k1);
    c0 = n0;
    c1 = uint32_t(p1);
    c2 = n2;
    c3 = uint32_t(p0);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// u = (floor(w / 2^9) + 1/2) * 2^-23: exact in float and double. In float it is
// built as (1 + m 2^-23) - (1 - 2^-24) with m = floor(w / 2^9) placed in the
// mantissa of 1.0 by one funnel shift; the difference (2m + 1) 2^-24 is exact.
__device__ __forceinline__ float unit_uniform(uint32_t w) {
  return __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u)) - 0x1.fffffep-1f;
}
__device__ __forceinline__ double unit_uniform_d(uint32_t w) {
  return (double(w >> 9) + 0.5) * 0x1p-23;
}
// ln u in double; for u >= 1/2, u - 1 is exact and log1p keeps full accuracy.
__device__ __forceinline__ double log_uniform_d(double u) {
  return u >= 0.5 ? log1p(u - 1.0) : log(u);
}

// ln u of the accept test's uniform of chain r at draft position j: Philox
// counter (0, pos0[b] + j, r, accept purpose), first word.
__device__ __forceinline__ double accept_log_u(uint64_t seed, const int64_t* pos0, int64_t b,
                                               int64_t j, int64_t r) {
  const uint64_t pos = uint64_t(pos0 ? pos0[b] : 0) + uint64_t(j);
  const Philox4 w = philox4x32_10(0u, uint32_t(pos), uint32_t(r), kPurposeAccept, uint32_t(seed),
                                  uint32_t(seed >> 32));
  return log_uniform_d(unit_uniform_d(w.w[0]));
}

// ---------------------------------------------------------------------------
// Device-side index checks (a build with -DSV_DEVICE_CHECKS): a work unit checks
// the indices it derived against the sizes it was launched with before it
// touches memory; a failed check is counted in sv_check_count (read by
// specverify_check_count) and the unit is skipped. In the product build sv_ok
// is true and the checks fold away.
#ifdef SV_DEVICE_CHECKS
__device__ unsigned int sv_check_count;
__device__ __forceinline__ bool sv_ok(bool ok) {
  if (!ok) atomicAdd(&sv_check_count, 1u);
  return ok;
}
#else
__device__ __forceinline__ bool sv_ok(bool) { return true; }
#endif

// ---------------------------------------------------------------------------
// Logit access. A "vector" is 8 consecutive logits starting at a multiple of 8.
template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t e) {
  if constexpr (DT == SV_BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[e];
    return __uint_as_float(uint32_t(h) << 16);
  } else {
    return reinterpret_cast<const float*>(row)[e];
  }
}

// Raw storage of one vector: 4 dwords of bf16 pairs, or 8 floats.
template <int DT>
struct RawVec {
  uint32_t w[DT == SV_BF16 ? 4 : 8];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// All 8 ids of vector vi must lie inside the row. NT: non-temporal 128-bit loads
// (logits are read once; streaming them past the caches measured ~8% faster).
template <int DT, bool VEC, bool NT = false>
__device__ __forceinline__ RawVec<DT> load_vec(const void* row, int64_t vi) {
  RawVec<DT> r;
  if constexpr (VEC) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + (DT == SV_BF16 ? vi : 2 * vi);
    const u32x4 a = NT ? __builtin_nontemporal_load(p) : p[0];
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    if constexpr (DT == SV_F32) {
      const u32x4 b = NT ? __builtin_nontemporal_load(p + 1) : p[1];
      r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    }
  } else {
    if constexpr (DT == SV_BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + kVec * vi;
#pragma unroll
      for (int i = 0; i < 4; ++i) r.w[i] = uint32_t(p[2 * i]) | (uint32_t(p[2 * i + 1]) << 16);
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + kVec * vi;
#pragma unroll
      for (int i = 0; i < 8; ++i) r.w[i] = p[i];
    }
  }
  return r;
}

template <int DT>
__device__ __forceinline__ float vec_elem(const RawVec<DT>& r, int t) {
  if constexpr (DT == SV_BF16) {
    const uint32_t w = r.w[t >> 1];
    return __uint_as_float((t & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return __uint_as_float(r.w[t]);
  }
}

// Nonzero when some slot of the vector holds a NaN, from the raw bits: with
// the sign cleared a bf16 half (or an f32 word) is a NaN iff it exceeds the
// +inf pattern 0x7F80 (0x7F800000), i.e. iff adding 0x7F (0x7FFFFF) carries
// into its top bit; the low half's sum stays below 2^16, so the halves of a
// word do not interact. Integer ops on packed words, no unpacking.
template <int DT>
__device__ __forceinline__ uint32_t nan_bits(const RawVec<DT>& r) {
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < (DT == SV_BF16 ? 4 : 8); ++i) {
    if constexpr (DT == SV_BF16) acc |= ((r.w[i] & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
    else acc |= ((r.w[i] & 0x7FFFFFFFu) + 0x007FFFFFu) & 0x80000000u;
  }
  return acc;
}

// A vector that reads -inf in every slot.
template <int DT>
__device__ __forceinline__ RawVec<DT> neg_inf_vec() {
  RawVec<DT> r;
  if constexpr (DT == SV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = 0xFF80FF80u;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.w[i] = 0xFF800000u;
  }
  return r;
}

// Vector vi of a row of V logits, ids >= V reading -inf (only a row's last
// vector can be partial; it is read element by element).
template <int DT, bool VEC>
__device__ __forceinline__ RawVec<DT> load_vec_bounded(const void* row, int64_t vi, int64_t V) {
  if ((vi + 1) * kVec <= V) return load_vec<DT, VEC>(row, vi);
  RawVec<DT> r = neg_inf_vec<DT>();
#pragma unroll
  for (int t = 0; t < kVec; ++t) {
    const int64_t e = vi * kVec + t;
    if (e < V) {
      if constexpr (DT == SV_BF16) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(row)[e];
        r.w[t >> 1] = (t & 1) ? ((r.w[t >> 1] & 0x0000FFFFu) | (h << 16))
                              : ((r.w[t >> 1] & 0xFFFF0000u) | h);
      } else {
        r.w[t] = reinterpret_cast<const uint32_t*>(row)[e];
      }
    }
  }
  return r;
}

__device__ __forceinline__ const void* row_ptr(const void* base, int esz, int64_t off_elems) {
  return reinterpret_cast<const char*>(base) + off_elems * esz;
}

__device__ __forceinline__ void better_max(float& m, int32_t& i, float om, int32_t oi) {
  if (om > m || (om == m && oi < i)) {
    m = om;
    i = oi;
  }
}

// Lane moves inside rows of 16 lanes by DPP (a VALU operand modifier, no
// LDS round trip): quad_perm [1,0,3,2] and [2,3,0,1] (lane ^ 1, lane ^ 2),
// row_half_mirror (i <-> 7 - i within 8 lanes) and row_mirror (i <-> 15 - i
// within 16). Applied in that order, each pairs lanes whose partial results
// cover disjoint groups, so after the four every lane of a row holds its
// row's result (for order-free operations such as min and max).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp64(double x) {
  const uint64_t b = uint64_t(__double_as_longlong(x));
  const uint64_t lo = dpp32<CTRL>(uint32_t(b)), hi = dpp32<CTRL>(uint32_t(b >> 32));
  return __longlong_as_double(int64_t((hi << 32) | lo));
}
__device__ __forceinline__ double readlane64(double x, int l) {
  const uint64_t b = uint64_t(__double_as_longlong(x));
  const uint64_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), l));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), l));
  return __longlong_as_double(int64_t((hi << 32) | lo));
}

// A row's 8 lanes (kRowLanes) combined by DPP: lane ^ 1, lane ^ 2, then the
// two quads (row_half_mirror); every lane of the 8 gets the result. The
// argmax is order-free; the sum's order is fixed, and the draws' prologue
// and finalize_rows_kernel both use it, so a row gets the same bits from
// either.
__device__ __forceinline__ void group8_argmax(float& m, int32_t& i) {
  better_max(m, i, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(m))), int32_t(dpp32<kDppXor1>(uint32_t(i))));
  better_max(m, i, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(m))), int32_t(dpp32<kDppXor2>(uint32_t(i))));
  better_max(m, i, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(m))),
             int32_t(dpp32<kDppHalfMirror>(uint32_t(i))));
}
// The wavefront's minimum in every lane (DPP inside rows, then the rows).
__device__ __forceinline__ float wave_min(float x) {
  x = fminf(x, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(x))));
  x = fminf(x, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(x))));
  x = fminf(x, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(x))));
  x = fminf(x, __uint_as_float(dpp32<kDppMirror>(__float_as_uint(x))));
  float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r)
    w = fminf(w, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16 * r)));
  return w;
}
// The wavefront's sum in every lane, rows added in a fixed order.
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp64<kDppXor1>(x);
  x += dpp64<kDppXor2>(x);
  x += dpp64<kDppHalfMirror>(x);
  x += dpp64<kDppMirror>(x);
  double w = readlane64(x, 0);
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r) w += readlane64(x, 16 * r);
  return w;
}
// The wavefront's largest value and its lowest id (better_max), in every lane.
__device__ __forceinline__ void wave_argmax(float& m, int32_t& i) {
  better_max(m, i, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(m))), int32_t(dpp32<kDppXor1>(uint32_t(i))));
  better_max(m, i, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(m))), int32_t(dpp32<kDppXor2>(uint32_t(i))));
  better_max(m, i, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(m))),
             int32_t(dpp32<kDppHalfMirror>(uint32_t(i))));
  better_max(m, i, __uint_as_float(dpp32<kDppMirror>(__float_as_uint(m))), int32_t(dpp32<kDppMirror>(uint32_t(i))));
  float wm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
  int32_t wi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r)
    better_max(wm, wi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16 * r)),
               __builtin_amdgcn_readlane(i, 16 * r));
  m = wm;
  i = wi;
}
__device__ __forceinline__ double group8_sum(double x) {
  x += dpp64<kDppXor1>(x);
  x += dpp64<kDppXor2>(x);
  x += dpp64<kDppHalfMirror>(x);
  return x;
}

// ---------------------------------------------------------------------------
// Rows and their place in the flattened stream. Target rows come first, in
// (b, j) order; then the K*G draft rows of every batch row that needs them, in
// (b, k, j) order. In compact mode only batch rows with T > 0 contribute draft
// rows; otherwise all do and greedy ones are skipped in place.
struct RowSet {
  const void* t;
  int64_t tsb, tsj;
  const void* d;
  int64_t dsb, dsk, dsj;
  int64_t B, P, K, G;
  const float* temp;
};

// Stream chunks: every stream row is cut into chunks of kWave * chunk_lanes(DT)
// vectors (8 KB), one partial per chunk, stored row-major: part[rho * cpr + j].
template <int DT>
constexpr int chunk_lanes() { return DT == SV_BF16 ? 8 : 4; }  // vectors per lane per chunk
inline int64_t chunk_vectors(int dtype) { return int64_t(kWave) * (dtype == SV_BF16 ? 8 : 4); }

struct RowStat {
  double lnz;
  float m;
  int32_t idx;
  bool bad;  // the row is an input error (row_bad)
};

// 2^e for a rescaling exponent e <= 0 between partial sums, in single
// precision: about 1e-7 relative per term, far inside the normaliser tolerance.
__device__ __forceinline__ double exp2_scale(double e) {
  return double(__builtin_amdgcn_exp2f(float(e)));
}

// Fold chunk partial q into a lane's running (m, idx, s); s stays relative to
// m in units of k2 = float(log2(e) / T). A partial whose maximum is -inf, and
// every partial of a greedy row, carries s = 0, or NaN when its chunk held a
// NaN; that s is added as it is, so a NaN anywhere in a row reaches the row's
// sum (a +inf logit makes its chunk's sum NaN too).
__device__ __forceinline__ void fold_partial(float& m, int32_t& idx, double& s, const RowPartial& q,
                                             bool sampled, double k2) {
  float bm = m;
  int32_t bi = idx;
  better_max(bm, bi, q.m, q.idx);
  if (sampled) {
    if (bm > -INFINITY && m > -INFINITY) s *= exp2_scale((double(m) - double(bm)) * k2);
    s += q.m > -INFINITY ? q.s * exp2_scale((double(q.m) - double(bm)) * k2) : q.s;
  } else {
    s += q.s;
  }
  m = bm;
  idx = bi;
}

// A needed row is an input error when its largest logit is not finite (every
// entry -inf, or a +inf) or it holds a NaN (its folded sum is NaN).
__device__ __forceinline__ bool row_bad(float M, double sr) {
  return !(M > -INFINITY && M < INFINITY && sr == sr);
}

// ln Z of a row from its maximum M and its folded sum sr (relative to M):
// ln sum exp(z / T) for T > 0, max z for T == 0, NaN for other T and for rows
// holding a NaN or (T > 0) a +inf; an all -inf row gives -inf.
__device__ __forceinline__ double row_lnz(float M, double sr, float T) {
  if (!(sr == sr)) return NAN;
  if (T > 0.0f) return M > -INFINITY ? double(M) / double(T) + log(sr) : double(M);
  if (T == 0.0f) return double(M);
  return NAN;
}

// Statistics of one stream row by a group of kRowLanes consecutive lanes, for
// rows of few chunks: lane gl of the group folds chunks gl, gl + 8, ..., four
// loads in flight at a time (has == false: the lane folds nothing), and
// group_reduce_row combines the group in a fixed order (group8_sum). The
// draws' prologue folds and combines its rows in this same order, inline, so
// that both give a row the same bits. Every lane of the wavefront calls
// group_reduce_row; all lanes of a group get the result (lnZ as row_lnz).
constexpr int kRowLanes = 8;

__device__ __forceinline__ void group_fold(const RowPartial* __restrict__ part, int64_t rho,
                                           bool has, int64_t cpr, int gl, bool sampled, double k2,
                                           float& m, int32_t& idx, double& s) {
  m = -INFINITY;
  idx = INT_MAX;
  s = 0.0;
  for (int64_t c0 = gl; c0 < cpr; c0 += 4 * kRowLanes) {
    RowPartial q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + int64_t(u) * kRowLanes;
      q[u] = (has && c < cpr) ? part[rho * cpr + c] : RowPartial{-INFINITY, INT_MAX, 0.0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) fold_partial(m, idx, s, q[u], sampled, k2);
  }
}

__device__ __forceinline__ RowStat group_reduce_row(float m, int32_t idx, double s, float T) {
  const bool sampled = T > 0.0f;
  const double k2 = double(kLog2e / T);
  float M = m;
  int32_t I = idx;
  group8_argmax(M, I);
  double sr = (sampled && M > -INFINITY && m > -INFINITY) ? s * exp2_scale((double(m) - double(M)) * k2) : s;
  sr = group8_sum(sr);
  RowStat out;
  out.m = M;
  out.idx = I;
  out.lnz = row_lnz(M, sr, T);
  out.bad = row_bad(M, sr);
  return out;
}

// ---------------------------------------------------------------------------
// Which batch rows need draft rows: a ballot mask per 64 batch rows and an
// exclusive prefix of their counts, built in LDS by every stream workgroup.
struct SampledTable {
  uint64_t mask[kMaxCompactB / 64];
  int32_t pref[kMaxCompactB / 64 + 1];
  int32_t wsum[kStreamWaves];
};

__device__ void build_sampled_table(const float* __restrict__ temp, int64_t B, SampledTable& tab) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nchunks = int((B + 63) / 64);
  for (int c = wid; c < nchunks; c += kStreamWaves) {
    const int64_t b = int64_t(c) * 64 + lane;
    const bool s = b < B && temp[b] > 0.0f;
    const uint64_t m = __ballot(s);
    if (lane == 0) tab.mask[c] = m;
  }
  __syncthreads();
  // inclusive scan of per-chunk counts, one chunk per thread (nchunks <= 256)
  int x = int(threadIdx.x) < nchunks ? __popcll(tab.mask[threadIdx.x]) : 0;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tab.wsum[wid] = x;
  __syncthreads();
  for (int w = 0; w < wid; ++w) x += tab.wsum[w];
  if (int(threadIdx.x) < nchunks) tab.pref[threadIdx.x + 1] = x;
  if (threadIdx.x == 0) tab.pref[0] = 0;
  __syncthreads();
}

// Batch row of the s-th sampled batch row (0-based).
__device__ int64_t select_sampled(const SampledTable& tab, int nchunks, int64_t s) {
  int lo = 0, hi = nchunks - 1;
  while (lo < hi) {  // last chunk c with pref[c] <= s
    const int mid = (lo + hi + 1) >> 1;
    if (tab.pref[mid] <= s) lo = mid;
    else hi = mid - 1;
  }
  // the r-th (from 0) set bit of the chunk's mask, by halving: keep the low
  // half while it holds more than r set bits, else skip it
  uint64_t m = tab.mask[lo];
  int r = int(s - tab.pref[lo]);
  int pos = 0;
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    const int c = __popcll(m & ((uint64_t(1) << w) - 1));
    if (r >= c) {
      r -= c;
      m >>= w;
      pos += w;
    }
  }
  return int64_t(lo) * 64 + pos;
}

// Division of n < 2^31 by an invariant divisor d >= 1 as a multiply-high and a
// shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, figure 4.1): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l. mulhi(m, n)
// is at most n, so the sum stays below 2^32 for n < 2^31.
struct FastDiv {
  uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{d, uint32_t(m), l};
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.l;
}

struct StreamArgs {
  RowSet rs;
  int64_t V, vpr;
  int64_t cpr;           // chunks per row
  int64_t nrows;         // stream rows (recomputed on the device in compact mode)
  int compact;
  RowPartial* part;      // [B*(P+K*G)][cpr]: slot b*P+j, then B*P + (b*K+k)*G+j
  int32_t* rank_out;     // [B + 1]: sampled batch rows before b; [B] = their total
  uint32_t* clear;       // [nclear] per-chain counters the next launch counts on, zeroed here
  int64_t nclear;
  // The step: one more workgroup than the stream needs gathers tok_aux [B*K*G]
  // (gather_tokens) instead of streaming; null otherwise.
  TokenAux* tok_aux;
  const int32_t* tokens;  // [B, K, G]
  const int64_t* pos0;
  uint64_t seed;
  // The chunk-index divisions (by cpr, P, K*G, G) as multiply-shifts: every
  // chunk index is below 2^31 (the host rejects larger calls).
  FastDiv by_cpr, by_p, by_kg, by_g;
  float win_scale;  // window_scale of the launch (set with the grid)
};

// The chunk of a persistent workgroup's i-th claim. Claims i < i0 take whole
// windows of nblk chunks: chunk nblk*i + ((g + (i mod 32)) mod nblk) for
// workgroup g of nblk. Without the rotation a row's short last chunk would fall
// on the same few workgroups every time (all of them when nblk is a multiple of
// the chunks per row, e.g. 256 workgroups and 32 chunks), which would then idle
// while the others stream. Claims i >= i0 take windows of E = ceil(nblk / 2)
// chunks shared by the even workgroups alone (rotated the same way): the
// workgroups are dealt to the 8 XCDs round robin, and the odd XCDs stream ~5%
// slower than the even ones (device-clock traces: B=512 K=4 gamma=8, even XCDs
// end at ~816 us, odd ones at ~857 us), so the even ones take the last ~5%.
// Chunks rise with i, so a workgroup's first one past the end ends its loop
// (odd workgroups: every claim from i0 on). !TAIL: whole windows only (a
// separate kernel, as the check alone measured +0.35 us per step at B=64
// gamma=8 V=128256, where it never applies).
template <bool TAIL>
__device__ __forceinline__ int64_t claimed_chunk(uint32_t i, int64_t nblk, uint32_t i0) {
  if (!TAIL || i < i0) {
    int64_t o = int64_t(blockIdx.x) + int64_t(nblk >= 32 ? (i & 31u) : 0u);
    if (o >= nblk) o -= nblk;
    return o + nblk * int64_t(i);
  }
  if (blockIdx.x & 1u) return INT64_MAX;
  const int64_t E = (nblk + 1) / 2;
  const uint32_t j = i - i0;
  int64_t o = int64_t(blockIdx.x / 2u) + int64_t(E >= 32 ? (j & 31u) : 0u);
  if (o >= E) o -= E;
  return int64_t(i0) * nblk + o + E * int64_t(j);
}

// The whole windows before the even workgroups take over, as a factor on the
// unit count: 1 / (nblk + E/20), so that the even workgroups' extra share is
// ~5% of theirs; 0 (no such windows) for grids under 64 workgroups, and where a
// workgroup reads fewer than 192 chunks (12 per wavefront; `chunks` per unit):
// there the even workgroups' extra chunk per wavefront outlasts the 5% (B=64
// gamma=8 V=128256, 136 chunks per workgroup: 67.4 vs 66.4 us per step;
// B=256 gamma=4 V=151936, 260: 121.7 vs 122.8 us; B=512 K=4 gamma=8, 2624:
// 1112 vs 1125 us). In float32, on the host: a count off by one moves a few
// chunks between the two kinds of windows, and every count maps the chunks one
// to one. The stream kernel uses it (the overlap sweep of the acceptance
// probability claims whole windows only).
inline float window_scale(int64_t total, int64_t nblk, int64_t chunks) {
  if (nblk < 64 || total * chunks < 192 * nblk) return 0.0f;
  return 20.0f / float(20 * nblk + (nblk + 1) / 2);
}
__device__ __forceinline__ uint32_t full_windows(int64_t total, float scale) {
  return scale > 0.0f ? uint32_t(float(uint32_t(total)) * scale) : UINT32_MAX;
}

// The step's token gather (the stream grid's extra, last workgroup): for every
// (chain, position) the logits at the draft token, read only for sampled rows
// and valid tokens, and ln u of the accept uniform (Philox counter (0,
// position, chain, accept purpose)), so that the draws' prologue finds them
// with one load that depends on nothing. With one workgroup per CU this
// workgroup starts when the first streaming one ends.
template <int DT>
__device__ void gather_tokens(const StreamArgs& a) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  const RowSet& rs = a.rs;
  for (int64_t i = threadIdx.x; i < rs.B * rs.K * rs.G; i += kStreamBlock) {
    const int64_t chain = int64_t(fast_div(uint32_t(i), a.by_g));
    const int64_t j = i - chain * rs.G;
    const int64_t b = int64_t(uint32_t(chain) / uint32_t(rs.K));
    const int64_t k = chain - b * rs.K;
    const int32_t x = a.tokens[i];
    float zt = 0.0f, zd = 0.0f;
    if (!(x < 0 || int64_t(x) >= a.V) && rs.temp[b] > 0.0f) {
      zt = load_one<DT>(row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj), x);
      zd = load_one<DT>(row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj), x);
    }
    a.tok_aux[i] = TokenAux{zt, zd, accept_log_u(a.seed, a.pos0, b, j, chain)};
  }
}

// Persistent workgroups (one per CU) walk the chunks of the flattened stream
// round robin (workgroup g owns chunks g, g + G, g + 2G, ...; its wavefronts
// claim them in order), so at any moment the grid reads one moving window of
// the rows. A chunk's loads are all issued before any is used. Sampled rows: chunk maximum M and s = sum 2^((z - M) * k2);
// greedy rows: maximum and lowest argmax; ARGMAX_ALL: argmax of sampled rows too.
template <int DT, bool VEC, bool ARGMAX_ALL, bool TAIL>
__global__ __launch_bounds__(kStreamBlock) void stream_kernel(StreamArgs a) {
  __shared__ SampledTable tab;
  __shared__ uint32_t s_claim;
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  constexpr int CL = chunk_lanes<DT>();
  const RowSet& rs = a.rs;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t BP = rs.B * rs.P;
  const int64_t KG = rs.K * rs.G;
  const int nchunks = int((rs.B + 63) / 64);
  int64_t nrows = a.nrows;
  const int64_t nblk = int64_t(gridDim.x) - (a.tok_aux ? 1 : 0);  // streaming workgroups
  if (a.tok_aux && int64_t(blockIdx.x) == nblk) {
    gather_tokens<DT>(a);
    return;
  }
  if (threadIdx.x == 0) s_claim = 0u;
  for (int64_t i = int64_t(blockIdx.x) * kStreamBlock + threadIdx.x; i < a.nclear;
       i += nblk * kStreamBlock)
    a.clear[i] = 0u;
  __syncthreads();
  if (a.compact) {
    build_sampled_table(rs.temp, rs.B, tab);
    nrows = BP + int64_t(tab.pref[nchunks]) * KG;
    if (blockIdx.x == 0 && a.rank_out) {
      for (int64_t b = threadIdx.x; b < rs.B; b += kStreamBlock) {
        const int c = int(b >> 6);
        a.rank_out[b] = tab.pref[c] + __popcll(tab.mask[c] & ((1ull << (b & 63)) - 1ull));
      }
      if (threadIdx.x == 0) a.rank_out[rs.B] = tab.pref[nchunks];
    }
  }
  const int64_t cv = int64_t(kWave) * CL;
  const int64_t total = nrows * a.cpr;
  const bool v_tail = (a.V % kVec) != 0;
  const uint32_t i0 = TAIL ? full_windows(total, a.win_scale) : UINT32_MAX;
  // the workgroup's wavefronts claim its chunks in order
  uint32_t claim = 0;
  if (lane == 0) claim = atomicAdd(&s_claim, 1u);
  int64_t c = claimed_chunk<TAIL>(__builtin_amdgcn_readfirstlane(claim), nblk, i0);
  while (c < total) {
    uint32_t next = 0;
    if (lane == 0) next = atomicAdd(&s_claim, 1u);  // the next claim, answered during the loads
    const int64_t rho = fast_div(uint32_t(c), a.by_cpr);
    const int64_t v0 = (c - rho * a.cpr) * cv;
    const int64_t v1 = v0 + cv < a.vpr ? v0 + cv : a.vpr;
    const void* row;
    int64_t b;
    int64_t slot = rho;  // partials sit by batch row: target rows, then draft rows (b, k, j)
    bool is_draft, unit_ok;
    if (rho < BP) {
      b = fast_div(uint32_t(rho), a.by_p);
      const int64_t j = rho - b * rs.P;
      row = row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj);
      is_draft = false;
      unit_ok = sv_ok(b < rs.B && j < rs.P);
    } else {
      const int64_t d = rho - BP;
      const int64_t sidx = fast_div(uint32_t(d), a.by_kg);
      b = a.compact ? select_sampled(tab, nchunks, sidx) : sidx;
      const int64_t rem = d - sidx * KG;
      const int64_t k = fast_div(uint32_t(rem), a.by_g);
      const int64_t j = rem - k * rs.G;
      row = row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj);
      is_draft = true;
      slot = BP + b * KG + rem;
      unit_ok = sv_ok(b < rs.B && k < rs.K && j < rs.G);
    }
    unit_ok = unit_ok && sv_ok(slot < BP + rs.B * KG && c - rho * a.cpr < a.cpr && v0 < v1);
    // In compact mode every streamed draft row belongs to a sampled batch row,
    // so the chunk's loads go out before the temperature arrives; otherwise a
    // greedy row's draft logits are skipped, never read.
    const bool skip = !unit_ok || (is_draft && !a.compact && !(rs.temp[b] > 0.0f));
    RowPartial out{-INFINITY, INT_MAX, 0.0};
    if (!skip) {
      RawVec<DT> r[CL];
#pragma unroll
      for (int u = 0; u < CL; ++u) {
        const int64_t vi = v0 + lane + int64_t(kWave) * u;
        if (vi >= v1) r[u] = neg_inf_vec<DT>();
        else if (v_tail && vi == a.vpr - 1) r[u] = load_vec_bounded<DT, VEC>(row, vi, a.V);
        else r[u] = load_vec<DT, VEC, true>(row, vi);
      }
      const float T = rs.temp[b];
      const bool sampled = T > 0.0f;
      float am = -INFINITY;
      int32_t ai = INT_MAX;
      uint32_t nan_seen = 0;  // greedy rows: a NaN anywhere in the chunk
      if (!sampled || ARGMAX_ALL) {
#pragma unroll
        for (int u = 0; u < CL; ++u) nan_seen |= nan_bits<DT>(r[u]);
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int q = 0; q < kVec; ++q) {
            const float x = vec_elem<DT>(r[u], q);
            if (x > am) {
              am = x;
              ai = int32_t((v0 + lane + int64_t(kWave) * u) * kVec + q);
            }
          }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
          const float om = __shfl_xor(am, off, kWave);
          const int32_t oi = __shfl_xor(ai, off, kWave);
          better_max(am, ai, om, oi);
        }
      }
      if (sampled) {
        const float k2 = kLog2e / T;
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int q = 0; q < kVec; ++q) m = fmaxf(m, vec_elem<DT>(r[u], q));
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        // re-read the raw words below rather than keep 64 unpacked values live
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int i = 0; i < (DT == SV_BF16 ? 4 : 8); ++i) asm volatile("" : "+v"(r[u].w[i]));
        double sum = 0.0;
        if (m != -INFINITY) {
          // 2^(z*k2 - c) with c = float(m*k2); d = m*k2 - c exactly (fma), and
          // 2^((z - m)*k2) = 2^(z*k2 - c) * 2^(-d) with |d| < 1e-4: 1 - d ln 2.
          const float c = m * k2;
          const float d = fmaf(m, k2, -c);
#pragma unroll
          for (int u = 0; u < CL; ++u) {
            float sv = 0.0f;
#pragma unroll
            for (int q = 0; q < kVec; ++q)
              sv += __builtin_amdgcn_exp2f(fmaf(vec_elem<DT>(r[u], q), k2, -c));
            sum += double(sv);
          }
#pragma unroll
          for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
          sum *= 1.0 - double(d) * 0.69314718055994530942;
        } else {
          // every entry -inf or NaN (fmaxf passes NaN by): carry a NaN in the sum
#pragma unroll
          for (int u = 0; u < CL; ++u) nan_seen |= nan_bits<DT>(r[u]);
          if (__ballot(nan_seen != 0)) sum = NAN;
        }
        out = RowPartial{m, ai, sum};
      } else {
        out = RowPartial{am, ai, __ballot(nan_seen != 0) ? double(NAN) : 0.0};
      }
    }
    if (lane == 0 && unit_ok) a.part[slot * a.cpr + (c - rho * a.cpr)] = out;
    c = claimed_chunk<TAIL>(__builtin_amdgcn_readfirstlane(next), nblk, i0);
  }
}

// ln Z and argmax of every row (specverify_normalize): eight lanes per row, the
// same fold and reduction order as the draws' prologue, so both give a row the
// same bits. Rows number fewer than 2^31 (the stream's chunk limit).
constexpr int kFinBlock = 256;

__global__ __launch_bounds__(kFinBlock) void finalize_rows_kernel(const RowPartial* __restrict__ part,
                                                                  int64_t nrows, int64_t cpr, int64_t P,
                                                                  const float* __restrict__ temp,
                                                                  double* __restrict__ lnz,
                                                                  int32_t* __restrict__ amax) {
  const int64_t rho = int64_t(blockIdx.x) * (kFinBlock / kRowLanes) + threadIdx.x / kRowLanes;
  const int gl = threadIdx.x % kRowLanes;
  const bool has = rho < nrows;
  const float T = has ? temp[uint32_t(rho) / uint32_t(P)] : 1.0f;
  float m;
  int32_t idx;
  double s;
  group_fold(part, rho, has, cpr, gl, T > 0.0f, double(kLog2e / T), m, idx, s);
  const RowStat st = group_reduce_row(m, idx, s, T);
  if (has && gl == 0) {
    lnz[rho] = st.lnz;
    if (amax) amax[rho] = st.idx == INT_MAX ? 0 : st.idx;
  }
}

// ---------------------------------------------------------------------------
// Hand-offs between workgroups of one launch: data are published with relaxed
// agent-scope atomic stores, which gfx950 writes through to the device
// coherence point, and read with relaxed agent-scope atomic loads, which read
// the coherent copy; the publisher waits for its stores to be acknowledged
// (vmcnt = 0) before the counter bump that announces them, and the reader
// loads only after its own bump has returned. The memory model's
// release/acquire on the bump would add an L2 write-back before it and an L2
// invalidate after it; the invalidate drops the rows that the XCD's other
// workgroups are scanning (17 us more per step at B=64, gamma=8, V=128256).
__device__ __forceinline__ void pub64(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t bump32(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wavefront's earlier memory operations have completed.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void pub_cand(Cand* p, const Cand& c) {
  pub64(p, uint64_t(__double_as_longlong(c.score)));
  pub64(reinterpret_cast<char*>(p) + 8, uint64_t(uint32_t(c.id)));
}
__device__ __forceinline__ Cand get_cand(const Cand* p) {
  const uint64_t a = get64(p);
  const uint64_t b = get64(reinterpret_cast<const char*>(p) + 8);
  return Cand{__longlong_as_double(int64_t(a)), int32_t(uint32_t(b)), 0};
}

// ---------------------------------------------------------------------------
__device__ __forceinline__ bool cand_less(float ka, int32_t ia, float kb, int32_t ib) {
  return ka < kb || (ka == kb && ia < ib);
}

// The best two of two sorted pairs, by selects only (no branches, so the
// pair stays in registers).
__device__ __forceinline__ Top2 top2_merge(const Top2& a, const Top2& b) {
  const bool bf = cand_less(b.k1, b.i1, a.k1, a.i1);  // b holds the overall best
  Top2 r;
  r.k1 = bf ? b.k1 : a.k1;
  r.i1 = bf ? b.i1 : a.i1;
  r.t1 = bf ? b.t1 : a.t1;
  r.d1 = bf ? b.d1 : a.d1;
  // second: the loser's best against the winner's second
  const float xk = bf ? a.k1 : b.k1, yk = bf ? b.k2 : a.k2;
  const int32_t xi = bf ? a.i1 : b.i1, yi = bf ? b.i2 : a.i2;
  const float xt = bf ? a.t1 : b.t1, yt = bf ? b.t2 : a.t2;
  const float xd = bf ? a.d1 : b.d1, yd = bf ? b.d2 : a.d2;
  const bool xs = cand_less(xk, xi, yk, yi);
  r.k2 = xs ? xk : yk;
  r.i2 = xs ? xi : yi;
  r.t2 = xs ? xt : yt;
  r.d2 = xs ? xd : yd;
  return r;
}

// A scan's running best two, each candidate packed into one double: the key's
// float bits above the id. Keys are +inf or positive normal floats (E_v is at
// least -log2(1 - 2^-24) and w_v at most about 1, so a key exceeds 8e-8), which
// makes every packed value a finite normal double, and doubles of positive sign
// order as their bit patterns do: by key, then by id. Keeping the best two is
// then three float64 min/max instructions per id, and the logits of the two
// that survive the wavefront's merge are read again from the row (with_logits).
struct Best2 {
  double c1, c2;  // c1 <= c2
};

__device__ __forceinline__ double cand_pack(float key, int32_t id) {
  return __hiloint2double(__float_as_int(key), id);
}
__device__ __forceinline__ int32_t cand_id(double c) { return __double2loint(c); }
__device__ __forceinline__ float cand_key(double c) { return __int_as_float(__double2hiint(c)); }

__device__ __forceinline__ Best2 best2_empty() {
  const double e = cand_pack(INFINITY, INT_MAX);
  return Best2{e, e};
}

__device__ __forceinline__ void best2_push(Best2& s, double c) {
  s.c2 = fmin(s.c2, fmax(s.c1, c));
  s.c1 = fmin(s.c1, c);
}

__device__ __forceinline__ void best2_merge(Best2& v, double o1, double o2) {
  v.c2 = fmin(fmax(v.c1, o1), fmin(v.c2, o2));
  v.c1 = fmin(v.c1, o1);
}

// The wavefront's best two in every lane: DPP inside each row of 16 lanes,
// then the four rows' results read from lanes 0, 16, 32 and 48.
__device__ __forceinline__ Best2 wave_best2(Best2 v) {
  best2_merge(v, dpp64<kDppXor1>(v.c1), dpp64<kDppXor1>(v.c2));
  best2_merge(v, dpp64<kDppXor2>(v.c1), dpp64<kDppXor2>(v.c2));
  best2_merge(v, dpp64<kDppHalfMirror>(v.c1), dpp64<kDppHalfMirror>(v.c2));
  best2_merge(v, dpp64<kDppMirror>(v.c1), dpp64<kDppMirror>(v.c2));
  Best2 w{readlane64(v.c1, 0), readlane64(v.c2, 0)};
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r) best2_merge(w, readlane64(v.c1, 16 * r), readlane64(v.c2, 16 * r));
  return w;
}

// The wavefront's best (float64 score, id) in every lane: the highest score,
// ties to the lowest id (order-free, so DPP inside rows, then the rows).
__device__ __forceinline__ void cand_better(double& bs, int32_t& id, double ob, int32_t oi) {
  if (ob > bs || (ob == bs && oi < id)) {
    bs = ob;
    id = oi;
  }
}
__device__ __forceinline__ void wave_best_cand(double& bs, int32_t& id) {
  cand_better(bs, id, dpp64<kDppXor1>(bs), int32_t(dpp32<kDppXor1>(uint32_t(id))));
  cand_better(bs, id, dpp64<kDppXor2>(bs), int32_t(dpp32<kDppXor2>(uint32_t(id))));
  cand_better(bs, id, dpp64<kDppHalfMirror>(bs), int32_t(dpp32<kDppHalfMirror>(uint32_t(id))));
  cand_better(bs, id, dpp64<kDppMirror>(bs), int32_t(dpp32<kDppMirror>(uint32_t(id))));
  double wb = readlane64(bs, 0);
  int32_t wi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 1; r < kWave / 16; ++r)
    cand_better(wb, wi, readlane64(bs, 16 * r), __builtin_amdgcn_readlane(id, 16 * r));
  bs = wb;
  id = wi;
}

// The wavefront's best two (every lane holds them) with their target and draft
// logits, read again from the rows by lanes 0 and 1; ids past the row (a
// partial last vector) read -inf, as the scan saw them. Valid in every lane.
template <int DT>
__device__ __forceinline__ Top2 with_logits(const Best2& b, const void* row_t, const void* row_d,
                                            bool residual, int64_t V) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t id = cand_id(lane == 0 ? b.c1 : b.c2);
  float zt = -INFINITY, zd = -INFINITY;
  if (lane < 2 && id < V) {
    zt = load_one<DT>(row_t, id);
    if (residual) zd = load_one<DT>(row_d, id);
  }
  auto lane_f = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return Top2{cand_key(b.c1), cand_id(b.c1), lane_f(zt, 0), lane_f(zd, 0),
              cand_key(b.c2), cand_id(b.c2), lane_f(zt, 1), lane_f(zd, 1)};
}

// What a scan needs to know about the draw.
struct DrawParams {
  float k2;     // log2(e) / T
  float L2t;    // ln Z of the target row, in log2 units
  float D2;     // (ln Z_t - ln Z_d) in log2 units (residual draws)
  uint32_t pos, r, s0, s1;
};

// Exponential-race keys of the 8 ids of vector vi: key_v = E_v / w_v with
// E_v = -log2 u_v (a constant factor ln 2 does not move the argmin) and w_v
// the unnormalised weight, 2^(z_t*k2 - L2t) = p_v for the bonus draw, and
// p_v - q_v with q_v = p_v * 2^((z_d - z_t)*k2 + D2) for the residual draw.
// Ids >= V (a row's last, partial vector) hold -inf logits (load_vec_bounded),
// so their weight is 0 or NaN and their key +inf.
template <int DT, bool RESIDUAL>
__device__ __forceinline__ void score_vec(const RawVec<DT>& rt, const RawVec<DT>& rd, int64_t vi,
                                          const DrawParams& dp, Best2& best) {
  const uint32_t c0 = uint32_t(vi * 2);
  const Philox4 lo = philox4x32_10(c0, dp.pos, dp.r, kPurposeSample, dp.s0, dp.s1);
  const Philox4 hi = philox4x32_10(c0 + 1u, dp.pos, dp.r, kPurposeSample, dp.s0, dp.s1);
#pragma unroll
  for (int t = 0; t < kVec; ++t) {
    const float zt = vec_elem<DT>(rt, t);
    const float zd = RESIDUAL ? vec_elem<DT>(rd, t) : 0.0f;
    const float a2 = fmaf(zt, dp.k2, -dp.L2t);
    float w = __builtin_amdgcn_exp2f(a2);
    if constexpr (RESIDUAL) w -= __builtin_amdgcn_exp2f(a2 + fmaf(zd - zt, dp.k2, dp.D2));
    const uint32_t word = t < 4 ? lo.w[t] : hi.w[t - 4];
    const float e2 = -__builtin_amdgcn_logf(unit_uniform(word));
    // w <= 0 (and NaN, from -inf logits) give +inf: rcp(+0) = +inf and e2 > 0
    const float key = e2 * __builtin_amdgcn_rcpf(fmaxf(w, 0.0f));
    best2_push(best, cand_pack(key, int32_t(vi * kVec + t)));
  }
}

// score_vec with an exact filter. -ln u >= 1 - u and w_v <= p_v give
// key_v >= (1 - u_v) / (ln 2 * p_v); an id is skipped only when that bound,
// less a relative 1e-5 that covers the float rounding of both sides (a few
// units in the last place), still exceeds thr, a key that two candidates of
// one lane already beat, so it cannot enter the wave's best two. The log, the
// draft term, the reciprocal and the insertion run only for ids some lane of
// the wave keeps; a kept id's key is computed exactly as in score_vec.
template <int DT, bool RESIDUAL>
__device__ __forceinline__ void score_vec_filtered(const RawVec<DT>& rt, const RawVec<DT>& rd,
                                                   int64_t vi, const DrawParams& dp, float thr,
                                                   Best2& best) {
  const uint32_t c0 = uint32_t(vi * 2);
  const Philox4 lo = philox4x32_10(c0, dp.pos, dp.r, kPurposeSample, dp.s0, dp.s1);
  const Philox4 hi = philox4x32_10(c0 + 1u, dp.pos, dp.r, kPurposeSample, dp.s0, dp.s1);
  const float bound = thr * (0.69314718f * (1.0f + 1e-5f));
#pragma unroll
  for (int t = 0; t < kVec; ++t) {
    const float zt = vec_elem<DT>(rt, t);
    const float a2 = fmaf(zt, dp.k2, -dp.L2t);
    const float p = __builtin_amdgcn_exp2f(a2);
    const uint32_t word = t < 4 ? lo.w[t] : hi.w[t - 4];
    const float u = unit_uniform(word);
    const bool keep = !(1.0f - u > bound * p);
    if (__ballot(keep)) {
      if (keep) {
        const float zd = RESIDUAL ? vec_elem<DT>(rd, t) : 0.0f;
        float w = p;
        if constexpr (RESIDUAL) w -= __builtin_amdgcn_exp2f(a2 + fmaf(zd - zt, dp.k2, dp.D2));
        const float e2 = -__builtin_amdgcn_logf(u);
        const float key = e2 * __builtin_amdgcn_rcpf(fmaxf(w, 0.0f));
        best2_push(best, cand_pack(key, int32_t(vi * kVec + t)));
      }
    }
  }
}

// Float64 re-score of a block's best two, ln w_v + G_v with G_v = -ln(-ln u_v)
// (w_v = p_v - q_v, or p_v for the bonus draw), by lanes 0-3 of the calling
// wavefront; every lane returns the winner (score -inf and id INT_MAX if none).
__device__ __forceinline__ Cand rescore_top2(const Top2& all, bool residual, double T, double lzt,
                                             double lzd, uint32_t pos, uint32_t r, uint32_t s0,
                                             uint32_t s1) {
  // Four lanes: 0 and 1 take -ln u of the two candidates, 2 and 3 their
  // residual factor 1 - exp(lq - lp) (1 for the bonus draw, 0 off the
  // support) and ln p; then one logarithm in all four gives G = -ln(-ln u)
  // and ln(1 - q/p), and each score is ln p + ln(1 - q/p) + G: the same
  // operations in the same order as one lane per candidate doing both chains
  // (same outputs), with one logarithm less on the way (B=64 gamma=8
  // V=128256: 65.9 vs 66.5 us per step; B=1 gamma=4 V=32000: 15.1 vs 15.5).
  const int lane = threadIdx.x & (kWave - 1);
  const bool second = (lane & 1) != 0;
  const int32_t v = second ? all.i2 : all.i1;
  const bool valid = !(v < 0 || v == INT_MAX);
  double y = 1.0, lp = 0.0;
  if (lane < 4 && valid) {
    if (lane < 2) {
      const Philox4 blk = philox4x32_10(uint32_t(v) >> 2, pos, r, kPurposeSample, s0, s1);
      const uint32_t k = uint32_t(v) & 3u;
      const uint32_t word = k == 0u ? blk.w[0] : k == 1u ? blk.w[1] : k == 2u ? blk.w[2] : blk.w[3];
      // u - 1 is exact for every u here ((k + 1/2) 2^-23: 24 significant
      // bits), so log1p keeps full accuracy over the whole range and both
      // lanes take one path (B=256 gamma=4 V=151936: 119.9 vs 120.3 us)
      y = -log1p(unit_uniform_d(word) - 1.0);
    } else {
      lp = double(second ? all.t2 : all.t1) / T - lzt;
      if (residual) {
        const double lq = double(second ? all.d2 : all.d1) / T - lzd;
        const double dd = lq - lp;
        y = dd < 0.0 ? -expm1(dd) : 0.0;
      }
    }
  }
  const double ly = log(y);
  const bool v1 = !(all.i1 < 0 || all.i1 == INT_MAX), v2 = !(all.i2 < 0 || all.i2 == INT_MAX);
  const double sc1 = v1 ? (residual ? readlane64(lp, 2) + readlane64(ly, 2) : readlane64(lp, 2)) -
                              readlane64(ly, 0)
                        : -INFINITY;
  const double sc2 = v2 ? (residual ? readlane64(lp, 3) + readlane64(ly, 3) : readlane64(lp, 3)) -
                              readlane64(ly, 1)
                        : -INFINITY;
  Cand c{sc1, all.i1, 0};
  if (sc2 > sc1 || (sc2 == sc1 && all.i2 < all.i1)) c = Cand{sc2, all.i2, 0};
  if (c.score == -INFINITY) c.id = INT_MAX;
  return c;
}

// Scan one split of the row pair (residual: target and draft row n; else the
// target row alone). Each wavefront takes a contiguous quarter of the split and
// lane l reads vectors vi0 + kWave*it (it < kSampleIters), so the loads of a
// lane share one address and differ by immediate offsets; all of them are
// issued before any is scored, and the scoring loop is not unrolled (it walks
// a window of registers that shifts by one vector per pass).
//
// When no vector of the split is partial (every split when V is a multiple of
// 8, else all but the row's last), the loads are issued unconditionally (lanes
// past the row load the row's last vector and never score it) and the scoring
// is unrolled, so vector it waits only for its own loads and the arithmetic of
// the first vectors overlaps the arrival of the later ones. FILTER: after every
// other vector the wavefront's smallest second-best key bounds the ids worth scoring
// (score_vec_filtered); it pays where the draws are bound by arithmetic (grids
// of several rounds) and costs latency where a single round of workgroups is
// bound by its dependent steps.
template <int DT, bool VEC, bool RESIDUAL, bool FILTER, int SI, bool ACC = false>
__device__ __forceinline__ Best2 scan_split(const void* row_t, const void* row_d, int64_t split,
                                           int64_t V, const DrawParams& dp,
                                           const Best2& init = best2_empty()) {
  constexpr int64_t kSplitVecs = int64_t(kBlock) * SI;  // vectors per split
  const int64_t vpr = (V + kVec - 1) / kVec;
  const int64_t vi0 = split * kSplitVecs +
                      int64_t(threadIdx.x / kWave) * (kWave * SI) + (threadIdx.x & (kWave - 1));
  const bool whole = VEC && (V % kVec == 0 || (split + 1) * kSplitVecs < vpr);
  if (whole) {
    RawVec<DT> wt[SI], wd[SI];
#pragma unroll
    for (int it = 0; it < SI; ++it) {
      const int64_t vi = vi0 + int64_t(kWave) * it;
      const int64_t vc = vi < vpr ? vi : vpr - 1;
      wt[it] = load_vec<DT, true>(row_t, vc);
      if constexpr (RESIDUAL) wd[it] = load_vec<DT, true>(row_d, vc);
    }
    Best2 best = ACC ? init : best2_empty();
    if constexpr (FILTER) {
      // two keys of one lane are at most thr (ACC: the earlier splits' too)
      float thr = ACC ? wave_min(cand_key(best.c2)) : INFINITY;
#pragma unroll
      for (int it = 0; it < SI; ++it) {
        const int64_t vi = vi0 + int64_t(kWave) * it;
        if (vi < vpr)
          score_vec_filtered<DT, RESIDUAL>(wt[it], RESIDUAL ? wd[it] : wt[it], vi, dp, thr, best);
        // after every other vector: an older bound is still a bound, and the
        // reduction costs more than the tighter one saves (B=512 K=4 gamma=8:
        // 1113.5 vs 1116.9 us per step; every vector or every fourth: no better)
        if ((it & 1) == 0 && it + 1 < SI) thr = wave_min(cand_key(best.c2));
      }
    } else {
#pragma unroll
      for (int it = 0; it < SI; ++it) {
        const int64_t vi = vi0 + int64_t(kWave) * it;
        if (vi < vpr) score_vec<DT, RESIDUAL>(wt[it], RESIDUAL ? wd[it] : wt[it], vi, dp, best);
      }
    }
    return best;
  }
  RawVec<DT> rt[SI], rd[SI];
#pragma unroll
  for (int it = 0; it < SI; ++it) {
    const int64_t vi = vi0 + int64_t(kWave) * it;
    const bool inside = vi < vpr;
    rt[it] = inside ? load_vec_bounded<DT, VEC>(row_t, vi, V) : neg_inf_vec<DT>();
    rd[it] = inside && RESIDUAL ? load_vec_bounded<DT, VEC>(row_d, vi, V) : rt[it];
  }
  Best2 best = ACC ? init : best2_empty();
#pragma unroll 1
  for (int it = 0; it < SI; ++it) {
    const int64_t vi = vi0 + int64_t(kWave) * it;
    if (vi < vpr) score_vec<DT, RESIDUAL>(rt[0], rd[0], vi, dp, best);
#pragma unroll
    for (int q = 0; q + 1 < SI; ++q) {
      rt[q] = rt[q + 1];
      rd[q] = rd[q + 1];
    }
  }
  return best;
}

// The token drawn from p (target row at ln Z = lzt) by one wavefront over the
// whole row: the fallback for an empty residual support, which only rounding
// can produce (cold code: never fetched unless taken). Every lane returns the
// id (INT_MAX if the row has no candidate).
template <int DT, bool VEC>
__device__ __forceinline__ int32_t draw_from_p(const void* row_t, int64_t V, double T, double lzt,
                                            DrawParams dp) {
  const int lane = threadIdx.x & (kWave - 1);
  dp.D2 = 0.0f;
  const int64_t vpr = (V + kVec - 1) / kVec;
  Best2 fb = best2_empty();
  for (int64_t vi = lane; vi < vpr; vi += kWave) {
    const RawVec<DT> pt = load_vec_bounded<DT, VEC>(row_t, vi, V);
    score_vec<DT, false>(pt, pt, vi, dp, fb);
  }
  const Top2 all = with_logits<DT>(wave_best2(fb), row_t, row_t, false, V);
  const int32_t id = rescore_top2(all, false, T, lzt, 0.0, dp.pos, dp.r, dp.s0, dp.s1).id;
  return __builtin_amdgcn_readlane(id, 0);
}

struct ChainArgs {
  RowSet rs;
  int64_t V;
  const RowPartial* part;    // stream chunk partials by batch-row slot
  int64_t cpr;               // chunks per row
  const int32_t* tokens;     // [B, K, G]
  const TokenAux* tok_aux;   // [B, K, G], from the stream kernel's token gather
  uint64_t seed;
  const int64_t* pos0;
  // outputs (split 0 of the draw kernel's chain; out_token of a sampled chain: its last split)
  int32_t* accept_len;
  int32_t* out_token;
  float* logp;
  float* logq;
  double* lnz_t_out;
  double* lnz_d_out;
  int32_t* dev_err;
  // given-n mode (specverify_residual_sample)
  const double* lnz_t_in;    // [B, G+1]
  const double* lnz_d_in;    // [B, K, G]
  const int32_t* amax_in;    // [B, G+1]
  const int32_t* n_in;       // [B, K]
  // draw kernel (split 0) or given_kernel -> (finish kernel)
  int64_t nsplit;
  Cand* cand;                // [B*K][nsplit]
  ChainInfo* info;           // [B*K]
  uint32_t* cnt;             // [B*K] splits done per chain, or null: finish_kernel picks the token
  // workgroup -> (chain, split) and chain -> (b, k) as multiply-shifts (B*K*nsplit < 2^31);
  // the fused draw kernel divides in 32 bits instead (measured faster there)
  FastDiv by_nsplit, by_k;
};

// specverify_residual_sample: one thread per chain turns the given n and
// normalisers into the draw kernel's ChainInfo (greedy rows: the token is the
// target row's argmax at n).
__global__ __launch_bounds__(kBlock) void given_kernel(ChainArgs a, int64_t chains) {
  const int64_t chain = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (chain >= chains) return;
  const RowSet& rs = a.rs;
  const int64_t b = fast_div(uint32_t(chain), a.by_k);
  const int G = int(rs.G);
  const int P = G + 1;
  const float T = rs.temp[b];
  const bool sampled = T > 0.0f;
  if (a.cnt) a.cnt[chain] = 0u;  // the draw launch counts this chain's splits from zero
  const int32_t n0 = a.n_in[chain];
  const int n = (n0 < 0 || n0 > G) ? -1 : n0;
  if (T == 0.0f && n >= 0) a.out_token[chain] = a.amax_in[b * P + n];
  ChainInfo ci;
  ci.n = (n >= 0 && sampled) ? n : -1;
  ci.lzt = n >= 0 ? a.lnz_t_in[b * P + n] : 0.0;
  ci.lzd = (n >= 0 && n < G && sampled) ? a.lnz_d_in[chain * G + n] : 0.0;
  ci.pad[0] = ci.pad[1] = ci.pad[2] = 0;
  a.info[chain] = ci;
}

// Per-chain prologue of the step's draw kernel: every split of a chain derives
// the chain's n itself, so no separate accept launch sits between the stream
// and the draws. The rows' ln Z come from the stream partials with 8 lanes per
// row (up to 32 rows per pass of the workgroup, a 3-step reduction per row,
// in the order of group_fold and group_reduce_row, written out here so the
// draft-token logits load while the partials fold). Split 0 writes the
// chain's outputs. Returns n in LDS (-1: nothing to draw or an error).
constexpr int kRowsPerPass = kBlock / kRowLanes;

template <int DT>
__device__ void chain_prologue(const ChainArgs& a, int64_t chain, bool lead, double* s_lnz,
                               int32_t* s_amax, int32_t* s_rowbad, int32_t* s_n) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  const RowSet& rs = a.rs;
  const int64_t b = int64_t(uint32_t(chain) / uint32_t(rs.K));
  const int64_t k = chain - b * rs.K;
  const int G = int(rs.G);
  const int P = G + 1;
  const int t = threadIdx.x;
  if (!sv_ok(chain < rs.B * rs.K)) {  // uniform in the workgroup
    if (t == 0) *s_n = -1;
    __syncthreads();
    return;
  }
  const float T = rs.temp[b];
  const bool sampled = T > 0.0f;
  const bool greedy = T == 0.0f;
  const double k2 = double(kLog2e / T);
  // The draft tokens, the logits at them and the accept uniforms (gathered by
  // the stream kernel when tok_aux is set, else loaded and drawn here) go
  // through the last wavefront, whose loads then wait on nothing of the
  // partials' (it folds rows only when a chain has more than 24 rows); LDS
  // hands them over.
  __shared__ int32_t s_tok[SV_MAX_GAMMA];
  __shared__ float s_zt[SV_MAX_GAMMA], s_zd[SV_MAX_GAMMA];
  __shared__ double s_logu[SV_MAX_GAMMA];
  constexpr int kTokWave = (kBlock / kWave - 1) * kWave;
  if (t >= kTokWave && t - kTokWave < G) {
    const int j = t - kTokWave;
    const int32_t x = a.tokens[chain * G + j];
    TokenAux q{0.0f, 0.0f, 0.0};
    if (a.tok_aux) {
      q = a.tok_aux[chain * G + j];
    } else {
      if (!(x < 0 || int64_t(x) >= a.V) && sampled) {
        q.zt = load_one<DT>(row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj), x);
        q.zd = load_one<DT>(row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj), x);
      }
      q.log_u = accept_log_u(a.seed, a.pos0, b, j, chain);
    }
    s_tok[j] = x;
    s_zt[j] = q.zt;
    s_zd[j] = q.zd;
    s_logu[j] = q.log_u;
  }
  const int grp = t / kRowLanes;
  const int gl = t % kRowLanes;
  const int nr = P + (sampled ? G : 0);
  int32_t bad = 0;
  for (int base = 0; base < nr; base += kRowsPerPass) {
    const int ri = base + grp;
    const bool has = ri < nr;
    const int64_t rho = !has ? 0 : ri < P ? b * P + ri : rs.B * P + chain * G + (ri - P);
    float m = -INFINITY;
    int32_t idx = INT_MAX;
    double s = 0.0;
    for (int64_t c0 = gl; c0 < a.cpr; c0 += 4 * kRowLanes) {
      RowPartial q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + int64_t(u) * kRowLanes;
        q[u] = (has && c < a.cpr) ? a.part[rho * a.cpr + c] : RowPartial{-INFINITY, INT_MAX, 0.0};
      }
      // a sampled row needs the maximum alone (the same value), a greedy one
      // its lowest argmax too
      if (sampled) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float bm = fmaxf(m, q[u].m);
          if (bm > -INFINITY && m > -INFINITY) s *= exp2_scale((double(m) - double(bm)) * k2);
          s += q[u].m > -INFINITY ? q[u].s * exp2_scale((double(q[u].m) - double(bm)) * k2) : q[u].s;
          m = bm;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) fold_partial(m, idx, s, q[u], sampled, k2);
      }
    }
    // combine the 8 lanes of each row in a fixed order
    float M = m;
    int32_t I = idx;
    if (sampled) {
      M = fmaxf(M, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(M))));
      M = fmaxf(M, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(M))));
      M = fmaxf(M, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(M))));
    } else {
      group8_argmax(M, I);
    }
    double sr = (sampled && M > -INFINITY && m > -INFINITY) ? s * exp2_scale((double(m) - double(M)) * k2) : s;
    sr = group8_sum(sr);
    if (has && gl == 0) {
      const double lnz = row_lnz(M, sr, T);
      s_lnz[ri] = lnz;
      if (row_bad(M, sr)) bad = SV_ERR_ROW;
      if (ri < P) {
        s_amax[ri] = I == INT_MAX ? 0 : I;
        if (lead && k == 0 && a.lnz_t_out) a.lnz_t_out[b * P + ri] = lnz;
      } else if (lead && a.lnz_d_out) {
        a.lnz_d_out[chain * G + (ri - P)] = lnz;
      }
    }
  }
  if (gl == 0) s_rowbad[grp] = bad;
  __syncthreads();
  // accept tests of the G positions in wavefront 0, first rejection by ballot
  if (t < kWave) {
    bool acc = false;
    bool tok_bad = false;
    if (t < G) {
      const int j = t;
      const int32_t x = s_tok[j];
      tok_bad = x < 0 || int64_t(x) >= a.V;
      double lp = 0.0, lq = 0.0;
      if (!tok_bad) {
        if (sampled) {
          lp = double(s_zt[j]) / double(T) - s_lnz[j];
          lq = double(s_zd[j]) / double(T) - s_lnz[P + j];
          acc = s_logu[j] < lp - lq;
        } else if (greedy) {
          acc = x == s_amax[j];
          lp = acc ? 0.0 : -INFINITY;
          lq = 0.0;
        }
      }
      if (lead && a.logp) a.logp[chain * G + j] = float(lp);
      if (lead && a.logq) a.logq[chain * G + j] = float(lq);
    }
    const uint64_t acc_mask = __ballot(acc);
    const uint64_t bad_mask = __ballot(tok_bad);
    if (t == 0) {
      const int n = __builtin_ctzll(~acc_mask);  // leading accepts (<= G: bit G of ~mask is set)
      int32_t err = 0;
      for (int g = 0; g < kRowsPerPass; ++g) err |= s_rowbad[g];
      if (bad_mask) err |= SV_ERR_TOKEN;
      if (!(sampled || greedy)) err |= SV_ERR_TEMP;
      *s_n = (err || !sampled) ? -1 : n;
      if (lead) {
        if (err) {
          a.accept_len[chain] = -1;
          a.out_token[chain] = -1;
          if (a.dev_err) atomicOr(a.dev_err, err);
        } else {
          a.accept_len[chain] = n;
          if (greedy) a.out_token[chain] = s_amax[n];
        }
        ChainInfo ci;
        ci.n = (!err && sampled) ? n : -1;
        ci.lzt = !err ? s_lnz[n] : 0.0;
        ci.lzd = (!err && sampled && n < G) ? s_lnz[P + n] : 0.0;
        ci.pad[0] = ci.pad[1] = ci.pad[2] = 0;
        a.info[chain] = ci;  // for finish_kernel past the counted chains
      }
    }
  }
  __syncthreads();
}

// The step's accept stage as its own launch, for grids too large to be
// resident at once (then every split repeating the prologue would cost a
// round of latency per dispatch round): one workgroup per chain runs the
// draws' prologue once (the same fold order, so the same ln Z bits) and
// leaves n and the normalisers in ChainInfo for the draw kernel.
template <int DT>
__global__ __launch_bounds__(kBlock) void accept_kernel(ChainArgs a) {
  __shared__ double s_lnz[kMaxRowsPerChain];
  __shared__ int32_t s_amax[SV_MAX_GAMMA + 1];
  __shared__ int32_t s_rowbad[kRowsPerPass];
  __shared__ int32_t s_n;
  chain_prologue<DT>(a, blockIdx.x, true, s_lnz, s_amax, s_rowbad, &s_n);
}

// One workgroup per (chain, split of kSplit ids). FUSED (the step): the
// workgroup derives n and the normalisers itself (chain_prologue); otherwise
// (specverify_residual_sample) it reads them from given_kernel's ChainInfo. At least 4 waves per SIMD: 16 workgroups' worth of waves per CU,
// so the usual grids run in one round.
template <int DT, bool VEC, bool FUSED, int SI>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 8)))
void draw_kernel(ChainArgs a) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  __shared__ Top2 s_top[kWavesPerBlock];
  __shared__ double s_lnz[kMaxRowsPerChain];
  __shared__ int32_t s_amax[SV_MAX_GAMMA + 1];
  __shared__ int32_t s_rowbad[kRowsPerPass];
  __shared__ int32_t s_n;
  const RowSet& rs = a.rs;
  const int64_t chain = FUSED ? int64_t(uint32_t(blockIdx.x) / uint32_t(a.nsplit))
                              : int64_t(fast_div(blockIdx.x, a.by_nsplit));
  const int64_t split = blockIdx.x - chain * a.nsplit;
  const int G = int(rs.G);
  int n;
  double lzt_c, lzd_c;
  if (FUSED) {
    chain_prologue<DT>(a, chain, split == 0, s_lnz, s_amax, s_rowbad, &s_n);
    n = s_n;
    if (n < 0) return;  // uniform across the workgroup: this chain draws nothing
    lzt_c = s_lnz[n];
    lzd_c = n < G ? s_lnz[G + 1 + n] : 0.0;
  } else {
    const ChainInfo ci = a.info[chain];
    n = ci.n;
    if (n < 0) return;
    lzt_c = ci.lzt;
    lzd_c = ci.lzd;
  }
  if (!sv_ok(n <= G && chain < rs.B * rs.K && split < a.nsplit)) return;
  const int64_t b = FUSED ? int64_t(uint32_t(chain) / uint32_t(rs.K)) : int64_t(fast_div(uint32_t(chain), a.by_k));
  const int64_t k = chain - b * rs.K;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const float T = rs.temp[b];

  // Scan this split of the row pair, then re-score its best two in float64.
  const bool residual = n < G;
  const void* row_t = row_ptr(rs.t, esz, b * rs.tsb + int64_t(n) * rs.tsj);
  const void* row_d =
      residual ? row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + int64_t(n) * rs.dsj) : row_t;
  const double lzt = lzt_c;
  const double lzd = residual ? lzd_c : 0.0;
  DrawParams dp;
  dp.k2 = kLog2e / T;
  dp.L2t = float(lzt * kLog2eD);
  dp.D2 = residual ? float((lzt - lzd) * kLog2eD) : 0.0f;
  dp.pos = uint32_t(uint64_t(a.pos0 ? a.pos0[b] : 0) + uint64_t(n));
  dp.r = uint32_t(chain);
  dp.s0 = uint32_t(a.seed);
  dp.s1 = uint32_t(a.seed >> 32);
  // the fused kernel runs one round of workgroups (latency-bound); the
  // separate-accept path serves grids of several rounds
  const Best2 best = residual ? scan_split<DT, VEC, true, !FUSED, SI>(row_t, row_d, split, a.V, dp)
                              : scan_split<DT, VEC, false, !FUSED, SI>(row_t, row_d, split, a.V, dp);
  // the logit loads of the wavefront's best two overlap the wait for the others
  const Top2 wbest = with_logits<DT>(wave_best2(best), row_t, row_d, residual, a.V);
  if (lane == 0) s_top[t / kWave] = wbest;
  __syncthreads();
  if (t >= kWave) return;  // wavefront 0 merges, publishes and, if last, selects
  Top2 all = s_top[0];
  for (int w = 1; w < kWavesPerBlock; ++w) all = top2_merge(all, s_top[w]);
  const Cand c = rescore_top2(all, residual, double(T), lzt, lzd, dp.pos, dp.r, dp.s0, dp.s1);
  uint32_t prev = 0;
  if (lane == 0) {
    if (!a.cnt) {
      a.cand[chain * a.nsplit + split] = c;
    } else {
      pub_cand(a.cand + chain * a.nsplit + split, c);
      stores_done();
      prev = bump32(a.cnt + chain);
    }
  }
  if (!a.cnt || __builtin_amdgcn_readfirstlane(prev) != uint32_t(a.nsplit - 1)) return;
  // The chain's last split picks the token: the best float64 score over the
  // splits (ties to the lowest id); no candidate anywhere means an empty
  // residual support (rounding only), drawn from p_n with the same noise.
  double bs = -INFINITY;
  int32_t id = INT_MAX;
  for (int64_t sp = lane; sp < a.nsplit; sp += kWave) {
    const Cand q = get_cand(a.cand + chain * a.nsplit + sp);
    if (q.score > bs || (q.score == bs && q.id < id)) {
      bs = q.score;
      id = q.id;
    }
  }
  wave_best_cand(bs, id);
  if (id == INT_MAX) id = draw_from_p<DT, VEC>(row_t, a.V, double(T), lzt, dp);
  if (lane == 0) a.out_token[chain] = id == INT_MAX ? -1 : id;
}

// Grids of many chains (after accept_kernel): one workgroup per chain scans
// the chain's whole row pair, split after split, keeping every lane's best two
// (and the filter's bound) across the splits, then merges and re-scores them
// once; no other workgroup takes part, so nothing is handed over.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 8)))
void draw_chain_kernel(ChainArgs a) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  __shared__ Top2 s_top[kWavesPerBlock];
  const RowSet& rs = a.rs;
  const int64_t chain = blockIdx.x;
  const ChainInfo ci = a.info[chain];
  const int n = ci.n;
  const int G = int(rs.G);
  if (n < 0) return;  // uniform: this chain draws nothing
  if (!sv_ok(n <= G && chain < rs.B * rs.K)) return;
  const int64_t b = int64_t(fast_div(uint32_t(chain), a.by_k));
  const int64_t k = chain - b * rs.K;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const float T = rs.temp[b];
  const bool residual = n < G;
  const void* row_t = row_ptr(rs.t, esz, b * rs.tsb + int64_t(n) * rs.tsj);
  const void* row_d =
      residual ? row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + int64_t(n) * rs.dsj) : row_t;
  const double lzt = ci.lzt;
  const double lzd = residual ? ci.lzd : 0.0;
  DrawParams dp;
  dp.k2 = kLog2e / T;
  dp.L2t = float(lzt * kLog2eD);
  dp.D2 = residual ? float((lzt - lzd) * kLog2eD) : 0.0f;
  dp.pos = uint32_t(uint64_t(a.pos0 ? a.pos0[b] : 0) + uint64_t(n));
  dp.r = uint32_t(chain);
  dp.s0 = uint32_t(a.seed);
  dp.s1 = uint32_t(a.seed >> 32);
  const int64_t nsplit = (a.V + kSplit - 1) / kSplit;
  Best2 best = best2_empty();
  for (int64_t sp = 0; sp < nsplit; ++sp)
    best = residual ? scan_split<DT, VEC, true, true, kSampleIters, true>(row_t, row_d, sp, a.V, dp, best)
                    : scan_split<DT, VEC, false, true, kSampleIters, true>(row_t, row_d, sp, a.V, dp, best);
  const Top2 wbest = with_logits<DT>(wave_best2(best), row_t, row_d, residual, a.V);
  if (lane == 0) s_top[t / kWave] = wbest;
  __syncthreads();
  if (t >= kWave) return;
  Top2 all = s_top[0];
  for (int w = 1; w < kWavesPerBlock; ++w) all = top2_merge(all, s_top[w]);
  const Cand c = rescore_top2(all, residual, double(T), lzt, lzd, dp.pos, dp.r, dp.s0, dp.s1);
  int32_t id = c.score == -INFINITY ? INT_MAX : c.id;
  if (id == INT_MAX) id = draw_from_p<DT, VEC>(row_t, a.V, double(T), lzt, dp);
  if (lane == 0) a.out_token[chain] = id == INT_MAX ? -1 : id;
}

// One wavefront per chain: the best float64 score over the splits wins (ties
// to the lowest id). No candidate anywhere means an empty residual support
// (reachable only by rounding): the token is then drawn from p_n with the same
// noise by a pass over the whole row.
template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void finish_kernel(const void* tgt, int64_t tsb, int64_t tsj,
                                                       int64_t K, int64_t G, int64_t V,
                                                       const float* __restrict__ temp,
                                                       uint64_t seed, const int64_t* pos0,
                                                       const ChainInfo* __restrict__ info,
                                                       const Cand* __restrict__ cand,
                                                       int64_t nsplit,
                                                       int32_t* __restrict__ out_token) {
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  const int64_t chain = blockIdx.x;
  const ChainInfo ci = info[chain];
  const int n = ci.n;
  if (n < 0 || !sv_ok(n <= G)) return;
  const int lane = threadIdx.x;
  double best = -INFINITY;
  int32_t id = INT_MAX;
  for (int64_t sp = lane; sp < nsplit; sp += kWave) {
    const Cand c = cand[chain * nsplit + sp];
    if (c.score > best || (c.score == best && c.id < id)) {
      best = c.score;
      id = c.id;
    }
  }
  wave_best_cand(best, id);
  if (id == INT_MAX) {
    const int64_t b = chain / K;
    const float T = temp[b];
    const void* row_t = row_ptr(tgt, esz, b * tsb + int64_t(n) * tsj);
    DrawParams dp;
    dp.k2 = kLog2e / T;
    dp.L2t = float(ci.lzt * kLog2eD);
    dp.D2 = 0.0f;
    dp.pos = uint32_t(uint64_t(pos0 ? pos0[b] : 0) + uint64_t(n));
    dp.r = uint32_t(chain);
    dp.s0 = uint32_t(seed);
    dp.s1 = uint32_t(seed >> 32);
    id = draw_from_p<DT, VEC>(row_t, V, double(T), ci.lzt, dp);
  }
  if (lane == 0) out_token[chain] = id == INT_MAX ? -1 : id;
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
// Acceptance probability alpha_j = sum_v min(p_j(v), q_j(v)) per chain and draft
// position, and the accept-length law P(n = m) = alpha_0..alpha_{m-1} (1 - alpha_m)
// (P(n = gamma) = alpha_0..alpha_{gamma-1}), from the normalisers of a step.

// Per (chain, position, chunk): the chunk's sum of min(p, q) (sampled rows), or
// the chunk maxima and their lowest ids of the target and draft rows (greedy).
struct alignas(8) OverlapPartial {
  double s;
  float mt, md;
  int32_t it, id;
};

struct OverlapArgs {
  RowSet rs;
  int64_t V, vpr, cpr;
  const double* lnz_t;     // [B, G+1]
  const double* lnz_d;     // [B, K, G]
  OverlapPartial* part;    // [(b*K + k)*G + j][cpr]
  FastDiv by_cpr, by_g;    // unit indices are below 2^31 (checked on the host)
};

// One sweep over the target rows 0..G-1 and every draft row. A unit is
// (b, j, chunk): the target chunk is loaded once and kept in registers while
// the K draft chunks of the same (b, j) are read against it. Since 2^x is
// increasing, min(p, q) = 2^min(e_p, e_q) with e = (z / T - ln Z) log2(e): one
// exp2 per pair. Each lane writes e = (z - m) k + (m k - ln Z log2 e) around its
// own largest logit m of that row (one m for the target, one for the draft),
// with the offset in float64: the offset is then log2 of the lane's largest
// term, so the float32 exponent carries no cancellation error where the terms
// are large; per-vector sums in float32, lane sums in float64. Persistent: one workgroup per CU claiming
// units from an LDS counter.
template <int DT, bool VEC>
__global__ __launch_bounds__(kStreamBlock) void overlap_kernel(OverlapArgs a) {
  __shared__ uint32_t s_claim;
  constexpr int CL = chunk_lanes<DT>();
  const RowSet& rs = a.rs;
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x == 0) s_claim = 0u;
  __syncthreads();
  const int64_t G = rs.G;
  const int64_t cv = int64_t(kWave) * CL;
  const int64_t total = rs.B * G * a.cpr;
  const int64_t nblk = gridDim.x;
  const bool v_tail = (a.V % kVec) != 0;
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  // whole windows only: the even XCDs' tail windows measured mixed here
  // (B=256 gamma=4 V=151936: 104.7 vs 105.7 us; B=512 K=4 gamma=8: 938 vs 931)
  const uint32_t i0 = UINT32_MAX;
  uint32_t claim = 0;
  if (lane == 0) claim = atomicAdd(&s_claim, 1u);
  int64_t c = claimed_chunk<false>(__builtin_amdgcn_readfirstlane(claim), nblk, i0);
  while (c < total) {
    uint32_t next = 0;
    if (lane == 0) next = atomicAdd(&s_claim, 1u);
    const int64_t bj = fast_div(uint32_t(c), a.by_cpr);
    const int64_t chunk = c - bj * a.cpr;
    const int64_t b = fast_div(uint32_t(bj), a.by_g);
    const int64_t j = bj - b * G;
    const int64_t v0 = chunk * cv;
    const int64_t v1 = v0 + cv < a.vpr ? v0 + cv : a.vpr;
    if (!sv_ok(b < rs.B && j < G && chunk < a.cpr && v0 < v1)) {
      c = claimed_chunk<false>(__builtin_amdgcn_readfirstlane(next), nblk, i0);
      continue;
    }
    const float T = rs.temp[b];
    const bool sampled = T > 0.0f;
    const void* trow = row_ptr(rs.t, esz, b * rs.tsb + j * rs.tsj);
    RawVec<DT> rt[CL];
#pragma unroll
    for (int u = 0; u < CL; ++u) {
      const int64_t vi = v0 + lane + int64_t(kWave) * u;
      if (vi >= v1) rt[u] = neg_inf_vec<DT>();
      else if (v_tail && vi == a.vpr - 1) rt[u] = load_vec_bounded<DT, VEC>(trow, vi, a.V);
      else rt[u] = load_vec<DT, VEC, true>(trow, vi);
    }
    const double k2 = kLog2eD / double(T);
    const float k2f = float(k2);
    const double l2t = sampled ? a.lnz_t[b * (G + 1) + j] * kLog2eD : 0.0;
    // greedy rows: the target chunk's maximum and lowest id, shared by the K drafts
    float tm = -INFINITY;
    int32_t ti = INT_MAX;
    if (!sampled) {
#pragma unroll
      for (int u = 0; u < CL; ++u)
#pragma unroll
        for (int q = 0; q < kVec; ++q) {
          const float x = vec_elem<DT>(rt[u], q);
          if (x > tm) {
            tm = x;
            ti = int32_t((v0 + lane + int64_t(kWave) * u) * kVec + q);
          }
        }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        const float om = __shfl_xor(tm, off, kWave);
        const int32_t oi = __shfl_xor(ti, off, kWave);
        better_max(tm, ti, om, oi);
      }
    }
    for (int64_t k = 0; k < rs.K; ++k) {
      const int64_t chain = b * rs.K + k;
      const void* drow = row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + j * rs.dsj);
      RawVec<DT> rd[CL];
#pragma unroll
      for (int u = 0; u < CL; ++u) {
        const int64_t vi = v0 + lane + int64_t(kWave) * u;
        if (vi >= v1) rd[u] = neg_inf_vec<DT>();
        else if (v_tail && vi == a.vpr - 1) rd[u] = load_vec_bounded<DT, VEC>(drow, vi, a.V);
        else rd[u] = load_vec<DT, VEC, true>(drow, vi);
      }
      OverlapPartial out{0.0, tm, -INFINITY, ti, INT_MAX};
      if (sampled) {
        const double l2d = a.lnz_d[chain * G + j] * kLog2eD;
        float mt = -INFINITY, md = -INFINITY;
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int q = 0; q < kVec; ++q) {
            mt = fmaxf(mt, vec_elem<DT>(rt[u], q));
            md = fmaxf(md, vec_elem<DT>(rd[u], q));
          }
        // re-read the raw words below rather than keep 128 unpacked values live
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int i = 0; i < (DT == SV_BF16 ? 4 : 8); ++i) {
            asm volatile("" : "+v"(rt[u].w[i]));
            asm volatile("" : "+v"(rd[u].w[i]));
          }
        double sum = 0.0;
        if (mt > -INFINITY && md > -INFINITY) {  // else p or q is 0 on every id of the lane
          const float at = float(double(mt) * k2 - l2t);
          const float ad = float(double(md) * k2 - l2d);
#pragma unroll
          for (int u = 0; u < CL; ++u) {
            float sv = 0.0f;
#pragma unroll
            for (int q = 0; q < kVec; ++q) {
              // -inf logits (and ids past V) give exp2(-inf) = 0
              const float ep = fmaf(vec_elem<DT>(rt[u], q) - mt, k2f, at);
              const float eq = fmaf(vec_elem<DT>(rd[u], q) - md, k2f, ad);
              sv += __builtin_amdgcn_exp2f(fminf(ep, eq));
            }
            sum += double(sv);
          }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
        out.s = sum;
      } else {
        float dm = -INFINITY;
        int32_t di = INT_MAX;
#pragma unroll
        for (int u = 0; u < CL; ++u)
#pragma unroll
          for (int q = 0; q < kVec; ++q) {
            const float x = vec_elem<DT>(rd[u], q);
            if (x > dm) {
              dm = x;
              di = int32_t((v0 + lane + int64_t(kWave) * u) * kVec + q);
            }
          }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
          const float om = __shfl_xor(dm, off, kWave);
          const int32_t oi = __shfl_xor(di, off, kWave);
          better_max(dm, di, om, oi);
        }
        out.md = dm;
        out.id = di;
      }
      if (lane == 0) a.part[(chain * G + j) * a.cpr + chunk] = out;
    }
    c = claimed_chunk<false>(__builtin_amdgcn_readfirstlane(next), nblk, i0);
  }
}

// One wavefront per chain: alpha_j from the chunk partials (a fixed-order
// float64 sum; greedy rows: do the two rows' lowest argmaxes agree), then the
// accept-length law.
constexpr int kAlphaBatch = 8;
__global__ __launch_bounds__(kBlock) void alpha_law_kernel(const OverlapPartial* __restrict__ part,
                                                           int64_t chains, int64_t K, int64_t G,
                                                           int64_t cpr,
                                                           const float* __restrict__ temp,
                                                           double* __restrict__ alpha,
                                                           double* __restrict__ law) {
  const int64_t chain = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (chain >= chains) return;
  const int lane = threadIdx.x & (kWave - 1);
  const float T = temp[chain / K];
  const bool sampled = T > 0.0f;
  const bool greedy = T == 0.0f;
  double reach = 1.0;  // P(n >= j), kept by every lane
  // kAlphaBatch positions at a time: their partials' loads all go out before
  // any is folded (one round of memory latency per batch, not per position)
  for (int64_t j0 = 0; j0 < G; j0 += kAlphaBatch) {
    double s[kAlphaBatch];
    float tm[kAlphaBatch], dm[kAlphaBatch];
    int32_t ti[kAlphaBatch], di[kAlphaBatch];
#pragma unroll
    for (int q = 0; q < kAlphaBatch; ++q) {
      s[q] = 0.0;
      tm[q] = dm[q] = -INFINITY;
      ti[q] = di[q] = INT_MAX;
    }
    for (int64_t c = lane; c < cpr; c += kWave) {
      OverlapPartial p[kAlphaBatch];
#pragma unroll
      for (int q = 0; q < kAlphaBatch; ++q)
        if (j0 + q < G) p[q] = part[(chain * G + j0 + q) * cpr + c];
#pragma unroll
      for (int q = 0; q < kAlphaBatch; ++q)
        if (j0 + q < G) {
          s[q] += p[q].s;
          better_max(tm[q], ti[q], p[q].mt, p[q].it);
          better_max(dm[q], di[q], p[q].md, p[q].id);
        }
    }
#pragma unroll
    for (int q = 0; q < kAlphaBatch; ++q) {
      if (j0 + q >= G) break;  // uniform
      // a sampled chain needs the sum alone, a greedy one the two argmaxes alone
      if (sampled) {
        s[q] = wave_sum(s[q]);
      } else if (greedy) {
        wave_argmax(tm[q], ti[q]);
        wave_argmax(dm[q], di[q]);
      }
      const int64_t j = j0 + q;
      const double aj = sampled ? s[q] : greedy ? (ti[q] == di[q] ? 1.0 : 0.0) : double(NAN);
      if (lane == 0) {
        alpha[chain * G + j] = aj;
        if (law) law[chain * (G + 1) + j] = reach * (1.0 - aj);
      }
      reach *= aj;
    }
  }
  if (lane == 0 && law) law[chain * (G + 1) + G] = reach;
}

// ---------------------------------------------------------------------------
// Speculation cache: for every chain and outcome n = j, the F_j most likely
// emitted tokens -- the largest max(p_j - q_j, 0) for j < gamma, the largest
// p_gamma for j = gamma, the largest raw target logits for greedy rows (ties
// to the lowest id) -- and the lookup of a step's (n, y) among them.

constexpr int kTopFBlock = 256;
constexpr int kTopFCap = 4096;                   // LDS candidate buffer (entries)
constexpr int kTopFWaves = kTopFBlock / kWave;
constexpr int kTopFWaveCap = kTopFCap / kTopFWaves;  // one wavefront's region of the buffer
constexpr int kTopFCut = 256;                    // a region past this many entries is cut
static_assert(kTopFCut + kWave * kVec <= kTopFWaveCap, "a step's admissions fit a region");
constexpr int kTopFSample = 8;                   // passes sampled for the first threshold
constexpr int kTopFSampleWide = 16;              // ... when the grid is 1 to 8 workgroups per CU
constexpr int kTopFWideRowsPerCU = 8;
constexpr int kTopFDepth = 4;                    // vectors per thread loaded one pass ahead
static_assert(SV_MAX_FANOUT <= kTopFBlock, "the first threshold is one of the threads' maxima");

struct TopFArgs {
  RowSet rs;
  int64_t V, vpr;
  const double* lnz_t;   // [B, G+1]
  const double* lnz_d;   // [B, K, G]
  int32_t fan[SV_MAX_GAMMA + 1];
  int32_t off[SV_MAX_GAMMA + 2];
  int64_t ftot;
  int32_t* cand;         // [B*K][ftot]
  float* cand_w;         // [B*K][ftot] or null
  int bonus_last;        // workgroup order: rows j < gamma first, then the j = gamma rows
};

__device__ __forceinline__ bool topf_before(float sa, int32_t ia, float sb, int32_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Bitonic sort of n entries (n <= kTopFCap, padded to a power of two with
// entries that sort last) into best-first order, by the whole workgroup.
__device__ void topf_sort(float* sw, int32_t* si, int n) {
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = n + int(threadIdx.x); i < n2; i += kTopFBlock) {
    sw[i] = -INFINITY;
    si[i] = INT_MAX;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < n2; i += kTopFBlock) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const bool first = (i & k) == 0;
          const bool later_is_better = topf_before(sw[ixj], si[ixj], sw[i], si[i]);
          if (later_is_better == first) {
            const float tw = sw[i];
            const int32_t ti = si[i];
            sw[i] = sw[ixj];
            si[i] = si[ixj];
            sw[ixj] = tw;
            si[ixj] = ti;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Barrier for LDS hand-offs only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders one wavefront's LDS accesses: its earlier ones complete before any
// later one issues (for data handed between its own lanes).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// topf_sort for the n <= kTopFWaveCap entries of one wavefront's region, by
// that wavefront alone (no workgroup barrier).
__device__ void topf_wave_sort(float* sw, int32_t* si, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = n + lane; i < n2; i += kWave) {
    sw[i] = -INFINITY;
    si[i] = INT_MAX;
  }
  wave_lds_sync();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = lane; i < n2; i += kWave) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const bool first = (i & k) == 0;
          const bool later_is_better = topf_before(sw[ixj], si[ixj], sw[i], si[i]);
          if (later_is_better == first) {
            const float tw = sw[i];
            const int32_t ti = si[i];
            sw[i] = sw[ixj];
            si[i] = si[ixj];
            sw[ixj] = tw;
            si[ixj] = ti;
          }
        }
      }
      wave_lds_sync();
    }
  }
}

// One workgroup per (chain, outcome j) with F_j > 0. A streaming selection:
// ids whose score reaches the current threshold go to their wavefront's region
// of an LDS buffer (slots from ballots); past 256 entries a wavefront sorts its
// region, cuts it to the best F_j and raises its threshold to the F_j-th score,
// without waiting for the others; at the end the regions are merged and
// sorted. The first threshold is the F_j-th largest of the threads' maxima
// over a sample of passes spread over the row (F_j distinct ids reach it, so
// it is no higher than the row's F_j-th score). The next pass's vectors load
// while the current one is scored. Scores: residual or target weights in
// float32 (the exponent split in two floats so that large z/T costs no
// precision; a residual's draft term only where the target term reaches the
// threshold), raw logits for greedy rows; -inf = not a candidate.
template <int DT, bool VEC, int NS>
__global__ __launch_bounds__(kTopFBlock) void topf_kernel(TopFArgs a) {
  __shared__ float sw[kTopFCap];
  __shared__ int32_t si[kTopFCap];
  __shared__ float s_max[kTopFBlock];
  __shared__ int s_wcnt[kTopFWaves];
  __shared__ float s_thr;
  constexpr int esz = DT == SV_BF16 ? 2 : 4;
  const RowSet& rs = a.rs;
  const int64_t G = rs.G;
  // bonus_last: the rows j < gamma (two logit rows each) first and the j = gamma
  // rows (one) last, so that where some CUs hold one workgroup more than others
  // (a grid of one round) the extra ones are the cheaper rows; otherwise
  // chain-major.
  const int64_t x = blockIdx.x;
  const int64_t nres = a.bonus_last ? rs.B * rs.K * G : 0;
  const int64_t chain = x < nres ? x / G : a.bonus_last ? x - nres : x / (G + 1);
  const int j = x < nres ? int(x - chain * G) : a.bonus_last ? int(G) : int(x - chain * (G + 1));
  if (!sv_ok(chain < rs.B * rs.K && j >= 0 && j <= G)) return;
  const int F = a.fan[j];
  if (F == 0) return;
  const int tid = threadIdx.x;
  const int64_t b = chain / rs.K;
  const int64_t k = chain - b * rs.K;
  const float T = rs.temp[b];
  const bool sampled = T > 0.0f;
  const bool greedy = T == 0.0f;
  const bool residual = sampled && j < G;
  int32_t* out = a.cand + chain * a.ftot + a.off[j];
  float* outw = a.cand_w ? a.cand_w + chain * a.ftot + a.off[j] : nullptr;
  if (!(sampled || greedy)) {
    for (int i = tid; i < F; i += kTopFBlock) {
      out[i] = -1;
      if (outw) outw[i] = -INFINITY;
    }
    return;
  }
  const void* trow = row_ptr(rs.t, esz, b * rs.tsb + int64_t(j) * rs.tsj);
  const void* drow = residual ? row_ptr(rs.d, esz, b * rs.dsb + k * rs.dsk + int64_t(j) * rs.dsj)
                              : trow;
  // a2 = z k2 - ln Z log2 e as fma(z, k_hi, -c_hi) + fma(z, k_lo, -c_lo)
  const double k2d = sampled ? kLog2eD / double(T) : 0.0;
  const float k_hi = float(k2d);
  const float k_lo = float(k2d - double(k_hi));
  const double l2t = sampled ? a.lnz_t[b * (G + 1) + j] * kLog2eD : 0.0;
  const float c_hi = float(l2t);
  const float c_lo = float(l2t - double(c_hi));
  const float d2 = residual ? float((a.lnz_t[b * (G + 1) + j] - a.lnz_d[chain * G + j]) * kLog2eD)
                            : 0.0f;
  // The weight (float32 score) of id vi*8+t; -inf: not a candidate.
  auto score_at = [&](const RawVec<DT>& rt, const RawVec<DT>& rd, int t) {
    const float zt = vec_elem<DT>(rt, t);
    if (greedy) return zt;
    const float a2 = fmaf(zt, k_hi, -c_hi) + fmaf(zt, k_lo, -c_lo);
    float w = __builtin_amdgcn_exp2f(a2);
    if (residual) w -= __builtin_amdgcn_exp2f(a2 + fmaf(vec_elem<DT>(rd, t) - zt, k_hi, d2));
    return w > 0.0f ? w : -INFINITY;
  };
  // First threshold: the F-th largest of the threads' maxima over a sample of
  // NS passes spread evenly over the row. The sampled ids are
  // distinct, so at least F of them reach it and it is no higher than the
  // row's F-th weight; being taken over the whole row, it admits far fewer
  // ids than the first pass alone would (fewer sorts of the buffer).
  {
    const int64_t passes = (a.vpr + kTopFBlock - 1) / kTopFBlock;
    const int64_t pstride = passes > NS ? passes / NS : 1;
    RawVec<DT> st[NS], sd[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t vi = int64_t(i) * pstride * kTopFBlock + tid;
      st[i] = neg_inf_vec<DT>();
      sd[i] = st[i];
      if (vi < a.vpr) {
        st[i] = load_vec_bounded<DT, VEC>(trow, vi, a.V);
        if (residual) sd[i] = load_vec_bounded<DT, VEC>(drow, vi, a.V);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int t = 0; t < kVec; ++t) mx = fmaxf(mx, score_at(st[i], sd[i], t));
    s_max[tid] = mx;
    __syncthreads();
    for (int kk = 2; kk <= kTopFBlock; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        const int ixj = tid ^ jj;
        float mine = s_max[tid], other = s_max[ixj];
        lds_barrier();
        if (ixj > tid) {
          const bool first = (tid & kk) == 0;
          if ((other > mine) == first) {
            s_max[tid] = other;
            s_max[ixj] = mine;
          }
        }
        lds_barrier();
      }
    }
    if (tid == 0) s_thr = s_max[F - 1];
  }
  // kTopFDepth vectors per thread per pass, the next pass's loaded while this
  // one is scored; each vector's ids are admitted (and the wavefront's region
  // cut) in turn, so a step adds at most one vector per lane to a region.
  constexpr int64_t kPass = int64_t(kTopFBlock) * kTopFDepth;
  RawVec<DT> nt[kTopFDepth], nd[kTopFDepth];
#pragma unroll
  for (int u = 0; u < kTopFDepth; ++u) {
    const int64_t vi = int64_t(u) * kTopFBlock + tid;
    nt[u] = neg_inf_vec<DT>();
    nd[u] = nt[u];
    if (vi < a.vpr) {
      nt[u] = load_vec_bounded<DT, VEC>(trow, vi, a.V);
      if (residual) nd[u] = load_vec_bounded<DT, VEC>(drow, vi, a.V);
    }
  }
  __syncthreads();
  // Each wavefront admits into its own region with its own threshold (the
  // sampled one, raised to its region's F-th score at each cut): an id below
  // it has F better ids in that region, so the union of the regions' best F
  // holds the row's best F.
  const int wv = tid / kWave;
  const int lane = tid % kWave;
  float* rw = sw + wv * kTopFWaveCap;
  int32_t* ri = si + wv * kTopFWaveCap;
  int wcnt = 0;
  float thr = s_thr;
  for (int64_t pbase = 0; pbase < a.vpr; pbase += kPass) {
    RawVec<DT> ct[kTopFDepth], cd[kTopFDepth];
#pragma unroll
    for (int u = 0; u < kTopFDepth; ++u) {
      ct[u] = nt[u];
      cd[u] = nd[u];
      const int64_t vn = pbase + kPass + int64_t(u) * kTopFBlock + tid;
      if (vn < a.vpr) {
        nt[u] = load_vec_bounded<DT, VEC>(trow, vn, a.V);
        if (residual) nd[u] = load_vec_bounded<DT, VEC>(drow, vn, a.V);
      }
    }
#pragma unroll
    for (int u = 0; u < kTopFDepth; ++u) {
      const int64_t vi = pbase + int64_t(u) * kTopFBlock + tid;
      if (pbase + int64_t(u) * kTopFBlock >= a.vpr) break;   // uniform: the row has ended
      float sc[kVec];
      if (residual) {
        // w = 2^a2 minus a non-negative term, so w <= 2^a2 exactly: unless an
        // id of the wavefront has 2^a2 at the threshold, none can be admitted
        // and the draft term is skipped (the same operations as score_at)
        float a2[kVec], e1[kVec];
        bool need = false;
#pragma unroll
        for (int t = 0; t < kVec; ++t) {
          const float zt = vec_elem<DT>(ct[u], t);
          a2[t] = fmaf(zt, k_hi, -c_hi) + fmaf(zt, k_lo, -c_lo);
          e1[t] = __builtin_amdgcn_exp2f(a2[t]);
          need = need || e1[t] >= thr;
        }
        if (__any(need && vi < a.vpr)) {
#pragma unroll
          for (int t = 0; t < kVec; ++t) {
            const float zt = vec_elem<DT>(ct[u], t);
            const float w = e1[t] - __builtin_amdgcn_exp2f(a2[t] + fmaf(vec_elem<DT>(cd[u], t) - zt, k_hi, d2));
            sc[t] = vi < a.vpr && w > 0.0f ? w : -INFINITY;
          }
        } else {
#pragma unroll
          for (int t = 0; t < kVec; ++t) sc[t] = -INFINITY;
        }
      } else {
#pragma unroll
        for (int t = 0; t < kVec; ++t) sc[t] = vi < a.vpr ? score_at(ct[u], cd[u], t) : -INFINITY;
      }
      // admit into this wavefront's region: slots from ballots, no atomics;
      // most steps admit nothing anywhere in the wavefront and skip it all
      bool keep[kVec];
      bool any = false;
#pragma unroll
      for (int t = 0; t < kVec; ++t) {
        keep[t] = sc[t] > -INFINITY && sc[t] >= thr;
        any = any || keep[t];
      }
      if (__any(any)) {
        int base = wcnt;
#pragma unroll
        for (int t = 0; t < kVec; ++t) {
          const uint64_t bal = __ballot(keep[t]);
          if (keep[t]) {
            const int slot = base + int(__builtin_amdgcn_mbcnt_hi(
                                        uint32_t(bal >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0u)));
            rw[slot] = sc[t];
            ri[slot] = int32_t(vi * kVec + t);
          }
          base += __popcll(bal);
        }
        wcnt = base;
      }
      if (wcnt > kTopFCut) {  // uniform in the wavefront: cut its region to the best F
        wave_lds_sync();
        topf_wave_sort(rw, ri, wcnt);
        if (wcnt >= F) {
          const float f = rw[F - 1];
          if (f > thr) thr = f;
        }
        wcnt = wcnt < F ? wcnt : F;
      }
    }
  }
  // merge the regions: each wavefront moves its entries behind the earlier ones'
  if (lane == 0) s_wcnt[wv] = wcnt;
  __syncthreads();
  int off = 0, cnt = 0;
#pragma unroll
  for (int w = 0; w < kTopFWaves; ++w) {
    off += w < wv ? s_wcnt[w] : 0;
    cnt += s_wcnt[w];
  }
  if (wv > 0)
    for (int i = lane; i < wcnt; i += kWave) {
      sw[off + i] = rw[i];
      si[off + i] = ri[i];
    }
  __syncthreads();
  topf_sort(sw, si, cnt);
  for (int i = tid; i < F; i += kTopFBlock) {
    const bool have = i < cnt;
    out[i] = have ? si[i] : -1;
    if (outw) outw[i] = have ? sw[i] : -INFINITY;
  }
}

// One thread per chain: the slot of the emitted token among the candidates of
// the chain's outcome (accept length n), or -1.
__global__ __launch_bounds__(kBlock) void cache_lookup_kernel(const int32_t* __restrict__ cand,
                                                              TopFArgs a, int64_t chains,
                                                              const int32_t* __restrict__ n_in,
                                                              const int32_t* __restrict__ y_in,
                                                              int32_t* __restrict__ slot) {
  const int64_t chain = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (chain >= chains) return;
  const int32_t n = n_in[chain];
  const int32_t y = y_in[chain];
  int32_t hit = -1;
  if (n >= 0 && n <= a.rs.G && y >= 0) {
    const int32_t* c = cand + chain * a.ftot;
    for (int32_t i = a.off[n]; i < a.off[n + 1]; ++i)
      if (c[i] == y) {
        hit = i;
        break;
      }
  }
  slot[chain] = hit;
}

// ---------------------------------------------------------------------------
// Branch pruning before verification: per branch, the running sum of ln q over
// the draft positions (float64, in order), the confident prefix L (positions
// whose running sum is >= ln tau) and, per batch row, the `keep` branches of
// largest L (ties: larger sum over the prefix, then lower k). One thread per
// batch row.
__global__ __launch_bounds__(kBlock) void branch_prune_kernel(const float* __restrict__ logq,
                                                              int64_t B, int64_t K, int64_t G,
                                                              double log_tau, int64_t keep,
                                                              int32_t* __restrict__ keep_mask,
                                                              int32_t* __restrict__ prefix_len,
                                                              double* __restrict__ conf) {
  const int64_t b = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (b >= B) return;
  int32_t len[SV_MAX_CHAIN_DECISIONS];
  double last[SV_MAX_CHAIN_DECISIONS];
  for (int64_t k = 0; k < K; ++k) {
    double c = 0.0;
    int32_t L = 0;
    double at = -INFINITY;
    for (int64_t j = 0; j < G; ++j) {
      c += double(logq[(b * K + k) * G + j]);
      if (conf) conf[(b * K + k) * G + j] = c;
      if (c >= log_tau) {
        ++L;
        at = c;
      }
    }
    len[k] = L;
    last[k] = at;
  }
  for (int64_t k = 0; k < K; ++k) {
    // rank of branch k: branches ordered before it
    int64_t ahead = 0;
    for (int64_t o = 0; o < K; ++o) {
      if (o == k) continue;
      const bool before = len[o] > len[k] || (len[o] == len[k] && last[o] > last[k]) ||
                          (len[o] == len[k] && last[o] == last[k] && o < k);
      ahead += before ? 1 : 0;
    }
    keep_mask[b * K + k] = ahead < keep ? 1 : 0;
    if (prefix_len) prefix_len[b * K + k] = len[k];
  }
}

// ---------------------------------------------------------------------------
// Host side.

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Steps whose draw grid is small take narrower splits (down to 2048 ids, one
// vector per thread) while the grid stays within half the CUs: each scan is
// then shorter, and a chain's latency is what such a step waits for. The
// candidate region holds the narrow count where chains * ceil(V / 2048) <=
// kNarrowMaxSplits.
constexpr int64_t kNarrowSplit = int64_t(kBlock) * kVec;
constexpr int64_t kNarrowMaxSplits = 1024;

struct Layout {
  int64_t vpr, cpr, nrows, chains, nsplit;
  size_t off_part, off_rank, off_info, off_top, off_tok, total;
};

// Chain counters at the start of every workspace. The first launch of every
// call that counts on them zeroes the ones it uses (the stream kernel, or
// given_kernel), so a workspace needs no preparation and an interrupted call
// leaves nothing behind. Steps with more chains pick their tokens in
// finish_kernel.
constexpr int64_t kMaxCountedChains = 65536;
constexpr size_t kCounterBytes = kMaxCountedChains * sizeof(uint32_t);

// One chunk partial per (stream row, chunk); every row of the batch counted.
Layout make_layout(int64_t B, int64_t nrows, int64_t chains, int64_t V, int dtype,
                   int64_t ntok = 0) {
  Layout L;
  L.vpr = (V + kVec - 1) / kVec;
  const int64_t cv = chunk_vectors(dtype);
  L.cpr = (L.vpr + cv - 1) / cv;
  L.nrows = nrows;
  L.chains = chains;
  L.nsplit = (V + kSplit - 1) / kSplit;
  L.off_part = kCounterBytes;
  L.off_rank = align256(L.off_part + size_t(nrows) * size_t(L.cpr) * sizeof(RowPartial));
  L.off_info = align256(L.off_rank + size_t(B + 1) * sizeof(int32_t));
  L.off_top = align256(L.off_info + size_t(chains) * sizeof(ChainInfo));
  const int64_t narrow = (V + kNarrowSplit - 1) / kNarrowSplit;
  const int64_t slots = chains * narrow <= kNarrowMaxSplits ? narrow : L.nsplit;
  L.off_tok = align256(L.off_top + size_t(chains) * size_t(slots) * sizeof(Cand));
  L.total = align256(L.off_tok + size_t(ntok) * sizeof(TokenAux));
  return L;
}

// Compute units of the current device (cached per device; only speed
// depends on it).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Workgroups of one stream-kernel instantiation resident on the device at
// once: the persistent grid (cached per device; only speed depends on it).
template <int DT, bool VEC, bool ARGMAX_ALL>
int64_t stream_blocks() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, stream_kernel<DT, VEC, ARGMAX_ALL, false>,
                                                   kStreamBlock, 0) != hipSuccess ||
      blocks <= 0)
    blocks = 1;
  const int64_t n = int64_t(cus) * blocks;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s, int esz) { return (s * esz) % 16 == 0; }
int check_dtype(int dtype) { return (dtype == SV_F32 || dtype == SV_BF16) ? SV_OK : SV_EDTYPE; }
int esize(int dtype) { return dtype == SV_BF16 ? 2 : 4; }
int launch_status() { return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP; }

// ev0 / ev1 (timing hook): events the launch itself marks with the kernel's
// start and end (hipExtLaunchKernel), so their elapsed time is the kernel's
// execution alone, as a profiler reports it.
template <int DT, bool VEC, bool ARGMAX_ALL>
void launch_stream_t(StreamArgs sa, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  int64_t grid = stream_blocks<DT, VEC, ARGMAX_ALL>();
  const int64_t need = (sa.nrows * sa.cpr + kStreamWaves - 1) / kStreamWaves;
  if (grid > need) grid = need;
  sa.win_scale = window_scale(sa.nrows * sa.cpr, grid, 1);  // compact mode: the all-sampled bound
  if (sa.tok_aux) grid += 1;  // the token gather
  // direct launches (a kernel picked through a function pointer is an
  // indirect call, which function-type sanitizers instrument)
  if (sa.win_scale > 0.0f) {
    if (ev0)
      hipExtLaunchKernelGGL((stream_kernel<DT, VEC, ARGMAX_ALL, true>), dim3(unsigned(grid)),
                            dim3(kStreamBlock), 0, st, ev0, ev1, 0u, sa);
    else
      hipLaunchKernelGGL((stream_kernel<DT, VEC, ARGMAX_ALL, true>), dim3(unsigned(grid)),
                         dim3(kStreamBlock), 0, st, sa);
  } else {
    if (ev0)
      hipExtLaunchKernelGGL((stream_kernel<DT, VEC, ARGMAX_ALL, false>), dim3(unsigned(grid)),
                            dim3(kStreamBlock), 0, st, ev0, ev1, 0u, sa);
    else
      hipLaunchKernelGGL((stream_kernel<DT, VEC, ARGMAX_ALL, false>), dim3(unsigned(grid)),
                         dim3(kStreamBlock), 0, st, sa);
  }
}

void launch_stream_dt(int dtype, bool vec, bool argmax_all, const StreamArgs& sa, hipStream_t st,
                      hipEvent_t e0, hipEvent_t e1) {
  if (dtype == SV_BF16) {
    if (vec) argmax_all ? launch_stream_t<SV_BF16, true, true>(sa, st, e0, e1)
                        : launch_stream_t<SV_BF16, true, false>(sa, st, e0, e1);
    else argmax_all ? launch_stream_t<SV_BF16, false, true>(sa, st, e0, e1)
                    : launch_stream_t<SV_BF16, false, false>(sa, st, e0, e1);
    return;
  }
  if (vec) argmax_all ? launch_stream_t<SV_F32, true, true>(sa, st, e0, e1)
                      : launch_stream_t<SV_F32, true, false>(sa, st, e0, e1);
  else argmax_all ? launch_stream_t<SV_F32, false, true>(sa, st, e0, e1)
                  : launch_stream_t<SV_F32, false, false>(sa, st, e0, e1);
}

// Events the next streaming-kernel launch of this host thread records around
// itself (specverify_time_next_stream_kernel); taken, and so cleared, by it.
thread_local hipEvent_t t_ev_before = nullptr;
thread_local hipEvent_t t_ev_after = nullptr;

void launch_stream(int dtype, bool vec, bool argmax_all, StreamArgs sa, hipStream_t st) {
  const hipEvent_t ev_before = t_ev_before, ev_after = t_ev_after;
  t_ev_before = t_ev_after = nullptr;
  // chunk indices are below 2^31 (stream_chunks_ok): the kernel divides by
  // multiply-shift
  const int64_t kg = sa.rs.K * sa.rs.G;
  sa.by_cpr = make_fastdiv(uint32_t(sa.cpr));
  sa.by_p = make_fastdiv(uint32_t(sa.rs.P));
  sa.by_kg = make_fastdiv(uint32_t(kg > 0 ? kg : 1));
  sa.by_g = make_fastdiv(uint32_t(sa.rs.G > 0 ? sa.rs.G : 1));
  launch_stream_dt(dtype, vec, argmax_all, sa, st, ev_before, ev_after);
}

// Workgroups of the fused draw kernel resident on the device at once (cached per
// device).
template <int DT, bool VEC>
int64_t draw_resident() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, draw_kernel<DT, VEC, true, kSampleIters>, kBlock,
                                                   0) != hipSuccess ||
      blocks <= 0)
    blocks = 4;
  const int64_t n = int64_t(cus) * blocks;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Draws whose grid needs many rounds of resident workgroups take splits of
// twice the ids (half the workgroups, each scanning 8 vectors per thread): the
// per-workgroup prologue is paid half as often, and the last round's imbalance
// is a small part of the whole. B=512 K=4 gamma=8 (25 rounds): 1198 vs 1228 us
// per step; B=256 K=1 gamma=4 (4 rounds) measured slower this way (137 vs 131).
constexpr int64_t kWideRounds = 8;
// From this many chains per CU, one workgroup per chain scans the whole row
// pair (draw_chain_kernel) instead of one per split.
constexpr int64_t kChainsPerCuWhole = 4;

template <int DT, bool VEC>
void launch_chain_finish(ChainArgs ca, bool given, hipStream_t st) {
  const int64_t chains = ca.rs.B * ca.rs.K;
  const bool fused = !given && chains * ca.nsplit <= draw_resident<DT, VEC>();
  // bf16 only: eight float32 vectors per thread and row do not fit the registers
  const bool wide = DT == SV_BF16 && !fused &&
                    chains * ca.nsplit >= kWideRounds * draw_resident<DT, VEC>();
  if (wide) {
    ca.nsplit = (ca.V + 2 * kSplit - 1) / (2 * kSplit);  // at most the workspace's count
    ca.by_nsplit = make_fastdiv(uint32_t(ca.nsplit));
  }
  // a fused grid of at most one split per two CUs: vectors per thread 4 -> 2 -> 1
  // (B=1 K=1 gamma=4 V=32000: 15.7 vs 17.5 us per step; B=16 gamma=5: 18.9 vs
  // 19.7; one split per CU measured slower at B=16)
  int si = kSampleIters;
  if (fused) {
    const int64_t cap = std::min<int64_t>(device_cus() / 2, kNarrowMaxSplits / 2);
    for (int s = kSampleIters / 2; s >= 1; s /= 2) {
      const int64_t ids = int64_t(kBlock) * kVec * s;
      const int64_t ns = (ca.V + ids - 1) / ids;
      if (chains * ns > cap) break;
      si = s;
      ca.nsplit = ns;
    }
    ca.by_nsplit = make_fastdiv(uint32_t(ca.nsplit));
  }
  const dim3 grid{unsigned(chains * ca.nsplit), 1u, 1u};
  auto draws = [&]() {
    if constexpr (DT == SV_BF16)
      if (wide) {
        hipLaunchKernelGGL((draw_kernel<DT, VEC, false, 2 * kSampleIters>), grid, dim3(kBlock), 0,
                           st, ca);
        return;
      }
    hipLaunchKernelGGL((draw_kernel<DT, VEC, false, kSampleIters>), grid, dim3(kBlock), 0, st, ca);
  };
  if (given) {
    hipLaunchKernelGGL(given_kernel, dim3(unsigned((chains + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, st, ca, chains);
    draws();
  } else if (fused) {
    // every split derives n itself: one launch fewer, one prologue per workgroup
    if (si == 1)
      hipLaunchKernelGGL((draw_kernel<DT, VEC, true, 1>), grid, dim3(kBlock), 0, st, ca);
    else if (si == 2)
      hipLaunchKernelGGL((draw_kernel<DT, VEC, true, 2>), grid, dim3(kBlock), 0, st, ca);
    else
      hipLaunchKernelGGL((draw_kernel<DT, VEC, true, kSampleIters>), grid, dim3(kBlock), 0, st, ca);
  } else {
    // more workgroups than fit at once: n per chain in its own launch
    hipLaunchKernelGGL((accept_kernel<DT>), dim3(unsigned(chains)), dim3(kBlock), 0, st, ca);
    if (chains >= kChainsPerCuWhole * device_cus()) {
      hipLaunchKernelGGL((draw_chain_kernel<DT, VEC>), dim3(unsigned(chains)), dim3(kBlock), 0, st, ca);
      return;
    }
    draws();
  }
  if (ca.cnt) return;  // the chains' last splits picked the tokens
  const RowSet& rs = ca.rs;
  hipLaunchKernelGGL((finish_kernel<DT, VEC>), dim3(unsigned(chains)), dim3(kWave), 0, st, rs.t,
                     rs.tsb, rs.tsj, rs.K, rs.G, ca.V, rs.temp, ca.seed, ca.pos0, ca.info,
                     ca.cand, ca.nsplit, ca.out_token);
}

void launch_chain(int dtype, bool vec, ChainArgs ca, bool given, hipStream_t st) {
  ca.by_nsplit = make_fastdiv(uint32_t(ca.nsplit));
  ca.by_k = make_fastdiv(uint32_t(ca.rs.K));
  if (dtype == SV_BF16) {
    if (vec) launch_chain_finish<SV_BF16, true>(ca, given, st);
    else launch_chain_finish<SV_BF16, false>(ca, given, st);
  } else {
    if (vec) launch_chain_finish<SV_F32, true>(ca, given, st);
    else launch_chain_finish<SV_F32, false>(ca, given, st);
  }
}

bool sizes_ok(int64_t B, int64_t K, int64_t G, int64_t V) {
  if (!(B >= 1 && K >= 1 && G >= 1 && G <= SV_MAX_GAMMA && K * G <= SV_MAX_CHAIN_DECISIONS &&
        V >= 1 && V < (int64_t(1) << 31)))
    return false;
  const int64_t nsplit = (V + kSplit - 1) / kSplit;
  return B <= (int64_t(1) << 31) / (G + 1) / (K + 1) && B * K * nsplit < (int64_t(1) << 31);
}

bool workspace_ok(void* ws, size_t have, size_t need, int* status) {
  if (ws == nullptr || have < need) {
    *status = SV_EWORKSPACE;
    return false;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    *status = SV_EALIGN;
    return false;
  }
  return true;
}

// The stream kernel indexes chunks in 32 bits: fewer than 2^31 chunks per call
// (2^31 chunks of 8 KB are 16 TiB of logits).
bool stream_chunks_ok(const Layout& L) { return L.nrows * L.cpr < (int64_t(1) << 31); }

Layout step_layout(int64_t B, int64_t K, int64_t G, int64_t V, int dtype) {
  return make_layout(B, B * (G + 1) + B * K * G, B * K, V, dtype, B * K * G);
}

bool logits_vec_ok(const void* t, const void* d, int esz, int64_t tsb, int64_t tsj, int64_t dsb,
                   int64_t dsk, int64_t dsj) {
  return aligned16(t) && aligned16(d) && stride_ok(tsb, esz) && stride_ok(tsj, esz) &&
         stride_ok(dsb, esz) && stride_ok(dsk, esz) && stride_ok(dsj, esz);
}

// The acceptance-probability sweep: one partial per (chain, position, chunk),
// after the counter region (which it never touches).
size_t overlap_layout_bytes(int64_t B, int64_t K, int64_t G, int64_t V, int dtype) {
  const int64_t vpr = (V + kVec - 1) / kVec;
  const int64_t cv = chunk_vectors(dtype);
  const int64_t cpr = (vpr + cv - 1) / cv;
  return kCounterBytes +
         align256(size_t(B) * size_t(K) * size_t(G) * size_t(cpr) * sizeof(OverlapPartial));
}

template <int DT, bool VEC>
int64_t overlap_blocks() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, overlap_kernel<DT, VEC>,
                                                   kStreamBlock, 0) != hipSuccess ||
      blocks <= 0)
    blocks = 1;
  const int64_t n = int64_t(cus) * blocks;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int DT, bool VEC>
void launch_overlap(const OverlapArgs& oa, int64_t units, hipStream_t st) {
  int64_t grid = overlap_blocks<DT, VEC>();
  const int64_t need = (units + kStreamWaves - 1) / kStreamWaves;
  if (grid > need) grid = need;
  hipLaunchKernelGGL((overlap_kernel<DT, VEC>), dim3(unsigned(grid)), dim3(kStreamBlock), 0, st,
                     oa);
}

// Outcome fan-out (host array [G+1]) into the kernel arguments; false if any
// entry is outside [0, SV_MAX_FANOUT].
bool fill_fanout(const int32_t* fan, int64_t G, TopFArgs& a) {
  int64_t off = 0;
  for (int64_t j = 0; j <= G; ++j) {
    if (fan[j] < 0 || fan[j] > SV_MAX_FANOUT) return false;
    a.fan[j] = fan[j];
    a.off[j] = int32_t(off);
    off += fan[j];
  }
  a.off[G + 1] = int32_t(off);
  a.ftot = off;
  return true;
}

template <int DT, bool VEC>
void launch_topf(bool wide, dim3 grid, hipStream_t st, const TopFArgs& ta) {
  if (wide)
    hipLaunchKernelGGL((topf_kernel<DT, VEC, kTopFSampleWide>), grid, dim3(kTopFBlock), 0, st, ta);
  else
    hipLaunchKernelGGL((topf_kernel<DT, VEC, kTopFSample>), grid, dim3(kTopFBlock), 0, st, ta);
}

int step_checks(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                int64_t d_stride_j, const float* temperature, const int32_t* accept_len,
                const int32_t* out_token);
int step_launch(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                int64_t d_stride_j, const float* temperature, uint64_t seed, const int64_t* pos0,
                int32_t* accept_len, int32_t* out_token, float* logp, float* logq,
                double* lnZ_target, double* lnZ_draft, int32_t* device_error, void* workspace,
                hipStream_t st);

}  // namespace

// Scratch of specverify_step_noalloc, for callers that cannot allocate: one
// copy per GPU, resident from the library's load on that GPU until the process
// ends. Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol): scratch_address() looks up each device's
// own address once, with that device current, and every launch uses that.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

int scratch_address(void** out) {
  static std::atomic<void*> cache[kMaxDevices];
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_EHIP;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> hold(lock);
    p = cache[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return SV_EHIP;
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SV_OK;
}

}  // namespace

extern "C" {

size_t specverify_workspace_size(int64_t B, int64_t K, int64_t gamma, int64_t V, int dtype) {
  if (check_dtype(dtype) != SV_OK) return 0;
  if (K == 0) {  // specverify_normalize: P = gamma + 1 rows per batch row
    if (B < 1 || gamma < 0 || V < 1 || V >= (int64_t(1) << 31) ||
        B > (int64_t(1) << 40) / (gamma + 1))
      return 0;
    return make_layout(B, B * (gamma + 1), 0, V, dtype).total;
  }
  if (!sizes_ok(B, K, gamma, V)) return 0;
  return step_layout(B, K, gamma, V, dtype).total;
}

int specverify_normalize(const void* logits, int dtype, int64_t B, int64_t P, int64_t V,
                         int64_t stride_b, int64_t stride_p, const float* temperature,
                         double* lnZ, int32_t* argmax, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!logits || !temperature || !lnZ) return SV_EINVAL;
  if (B < 1 || P < 1 || V < 1 || V >= (int64_t(1) << 31) || stride_b < 0 || stride_p < 0 ||
      B > (int64_t(1) << 40) / P)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  const Layout L = make_layout(B, B * P, 0, V, dtype);
  if (!stream_chunks_ok(L)) return SV_EINVAL;
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  const int esz = esize(dtype);
  const bool vec = aligned16(logits) && stride_ok(stride_b, esz) && stride_ok(stride_p, esz);
  auto* base = reinterpret_cast<char*>(workspace);
  auto* part = reinterpret_cast<RowPartial*>(base + L.off_part);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  StreamArgs sa{};
  sa.rs = RowSet{logits, stride_b, stride_p, nullptr, 0, 0, 0, B, P, 0, 1, temperature};
  sa.V = V;
  sa.vpr = L.vpr;
  sa.cpr = L.cpr;
  sa.nrows = B * P;
  sa.compact = 0;
  sa.part = part;
  sa.rank_out = nullptr;
  launch_stream(dtype, vec, argmax != nullptr, sa, st);
  constexpr int kFinRows = kFinBlock / kRowLanes;
  hipLaunchKernelGGL(finalize_rows_kernel, dim3(unsigned((B * P + kFinRows - 1) / kFinRows)),
                     dim3(kFinBlock), 0, st, part, B * P, L.cpr, P, temperature, lnZ, argmax);
  return launch_status();
}

int specverify_accept(const float* logp, const float* logq, int64_t B, int64_t K, int64_t gamma,
                      uint64_t seed, const int64_t* pos0, int32_t* accept_len,
                      uint32_t* accept_bits, void* stream) {
  if (!logp || !logq || !accept_len) return SV_EINVAL;
  if (B < 1 || K < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || B > (int64_t(1) << 31) / K)
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
  const Layout L = step_layout(B, K, gamma, V, dtype);
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  const int esz = esize(dtype);
  const bool vec = logits_vec_ok(target_logits, draft_logits, esz, t_stride_b, t_stride_j,
                                 d_stride_b, d_stride_k, d_stride_j);
  auto* base = reinterpret_cast<char*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  ChainArgs ca{};
  ca.rs = RowSet{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                 d_stride_j, B, gamma + 1, K, gamma, temperature};
  ca.V = V;
  ca.seed = seed;
  ca.pos0 = pos0;
  ca.out_token = out_token;
  ca.lnz_t_in = lnZ_target;
  ca.lnz_d_in = lnZ_draft;
  ca.amax_in = argmax_target;
  ca.n_in = accept_len;
  ca.nsplit = L.nsplit;
  ca.cand = reinterpret_cast<Cand*>(base + L.off_top);
  ca.info = reinterpret_cast<ChainInfo*>(base + L.off_info);
  ca.cnt = B * K <= kMaxCountedChains ? reinterpret_cast<uint32_t*>(base) : nullptr;
  launch_chain(dtype, vec, ca, true, st);
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
  int status = step_checks(target_logits, draft_logits, dtype, draft_tokens, B, K, gamma, V,
                           t_stride_b, t_stride_j, d_stride_b, d_stride_k, d_stride_j,
                           temperature, accept_len, out_token);
  if (status != SV_OK) return status;
  const Layout L = step_layout(B, K, gamma, V, dtype);
  if (!workspace_ok(workspace, workspace_bytes, L.total, &status)) return status;
  return step_launch(target_logits, draft_logits, dtype, draft_tokens, B, K, gamma, V,
                     t_stride_b, t_stride_j, d_stride_b, d_stride_k, d_stride_j, temperature,
                     seed, pos0, accept_len, out_token, logp, logq, lnZ_target, lnZ_draft,
                     device_error, workspace, reinterpret_cast<hipStream_t>(stream));
}

int specverify_step_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                            const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma,
                            int64_t V, int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b,
                            int64_t d_stride_k, int64_t d_stride_j, const float* temperature,
                            uint64_t seed, const int64_t* pos0, int32_t* accept_len,
                            int32_t* out_token, float* logp, float* logq, double* lnZ_target,
                            double* lnZ_draft, int32_t* device_error, void* stream) {
  int status = step_checks(target_logits, draft_logits, dtype, draft_tokens, B, K, gamma, V,
                           t_stride_b, t_stride_j, d_stride_b, d_stride_k, d_stride_j,
                           temperature, accept_len, out_token);
  if (status != SV_OK) return status;
  if (step_layout(B, K, gamma, V, dtype).total > size_t(SV_NOALLOC_SCRATCH_BYTES))
    return SV_ESCRATCH;
  void* ws = nullptr;
  status = scratch_address(&ws);
  if (status != SV_OK) return status;
  return step_launch(target_logits, draft_logits, dtype, draft_tokens, B, K, gamma, V,
                     t_stride_b, t_stride_j, d_stride_b, d_stride_k, d_stride_j, temperature,
                     seed, pos0, accept_len, out_token, logp, logq, lnZ_target, lnZ_draft,
                     device_error, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int step_checks(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                int64_t d_stride_j, const float* temperature, const int32_t* accept_len,
                const int32_t* out_token) {
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !accept_len ||
      !out_token)
    return SV_EINVAL;
  if (!sizes_ok(B, K, gamma, V)) return SV_EINVAL;
  if (t_stride_b < 0 || t_stride_j < 0 || d_stride_b < 0 || d_stride_k < 0 || d_stride_j < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  if (!stream_chunks_ok(step_layout(B, K, gamma, V, dtype))) return SV_EINVAL;
  return SV_OK;
}

// The step's launches on stream st with a workspace already checked for size
// and alignment.
int step_launch(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                int64_t d_stride_j, const float* temperature, uint64_t seed, const int64_t* pos0,
                int32_t* accept_len, int32_t* out_token, float* logp, float* logq,
                double* lnZ_target, double* lnZ_draft, int32_t* device_error, void* workspace,
                hipStream_t st) {
  const Layout L = step_layout(B, K, gamma, V, dtype);
  const int esz = esize(dtype);
  const bool vec = logits_vec_ok(target_logits, draft_logits, esz, t_stride_b, t_stride_j,
                                 d_stride_b, d_stride_k, d_stride_j);
  auto* base = reinterpret_cast<char*>(workspace);
  auto* part = reinterpret_cast<RowPartial*>(base + L.off_part);
  auto* rank = reinterpret_cast<int32_t*>(base + L.off_rank);
  const RowSet rs{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                  d_stride_j, B, gamma + 1, K, gamma, temperature};
  const int compact = B <= kMaxCompactB ? 1 : 0;

  StreamArgs sa{};
  sa.rs = rs;
  sa.V = V;
  sa.vpr = L.vpr;
  sa.cpr = L.cpr;
  sa.nrows = L.nrows;
  sa.compact = compact;
  sa.part = part;
  sa.rank_out = compact ? rank : nullptr;
  sa.clear = B * K <= kMaxCountedChains ? reinterpret_cast<uint32_t*>(base) : nullptr;
  sa.nclear = sa.clear ? B * K : 0;
  // The token gather takes one workgroup of the stream's grid: with at most
  // one (chain, position) per thread it ends well before the stream does (it
  // starts when the first streaming workgroup ends); larger batches draw the
  // accept uniforms in the draws' prologue instead (B=512 K=4 gamma=8: the
  // gather's 16 rounds of scattered loads lengthened the stream by ~38 us).
  TokenAux* tok_aux =
      B * K * gamma <= kStreamBlock ? reinterpret_cast<TokenAux*>(base + L.off_tok) : nullptr;
  sa.tok_aux = tok_aux;
  sa.tokens = draft_tokens;
  sa.pos0 = pos0;
  sa.seed = seed;
  launch_stream(dtype, vec, false, sa, st);

  ChainArgs ca{};
  ca.rs = rs;
  ca.V = V;
  ca.part = part;
  ca.cpr = L.cpr;
  ca.tokens = draft_tokens;
  ca.tok_aux = tok_aux;
  ca.seed = seed;
  ca.pos0 = pos0;
  ca.accept_len = accept_len;
  ca.out_token = out_token;
  ca.logp = logp;
  ca.logq = logq;
  ca.lnz_t_out = lnZ_target;
  ca.lnz_d_out = lnZ_draft;
  ca.dev_err = device_error;
  ca.nsplit = L.nsplit;
  ca.cand = reinterpret_cast<Cand*>(base + L.off_top);
  ca.info = reinterpret_cast<ChainInfo*>(base + L.off_info);
  ca.cnt = B * K <= kMaxCountedChains ? reinterpret_cast<uint32_t*>(base) : nullptr;
  launch_chain(dtype, vec, ca, false, st);
  return launch_status();
}

}  // namespace

extern "C" {

const char* specverify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (null pointer, size or stride out of range)";
    case SV_EDTYPE: return "unknown logit dtype";
    case SV_EWORKSPACE: return "workspace missing or too small";
    case SV_EALIGN: return "workspace not 256-byte aligned";
    case SV_EHIP: return "HIP kernel launch failed";
    case SV_ESCRATCH:
      return "sizes need more scratch than specverify_step_noalloc holds "
             "(SV_NOALLOC_SCRATCH_BYTES); use specverify_step with a workspace";
    case SV_ENOCHECKS: return "library built without device-side index checks";
    default: return "unknown status";
  }
}

size_t specverify_accept_prob_workspace_size(int64_t B, int64_t K, int64_t gamma, int64_t V,
                                             int dtype) {
  if (check_dtype(dtype) != SV_OK || !sizes_ok(B, K, gamma, V)) return 0;
  return overlap_layout_bytes(B, K, gamma, V, dtype);
}

int specverify_accept_prob(const void* target_logits, const void* draft_logits, int dtype,
                           int64_t B, int64_t K, int64_t gamma, int64_t V, int64_t t_stride_b,
                           int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                           int64_t d_stride_j, const float* temperature, const double* lnZ_target,
                           const double* lnZ_draft, double* alpha, double* law, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !temperature || !lnZ_target || !lnZ_draft || !alpha)
    return SV_EINVAL;
  if (!sizes_ok(B, K, gamma, V)) return SV_EINVAL;
  if (t_stride_b < 0 || t_stride_j < 0 || d_stride_b < 0 || d_stride_k < 0 || d_stride_j < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  int status = SV_OK;
  if (!workspace_ok(workspace, workspace_bytes, overlap_layout_bytes(B, K, gamma, V, dtype),
                    &status))
    return status;
  const int esz = esize(dtype);
  const bool vec = logits_vec_ok(target_logits, draft_logits, esz, t_stride_b, t_stride_j,
                                 d_stride_b, d_stride_k, d_stride_j);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  OverlapArgs oa{};
  oa.rs = RowSet{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                 d_stride_j, B, gamma + 1, K, gamma, temperature};
  oa.V = V;
  oa.vpr = (V + kVec - 1) / kVec;
  const int64_t cv = chunk_vectors(dtype);
  oa.cpr = (oa.vpr + cv - 1) / cv;
  oa.lnz_t = lnZ_target;
  oa.lnz_d = lnZ_draft;
  oa.part = reinterpret_cast<OverlapPartial*>(reinterpret_cast<char*>(workspace) + kCounterBytes);
  const int64_t units = B * gamma * oa.cpr;
  if (units >= (int64_t(1) << 31)) return SV_EINVAL;  // 32-bit unit indices
  oa.by_cpr = make_fastdiv(uint32_t(oa.cpr));
  oa.by_g = make_fastdiv(uint32_t(gamma));
  if (dtype == SV_BF16) {
    if (vec) launch_overlap<SV_BF16, true>(oa, units, st);
    else launch_overlap<SV_BF16, false>(oa, units, st);
  } else {
    if (vec) launch_overlap<SV_F32, true>(oa, units, st);
    else launch_overlap<SV_F32, false>(oa, units, st);
  }
  const int64_t chains = B * K;
  hipLaunchKernelGGL(alpha_law_kernel,
                     dim3(unsigned((chains + kWavesPerBlock - 1) / kWavesPerBlock)), dim3(kBlock),
                     0, st, oa.part, chains, K, gamma, oa.cpr, temperature, alpha, law);
  return launch_status();
}

int specverify_geometric_fanout(int64_t gamma, int64_t total, double ratio, int32_t* fanout) {
  if (!fanout || gamma < 1 || gamma > SV_MAX_GAMMA || total < 0 ||
      total > (gamma + 1) * int64_t(SV_MAX_FANOUT) || !(ratio > 0.0 && ratio <= 1.0))
    return SV_EINVAL;
  double share[SV_MAX_GAMMA + 1], exact[SV_MAX_GAMMA + 1], sum = 0.0;
  for (int64_t j = 0; j <= gamma; ++j) {
    share[j] = std::pow(ratio, double(j));
    sum += share[j];
  }
  int64_t used = 0;
  double rem[SV_MAX_GAMMA + 1];
  bool got[SV_MAX_GAMMA + 1];
  for (int64_t j = 0; j <= gamma; ++j) {
    exact[j] = double(total) * share[j] / sum;
    fanout[j] = int32_t(std::floor(exact[j]));
    rem[j] = exact[j] - double(fanout[j]);
    got[j] = false;
    used += fanout[j];
  }
  // one more to each of the largest remainders, ties to the smaller j
  for (int64_t left = total - used; left > 0; --left) {
    int64_t best = -1;
    double br = -1.0;
    for (int64_t j = 0; j <= gamma; ++j)
      if (!got[j] && rem[j] > br) {
        best = j;
        br = rem[j];
      }
    if (best < 0) break;
    got[best] = true;
    fanout[best] += 1;
  }
  for (int64_t j = 0; j <= gamma; ++j)
    if (fanout[j] > SV_MAX_FANOUT) return SV_EINVAL;
  return SV_OK;
}

int specverify_residual_topf(const void* target_logits, const void* draft_logits, int dtype,
                             int64_t B, int64_t K, int64_t gamma, int64_t V, int64_t t_stride_b,
                             int64_t t_stride_j, int64_t d_stride_b, int64_t d_stride_k,
                             int64_t d_stride_j, const float* temperature,
                             const double* lnZ_target, const double* lnZ_draft,
                             const int32_t* fanout, int32_t* cand, float* cand_weight,
                             void* stream) {
  if (!target_logits || !draft_logits || !temperature || !lnZ_target || !lnZ_draft || !fanout ||
      !cand)
    return SV_EINVAL;
  if (!sizes_ok(B, K, gamma, V)) return SV_EINVAL;
  if (t_stride_b < 0 || t_stride_j < 0 || d_stride_b < 0 || d_stride_k < 0 || d_stride_j < 0)
    return SV_EINVAL;
  if (check_dtype(dtype) != SV_OK) return SV_EDTYPE;
  TopFArgs ta{};
  if (!fill_fanout(fanout, gamma, ta)) return SV_EINVAL;
  if (ta.ftot == 0) return SV_OK;
  const int esz = esize(dtype);
  const bool vec = logits_vec_ok(target_logits, draft_logits, esz, t_stride_b, t_stride_j,
                                 d_stride_b, d_stride_k, d_stride_j);
  ta.rs = RowSet{target_logits, t_stride_b, t_stride_j, draft_logits, d_stride_b, d_stride_k,
                 d_stride_j, B, gamma + 1, K, gamma, temperature};
  ta.V = V;
  ta.vpr = (V + kVec - 1) / kVec;
  ta.lnz_t = lnZ_target;
  ta.lnz_d = lnZ_draft;
  ta.cand = cand;
  ta.cand_w = cand_weight;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t rows = B * K * (gamma + 1);
  const dim3 grid{unsigned(rows), 1u, 1u};
  // A wider sample gives a tighter first threshold (fewer admissions) for
  // twice the sample loads and more registers: it pays while the grid holds
  // one to a few workgroups per CU; below that the kernel is one workgroup's
  // latency, above it occupancy bounds the rate.
  const int64_t cus = device_cus();
  const bool wide = rows >= cus && rows <= int64_t(kTopFWideRowsPerCU) * cus;
  // at most three workgroups per CU: one round (B=64 gamma=8 V=128256: 126 vs
  // 139 us; grids of several rounds measured slower in this order)
  ta.bonus_last = rows <= 3 * cus ? 1 : 0;
  if (dtype == SV_BF16) {
    if (vec) launch_topf<SV_BF16, true>(wide, grid, st, ta);
    else launch_topf<SV_BF16, false>(wide, grid, st, ta);
  } else {
    if (vec) launch_topf<SV_F32, true>(wide, grid, st, ta);
    else launch_topf<SV_F32, false>(wide, grid, st, ta);
  }
  return launch_status();
}

int specverify_cache_lookup(const int32_t* cand, const int32_t* fanout, int64_t B, int64_t K,
                            int64_t gamma, const int32_t* accept_len, const int32_t* out_token,
                            int32_t* slot, void* stream) {
  if (!cand || !fanout || !accept_len || !out_token || !slot) return SV_EINVAL;
  if (B < 1 || K < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || B > (int64_t(1) << 40) / K)
    return SV_EINVAL;
  TopFArgs ta{};
  if (!fill_fanout(fanout, gamma, ta)) return SV_EINVAL;
  ta.rs.G = gamma;
  const int64_t chains = B * K;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(cache_lookup_kernel, dim3(unsigned((chains + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, st, cand, ta, chains, accept_len, out_token, slot);
  return launch_status();
}

int specverify_branch_prune(const float* logq, int64_t B, int64_t K, int64_t gamma,
                            double log_tau, int64_t keep, int32_t* keep_mask,
                            int32_t* prefix_len, double* conf, void* stream) {
  if (!logq || !keep_mask || B < 1 || K < 1 || gamma < 1 || gamma > SV_MAX_GAMMA ||
      K * gamma > SV_MAX_CHAIN_DECISIONS || keep < 0 || std::isnan(log_tau) ||
      B > (int64_t(1) << 40))
    return SV_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(branch_prune_kernel, dim3(unsigned((B + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, st, logq, B, K, gamma, log_tau, keep, keep_mask, prefix_len, conf);
  return launch_status();
}

int specverify_check_count(uint32_t* count, int reset) {
#ifdef SV_DEVICE_CHECKS
  if (!count) return SV_EINVAL;
  if (hipMemcpyFromSymbol(count, HIP_SYMBOL(sv_check_count), sizeof(uint32_t)) != hipSuccess)
    return SV_EHIP;
  if (reset) {
    const uint32_t zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(sv_check_count), &zero, sizeof zero) != hipSuccess)
      return SV_EHIP;
  }
  return SV_OK;
#else
  (void)count;
  (void)reset;
  return SV_ENOCHECKS;
#endif
}

int specverify_time_next_stream_kernel(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return SV_EINVAL;
  t_ev_before = static_cast<hipEvent_t>(before);
  t_ev_after = static_cast<hipEvent_t>(after);
  return SV_OK;
}

int specverify_version(void) { return 200; }

}  // extern "C"
