// One wave samples one row from its k candidates (GPT-OSS tail API page,
// parameter "sampling_params": per-row [top_k, top_p, temperature] plus the
// optional inverse-transform draw u, 0.5 when absent; temperature 0 is the
// greedy argmax of the GK decode design).  Shared by the standalone sampler
// kernel and the fused top-k + sampler kernel.
//
// Lane l owns candidates l*P .. l*P+P-1 (P = ceil(k/64)), so candidate order
// is lane order.  The softmax numerators, the running sums and both cut
// comparisons are evaluated in fp64:
//
//   kk = trunc(top_k), or k when top_k is not in [1, k+1)
//   T <= 0 (or NaN): token = idx[0]
//   e_i = exp((v_i - v_0) / T), i < kk;   S_i = e_0 + ... + e_i
//   m = 1 + min{i < kk : S_i >= top_p * S_{kk-1}}   (kk if none)
//   j = min{i < m : S_i > u * S_{m-1}}              (m-1 if none)
//   token = idx[j]
#pragma once

#include <climits>

#include "tail_internal.h"

namespace tail {

// vals / ix: the row's candidates in descending order (global or LDS memory).
// Returns the token on every lane.
template <int P, typename VP, typename IP>
__device__ inline int32_t sample_row_wave(VP vals, IP ix, int k, float top_k, float top_p,
                                          float temp, float u, int lane) {
  const int kk = (top_k >= 1.0f && top_k < float(k) + 1.0f) ? int(top_k) : k;
  if (!(temp > 0.0f)) return ix[0];

  const double v0 = vals[0], T = temp;
  double S[P];
  double run = 0.0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int i = lane * P + j;
    const double e = i < kk ? exp((double(vals[i]) - v0) / T) : 0.0;
    run += e;
    S[j] = run;
  }
  double incl = run;  // inclusive prefix of the lane totals, in lane order
  for (int off = 1; off < 64; off <<= 1) {
    const double t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const double excl = incl - run;
#pragma unroll
  for (int j = 0; j < P; ++j) S[j] += excl;

  // a lane's value read by every lane (the source lane is the same on all of
  // them: v_readlane, no LDS round trip)
  auto read_lane = [](double v, int src) {
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(b), src);
    const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(b >> 32), src);
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
  };
  auto S_at = [&](int i) {  // S_i broadcast from its owner lane
    double mine = 0.0;
#pragma unroll
    for (int j = 0; j < P; ++j)
      if (j == i % P) mine = S[j];
    return read_lane(mine, __builtin_amdgcn_readfirstlane(i / P));
  };

  // first candidate (in lane-major order) meeting a cut: the first lane with a
  // hit, then that lane's first hit
  auto first_hit = [&](int lim, double thr, bool inclusive) {
    int mine = INT_MAX;
#pragma unroll
    for (int j = P - 1; j >= 0; --j) {
      const int i = lane * P + j;
      if (i < lim && (inclusive ? S[j] >= thr : S[j] > thr)) mine = i;
    }
    const uint64_t hits = __ballot(mine != INT_MAX);
    return hits ? int(__builtin_amdgcn_readlane(uint32_t(mine), __ffsll((unsigned long long)hits) - 1))
                : INT_MAX;
  };

  const int first_p = first_hit(kk, double(top_p) * S_at(kk - 1), true);
  const int m = first_p == INT_MAX ? kk : first_p + 1;
  const int first = first_hit(m, double(u) * S_at(m - 1), false);
  return ix[first == INT_MAX ? m - 1 : first];
}

// Row parameters from a [gbs, ncols] fp32 array (u = 0.5 without a 4th column).
struct RowParams {
  float top_k, top_p, temp, u;
};
__device__ inline RowParams load_params(const float* params, int ncols, int row) {
  const float* p = params + size_t(row) * ncols;
  return RowParams{p[0], p[1], p[2], ncols == 4 ? p[3] : 0.5f};
}

}  // namespace tail
