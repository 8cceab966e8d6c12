// Per-row sampler over the top-k candidates (GPT-OSS tail API page,
// parameter "sampling_params": per-row [top_k, top_p, temperature] and the
// optional inverse-transform draw u, whose compiled-in default is 0.5; the
// greedy sampler of the GK decode design is the temperature-0 case).
//
// One wave per row; lane l holds candidates l*P .. l*P+P-1 (P = ceil(k/64)),
// so candidate order is lane order.  The softmax numerators, the running
// sums and the two cut comparisons are done in fp64, which keeps the CDF
// boundaries within ~1e-15 of an fp64 evaluation in candidate order.
//
//   kk = trunc(top_k), or k when top_k is not in [1, k+1)
//   T <= 0 (or NaN): token = idx[0]
//   e_i = exp((v_i - v_0) / T), i < kk;   S_i = e_0 + ... + e_i
//   m = 1 + min{i < kk : S_i >= top_p * S_{kk-1}}   (kk if none)
//   j = min{i < m : S_i > u * S_{m-1}}              (m-1 if none)
//   token = idx[j]
#include "tail_internal.h"

#include <climits>

namespace tail {
namespace {

constexpr int kRowsPerBlock = 4;

__device__ inline int wave_min_i32(int v) {
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}

template <int P>
__global__ __launch_bounds__(64 * kRowsPerBlock) void sample_kernel(
    const float* __restrict__ vals, const int32_t* __restrict__ idx, int gbs, int k,
    const float* __restrict__ params, int ncols, int32_t* __restrict__ tokens) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + wave;
  if (row >= gbs) return;
  const float* pr = params + size_t(row) * ncols;
  const float top_k = pr[0], top_p = pr[1], temp = pr[2];
  const float u = ncols == 4 ? pr[3] : 0.5f;
  const int kk = (top_k >= 1.0f && top_k < float(k) + 1.0f) ? int(top_k) : k;
  const float* v = vals + size_t(row) * k;
  const int32_t* ix = idx + size_t(row) * k;

  if (!(temp > 0.0f)) {
    if (lane == 0) tokens[row] = ix[0];
    return;
  }

  const double v0 = v[0], T = temp;
  double S[P];
  double run = 0.0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int i = lane * P + j;
    const double e = i < kk ? exp((double(v[i]) - v0) / T) : 0.0;
    run += e;
    S[j] = run;
  }
  // exclusive prefix of the lane totals, in lane order
  double incl = run;
  for (int off = 1; off < 64; off <<= 1) {
    const double t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const double excl = incl - run;
#pragma unroll
  for (int j = 0; j < P; ++j) S[j] += excl;

  auto S_at = [&](int i) {  // S_i, broadcast from its owner lane
    double mine = 0.0;
#pragma unroll
    for (int j = 0; j < P; ++j)
      if (j == i % P) mine = S[j];
    return __shfl(mine, i / P, 64);
  };

  const double total = S_at(kk - 1);
  const double pthr = double(top_p) * total;
  int first = INT_MAX;
#pragma unroll
  for (int j = P - 1; j >= 0; --j) {
    const int i = lane * P + j;
    if (i < kk && S[j] >= pthr) first = i;
  }
  first = wave_min_i32(first);
  const int m = first == INT_MAX ? kk : first + 1;

  const double uthr = double(u) * S_at(m - 1);
  first = INT_MAX;
#pragma unroll
  for (int j = P - 1; j >= 0; --j) {
    const int i = lane * P + j;
    if (i < m && S[j] > uthr) first = i;
  }
  first = wave_min_i32(first);
  const int jsel = first == INT_MAX ? m - 1 : first;
  if (lane == 0) tokens[row] = ix[jsel];
}

}  // namespace

hipError_t launch_sample(const float* vals, const int32_t* idx, int gbs, int k,
                         const float* params, int ncols, int32_t* tokens, hipStream_t st) {
  dim3 grid((gbs + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (k <= 64)
    hipLaunchKernelGGL(sample_kernel<1>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens);
  else if (k <= 128)
    hipLaunchKernelGGL(sample_kernel<2>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens);
  else if (k <= 256)
    hipLaunchKernelGGL(sample_kernel<4>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens);
  else if (k <= 512)
    hipLaunchKernelGGL(sample_kernel<8>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens);
  else
    hipLaunchKernelGGL(sample_kernel<16>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens);
  return hipGetLastError();
}

}  // namespace tail
