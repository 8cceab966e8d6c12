// Standalone per-row sampler kernel (tail_sample): one wave per row over the
// row's k candidates, see sampler_row.h for the rule.
#include "sampler_row.h"

namespace tail {
namespace {

constexpr int kRowsPerBlock = 4;

template <int P>
__global__ __launch_bounds__(64 * kRowsPerBlock) void sample_kernel(
    const float* __restrict__ vals, const int32_t* __restrict__ idx, int gbs, int k,
    const float* __restrict__ params, int ncols, int32_t* __restrict__ tokens) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + wave;
  if (row >= gbs) return;
  const RowParams p = load_params(params, ncols, row);
  const int32_t t = sample_row_wave<P>(vals + size_t(row) * k, idx + size_t(row) * k, k, p.top_k,
                                       p.top_p, p.temp, p.u, lane);
  if (lane == 0) tokens[row] = t;
}

}  // namespace

hipError_t launch_sample(const float* vals, const int32_t* idx, int gbs, int k,
                         const float* params, int ncols, int32_t* tokens, hipStream_t st) {
  dim3 grid((gbs + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
#define TAIL_SAMPLE_LAUNCH(P) \
  hipLaunchKernelGGL(sample_kernel<P>, grid, block, 0, st, vals, idx, gbs, k, params, ncols, tokens)
  if (k <= 64) TAIL_SAMPLE_LAUNCH(1);
  else if (k <= 128) TAIL_SAMPLE_LAUNCH(2);
  else if (k <= 256) TAIL_SAMPLE_LAUNCH(4);
  else if (k <= 512) TAIL_SAMPLE_LAUNCH(8);
  else TAIL_SAMPLE_LAUNCH(16);
#undef TAIL_SAMPLE_LAUNCH
  return hipGetLastError();
}

}  // namespace tail
