// Final RMSNorm of the post-MoE hidden rows (GPT-OSS tail API page,
// parameters "gamma", "eps", "hidden_actual", "hidden_states",
// "zero_interleaved_pad", "deferred_rms").
//
// One 256-thread workgroup per row.  The row is read once with coalesced
// loads, widened exactly to fp32 (fp16 via the hardware conversion, bf16 by a
// 16-bit shift), and its sum of squares is accumulated in fp64 in a fixed
// order (per-thread strided partials, then a fixed butterfly and a fixed
// cross-wave sum), so r is a correctly rounded fp32 of 1/sqrt(ms + eps) in
// all but pathological cases and every row gives the same bytes alone or in
// a batch.  Bytes moved per row: H * (dtype bytes + 4 for gamma + 4 for y).
#include "tail_internal.h"

#include <hip/hip_fp16.h>

namespace tail {
namespace {

constexpr int kThreads = 256;

template <int DT>
__device__ inline float load_hidden(const void* p, size_t i) {
  if constexpr (DT == 0) {
    return static_cast<const float*>(p)[i];
  } else if constexpr (DT == 1) {
    return __half2float(static_cast<const __half*>(p)[i]);
  } else {
    uint32_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(b << 16);
  }
}

__device__ inline double wave_sum(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const void* __restrict__ hidden,
                                                           const float* __restrict__ gamma, int H,
                                                           int H_u, int pad_s, float eps,
                                                           int deferred, float* __restrict__ y,
                                                           float* __restrict__ r_out) {
  __shared__ double s_part[kThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t base = size_t(row) * H;

  double ss = 0.0;
  for (int h = tid; h < H; h += kThreads) {
    bool pad = pad_s && (h % pad_s == pad_s - 1);
    if (!pad) {
      double x = load_hidden<DT>(hidden, base + h);
      ss = fma(x, x, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  double tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  double ms = tot / double(H_u);
  float r = float(1.0 / sqrt(ms + double(eps)));

  for (int h = tid; h < H; h += kThreads) {
    bool pad = pad_s && (h % pad_s == pad_s - 1);
    float out = 0.0f;
    if (!pad) {
      float x = load_hidden<DT>(hidden, base + h);
      float g = gamma[h];
      out = deferred ? x * g : (x * r) * g;
    }
    y[base + h] = out;
  }
  if (tid == 0 && r_out) r_out[row] = r;
}

}  // namespace

hipError_t launch_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H,
                          int H_u, int pad_s, float eps, bool deferred, float* y, float* r,
                          hipStream_t st) {
  dim3 grid(gbs), block(kThreads);
  switch (dtype) {
    case 0:
      hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), y, r);
      break;
    case 1:
      hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), y, r);
      break;
    default:
      hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), y, r);
      break;
  }
  return hipGetLastError();
}

}  // namespace tail
