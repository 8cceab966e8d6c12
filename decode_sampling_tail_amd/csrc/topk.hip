// Global top-k of every logit row over the full vocabulary (GPT-OSS tail API
// page: Background -- the global top-k is computed locally over the full
// vocabulary -- and parameter "k"), optionally followed by the row's sampler.
//
// The lm_head kernels write the group maxima the select needs in their
// epilogue; for other inputs group_max_kernel / span_max_kernel compute them
// in one pass over the logits.  select_kernel runs the select of
// select_row.h with one 1024-thread workgroup per row.
#include "select_row.h"

namespace tail {
namespace {

constexpr int kGmThreads = 256;
constexpr int kSelThreads = 1024;

__device__ inline uint32_t fold_key(float f, int fold) {
  uint32_t u = __float_as_uint(f);
  if (fold && (u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN -> -inf
  return float_key(__uint_as_float(u));
}

__global__ __launch_bounds__(kGmThreads) void group_max_kernel(const float* __restrict__ logits,
                                                               int V, int gs, int groups, int fold,
                                                               uint32_t* __restrict__ gkey) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x * (kGmThreads / 64) + wave;
  if (g >= groups) return;
  const int row = blockIdx.y;
  const int start = g * gs;
  const int n = min(gs, V - start);
  const float* p = logits + size_t(row) * V + start;
  uint32_t m = 0;
  if (gs >= 4) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
    for (int i = lane; i < n / 4; i += 64) {
      float4 v = p4[i];
      m = max(m, max(max(fold_key(v.x, fold), fold_key(v.y, fold)),
                     max(fold_key(v.z, fold), fold_key(v.w, fold))));
    }
  } else {
    for (int i = lane; i < n; i += 64) m = max(m, fold_key(p[i], fold));
  }
  m = wave_max_u32(m);
  if (lane == 0) gkey[size_t(row) * groups + g] = m;
}

// Group maxima for groups of 4 to 256 columns (q = gs / 4 float4 each):
// every lane of a wave loads float4s, SPAN of them in flight, and the q lanes
// of each group combine their keys in place (quad permutations and row
// mirrors up to 16 lanes, shuffles across rows for 32 and 64), so every load
// instruction moves 1 KB whatever the group size; the group's first lane
// writes its key.  (group_max_kernel, one wave per group, serves the other
// sizes.)  One row (small batches) takes one load per lane, so that more
// waves share its latency; four from 8 rows up.
template <int LQ, int SPAN>
__global__ __launch_bounds__(kGmThreads) void span_max_kernel(const float* __restrict__ logits,
                                                              int V, int groups, int fold,
                                                              uint32_t* __restrict__ gkey) {
  constexpr int Q = 1 << LQ;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y;
  const int nf = V >> 2;  // float4 per row (V is a multiple of 8)
  const float4* p = reinterpret_cast<const float4*>(logits + size_t(row) * V);
  const int f0 = (blockIdx.x * (kGmThreads / 64) + wave) * (64 * SPAN) + lane;
  float4 v[SPAN];
#pragma unroll
  for (int s = 0; s < SPAN; ++s) {
    const int f = f0 + 64 * s;
    v[s] = p[f < nf ? f : nf - 1];  // past the row: a valid element, not used
  }
#pragma unroll
  for (int s = 0; s < SPAN; ++s) {
    const int f = f0 + 64 * s;
    uint32_t m = 0u;
    if (f < nf)
      m = max(max(fold_key(v[s].x, fold), fold_key(v[s].y, fold)),
              max(fold_key(v[s].z, fold), fold_key(v[s].w, fold)));
    if constexpr (Q >= 2) m = max(m, dpp_mov<0xb1>(m, m));   // quad_perm [1,0,3,2]
    if constexpr (Q >= 4) m = max(m, dpp_mov<0x4e>(m, m));   // quad_perm [2,3,0,1]
    if constexpr (Q >= 8) m = max(m, dpp_mov<0x141>(m, m));  // row_half_mirror
    if constexpr (Q >= 16) m = max(m, dpp_mov<0x140>(m, m)); // row_mirror
    if constexpr (Q >= 32) m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
    if constexpr (Q >= 64) m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
    if ((lane & (Q - 1)) == 0 && f < nf) gkey[size_t(row) * groups + (f >> LQ)] = m;
  }
}

template <int P, bool MIRROR>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, int V, int gs, int groups, int k,
    const uint32_t* __restrict__ gkey, int fold, float* __restrict__ vals,
    int32_t* __restrict__ idx, uint32_t* __restrict__ taps, const float* __restrict__ params,
    int ncols, int32_t* __restrict__ tokens) {
  __shared__ SelShared s;
  select_row<kSelThreads, MIRROR>(s, threadIdx.x, blockIdx.x, logits, V, gs, groups, k, gkey, fold, vals, idx,
                                  taps, params, ncols, tokens,
                                  [&](SelShared& sh, const RowParams& prm, int lane) {
                                    return sample_row_wave<P>(sh.top_v, sh.top_i, k, prm.top_k,
                                                              prm.top_p, prm.temp, prm.u, lane);
                                  });
}

}  // namespace

hipError_t launch_group_max(const float* logits, int gbs, int V, const TopkGeom& geom, bool fold,
                            uint32_t* gkey, hipStream_t st) {
  const int gs = geom.gs;
  if (gs >= 4 && gs <= 256) {
    const int span = gbs < 8 ? 1 : 4;
    const int per_block = 64 * span * (kGmThreads / 64);  // float4 per workgroup
    dim3 grid((V / 4 + per_block - 1) / per_block, gbs);
#define TAIL_SPAN_MAX(LQ)                                                                       \
  do {                                                                                          \
    if (span == 1)                                                                              \
      hipLaunchKernelGGL((span_max_kernel<LQ, 1>), grid, dim3(kGmThreads), 0, st, logits, V,    \
                         geom.groups, int(fold), gkey);                                         \
    else                                                                                        \
      hipLaunchKernelGGL((span_max_kernel<LQ, 4>), grid, dim3(kGmThreads), 0, st, logits, V,    \
                         geom.groups, int(fold), gkey);                                         \
  } while (0)
    switch (gs) {
      case 4: TAIL_SPAN_MAX(0); break;
      case 8: TAIL_SPAN_MAX(1); break;
      case 16: TAIL_SPAN_MAX(2); break;
      case 32: TAIL_SPAN_MAX(3); break;
      case 64: TAIL_SPAN_MAX(4); break;
      case 128: TAIL_SPAN_MAX(5); break;
      default: TAIL_SPAN_MAX(6); break;
    }
#undef TAIL_SPAN_MAX
    return hipGetLastError();
  }
  const int gpb = kGmThreads / 64;
  dim3 g1((geom.groups + gpb - 1) / gpb, gbs);
  hipLaunchKernelGGL(group_max_kernel, g1, dim3(kGmThreads), 0, st, logits, V, geom.gs, geom.groups,
                     int(fold), gkey);
  return hipGetLastError();
}

namespace {
template <bool MIRROR>
void select_dispatch(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                     const uint32_t* gkey, bool fold, float* vals, int32_t* idx, uint32_t* taps,
                     const float* params, int ncols, int32_t* tokens, hipStream_t st) {
  dim3 grid(gbs), block(kSelThreads);
#define TAIL_SELECT_LAUNCH(P)                                                                  \
  hipLaunchKernelGGL((select_kernel<P, MIRROR>), grid, block, 0, st, logits, V, geom.gs,       \
                     geom.groups, k, gkey, int(fold), vals, idx, taps, params, ncols, tokens)
  if (k <= 64) TAIL_SELECT_LAUNCH(1);
  else if (k <= 128) TAIL_SELECT_LAUNCH(2);
  else if (k <= 256) TAIL_SELECT_LAUNCH(4);
  else if (k <= 512) TAIL_SELECT_LAUNCH(8);
  else TAIL_SELECT_LAUNCH(16);
#undef TAIL_SELECT_LAUNCH
}
}  // namespace

hipError_t launch_select(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                         const uint32_t* gkey, bool mirror, bool fold, float* vals, int32_t* idx,
                         uint32_t* taps, const float* params, int ncols, int32_t* tokens,
                         hipStream_t st) {
  if (mirror)
    select_dispatch<true>(logits, gbs, V, k, geom, gkey, fold, vals, idx, taps, params, ncols,
                          tokens, st);
  else
    select_dispatch<false>(logits, gbs, V, k, geom, gkey, fold, vals, idx, taps, params, ncols,
                           tokens, st);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                       uint32_t* gkey_ws, bool mirror, bool fold, float* vals, int32_t* idx,
                       uint32_t* taps, hipStream_t st) {
  hipError_t e = launch_group_max(logits, gbs, V, geom, fold, gkey_ws, st);
  if (e != hipSuccess) return e;
  return launch_select(logits, gbs, V, k, geom, gkey_ws, mirror, fold, vals, idx, taps, nullptr, 0,
                       nullptr, st);
}

}  // namespace tail
