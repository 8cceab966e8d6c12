// Internal declarations shared by the host API and the kernel translation
// units of the decode-tail library (gfx950 only).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tail {

// ------------------------------------------------------------ small helpers
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Unpadded lane u -> physical hidden lane h, when every group of s lanes ends
// with one pad lane (s = 0: no padding).
__host__ __device__ inline int phys_lane(int u, int s) { return s ? u + u / (s - 1) : u; }

// Order-preserving key of a float: larger float <=> larger unsigned key.
// -0.0 is canonicalized to +0.0 so the two compare equal.
__device__ inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Geometry of the top-k: the row is cut into groups of `gs` (a power of two)
// columns; there must be at least k groups so that the k-th largest group
// maximum bounds the k-th largest logit from below, and at most
// kMaxGroups of them so the group maxima of one row fit in LDS.
constexpr int kMaxGroups = 8192;
struct TopkGeom {
  int gs;      // group size (columns)
  int groups;  // ceil(V / gs)
};
inline bool topk_geometry(int V, int k, TopkGeom* g) {
  int gs = 256;
  while (gs > 1 && (V + gs - 1) / gs < k) gs >>= 1;
  while ((V + gs - 1) / gs > kMaxGroups) gs <<= 1;
  g->gs = gs;
  g->groups = (V + gs - 1) / gs;
  return g->groups >= k && g->groups <= kMaxGroups;
}

// Launchers (each defined next to its kernels).  They assume validated
// arguments and return the launch status.
hipError_t launch_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H, int H_u,
                          int pad_s, float eps, bool deferred, float* y, float* r, hipStream_t st);

hipError_t launch_lm_head_gemv(const float* y, int ldy, const uint16_t* w, const float* row_scale,
                               int gbs, int H_u, int pad_s, int V, float* logits, hipStream_t st);

hipError_t launch_topk(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                       uint32_t* gkey_ws, float* vals, int32_t* idx, hipStream_t st);

hipError_t launch_sample(const float* vals, const int32_t* idx, int gbs, int k,
                         const float* params, int ncols, int32_t* tokens, hipStream_t st);

}  // namespace tail
