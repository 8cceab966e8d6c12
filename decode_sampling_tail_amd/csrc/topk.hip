// Global top-k of every logit row over the full vocabulary (GPT-OSS tail API
// page: Background -- the global top-k is computed locally over the full
// vocabulary -- and parameter "k").
//
// Two kernels:
//
// 1. group_max_kernel: the row is cut into groups of gs columns (gs a power of
//    two chosen so there are at least k groups); one wave reduces one group to
//    the largest order-preserving key of its values.  This is the only pass
//    over the whole logit row (V * 4 bytes per row).
//
// 2. select_kernel: one 1024-thread workgroup per row.
//    a. t0 = the k-th largest group maximum (binary search on the key, counts
//       over LDS).  At least k groups have a maximum >= t0 and each such
//       maximum is an element, so at least k elements are >= t0: every member
//       of the top-k is >= t0, and only groups whose maximum is >= t0 can hold
//       one.  For Gaussian-like rows this leaves a few hundred candidates.
//    b. The waves scan only those groups and append every (key, index) with
//       key >= t0 to an LDS list (wave-aggregated atomic slot allocation).
//    c. Candidates are ranked by the composite 64-bit key
//       (value key << 32) | ~index, so larger value first and, for equal
//       values, lower index first; rank < k is written out.  Long lists are
//       first pruned to the keys >= the k-th largest value key.
//    d. If more than kCap candidates pass (massive ties), the exact k-th
//       largest value v* and, if needed, the index cut among the elements
//       equal to v* are found by counting passes over the candidate groups,
//       and only the k winners are collected.  Slow, but exact for any input.
//
// Values are copied from the logits themselves, so -0.0 keeps its sign while
// comparing equal to +0.0.
#include "tail_internal.h"

namespace tail {
namespace {

constexpr int kGmThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCap = 4096;                       // LDS candidate capacity
constexpr int kPerThread = kCap / kSelThreads;  // candidates per thread in registers

__device__ inline uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

__global__ __launch_bounds__(kGmThreads) void group_max_kernel(const float* __restrict__ logits,
                                                               int V, int gs, int groups,
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
      m = max(m, max(max(float_key(v.x), float_key(v.y)), max(float_key(v.z), float_key(v.w))));
    }
  } else {
    for (int i = lane; i < n; i += 64) m = max(m, float_key(p[i]));
  }
  m = wave_max_u32(m);
  if (lane == 0) gkey[size_t(row) * groups + g] = m;
}

struct SelShared {
  uint32_t g[kMaxGroups];  // group maximum keys of the row
  uint64_t c[kCap];        // candidate composite keys
  uint32_t red[2][kSelWaves];
  uint32_t cnt;
};

// Block-wide reductions; every thread gets the result.  Two alternating
// buffers make one barrier per call enough.
struct Block {
  SelShared& s;
  int wave, lane, parity;
  __device__ uint32_t sum(uint32_t v) {
    v = wave_sum_u32(v);
    if (lane == 0) s.red[parity][wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) t += s.red[parity][i];
    parity ^= 1;
    return t;
  }
  __device__ uint32_t maxv(uint32_t v) {
    v = wave_max_u32(v);
    if (lane == 0) s.red[parity][wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) t = max(t, s.red[parity][i]);
    parity ^= 1;
    return t;
  }
  __device__ uint32_t minv(uint32_t v) {
    v = wave_min_u32(v);
    if (lane == 0) s.red[parity][wave] = v;
    __syncthreads();
    uint32_t t = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) t = min(t, s.red[parity][i]);
    parity ^= 1;
    return t;
  }
};

__device__ inline uint64_t composite(uint32_t key, int e) {
  return (uint64_t(key) << 32) | uint64_t(~uint32_t(e));
}

// Append the lanes' (key, e) where pred holds; slots past kCap are counted
// but not stored.
__device__ inline void wave_append(SelShared& s, bool pred, uint32_t key, int e, int lane) {
  uint64_t mask = __ballot(pred);
  if (mask == 0) return;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&s.cnt, (uint32_t)__popcll(mask));
  base = __shfl((int)base, 0, 64);
  if (pred) {
    uint32_t pos = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (pos < kCap) s.c[pos] = composite(key, e);
  }
}

// Predicate of a candidate: key > kv, or key == kv and index < ilim.
__device__ inline bool wins(uint32_t key, int e, uint32_t kv, int ilim) {
  return key > kv || (key == kv && e < ilim);
}

// Visit every element of every group whose maximum is >= t0 (the only groups
// that can hold a top-k member).  Wave w takes groups w, w + 16, ...; each
// lane handles four consecutive columns per 256-column chunk.
template <typename F>
__device__ inline void for_candidate_groups(const SelShared& s, const float* row, int V, int gs,
                                            int groups, uint32_t t0, int wave, int lane, F&& f) {
  for (int g = wave; g < groups; g += kSelWaves) {
    if (s.g[g] < t0) continue;
    const int start = g * gs;
    const int n = min(gs, V - start);
    if (gs >= 4) {
      for (int i0 = 0; i0 < n; i0 += 256) {
        const int e0 = start + i0 + lane * 4;
        const bool in = i0 + lane * 4 < n;
        float4 v = in ? *reinterpret_cast<const float4*>(row + e0) : make_float4(0, 0, 0, 0);
        f(in, float_key(v.x), e0);
        f(in, float_key(v.y), e0 + 1);
        f(in, float_key(v.z), e0 + 2);
        f(in, float_key(v.w), e0 + 3);
      }
    } else {
      const bool in = lane < n;
      f(in, in ? float_key(row[start + lane]) : 0u, start + lane);
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ logits,
                                                             int V, int gs, int groups, int k,
                                                             const uint32_t* __restrict__ gkey,
                                                             float* __restrict__ vals,
                                                             int32_t* __restrict__ idx) {
  __shared__ SelShared s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row_id = blockIdx.x;
  const float* row = logits + size_t(row_id) * V;
  Block blk{s, wave, lane, 0};

  // a. group maxima -> t0, the k-th largest of them
  uint32_t lo_l = 0xFFFFFFFFu, hi_l = 0;
  for (int g = tid; g < groups; g += kSelThreads) {
    uint32_t v = gkey[size_t(row_id) * groups + g];
    s.g[g] = v;
    lo_l = min(lo_l, v);
    hi_l = max(hi_l, v);
  }
  if (tid == 0) s.cnt = 0;
  uint64_t lo = blk.minv(lo_l);
  uint64_t hi = uint64_t(blk.maxv(hi_l)) + 1;
  while (hi - lo > 1) {  // count(>= lo) >= k > count(>= hi)
    uint64_t mid = (lo + hi) >> 1;
    uint32_t c = 0;
    for (int g = tid; g < groups; g += kSelThreads) c += s.g[g] >= mid;
    if (blk.sum(c) >= uint32_t(k)) lo = mid; else hi = mid;
  }
  const uint32_t t0 = uint32_t(lo);

  // b. collect every element >= t0
  uint32_t kv = t0;
  int ilim = V;
  for_candidate_groups(s, row, V, gs, groups, t0, wave, lane,
                       [&](bool in, uint32_t key, int e) { wave_append(s, in && key >= t0, key, e, lane); });
  __syncthreads();
  uint32_t n = s.cnt;

  // d. too many candidates: find the exact cut by counting passes
  if (n > uint32_t(kCap)) {
    auto count = [&](uint32_t kv_, int ilim_) {
      uint32_t c = 0;
      for_candidate_groups(s, row, V, gs, groups, t0, wave, lane,
                           [&](bool in, uint32_t key, int e) { c += in && wins(key, e, kv_, ilim_); });
      return blk.sum(c);
    };
    uint64_t vlo = t0, vhi = hi;  // count(>= vlo) >= k > count(>= vhi)
    while (vhi - vlo > 1) {
      uint64_t mid = (vlo + vhi) >> 1;
      if (count(uint32_t(mid), V) >= uint32_t(k)) vlo = mid; else vhi = mid;
    }
    kv = uint32_t(vlo);
    if (count(kv, V) > uint32_t(kCap)) {  // ties at v*: keep the lowest indices
      int ilo = 0, ihi = V;               // count(kv, ilo) < k <= count(kv, ihi)
      while (ihi - ilo > 1) {
        int mid = (ilo + ihi) >> 1;
        if (count(kv, mid) >= uint32_t(k)) ihi = mid; else ilo = mid;
      }
      ilim = ihi;
    }
    __syncthreads();
    if (tid == 0) s.cnt = 0;
    __syncthreads();
    for_candidate_groups(s, row, V, gs, groups, t0, wave, lane, [&](bool in, uint32_t key, int e) {
      wave_append(s, in && wins(key, e, kv, ilim), key, e, lane);
    });
    __syncthreads();
    n = s.cnt;
  }

  // c. prune long lists to the keys >= the k-th largest value key
  if (n > uint32_t(2 * k)) {
    uint64_t mine[kPerThread];
    uint32_t mlo = 0xFFFFFFFFu, mhi = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      int i = tid + j * kSelThreads;
      mine[j] = i < int(n) ? s.c[i] : 0;
      if (i < int(n)) {
        mlo = min(mlo, uint32_t(mine[j] >> 32));
        mhi = max(mhi, uint32_t(mine[j] >> 32));
      }
    }
    uint64_t plo = blk.minv(mlo), phi = uint64_t(blk.maxv(mhi)) + 1;
    while (phi - plo > 1) {
      uint64_t mid = (plo + phi) >> 1;
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) c += (tid + j * kSelThreads < int(n)) && (mine[j] >> 32) >= mid;
      if (blk.sum(c) >= uint32_t(k)) plo = mid; else phi = mid;
    }
    const uint32_t vstar = uint32_t(plo);
    if (tid == 0) s.cnt = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      int i = tid + j * kSelThreads;
      bool keep = i < int(n) && uint32_t(mine[j] >> 32) >= vstar;
      uint64_t m = __ballot(keep);
      if (m) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&s.cnt, (uint32_t)__popcll(m));
        base = __shfl((int)base, 0, 64);
        if (keep) s.c[base + __popcll(m & ((1ull << lane) - 1ull))] = mine[j];
      }
    }
    __syncthreads();
    n = s.cnt;
  }

  // rank by composite key; the k best go out in order
  for (int i = tid; i < int(n); i += kSelThreads) {
    const uint64_t ci = s.c[i];
    uint32_t rank = 0;
    for (int j = 0; j < int(n); ++j) rank += s.c[j] > ci;
    if (rank < uint32_t(k)) {
      const int e = int(~uint32_t(ci));
      vals[size_t(row_id) * k + rank] = row[e];
      idx[size_t(row_id) * k + rank] = e;
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                       uint32_t* gkey_ws, float* vals, int32_t* idx, hipStream_t st) {
  const int gpb = kGmThreads / 64;
  dim3 g1((geom.groups + gpb - 1) / gpb, gbs);
  hipLaunchKernelGGL(group_max_kernel, g1, dim3(kGmThreads), 0, st, logits, V, geom.gs,
                     geom.groups, gkey_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(gbs), dim3(kSelThreads), 0, st, logits, V, geom.gs,
                     geom.groups, k, gkey_ws, vals, idx);
  return hipGetLastError();
}

}  // namespace tail
