// Final RMSNorm of the post-MoE hidden rows (GPT-OSS tail API page,
// parameters "gamma", "eps", "hidden_actual", "hidden_states",
// "zero_interleaved_pad", "deferred_rms").
//
// One 256-thread workgroup per row.  Each thread owns lanes t, t+256, ...
// of the row; up to 16 of them (H <= 4096) are loaded in one unrolled burst
// so the row costs one memory latency, and stay in registers for the output
// pass.  Longer rows are processed in bursts of 4096 lanes and re-read.  The
// values are widened exactly to fp32 (fp16 by the hardware conversion, bf16
// by a 16-bit shift); the sum of squares is accumulated in fp64 in a fixed
// order (per-thread ascending lanes, a fixed butterfly, a fixed cross-wave
// sum), so r = fp32(1/sqrt(ms + eps)) is the same for a row alone or in a
// batch.  Bytes per row: H * (dtype bytes + 4 gamma + 4 output).
#include "tail_internal.h"

namespace tail {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 16;  // lanes per thread per burst
constexpr int kBurst = kThreads * kPer;

__device__ inline double wave_sum(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ inline bool is_pad(int h, int pad_s) { return pad_s && (h % pad_s == pad_s - 1); }

// Bursts load every slot unconditionally (slots past the row from a clamped
// valid index) and zero the out-of-range slots after widening: a load inside
// a branch that widened its value (or that the compiler widened there) had
// to complete before the branch closed, one memory latency per element.
template <int DT>
__device__ inline void load_burst(const void* hidden, size_t base, int h0, int H, int pad_s, int tid,
                                  float (&x)[kPer]) {
  uint32_t xb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int h = h0 + tid + i * kThreads;
    xb[i] = load_bits<DT>(hidden, base + (h < H ? h : H - 1));
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int h = h0 + tid + i * kThreads;
    x[i] = (h < H && !is_pad(h, pad_s)) ? widen_bits<DT>(xb[i]) : 0.0f;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const void* __restrict__ hidden,
                                                           const float* __restrict__ gamma, int H,
                                                           int H_u, int pad_s, float eps,
                                                           int deferred, int page,
                                                           float* __restrict__ y,
                                                           float* __restrict__ r_out) {
  __shared__ double s_part[kThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t base = size_t(row) * H;

  float x[kPer];
  double ss = 0.0;
  for (int h0 = 0; h0 < H; h0 += kBurst) {
    load_burst<DT>(hidden, base, h0, H, pad_s, tid, x);
#pragma unroll
    for (int i = 0; i < kPer; ++i) ss = fma(double(x[i]), double(x[i]), ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  const double tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float r = float(1.0 / sqrt(tot / double(H_u) + double(eps)));

  for (int h0 = 0; h0 < H; h0 += kBurst) {
    if (H > kBurst) load_burst<DT>(hidden, base, h0, H, pad_s, tid, x);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int h = h0 + tid + i * kThreads;
      if (h < H) {
        float out = 0.0f;
        if (!is_pad(h, pad_s)) {
          const float g = gamma[h];
          out = deferred ? x[i] * g : (x[i] * r) * g;
          if (page) out = bf16_round(out);
        }
        y[base + h] = out;
      }
    }
  }
  if (tid == 0 && r_out) r_out[row] = r;
}

// ---------------------------------------------------------------------------
// Activation producer for the matrix-core lm_head.  One workgroup per batch
// row (rows gbs..rows_pad-1 are written as zeros).  K is the number of lanes
// the contraction runs over (H_u when pad lanes are skipped, else H); the
// mean square always divides by H_u.  The row's activation
//   NORM:  y = x * gamma (deferred rms; r is written to r_out) or (x * r) * gamma
//   !NORM: y = the given fp32 row
// is taken over the real lanes only (compacted: unpadded index u), zero-padded
// to Kp, and split into NT bf16 terms t_0 = bf16(y), t_1 = bf16(y - t_0),
// t_2 = bf16(y - t_0 - t_1) (round to nearest even; each difference is exact
// in fp32).
//
// Output layout (L): ready operand fragments of the matrix-core kernels,
// 1 KB each (64 lanes x 8 bf16).
//  L = 0, v_mfma_f32_16x16x32_bf16: row tile rt = rows 16 rt .. 16 rt + 15,
//    K block kb = unpadded lanes 32 kb .. 32 kb + 31; lane 16 g + s carries row
//    16 rt + s at K slots 8 g .. 8 g + 7, and K slot 8 g + j is unpadded lane
//    32 kb + 4 g + (j & 3) + 16 (j >> 2).  Ordered (term, row tile, K block),
//    so the fragments of one row tile for consecutive K blocks are contiguous.
//  L = 1, v_mfma_f32_32x32x16_bf16: row tile = rows 32 rt .. 32 rt + 31, K
//    block = unpadded lanes 16 kb .. 16 kb + 15; lane 32 h + n carries row
//    32 rt + n at unpadded lanes 16 kb + 8 h .. + 7 (natural order).  Ordered
//    (K block, term, row tile), so all the fragments one K-step of the
//    large-batch kernel reads are contiguous.
// Each thread produces one 16-byte lane (an "octet") per term.  gz (may be
// NULL): this row's [groups] entries are cleared (the matrix-core kernels
// combine the maxima of the key groups that straddle two of their tiles
// there with atomic maxima); fs_out (may be NULL): row 0 stores the
// large-batch kernel's select arguments there and clears their counters (its
// grid barrier's and row queue's).
__device__ inline uint16_t bf16_rne(float f) { return uint16_t(bf16_rne_bits(__float_as_uint(f))); }
__device__ inline float bf16_val(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int L>
__device__ inline int octet_lane(int o, int j) {  // unpadded lane of slot j of octet o
  if constexpr (L == 0) return 32 * (o / 4) + 4 * (o % 4) + (j & 3) + 16 * (j >> 2);
  else return 8 * o + j;
}

template <int DT, int NT, bool NORM, int L>
__global__ __launch_bounds__(kThreads) void split_kernel(const void* __restrict__ src,
                                                         const float* __restrict__ gamma, int H,
                                                         int H_u, int K, int pad_s, FastDiv pdiv,
                                                         float eps, int deferred, int gbs,
                                                         int rows_pad, int Kp,
                                                         uint16_t* __restrict__ act,
                                                         float* __restrict__ r_out,
                                                         uint32_t* __restrict__ gz, int groups,
                                                         FusedSelect fs, FusedSelect* fs_out) {
  __shared__ double s_part[kThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // 16-byte lane of octet o for term t
  auto lane_ptr = [&](int t, int o) {
    if constexpr (L == 0) {  // o = 4 kb + g
      const size_t frag = (size_t(t) * (rows_pad / 16) + row / 16) * (Kp / 32) + o / 4;
      return reinterpret_cast<uint4*>(act + (frag * 64 + (o % 4) * 16 + row % 16) * 8);
    } else {  // o = 2 kb + h
      const size_t frag = (size_t(o / 2) * NT + t) * (rows_pad / 32) + row / 32;
      return reinterpret_cast<uint4*>(act + (frag * 64 + (o % 2) * 32 + row % 32) * 8);
    }
  };
  if (gz && row < gbs)
    for (int i = tid; i < groups; i += kThreads) gz[size_t(row) * groups + i] = 0u;
  if (fs_out && row == 0) {
    if (tid == 0) *fs_out = fs;
    for (int i = tid; i < fs.nsync; i += kThreads) fs.sync[i] = 0u;
  }
  if (row >= gbs) {
    for (int o = tid; o < Kp / 8; o += kThreads)
#pragma unroll
      for (int t = 0; t < NT; ++t) *lane_ptr(t, o) = make_uint4(0, 0, 0, 0);
    return;
  }
  const size_t base = size_t(row) * H;
  constexpr int kOct = kPer / 8;  // octets per thread per burst
  // loads the lanes of octets o0 + tid + i * kThreads (zero past K)
  auto load_octets = [&](int o0, float (&x)[kOct][8], float (&g)[kOct][8]) {
    uint32_t xb[kOct][8];
#pragma unroll
    for (int i = 0; i < kOct; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = o0 + tid + i * kThreads;
        const int u = octet_lane<L>(o, j);
        const int uc = u < K ? u : K - 1;
        const int h = pad_s ? uc + int(fastdiv(uint32_t(uc), pdiv)) : uc;
        xb[i][j] = load_bits<DT>(src, base + h);
        g[i][j] = 1.0f;
        if constexpr (NORM) g[i][j] = gamma[h];
      }
#pragma unroll
    for (int i = 0; i < kOct; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = o0 + tid + i * kThreads;
        const int u = octet_lane<L>(o, j);
        x[i][j] = u < K ? widen_bits<DT>(xb[i][j]) : 0.0f;
      }
  };
  // splits and stores the loaded octets
  auto emit_octets = [&](int o0, const float (&x)[kOct][8], const float (&g)[kOct][8], float r) {
#pragma unroll
    for (int i = 0; i < kOct; ++i) {
      const int o = o0 + tid + i * kThreads;
      if (o >= Kp / 8) continue;
      uint16_t term[NT][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int u = octet_lane<L>(o, j);
        float y = 0.0f;
        if (u < K) {
          if constexpr (NORM) y = deferred ? x[i][j] * g[i][j] : (x[i][j] * r) * g[i][j];
          else y = x[i][j];
        }
        float rem = y;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          term[t][j] = bf16_rne(rem);
          rem = rem - bf16_val(term[t][j]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint4 v;
        v.x = uint32_t(term[t][0]) | (uint32_t(term[t][1]) << 16);
        v.y = uint32_t(term[t][2]) | (uint32_t(term[t][3]) << 16);
        v.z = uint32_t(term[t][4]) | (uint32_t(term[t][5]) << 16);
        v.w = uint32_t(term[t][6]) | (uint32_t(term[t][7]) << 16);
        *lane_ptr(t, o) = v;
      }
    }
  };
  auto finish_r = [&](double ss) {  // fixed-order block sum of the per-thread partials
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    const double tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    const float r = float(1.0 / sqrt(tot / double(H_u) + double(eps)));
    if (tid == 0 && r_out) r_out[row] = r;
    return r;
  };

  if (Kp / 8 <= kOct * kThreads) {
    // the whole row in one burst, kept in registers: one memory latency.
    // Deferred: the terms do not depend on r, so they are stored first and r
    // (a block reduction) is finished while the stores drain
    float x[kOct][8], g[kOct][8];
    load_octets(0, x, g);
    if (!NORM || deferred) emit_octets(0, x, g, 1.0f);
    if constexpr (NORM) {
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < kOct; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fma(double(x[i][j]), double(x[i][j]), ss);
      const float r = finish_r(ss);
      if (!deferred) emit_octets(0, x, g, r);
    }
    return;
  }
  // longer rows: the sum of squares first, then the split, burst by burst
  float r = 1.0f;
  if constexpr (NORM) {
    float x[kPer];
    double ss = 0.0;
    for (int h0 = 0; h0 < H; h0 += kBurst) {
      load_burst<DT>(src, base, h0, H, pad_s, tid, x);
#pragma unroll
      for (int i = 0; i < kPer; ++i) ss = fma(double(x[i]), double(x[i]), ss);
    }
    r = finish_r(ss);
  }
  for (int o0 = 0; o0 < Kp / 8; o0 += kOct * kThreads) {
    float x[kOct][8], g[kOct][8];
    load_octets(o0, x, g);
    emit_octets(o0, x, g, r);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H,
                          int H_u, int pad_s, float eps, bool deferred, bool page, float* y,
                          float* r, hipStream_t st) {
  dim3 grid(gbs), block(kThreads);
  switch (dtype) {
    case 0:
      hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), int(page), y, r);
      break;
    case 1:
      hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), int(page), y, r);
      break;
    default:
      hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, st, hidden, gamma, H, H_u, pad_s, eps,
                         int(deferred), int(page), y, r);
      break;
  }
  return hipGetLastError();
}

}  // namespace tail

namespace tail {

hipError_t launch_split(const void* src, int dtype, bool norm, const float* gamma, int gbs, int H,
                        int H_u, int K, int pad_s, float eps, bool deferred, int nt, int layout,
                        int rows_pad, int Kp, uint16_t* act, float* r, uint32_t* gz, int groups,
                        const FusedSelect& fs, FusedSelect* fs_out, hipStream_t st) {
  const FastDiv pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  dim3 grid(rows_pad), block(kThreads);
#define TAIL_SPLIT(DT, NT, NORM, L)                                                              \
  hipLaunchKernelGGL((split_kernel<DT, NT, NORM, L>), grid, block, 0, st, src, gamma, H, H_u, K, \
                     pad_s, pdiv, eps, int(deferred), gbs, rows_pad, Kp, act, r, gz, groups, fs, fs_out)
#define TAIL_SPLIT_DT(NT, L)                    \
  do {                                          \
    if (!norm) TAIL_SPLIT(0, NT, false, L);     \
    else if (dtype == 0) TAIL_SPLIT(0, NT, true, L); \
    else if (dtype == 1) TAIL_SPLIT(1, NT, true, L); \
    else TAIL_SPLIT(2, NT, true, L);            \
  } while (0)
  // two terms (the default precision) or one (the page-precision mode)
  if (nt == 2 && layout == 0) TAIL_SPLIT_DT(2, 0);
  else if (nt == 2 && layout == 1) TAIL_SPLIT_DT(2, 1);
  else if (nt == 1 && layout == 0) TAIL_SPLIT_DT(1, 0);
  else if (nt == 1 && layout == 1) TAIL_SPLIT_DT(1, 1);
  else return hipErrorInvalidValue;
#undef TAIL_SPLIT_DT
#undef TAIL_SPLIT
  return hipGetLastError();
}

}  // namespace tail
