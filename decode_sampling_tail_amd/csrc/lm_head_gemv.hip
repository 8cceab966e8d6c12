// lm_head contraction, weight-streaming form for small batches (GPT-OSS tail
// API page, parameter "lm_head_weight_t": [H, V] bf16, already transposed and
// C-contiguous), optionally with the final RMSNorm fused into its prologue
// (parameters "gamma", "eps", "hidden_actual", "deferred_rms").
//
// logits[b, v] = scale[b] * sum_u y[b, u] * W[h(u), v]
//
// The weight (K * V * 2 bytes, 1.16 GB for GPT-OSS) is read exactly once;
// that read is the roofline of the whole tail at small batch.
//
// Mapping: a workgroup of W waves (4 by default) owns a slab of 512 consecutive
// vocabulary columns; lane l of every wave owns columns 8l..8l+7 of the slab,
// read as one non-temporal 16-byte load per weight row (a wave reads 1 KB
// of a row per load).  The W waves split the K contraction lanes into W
// contiguous ranges and keep NB x 8 fp32 partial sums each; loads run one
// batch of U rows ahead of the FMAs.  Partials are combined through LDS in a
// fixed tree (step d adds wave w + d into wave w, d = W/2 .. 1; for W = 4:
// (p0+p2) + (p1+p3)), so a column's sum depends only on
// K and the shape, never on the column's position or on the other rows.
//
// Activations: SRC < 0 takes a given fp32 y [gbs, H], scale = row_scale (or
// 1).  SRC = -2 copies each wave's K range of the NB rows into an LDS table
// first (compacted over the K lanes, like the fused table below); SRC = -1,
// for rows too wide for LDS, reads y in the loop (row index wave-uniform), at
// the cost of NB x U extra loads per batch.  SRC = hidden
// dtype (0 fp32, 1 fp16, 2 bf16) fuses the RMSNorm: the prologue widens the
// NB hidden rows exactly, accumulates each row's sum of squares in fp64 in a
// fixed order (per wave over its lanes, then the W wave partials in order),
// and stores y compacted over the K lanes in LDS, with
// r = fp32(1 / sqrt(sum / H_u + eps)).  Deferred: each wave fills only its
// own K range with y = x * gamma, so no barrier delays the weight stream, and
// r (scale) is finished in the epilogue.  In-chain: the whole row's r comes
// first and y = (x * r) * gamma (scale = 1).
//
// Split K: a narrow vocabulary (one shard of a vocabulary-parallel layout)
// has too few 512-column slabs to fill the chip, so the K lanes are also cut
// into KC contiguous ranges, one per grid row (blockIdx.y); each workgroup
// writes its unscaled partial sums (and, for the deferred fused RMSNorm, its
// range's partial sum of squares) and reduce_kernel adds the KC partials in
// range order, finishes r, scales, and writes the logits and group maxima.
// KC depends only on V and K, so a row's logits do not depend on the batch.
//
// Page precision (parameters "deferred_rms" and "skip_nan_fold": one bf16
// rounding of the GEMM input per element, bf16 products summed in fp32):
// every activation is rounded to bf16 where it is formed (fused) or read
// (given y); the products with the bf16 weights are then exact in fp32.
#include "tail_internal.h"

namespace tail {
namespace {

constexpr int kSlab = 512;  // columns per workgroup
constexpr int kMaxNB = 8;   // batch rows per pass
// default shape: waves per workgroup and weight rows per load batch
constexpr int kWaves = 4;
constexpr int kUnroll = 6;
// K lanes per thread in one prologue burst (times NB rows held in registers)
template <int NB>
constexpr int kPrologueBurst = NB <= 4 ? 16 : 8;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The prologues load every slot of a burst unconditionally, slots past the
// range from a clamped valid lane, and zero those slots where the values are
// used: a load inside a branch that widened its value (or that the compiler
// widened there) had to complete before the branch closed, one memory
// latency per element.

// butterfly sums over the 64 lanes of NB independent values at once: every
// step exchanges all NB values before it waits, so the NB reductions share
// one chain of six exchanges (each value's order is the plain butterfly's)
template <int NB>
__device__ inline void wave_sums(double (&v)[NB]) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    double o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = __shfl_xor(v[b], off, 64);
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] += o[b];
  }
}

struct GemvArgs {
  const void* src;         // y fp32 [gbs, ldsrc] (SRC < 0) or hidden [gbs, ldsrc] (fused)
  int ldsrc;               // row stride of src (H)
  const float* gamma;      // fused only
  float eps;               // fused only
  int H_u;                 // fused only: mean-square divisor
  int deferred;            // fused only
  int page;                // round the activations to bf16
  const uint16_t* w;
  const float* row_scale;  // SRC < 0 only (may be NULL)
  int K, pad_s, V;
  FastDiv pdiv;
  float* logits;
  float* r_out;            // fused only (may be NULL): per-row r
  uint32_t* gkey;
  int groups, b0;
  int kc_n;      // K ranges (gridDim.y); > 1: partial sums go to part
  int gbs;       // rows of the whole call (partial buffer stride)
  float* part;   // [kc_n][gbs][V] partial sums (kc_n > 1)
  double* pss;   // [kc_n][gbs] partial sums of squares (kc_n > 1, fused deferred)
};

template <int NB, int SRC, int W = kWaves, int U = kUnroll>
__global__ __launch_bounds__(W * 64) void gemv_kernel(GemvArgs a) {
  constexpr int kThreads = W * 64;
  extern __shared__ __align__(16) unsigned char smem[];
  float4* s_red = reinterpret_cast<float4*>(smem);                         // [W/2][NB][kSlab/4]
  float* s_y = reinterpret_cast<float*>(smem + (W / 2) * NB * kSlab * 4);  // [NB][K] (fused, SRC = -2)
  __shared__ double s_part[NB][W];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int col = blockIdx.x * kSlab + lane * 8;
  const bool act = col < a.V;
  const int K = a.K, V = a.V, pad_s = a.pad_s;

  // this workgroup's K range, cut among its waves
  const int kc = blockIdx.y;
  const int kb0 = int((long long)K * kc / a.kc_n), kb1 = int((long long)K * (kc + 1) / a.kc_n);
  const int u0 = kb0 + ((kb1 - kb0) * wave) / W;
  const int u1 = kb0 + ((kb1 - kb0) * (wave + 1)) / W;
  int h = pad_s ? u0 + int(fastdiv(uint32_t(u0), a.pdiv)) : u0;
  int gpos = pad_s ? h % pad_s : 0;
  const uint16_t* wcol = a.w + col;

  uint4 wv[U];
  int hh[U];
  auto load_batch = [&](int u, uint4 (&dst)[U], int (&hd)[U]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      hd[j] = h;
      dst[j] = make_uint4(0, 0, 0, 0);
      if (u + j < u1 && act) dst[j] = load_stream(wcol + size_t(h) * V);
      ++h;
      if (pad_s && ++gpos == pad_s - 1) {
        ++h;
        gpos = 0;
      }
    }
  };
  // The first weight batch is in flight while the prologue runs.  Prologues
  // that build the LDS table issue their own first loads before it: loads
  // complete in issue order, so the table's arithmetic then waits only for
  // its inputs (small and mostly L2-resident), not for the weight batch
  // behind them
  bool table_first = SRC == -2;
  if constexpr (SRC >= 0) table_first = a.deferred != 0;
  if (!table_first) load_batch(u0, wv, hh);

  float scale[NB];
  bool scale_at_end = false;  // deferred fused RMSNorm: r is finished in the epilogue
  if constexpr (SRC >= 0) {
    const size_t rowbase = size_t(a.b0) * a.ldsrc;
    if (a.deferred) {
      // each wave builds only its own slice [u0, u1) of the y table and its
      // partial sums of squares: no workgroup barrier before the main loop.
      // One burst carries kBurst lanes per thread of gamma and of all NB rows
      // (one memory latency per burst rather than one per element or row);
      // a row's sum still runs over its lanes in ascending burst order
      constexpr int kBurst = kPrologueBurst<NB>;
      double ss[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ss[b] = 0.0;
      uint32_t xb[NB][kBurst];
      float g[kBurst];
      auto burst_load = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
          const int u = c0 + lane + 64 * i;
          const int uc = u < K ? u : K - 1;
          const int hp = pad_s ? uc + int(fastdiv(uint32_t(uc), a.pdiv)) : uc;
          g[i] = a.gamma[hp];
#pragma unroll
          for (int b = 0; b < NB; ++b)
            xb[b][i] = load_bits<SRC>(a.src, rowbase + size_t(b) * a.ldsrc + hp);
        }
      };
      auto burst_use = [&](int c0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < kBurst; ++i) {
            const int u = c0 + lane + 64 * i;
            const float x = u < u1 ? widen_bits<SRC>(xb[b][i]) : 0.0f;
            ss[b] = fma(double(x), double(x), ss[b]);
            if (u < u1) {
              const float yv = x * g[i];
              s_y[b * K + u] = a.page ? bf16_round(yv) : yv;
            }
          }
      };
      burst_load(u0);
      load_batch(u0, wv, hh);
      burst_use(u0);
      for (int c0 = u0 + 64 * kBurst; c0 < u1; c0 += 64 * kBurst) {
        burst_load(c0);
        burst_use(c0);
      }
      wave_sums<NB>(ss);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (lane == 0) s_part[b][wave] = ss[b];
        scale[b] = 1.0f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      scale_at_end = true;
    } else {
      // in-chain: r is needed before the contraction, so the whole rows
      // first, in bursts over all NB rows (a thread's lanes tid, tid + 256,
      // ... in ascending order)
      constexpr int kBurst = kPrologueBurst<NB>;
      double ss[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ss[b] = 0.0;
      for (int c0 = 0; c0 < K; c0 += kThreads * kBurst) {
        uint32_t xb[NB][kBurst];
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
          const int u = c0 + tid + kThreads * i;
          const int uc = u < K ? u : K - 1;
          const int hp = pad_s ? uc + int(fastdiv(uint32_t(uc), a.pdiv)) : uc;
#pragma unroll
          for (int b = 0; b < NB; ++b)
            xb[b][i] = load_bits<SRC>(a.src, rowbase + size_t(b) * a.ldsrc + hp);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < kBurst; ++i) {
            const int u = c0 + tid + kThreads * i;
            const float x = u < K ? widen_bits<SRC>(xb[b][i]) : 0.0f;
            ss[b] = fma(double(x), double(x), ss[b]);
            if (u < K) s_y[b * K + u] = x;
          }
      }
      wave_sums<NB>(ss);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (lane == 0) s_part[b][wave] = ss[b];
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        double tot = 0.0;  // the wave partials in wave order
#pragma unroll
        for (int w = 0; w < W; ++w) tot += s_part[b][w];
        const float r = float(1.0 / sqrt(tot / double(a.H_u) + double(a.eps)));
        scale[b] = 1.0f;
        for (int u = tid; u < K; u += kThreads) {
          const int hp = pad_s ? u + int(fastdiv(uint32_t(u), a.pdiv)) : u;
          const float yv = (s_y[b * K + u] * r) * a.gamma[hp];
          s_y[b * K + u] = a.page ? bf16_round(yv) : yv;
        }
        if (tid == 0 && kc == 0 && blockIdx.x == 0 && a.r_out) a.r_out[a.b0 + b] = r;
      }
      __syncthreads();
    }
  } else {
    if constexpr (SRC == -2) {
      // the wave's own K range of all NB rows, in bursts as the deferred
      // prologue above
      constexpr int kBurst = kPrologueBurst<NB>;
      const float* y0 = static_cast<const float*>(a.src) + size_t(a.b0) * a.ldsrc;
      float x[NB][kBurst];
      auto burst_load = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
          const int u = c0 + lane + 64 * i;
          const int uc = u < K ? u : K - 1;
          const int hp = pad_s ? uc + int(fastdiv(uint32_t(uc), a.pdiv)) : uc;
#pragma unroll
          for (int b = 0; b < NB; ++b) x[b][i] = y0[size_t(b) * a.ldsrc + hp];
        }
      };
      auto burst_use = [&](int c0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < kBurst; ++i) {
            const int u = c0 + lane + 64 * i;
            if (u < u1) s_y[b * K + u] = a.page ? bf16_round(x[b][i]) : x[b][i];
          }
      };
      burst_load(u0);
      load_batch(u0, wv, hh);
      burst_use(u0);
      for (int c0 = u0 + 64 * kBurst; c0 < u1; c0 += 64 * kBurst) {
        burst_load(c0);
        burst_use(c0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) scale[b] = a.row_scale ? a.row_scale[a.b0 + b] : 1.0f;
  }

  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;

  const float* yg = static_cast<const float*>(a.src) + size_t(a.b0) * a.ldsrc;
  const bool page_src = SRC == -1 && a.page;
  for (int u = u0; u < u1; u += U) {
    uint4 nx[U];
    int nh[U];
    if (u + U < u1) load_batch(u + U, nx, nh);
    // the batch's activations first (rows past the range read as 0 and their
    // weights were not loaded, so they add exact zeros), then the FMAs
    float yv[NB][U];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        yv[b][j] = 0.0f;
        if (u + j < u1) {
          if constexpr (SRC != -1) yv[b][j] = s_y[b * K + u + j];
          else yv[b][j] = page_src ? bf16_round(yg[size_t(b) * a.ldsrc + hh[j]])
                                   : yg[size_t(b) * a.ldsrc + hh[j]];
        }
      }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float wf[8] = {bf_lo(wv[j].x), bf_hi(wv[j].x), bf_lo(wv[j].y), bf_hi(wv[j].y),
                           bf_lo(wv[j].z), bf_hi(wv[j].z), bf_lo(wv[j].w), bf_hi(wv[j].w)};
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[b][c] = fmaf(yv[b][j], wf[c], acc[b][c]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      wv[j] = nx[j];
      hh[j] = nh[j];
    }
  }

  // fixed-order tree over the waves: step d pairs wave w with w + d
#pragma unroll
  for (int d = W / 2; d >= 1; d >>= 1) {
    if (wave >= d && wave < 2 * d) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s_red[((wave - d) * NB + b) * (kSlab / 4) + lane * 2] =
            make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
        s_red[((wave - d) * NB + b) * (kSlab / 4) + lane * 2 + 1] =
            make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
      }
    }
    __syncthreads();
    if (wave < d) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 p = s_red[(wave * NB + b) * (kSlab / 4) + lane * 2];
        const float4 q = s_red[(wave * NB + b) * (kSlab / 4) + lane * 2 + 1];
        acc[b][0] += p.x; acc[b][1] += p.y; acc[b][2] += p.z; acc[b][3] += p.w;
        acc[b][4] += q.x; acc[b][5] += q.y; acc[b][6] += q.z; acc[b][7] += q.w;
      }
    }
    __syncthreads();
  }

  if (wave == 0 && a.kc_n > 1) {
    // split K: the unscaled partial sums of this range (and, deferred fused,
    // its partial sum of squares); reduce_kernel finishes them
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (act) {
        float4* out = reinterpret_cast<float4*>(
            a.part + (size_t(kc) * a.gbs + a.b0 + b) * V + col);
        out[0] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
        out[1] = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
      }
      if (scale_at_end && lane == 0 && blockIdx.x == 0) {
        double tot = 0.0;  // the wave partials in wave order
#pragma unroll
        for (int w = 0; w < W; ++w) tot += s_part[b][w];
        a.pss[size_t(kc) * a.gbs + a.b0 + b] = tot;
      }
    }
  } else if (wave == 0) {
    if (scale_at_end) {  // every wave's partial sum of squares is visible after the tree
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        double tot = 0.0;  // the wave partials in wave order
#pragma unroll
        for (int w = 0; w < W; ++w) tot += s_part[b][w];
        const float r = float(1.0 / sqrt(tot / double(a.H_u) + double(a.eps)));
        scale[b] = r;
        if (lane == 0 && blockIdx.x == 0 && a.r_out) a.r_out[a.b0 + b] = r;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = scale[b];
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = acc[b][c] * s;
      if (act) {
        float4* out = reinterpret_cast<float4*>(a.logits + size_t(a.b0 + b) * V + col);
        out[0] = make_float4(o[0], o[1], o[2], o[3]);
        out[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
      if (a.gkey) {  // maxima of the 64-column groups: 8 lanes each
        uint32_t m = 0;
        if (act) {
#pragma unroll
          for (int c = 0; c < 8; ++c) m = max(m, float_key(o[c]));
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
        const int g = blockIdx.x * (kSlab / kFusedGroup) + lane / 8;
        if ((lane & 7) == 0 && g < a.groups) a.gkey[size_t(a.b0 + b) * a.groups + g] = m;
      }
    }
  }
}

// Split-K finish: one wave per (512-column slab, row); lane l owns columns
// 8 l .. 8 l + 7 of the slab.  Sums the kc_n partials in range order, then
// scales by row_scale (given), by r from the kc_n partial sums of squares
// (deferred fused RMSNorm; r also goes to r_out), or by 1.
__global__ __launch_bounds__(64) void reduce_kernel(const float* __restrict__ part,
                                                    const double* __restrict__ pss, int kc_n,
                                                    int gbs, int V, const float* __restrict__ row_scale,
                                                    int H_u, float eps, float* __restrict__ r_out,
                                                    float* __restrict__ logits,
                                                    uint32_t* __restrict__ gkey, int groups) {
  const int lane = threadIdx.x, b = blockIdx.y;
  const int col = blockIdx.x * kSlab + lane * 8;
  const bool act = col < V;
  float scale = 1.0f;
  if (pss) {
    double tot = 0.0;
    for (int kc = 0; kc < kc_n; ++kc) tot += pss[size_t(kc) * gbs + b];
    scale = float(1.0 / sqrt(tot / double(H_u) + double(eps)));
    if (lane == 0 && blockIdx.x == 0 && r_out) r_out[b] = scale;
  } else if (row_scale) {
    scale = row_scale[b];
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (act) {
    for (int kc = 0; kc < kc_n; ++kc) {
      const float4* p = reinterpret_cast<const float4*>(part + (size_t(kc) * gbs + b) * V + col);
      const float4 x = p[0], y = p[1];
      o[0] += x.x; o[1] += x.y; o[2] += x.z; o[3] += x.w;
      o[4] += y.x; o[5] += y.y; o[6] += y.z; o[7] += y.w;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= scale;
    float4* out = reinterpret_cast<float4*>(logits + size_t(b) * V + col);
    out[0] = make_float4(o[0], o[1], o[2], o[3]);
    out[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
  if (gkey) {
    uint32_t m = 0;
    if (act) {
#pragma unroll
      for (int c = 0; c < 8; ++c) m = max(m, float_key(o[c]));
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    const int g = blockIdx.x * (kSlab / kFusedGroup) + lane / 8;
    if ((lane & 7) == 0 && g < groups) gkey[size_t(b) * groups + g] = m;
  }
}

// Dynamic LDS above 64 KB needs the kernel's limit raised, once per device.
template <int NB, int SRC>
hipError_t raise_lds_limit() {
  static std::once_flag once[kMaxDevices];
  static hipError_t status[kMaxDevices];
  return per_device(once, status, [](int) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<NB, SRC>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  });
}

template <int SRC>
hipError_t launch_pass(int nb, dim3 grid, hipStream_t st, const GemvArgs& a) {
  const size_t lds = size_t(kWaves / 2) * nb * kSlab * 4 + (SRC != -1 ? size_t(nb) * a.K * 4 : 0);
#define TAIL_GEMV(NB)                                                                   \
  do {                                                                                  \
    if (lds > 64 * 1024) {                                                              \
      const hipError_t le = raise_lds_limit<NB, SRC>();                                 \
      if (le != hipSuccess) return le;                                                  \
    }                                                                                   \
    hipLaunchKernelGGL((gemv_kernel<NB, SRC>), grid, dim3(kWaves * 64), lds, st, a);    \
  } while (0)
  switch (nb) {
    case 1: TAIL_GEMV(1); break;
    case 2: TAIL_GEMV(2); break;
    case 3: TAIL_GEMV(3); break;
    case 4: TAIL_GEMV(4); break;
    case 5: TAIL_GEMV(5); break;
    case 6: TAIL_GEMV(6); break;
    case 7: TAIL_GEMV(7); break;
    default: TAIL_GEMV(8); break;
  }
#undef TAIL_GEMV
  return hipGetLastError();
}

}  // namespace

namespace {
// the reduction buffer and an NB x K fp32 activation table within the raised
// LDS limit
bool gemv_table_fits(int nb, int K) {
  return size_t(kWaves / 2) * nb * kSlab * 4 + size_t(nb) * K * 4 <= 96 * 1024;
}
}  // namespace

// K ranges for a V-column lm_head: one when the 512-column slabs fill the
// chip's 256 CUs, else enough to make about 384 workgroups, each keeping at
// least 256 K lanes (a design constant, so workspace sizes stay host-only).
int gemv_ksplit(int V, int K) {
  const int slabs = (V + kSlab - 1) / kSlab;
  if (slabs >= 256) return 1;
  int kc = (384 + slabs - 1) / slabs;
  const int cap = K / 256 > 1 ? K / 256 : 1;
  kc = kc < cap ? kc : cap;
  return kc > 16 ? 16 : (kc < 1 ? 1 : kc);
}

size_t gemv_part_bytes(int gbs, int K, int V) {
  const int kc = gemv_ksplit(V, K);
  if (kc <= 1) return 0;
  return align256(size_t(kc) * gbs * V * 4) + align256(size_t(kc) * gbs * 8);
}

bool gemv_fusable(int gbs, int K) { return gbs <= kGemvMaxBatch && gemv_table_fits(gbs, K); }

hipError_t launch_part_reduce(const float* part, int kc_n, int gbs, int V, const float* row_scale,
                              float* logits, uint32_t* gkey, hipStream_t st) {
  dim3 grid((V + kSlab - 1) / kSlab, gbs);
  hipLaunchKernelGGL(reduce_kernel, grid, dim3(64), 0, st, part, nullptr, kc_n, gbs, V, row_scale,
                     0, 0.0f, nullptr, logits, gkey, (V + kFusedGroup - 1) / kFusedGroup);
  return hipGetLastError();
}

namespace {
// the split-K finish (no-op for one K range)
hipError_t finish_ksplit(const GemvArgs& a, int gbs, const float* row_scale, bool deferred_fused,
                         int H_u, float eps, float* r_out, hipStream_t st) {
  if (a.kc_n <= 1) return hipSuccess;
  dim3 grid((a.V + kSlab - 1) / kSlab, gbs);
  hipLaunchKernelGGL(reduce_kernel, grid, dim3(64), 0, st, a.part,
                     deferred_fused ? a.pss : nullptr, a.kc_n, gbs, a.V, row_scale, H_u, eps, r_out,
                     a.logits, a.gkey, a.groups);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_lm_head_gemv(const float* y, int ldy, const uint16_t* w, const float* row_scale,
                               int gbs, int K, int pad_s, int V, bool page, float* logits,
                               uint32_t* gkey, void* part_ws, hipStream_t st) {
  GemvArgs a{};
  a.page = page ? 1 : 0;
  a.gbs = gbs;
  a.kc_n = gemv_ksplit(V, K);
  a.part = static_cast<float*>(part_ws);
  a.pss = reinterpret_cast<double*>(static_cast<char*>(part_ws) +
                                    align256(size_t(a.kc_n) * gbs * V * 4));
  a.src = y;
  a.ldsrc = ldy;
  a.w = w;
  a.row_scale = row_scale;
  a.K = K;
  a.pad_s = pad_s;
  a.V = V;
  a.pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  a.logits = logits;
  a.gkey = gkey;
  a.groups = (V + kFusedGroup - 1) / kFusedGroup;
  dim3 grid((V + kSlab - 1) / kSlab, a.kc_n);
  for (int b0 = 0; b0 < gbs; b0 += kMaxNB) {
    a.b0 = b0;
    const int nb = gbs - b0 < kMaxNB ? gbs - b0 : kMaxNB;
    const hipError_t e = gemv_table_fits(nb, K) ? launch_pass<-2>(nb, grid, st, a)
                                                : launch_pass<-1>(nb, grid, st, a);
    if (e != hipSuccess) return e;
  }
  return finish_ksplit(a, gbs, row_scale, false, 0, 0.0f, nullptr, st);
}

hipError_t launch_norm_gemv(const void* hidden, int dtype, const float* gamma, int gbs, int H,
                            int H_u, int K, int pad_s, float eps, bool deferred, bool page,
                            const uint16_t* w, int V, float* logits, float* r_out, uint32_t* gkey,
                            void* part_ws, hipStream_t st) {
  GemvArgs a{};
  a.page = page ? 1 : 0;
  a.gbs = gbs;
  a.kc_n = gemv_ksplit(V, K);
  a.part = static_cast<float*>(part_ws);
  a.pss = reinterpret_cast<double*>(static_cast<char*>(part_ws) +
                                    align256(size_t(a.kc_n) * gbs * V * 4));
  a.src = hidden;
  a.ldsrc = H;
  a.gamma = gamma;
  a.eps = eps;
  a.H_u = H_u;
  a.deferred = deferred ? 1 : 0;
  a.w = w;
  a.K = K;
  a.pad_s = pad_s;
  a.V = V;
  a.pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  a.logits = logits;
  a.r_out = r_out;
  a.gkey = gkey;
  a.groups = (V + kFusedGroup - 1) / kFusedGroup;
  a.b0 = 0;
  dim3 grid((V + kSlab - 1) / kSlab, a.kc_n);
  hipError_t e;
  switch (dtype) {
    case 0: e = launch_pass<0>(gbs, grid, st, a); break;
    case 1: e = launch_pass<1>(gbs, grid, st, a); break;
    default: e = launch_pass<2>(gbs, grid, st, a); break;
  }
  if (e != hipSuccess) return e;
  return finish_ksplit(a, gbs, nullptr, deferred, H_u, eps, r_out, st);
}

}  // namespace tail
