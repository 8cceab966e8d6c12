// lm_head contraction, weight-streaming form for small batches (GPT-OSS tail
// API page, parameter "lm_head_weight_t": [H, V] bf16, already transposed and
// C-contiguous).
//
// logits[b, v] = row_scale[b] * sum_h y[b, h] * W[h, v]
//
// The weight (H_u * V * 2 bytes, 1.16 GB for GPT-OSS) is read exactly once;
// that read is the roofline of the whole tail at small batch.
//
// Mapping: a 512-thread workgroup (8 waves) owns a slab of 512 consecutive
// vocabulary columns; lane l of every wave owns columns 8l..8l+7 of the slab,
// which it reads as one 16-byte load per weight row, so each wave reads a
// contiguous 1 KB of a row per load.  The 8 waves split the (unpadded) hidden
// lanes into 8 contiguous ranges; each keeps NB x 8 fp32 partial sums for the
// NB batch rows of this pass, reading y[b, h] through the scalar cache (the
// row index is wave-uniform).  Partials are combined through LDS in a fixed
// tree, ((p0+p4)+(p2+p6)) + ((p1+p5)+(p3+p7)), so a column's sum depends only
// on H_u and never on the column's position or on the other batch rows.
#include "tail_internal.h"

namespace tail {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kSlab = 512;  // columns per workgroup
constexpr int kUnroll = 8;  // weight rows in flight per lane
constexpr int kMaxNB = 8;   // batch rows per pass

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The weight is streamed once and never reused: non-temporal loads keep it
// from displacing useful lines and measurably raise the achieved bandwidth.
__device__ inline uint4 load_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int NB>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const float* __restrict__ y, int ldy,
                                                        const uint16_t* __restrict__ w,
                                                        const float* __restrict__ row_scale,
                                                        int H_u, int pad_s, int V,
                                                        float* __restrict__ logits,
                                                        uint32_t* __restrict__ gkey, int groups,
                                                        int b0) {
  __shared__ float4 s_red[4][NB][kSlab / 4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x * kSlab + lane * 8;
  const bool act = col < V;

  const int u0 = (wave * H_u) / kWaves;
  const int u1 = ((wave + 1) * H_u) / kWaves;
  int h = phys_lane(u0, pad_s);
  int gpos = pad_s ? h % pad_s : 0;

  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;

  const uint16_t* wcol = w + col;
  const float* yb = y + size_t(b0) * ldy;

  for (int u = u0; u < u1; u += kUnroll) {
    uint4 wv[kUnroll];
    int hh[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      hh[j] = h;
      wv[j] = make_uint4(0, 0, 0, 0);
      if (u + j < u1 && act) wv[j] = load_stream(wcol + size_t(h) * V);
      ++h;
      if (pad_s && ++gpos == pad_s - 1) {
        ++h;
        gpos = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      if (u + j < u1) {
        float wf[8] = {bf_lo(wv[j].x), bf_hi(wv[j].x), bf_lo(wv[j].y), bf_hi(wv[j].y),
                       bf_lo(wv[j].z), bf_hi(wv[j].z), bf_lo(wv[j].w), bf_hi(wv[j].w)};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float yv = yb[size_t(b) * ldy + hh[j]];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[b][c] = fmaf(yv, wf[c], acc[b][c]);
        }
      }
    }
  }

  // fixed-order tree over the 8 waves: step d pairs wave w with w + d
#pragma unroll
  for (int d = 4; d >= 1; d >>= 1) {
    if (wave >= d && wave < 2 * d) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s_red[wave - d][b][lane * 2] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
        s_red[wave - d][b][lane * 2 + 1] = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
      }
    }
    __syncthreads();
    if (wave < d) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float4 p = s_red[wave][b][lane * 2], q = s_red[wave][b][lane * 2 + 1];
        acc[b][0] += p.x; acc[b][1] += p.y; acc[b][2] += p.z; acc[b][3] += p.w;
        acc[b][4] += q.x; acc[b][5] += q.y; acc[b][6] += q.z; acc[b][7] += q.w;
      }
    }
    __syncthreads();
  }

  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = row_scale ? row_scale[b0 + b] : 1.0f;
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = acc[b][c] * s;
      if (act) {
        float4* out = reinterpret_cast<float4*>(logits + size_t(b0 + b) * V + col);
        out[0] = make_float4(o[0], o[1], o[2], o[3]);
        out[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
      if (gkey) {  // maxima of the 64-column groups: 8 lanes each
        uint32_t m = 0;
        if (act) {
#pragma unroll
          for (int c = 0; c < 8; ++c) m = max(m, float_key(o[c]));
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
        const int g = blockIdx.x * (kSlab / kFusedGroup) + lane / 8;
        if ((lane & 7) == 0 && g < groups) gkey[size_t(b0 + b) * groups + g] = m;
      }
    }
  }
}

template <int NB>
void launch_nb(dim3 grid, hipStream_t st, const float* y, int ldy, const uint16_t* w,
               const float* rs, int H_u, int pad_s, int V, float* logits, uint32_t* gkey,
               int groups, int b0) {
  hipLaunchKernelGGL(gemv_kernel<NB>, grid, dim3(kThreads), 0, st, y, ldy, w, rs, H_u, pad_s, V,
                     logits, gkey, groups, b0);
}

}  // namespace

hipError_t launch_lm_head_gemv(const float* y, int ldy, const uint16_t* w, const float* row_scale,
                               int gbs, int H_u, int pad_s, int V, float* logits, uint32_t* gkey,
                               hipStream_t st) {
  dim3 grid((V + kSlab - 1) / kSlab);
  const int groups = (V + kFusedGroup - 1) / kFusedGroup;
  for (int b0 = 0; b0 < gbs; b0 += kMaxNB) {
    int nb = gbs - b0 < kMaxNB ? gbs - b0 : kMaxNB;
    switch (nb) {
      case 1: launch_nb<1>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 2: launch_nb<2>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 3: launch_nb<3>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 4: launch_nb<4>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 5: launch_nb<5>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 6: launch_nb<6>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      case 7: launch_nb<7>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
      default: launch_nb<8>(grid, st, y, ldy, w, row_scale, H_u, pad_s, V, logits, gkey, groups, b0); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tail
