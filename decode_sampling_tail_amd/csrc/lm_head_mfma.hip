// lm_head contraction on the bf16 matrix cores, for batches beyond the
// weight-streaming GEMV (GPT-OSS tail API page, parameter "lm_head_weight_t":
// [H, V] bf16, already transposed and C-contiguous).
//
// logits[b, v] = row_scale[b] * sum_h (sum_t A_t[b, h]) * W[h, v]
//
// The fp32 activations arrive split into NT bf16 terms A_0 + A_1 (+ A_2)
// (each term the bf16 rounding of what the earlier terms left), so every
// product in v_mfma_f32_16x16x32_bf16 is exact and accumulates in fp32; two
// terms represent an activation to 2^-17 relative, three to 2^-26.  The
// weight itself is bf16 and is never rounded.
//
// Tiling: a workgroup owns VT consecutive vocabulary columns for BROWS =
// 16 * NBT batch rows and walks the (unpadded) hidden dimension in K-steps
// of KT (32 or 64) rows.  Per K-step the weight tile [KT x VT] is staged into
// LDS in its natural row-major form (row pitch 2 VT + 16 bytes) and each
// 16-column MFMA operand is read back with two ds_read_b64_tr_b16
// transposing reads; the activation tile [BROWS x KT] per term is staged next
// to it.  Loads of the next K-step go out (weight loads non-temporal) before
// the current step's MFMAs.  Waves form a WV x WB grid over (columns, rows);
// each wave owns (VT/WV) x (BROWS/WB) outputs.
//
// K order inside a 32-lane block: MFMA k-slot (g, j) (lane group g, element
// j) maps to block row 4g + (j & 3) + 16 (j >> 2), so one transposing read
// of the wave touches 16 consecutive LDS rows, 32 bytes of each.  The
// activation producer writes its terms in the same permuted order, so both
// operands agree on every k.
//
// Determinism: every output element is one fixed sequence of MFMAs (K-steps
// in order, terms in order), the same for every column and every row.
#include "tail_internal.h"

namespace tail {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int VT, int WV, int WB, int NBT, int NT, int KT>
struct Cfg {
  static constexpr int NW = WV * WB, NTH = NW * 64;
  static constexpr int VW = VT / WV, VTW = VW / 16;            // columns, 16-col tiles per wave
  static constexpr int BROWS = NBT * 16, BW = BROWS / WB, BTW = BW / 16;
  static constexpr int WROW = VT * 2 + 16;                     // LDS bytes per weight row
  static constexpr int BROW = KT * 2 + 16;                     // LDS bytes per activation row
  static constexpr int HCH = KT / 8;                           // 16-byte chunks per activation row
  static constexpr int WCH = KT * VT / 8, WPT = WCH / NTH;     // 16-byte weight chunks
  static constexpr int BCH = NT * BROWS * KT / 8, BPT = (BCH + NTH - 1) / NTH;
  static constexpr int GPW = VT / kFusedGroup;                 // key groups per workgroup
  static_assert(WCH % NTH == 0 && VW % 16 == 0 && BW % 16 == 0 && VT % kFusedGroup == 0 &&
                    kKStep % KT == 0 && KT % 32 == 0,
                "tile");
};

__device__ inline bf16x8 tr_operand(const unsigned char* s_w, int row, int col_bytes, int wrow) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(s_w + row * wrow + col_bytes));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(s_w + (row + 16) * wrow + col_bytes));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int VT, int WV, int WB, int NBT, int NT, int KT = 64>
__global__ __launch_bounds__(WV * WB * 64) void mfma_kernel(
    const uint16_t* __restrict__ act, int rows_pad, int Kp, const uint16_t* __restrict__ w, int V,
    int H_u, int pad_s, FastDiv pdiv, const float* __restrict__ row_scale, int gbs, int b0,
    float* __restrict__ logits, uint32_t* __restrict__ gkey, int groups) {
  using C = Cfg<VT, WV, WB, NBT, NT, KT>;
  __shared__ __align__(16) unsigned char s_w[KT * C::WROW];
  __shared__ __align__(16) unsigned char s_b[NT * C::BROWS * C::BROW];
  __shared__ uint32_t s_g[C::BROWS][C::GPW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % WV, wb = wave / WV;
  const int v0 = blockIdx.x * VT;
  const int nks = Kp / KT;  // Kp is a multiple of kKStep, which KT divides

  for (int i = tid; i < C::BROWS * C::GPW; i += C::NTH) (&s_g[0][0])[i] = 0u;

  uint4 wreg[C::WPT], breg[C::BPT];
  auto load_w = [&](int ks) {
#pragma unroll
    for (int i = 0; i < C::WPT; ++i) {
      const int c = tid + i * C::NTH, r = c / (VT / 8), cc = c % (VT / 8);
      const int u = ks * KT + r, col = v0 + cc * 8;
      wreg[i] = make_uint4(0, 0, 0, 0);
      if (u < H_u && col < V) {
        const int h = pad_s ? u + int(fastdiv(uint32_t(u), pdiv)) : u;
        wreg[i] = load_stream(w + size_t(h) * V + col);
      }
    }
  };
  auto load_b = [&](int ks) {
#pragma unroll
    for (int i = 0; i < C::BPT; ++i) {
      const int c = tid + i * C::NTH;
      breg[i] = make_uint4(0, 0, 0, 0);
      if (c < C::BCH) {
        const int t = c / (C::BROWS * C::HCH), rem = c % (C::BROWS * C::HCH);
        const int b = rem / C::HCH, hc = rem % C::HCH;
        const int row = b0 + b;
        if (row < rows_pad)
          breg[i] = *reinterpret_cast<const uint4*>(act + (size_t(t) * rows_pad + row) * Kp +
                                                    ks * KT + hc * 8);
      }
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int i = 0; i < C::WPT; ++i) {
      const int c = tid + i * C::NTH, r = c / (VT / 8), cc = c % (VT / 8);
      *reinterpret_cast<uint4*>(s_w + r * C::WROW + cc * 16) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::BPT; ++i) {
      const int c = tid + i * C::NTH;
      if (c < C::BCH) {
        const int t = c / (C::BROWS * C::HCH), rem = c % (C::BROWS * C::HCH);
        const int b = rem / C::HCH, hc = rem % C::HCH;
        *reinterpret_cast<uint4*>(s_b + (t * C::BROWS + b) * C::BROW + hc * 16) = breg[i];
      }
    }
  };

  f32x4 acc[C::VTW][C::BTW];
#pragma unroll
  for (int i = 0; i < C::VTW; ++i)
#pragma unroll
    for (int j = 0; j < C::BTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int s16 = lane & 15, kg = lane >> 4;
  // transposing-read supplier address inside a 32-row block: row 4g + (s >> 2)
  // (+16 for the second read), columns 4 (s & 3) .. +3 of the 16-column tile
  const int tr_row = 4 * kg + (s16 >> 2);
  const int tr_col = (wv * C::VW + 4 * (s16 & 3)) * 2;

  load_w(0);
  load_b(0);
  for (int ks = 0; ks < nks; ++ks) {
    __syncthreads();
    store_lds();
    if (ks + 1 < nks) {
      load_w(ks + 1);
      load_b(ks + 1);
    }
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < KT / 32; ++sb) {
      bf16x8 bfr[C::BTW][NT];
#pragma unroll
      for (int bt = 0; bt < C::BTW; ++bt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          bfr[bt][t] = *reinterpret_cast<const bf16x8*>(
              s_b + (t * C::BROWS + wb * C::BW + bt * 16 + s16) * C::BROW + (sb * 32 + 8 * kg) * 2);
#pragma unroll
      for (int vt = 0; vt < C::VTW; ++vt) {
        const bf16x8 a = tr_operand(s_w, sb * 32 + tr_row, tr_col + vt * 32, C::WROW);
#pragma unroll
        for (int bt = 0; bt < C::BTW; ++bt)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[vt][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr[bt][t], acc[vt][bt], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds v = 4 kg .. 4 kg + 3 of the tile for batch row s16
#pragma unroll
  for (int bt = 0; bt < C::BTW; ++bt) {
    const int bl = wb * C::BW + bt * 16 + s16;
    const int b = b0 + bl;
    const float sc = (b < gbs && row_scale) ? row_scale[b] : 1.0f;
#pragma unroll
    for (int vt = 0; vt < C::VTW; ++vt) {
      const int vl = wv * C::VW + vt * 16;
      const int v = v0 + vl + 4 * kg;
      const float4 o = make_float4(acc[vt][bt][0] * sc, acc[vt][bt][1] * sc, acc[vt][bt][2] * sc,
                                   acc[vt][bt][3] * sc);
      uint32_t m = 0;
      if (b < gbs && v < V) {
        *reinterpret_cast<float4*>(logits + size_t(b) * V + v) = o;
        m = max(max(float_key(o.x), float_key(o.y)), max(float_key(o.z), float_key(o.w)));
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
      if (gkey && kg == 0 && m) atomicMax(&s_g[bl][vl / kFusedGroup], m);
    }
  }
  if (gkey) {
    __syncthreads();
    for (int i = tid; i < C::BROWS * C::GPW; i += C::NTH) {
      const int bl = i / C::GPW, gl = i % C::GPW;
      const int b = b0 + bl, g = v0 / kFusedGroup + gl;
      if (b < gbs && g < groups) gkey[size_t(b) * groups + g] = s_g[bl][gl];
    }
  }
}

template <int VT, int WV, int WB, int NBT, int NT, int KT = 64>
hipError_t launch_cfg(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V, int H_u,
                      int pad_s, const float* row_scale, int gbs, int b0, float* logits,
                      uint32_t* gkey, hipStream_t st) {
  const FastDiv pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  const int groups = (V + kFusedGroup - 1) / kFusedGroup;
  dim3 grid((V + VT - 1) / VT), block(WV * WB * 64);
  hipLaunchKernelGGL((mfma_kernel<VT, WV, WB, NBT, NT, KT>), grid, block, 0, st, act, rows_pad, Kp, w, V,
                     H_u, pad_s, pdiv, row_scale, gbs, b0, logits, gkey, groups);
  return hipGetLastError();
}

}  // namespace

int mfma_terms(int gbs) { return gbs <= 64 ? 3 : 2; }

hipError_t launch_lm_head_mfma(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V,
                               int H_u, int pad_s, const float* row_scale, int gbs, float* logits,
                               uint32_t* gkey, hipStream_t st) {
  const int nt = mfma_terms(gbs);
  for (int b0 = 0; b0 < gbs; b0 += 256) {
    const int rows = gbs - b0 < 256 ? gbs - b0 : 256;
    const int nbt = (rows + 15) / 16;
    hipError_t e;
    if (nt == 3) {
      // 512-column tiles (393 workgroups for GPT-OSS, all resident at once)
      // and 32-row K-steps: about 32 KB of weight loads in flight per workgroup
      if (nbt <= 1) e = launch_cfg<512, 4, 1, 1, 3, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
      else if (nbt <= 2) e = launch_cfg<512, 4, 2, 2, 3, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
      else e = launch_cfg<512, 4, 2, 4, 3, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
    } else {
      if (nbt <= 8) e = launch_cfg<256, 2, 4, 8, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
      else e = launch_cfg<256, 2, 4, 16, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tail
