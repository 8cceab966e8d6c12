// lm_head contraction on the bf16 matrix cores, for batches beyond the
// weight-streaming GEMV (GPT-OSS tail API page, parameter "lm_head_weight_t":
// [H, V] bf16, already transposed and C-contiguous).
//
// logits[b, v] = row_scale[b] * sum_h (sum_t A_t[b, h]) * W[h, v]
//
// The fp32 activations arrive split into NT bf16 terms A_0 + A_1 (+ A_2)
// (each term the bf16 rounding of what the earlier terms left), so every
// product in v_mfma_f32_16x16x32_bf16 is exact and accumulates in fp32; two
// terms (the default) represent an activation to 2^-17 relative, three to
// 2^-26.  The page-precision mode uses one term: the activation rounded to
// bf16 once, as the page's parameter "deferred_rms" describes.  The weight
// itself is bf16 and is never rounded.
//
// Tiling: a workgroup owns VT consecutive vocabulary columns for BROWS =
// 16 * NBT batch rows and walks the (unpadded) hidden dimension in K-steps
// of KT (32 or 64) rows.  Per K-step the weight tile [KT x VT] is staged into
// LDS in its natural row-major form (row pitch 2 VT + 32 bytes) and each
// 16-column MFMA operand is read back with two ds_read_b64_tr_b16
// transposing reads; the activation tile [BROWS x KT] per term is staged next
// to it as the ready MFMA fragments the activation producer wrote (1 KB
// each, lane l's 16 bytes at 16 l), so its global loads, LDS stores and LDS
// reads are all linear, and the LDS accesses free of bank conflicts.
// Loads of the next K-step go out (weight loads non-temporal) before the
// current step's MFMAs.  Waves form a WV x WB grid over (columns, rows); each
// wave owns (VT/WV) x (BROWS/WB) outputs.
//
// K order inside a 32-lane block: MFMA k-slot (g, j) (lane group g, element
// j) maps to block row 4g + (j & 3) + 16 (j >> 2), so one transposing read
// of the wave touches 16 consecutive LDS rows, 32 bytes of each.  The
// activation producer writes its terms in the same permuted order, so both
// operands agree on every k.
//
// Determinism: every output element is one fixed sequence of MFMAs (K-steps
// in order, terms in order), the same for every column and every row.
//
// Split K (narrow vocabularies, e.g. one shard of a vocabulary-parallel
// layout, whose 512-column tiles cannot fill the chip): grid row kc of KC
// takes the K-steps [nks kc / KC, nks (kc + 1) / KC) and writes its unscaled
// partial sums; a fixed-order reduction (shared with the weight-streaming
// path) adds them, scales and writes the logits and group maxima.  KC depends
// only on V and K.
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
  static constexpr int WROW = VT * 2 + 32;                     // LDS bytes per weight row
  static constexpr int KB = KT / 32;                           // 32-lane K blocks per K-step
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

template <int VT, int WV, int WB, int NBT, int NT, int KT = 64, int MINB = 1, bool SPLIT = false>
__global__ __launch_bounds__(WV * WB * 64, MINB) void mfma_kernel(
    const uint16_t* __restrict__ act, int rows_pad, int Kp, const uint16_t* __restrict__ w, int V,
    int H_u, int pad_s, FastDiv pdiv, const float* __restrict__ row_scale, int gbs, int b0,
    float* __restrict__ logits, uint32_t* __restrict__ gkey, int groups, int kc_n,
    float* __restrict__ part) {
  using C = Cfg<VT, WV, WB, NBT, NT, KT>;
  __shared__ __align__(16) unsigned char s_w[KT * C::WROW];
  __shared__ __align__(16) unsigned char s_b[NT * C::BROWS * KT * 2];
  __shared__ uint32_t s_g[C::BROWS][C::GPW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % WV, wb = wave / WV;
  const int v0 = blockIdx.x * VT;
  const int nks = Kp / KT;  // Kp is a multiple of kKStep, which KT divides
  // this workgroup's K-steps (all of them unless K is split)
  const int ks0 = SPLIT ? int((long long)nks * blockIdx.y / kc_n) : 0;
  const int ks1 = SPLIT ? int((long long)nks * (blockIdx.y + 1) / kc_n) : nks;

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
        // chunk c = ((t * NBT + bt) * KB + sb) * 64 + l: lane l of the fragment
        // (term t, row tile b0 / 16 + bt, K block ks * KB + sb)
        const int l = c % 64, sb = (c / 64) % C::KB, bt = (c / (64 * C::KB)) % NBT;
        const int t = c / (64 * C::KB * NBT);
        const int rt = b0 / 16 + bt;
        if (rt < rows_pad / 16)
          breg[i] = *reinterpret_cast<const uint4*>(
              act + (((size_t(t) * (rows_pad / 16) + rt) * (Kp / 32) + ks * C::KB + sb) * 64 + l) * 8);
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
      // fragment layout: chunk c is lane (c % 64) of fragment (t, bt, K block) c / 64
      if (c < C::BCH) *reinterpret_cast<uint4*>(s_b + c * 16) = breg[i];
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

  load_w(ks0);
  load_b(ks0);
  for (int ks = ks0; ks < ks1; ++ks) {
    __syncthreads();
    store_lds();
    if (ks + 1 < ks1) {
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
              s_b + (((t * NBT + wb * C::BTW + bt) * C::KB + sb) * 64 + lane) * 16);
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
  if constexpr (SPLIT) {  // split K: unscaled partial sums of this K range
#pragma unroll
    for (int bt = 0; bt < C::BTW; ++bt) {
      const int b = b0 + wb * C::BW + bt * 16 + s16;
#pragma unroll
      for (int vt = 0; vt < C::VTW; ++vt) {
        const int v = v0 + wv * C::VW + vt * 16 + 4 * kg;
        if (b < gbs && v < V)
          *reinterpret_cast<float4*>(part + (size_t(blockIdx.y) * gbs + b) * V + v) =
              make_float4(acc[vt][bt][0], acc[vt][bt][1], acc[vt][bt][2], acc[vt][bt][3]);
      }
    }
    return;
  }
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

template <int VT, int WV, int WB, int NBT, int NT, int KT = 64, int MINB = 1>
hipError_t launch_cfg(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V, int H_u,
                      int pad_s, const float* row_scale, int gbs, int b0, float* logits,
                      uint32_t* gkey, int kc_n, float* part, hipStream_t st) {
  const FastDiv pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  const int groups = (V + kFusedGroup - 1) / kFusedGroup;
  dim3 grid((V + VT - 1) / VT, kc_n), block(WV * WB * 64);
  if (kc_n > 1)
    hipLaunchKernelGGL((mfma_kernel<VT, WV, WB, NBT, NT, KT, MINB, true>), grid, block, 0, st, act,
                       rows_pad, Kp, w, V, H_u, pad_s, pdiv, row_scale, gbs, b0, logits, gkey, groups,
                       kc_n, part);
  else
    hipLaunchKernelGGL((mfma_kernel<VT, WV, WB, NBT, NT, KT, MINB, false>), grid, block, 0, st, act,
                       rows_pad, Kp, w, V, H_u, pad_s, pdiv, row_scale, gbs, b0, logits, gkey, groups,
                       kc_n, part);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_terms(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V,
                        int H_u, int pad_s, const float* row_scale, int gbs, float* logits,
                        uint32_t* gkey, void* part_ws, hipStream_t st) {
  const int kc_n = mfma_ksplit(V, Kp);
  float* part = static_cast<float*>(part_ws);
  // up to 128 rows (larger batches run on the large-batch kernel)
  const int nbt = (gbs + 15) / 16;
  const int b0 = 0;
  hipError_t e;
  // 512-column tiles (393 workgroups for GPT-OSS) and 32-row K-steps; up to
  // 64 rows two workgroups share a CU, so all are resident at once
  if (nbt <= 1) e = launch_cfg<512, 4, 1, 1, NT, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
  else if (nbt <= 2) e = launch_cfg<512, 4, 1, 2, NT, 32, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
  else if (nbt <= 4) e = launch_cfg<512, 4, 1, 4, NT, 32, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
  else if (nbt <= 8) e = launch_cfg<512, 4, 2, 8, NT, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
  else e = hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  if (kc_n > 1) return launch_part_reduce(part, kc_n, gbs, V, row_scale, logits, gkey, st);
  return hipSuccess;
}

}  // namespace

int mfma_terms(int, bool page) { return page ? 1 : 2; }

// K ranges of the matrix-core lm_head: one when its 512-column tiles fill the
// chip's 256 CUs, else enough for about 384 workgroups, each keeping at least
// 8 K-steps of 32 (a design constant, so workspace sizes stay host-only).
int mfma_ksplit(int V, int Kp) {
  const int tiles = (V + 511) / 512;
  if (tiles >= 256) return 1;
  int kc = (384 + tiles - 1) / tiles;
  const int cap = Kp / 256 > 1 ? Kp / 256 : 1;
  kc = kc < cap ? kc : cap;
  return kc > 16 ? 16 : (kc < 1 ? 1 : kc);
}

size_t mfma_part_bytes(int gbs, int Kp, int V) {
  const int kc = mfma_ksplit(V, Kp);
  return kc > 1 ? align256(size_t(kc) * gbs * V * 4) : 0;
}

hipError_t launch_lm_head_mfma(const uint16_t* act, int nt, int rows_pad, int Kp, const uint16_t* w,
                               int V, int H_u, int pad_s, const float* row_scale, int gbs,
                               float* logits, uint32_t* gkey, void* part_ws, hipStream_t st) {
  if (nt == 2)
    return launch_terms<2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, logits, gkey,
                           part_ws, st);
  if (nt == 1)
    return launch_terms<1>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, logits, gkey,
                           part_ws, st);
  return hipErrorInvalidValue;
}

}  // namespace tail
