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

// Persistent form for batches above 64 rows, with direct global-to-LDS copies
// (global_load_lds_dwordx4) and an NS-stage LDS ring.
//
// The grid holds as many workgroups as fit on the device at once; workgroup
// w owns the contiguous range of 64-column key groups [w G' / P,
// (w + 1) G' / P) (P workgroups; G' is all G groups, or with leftover items,
// below, the P floor(G / P) that divide evenly), so every workgroup gets the
// same number of columns to within one group, and walks it in sub-tiles of
// VT columns (the last one may be narrower), one K-step of 32 rows at a time.  The K-steps of
// all its sub-tiles form one pipeline: the copies for step q + NS - 1 go out
// while step q runs, without passing through registers, so NS - 1 steps of
// memory latency are hidden; one barrier per step.  Wave (wv, wb) owns tiles
// wv * VTW .. wv * VTW + VTW - 1 (16 columns each) of the sub-tile for rows
// (wb * BTW .. wb * BTW + BTW - 1) * 16 of the 16 * NBT-row chunk.  A
// sub-tile's logits and its 64-column group maxima are written from the
// accumulators, without a barrier, after its last K-step.
//
// Weight stage: the [32 x VT] tile is stored unpadded (row pitch 2 VT bytes)
// with the 16-byte chunks of row r XOR-swizzled by 2 (r % 8); each copy moves
// 1 KB (1024 / (2 VT) whole rows), lane l fetching the global chunk that
// belongs in its LDS slot.  The transposing reads of half a wave touch rows
// with distinct r % 8, which the swizzle spreads over distinct 32-byte bank
// groups.  Activation stage: the 1 KB fragments of the step, one copy each.
//
// Rows past K and columns past V are fetched from clamped (valid) addresses:
// a clamped weight row meets zero activations, and clamped columns or row
// tiles only reach outputs that are never stored.
//
// Leftover items (two terms): when the groups do not divide evenly and the
// one extra group of some workgroups would cost them a whole extra pass (a
// step costs about the same however few columns it carries), the contiguous
// ranges cover only gmain = P * floor(G / P) groups and the columns past
// them are cut into VT-column regions, each dealt as WB items of one region
// x one row group (the BTW row tiles of the waves with that wb).  An item
// step carries two 32-row K blocks in the same stage bytes and copy count as
// a whole-pass step: block 0's weights in the weight slot, block 1's in the
// first half of the fragment slots, and the row group's fragments of both
// blocks in the second half.  An item so takes half a pass's steps; only its
// row group's waves run MFMAs and write outputs, and every element still
// takes its full K in order, so the logits are the same bytes.  The item
// steps continue the same pipeline in a loop of their own after the
// whole-pass steps (one loop choosing the step kind at run time scheduled
// the whole-pass steps worse).
template <int VT, int WV, int WB, int NBT, int NT, int NS>
struct DCfg {
  static constexpr int NW = WV * WB, NTH = NW * 64;
  static constexpr int VTW = VT / 16 / WV, BTW = NBT / WB;
  static constexpr int WPITCH = VT * 2, WBYTES = 32 * WPITCH;
  static constexpr int WINS = WBYTES / 1024, RPI = 1024 / WPITCH;  // weight copies, rows per copy
  static constexpr int BINS = NT * NBT, NINS = WINS + BINS;        // copies per step
  static constexpr int WAIT = NINS / NW;                           // fewest copies of any wave
  static constexpr int STAGE = WBYTES + BINS * 1024;
  // leftover items need two terms and a stage that holds two weight blocks
  // plus one row group's fragments of both
  static constexpr bool ITEMS = NT == 2 && 2 * WINS + 2 * NT * BTW == NINS;
  static_assert(VTW * 16 * WV == VT && VTW % 4 == 0 && BTW * WB == NBT && WPITCH <= 1024 &&
                    VT >= 128 && (VT & (VT - 1)) == 0 && WAIT >= 1 && NS >= 2 &&
                    WAIT * (NS - 2) < 64 && NS * STAGE <= 160 * 1024,
                "tile");
};

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ inline void wait_vmcnt() {
  // vmcnt field split over bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most W * n of this wave's memory operations are outstanding
// (n <= N, wave-uniform).
template <int W, int N>
__device__ inline void wait_steps(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<W * N>();
    else wait_steps<W, N - 1>(n);
  }
}

template <int VT, int WV, int WB, int NBT, int NT, int NS>
__global__ __launch_bounds__(WV * WB * 64) void dma_kernel(
    const uint16_t* __restrict__ act, int rows_pad, int Kp, const uint16_t* __restrict__ w, int V,
    int K, int pad_s, FastDiv pdiv, const float* __restrict__ row_scale, int gbs, int b0,
    float* __restrict__ logits, uint32_t* __restrict__ gkey, int groups, int gmain) {
  using C = DCfg<VT, WV, WB, NBT, NT, NS>;
  __shared__ __align__(1024) unsigned char smem[NS * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % WV, wb = wave / WV;
  const int s16 = lane & 15, kg = lane >> 4;
  const int P = gridDim.x;
  const int g0 = int((long long)blockIdx.x * gmain / P);
  const int g1 = int((long long)(blockIdx.x + 1) * gmain / P);
  const int c0 = g0 * kFusedGroup, c1 = min(g1 * kFusedGroup, V);
  const int nsub = (c1 - c0 + VT - 1) / VT;
  const int nks = Kp / 32;  // even: Kp is a multiple of 64
  const int nmain = nsub * nks;
  // leftover items (region, row group), blockIdx.x, blockIdx.x + P, ...; each
  // nks / 2 steps of two K blocks
  const int lcol0 = gmain * kFusedGroup;
  const int nitems = (C::ITEMS && lcol0 < V) ? (V - lcol0 + VT - 1) / VT * WB : 0;
  const int nitm = int(blockIdx.x) < nitems ? (nitems - 1 - int(blockIdx.x)) / P + 1 : 0;
  const int iks = nks / 2;
  const int total = nmain + nitm * iks;
  if (total <= 0) return;
  const int rtiles = rows_pad / 16;

  // item step q >= nmain: item id, its region's first column, first K block
  auto item_at = [&](int q, int& v0, int& kb) {
    const int id = int(blockIdx.x) + ((q - nmain) / iks) * P;
    v0 = lcol0 + (id / WB) * VT;
    kb = 2 * ((q - nmain) % iks);
    return id % WB;
  };

  // this wave's copies of item step q: copies [0, 2 WINS) the weights of
  // blocks kb and kb + 1, the rest the row group's fragments of both blocks
  // (block, term, row tile), in slot order
  auto issue_item = [&](int q) {
    int v0, kb;
    const int rg = item_at(q, v0, kb);
    unsigned char* st = smem + (q % NS) * C::STAGE;
    for (int i = wave; i < C::NINS; i += C::NW) {
      if (i < 2 * C::WINS) {
        const int blk = i / C::WINS, ks = kb + blk, ii = i - blk * C::WINS;
        const int r = ii * C::RPI + lane / (64 / C::RPI);
        const int p = lane % (64 / C::RPI);
        const int c = p ^ (2 * (r & 7));
        const int u = min(ks * 32 + r, K - 1);
        const int h = pad_s ? u + int(fastdiv(uint32_t(u), pdiv)) : u;
        const int col = min(v0 + c * 8, V - 8);
        __builtin_amdgcn_global_load_lds(w + size_t(h) * V + col, (lds_void*)(st + i * 1024), 16, 0,
                                         2 /* non-temporal */);
      } else {
        const int e = i - 2 * C::WINS;
        const int ks = kb + e / (NT * C::BTW), t = (e / C::BTW) % NT;
        const int rt = min(b0 / 16 + rg * C::BTW + e % C::BTW, rtiles - 1);
        __builtin_amdgcn_global_load_lds(
            act + (((size_t(t) * rtiles + rt) * (Kp / 32) + ks) * 64 + lane) * 8,
            (lds_void*)(st + i * 1024), 16, 0, 0);
      }
    }
  };

  // this wave's copies of step q into stage (q % NS)
  auto issue = [&](int q) {
    if (C::ITEMS && q >= nmain) {
      issue_item(q);
      return;
    }
    const int j = q / nks, ks = q % nks;
    const int v0 = c0 + j * VT;
    unsigned char* st = smem + (q % NS) * C::STAGE;
    for (int i = wave; i < C::NINS; i += C::NW) {
      if (i < C::WINS) {
        const int r = i * C::RPI + lane / (64 / C::RPI);
        const int p = lane % (64 / C::RPI);
        const int c = p ^ (2 * (r & 7));
        const int u = min(ks * 32 + r, K - 1);
        const int h = pad_s ? u + int(fastdiv(uint32_t(u), pdiv)) : u;
        const int col = min(v0 + c * 8, V - 8);
        __builtin_amdgcn_global_load_lds(w + size_t(h) * V + col, (lds_void*)(st + i * 1024), 16, 0,
                                         2 /* non-temporal */);
      } else {
        const int f = i - C::WINS, t = f / NBT, bt = f % NBT;
        const int rt = min(b0 / 16 + bt, rtiles - 1);
        __builtin_amdgcn_global_load_lds(
            act + (((size_t(t) * rtiles + rt) * (Kp / 32) + ks) * 64 + lane) * 8,
            (lds_void*)(st + C::WBYTES + f * 1024), 16, 0, 0);
      }
    }
  };

  f32x4 acc[C::VTW][C::BTW];
#pragma unroll
  for (int i = 0; i < C::VTW; ++i)
#pragma unroll
    for (int j = 0; j < C::BTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-row output scales, loaded once (a load in the epilogue would make the
  // compiler drain the copies in flight)
  float scale[C::BTW];
#pragma unroll
  for (int bt = 0; bt < C::BTW; ++bt) {
    const int b = b0 + (wb * C::BTW + bt) * 16 + s16;
    scale[bt] = (b < gbs && row_scale) ? row_scale[b] : 1.0f;
  }

  // Transposing reads: lane (g, s) supplies row r = 4 g + (s >> 2) of the
  // block (+16 for the second read) and bytes 8 (s & 3) .. +7 of the tile's
  // 32-byte column pair, whose chunks sit at (2 tile) ^ (2 (r % 8)).  They are
  // issued as inline assembly: the compiler cannot tell them apart from the
  // LDS the copies in flight are filling and would wait for every copy.
  const int tr_row = 4 * kg + (s16 >> 2);
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t smem_base = uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)smem));
  uint32_t tr_addr[C::VTW];
#pragma unroll
  for (int vt = 0; vt < C::VTW; ++vt) {
    const int tile = wv * C::VTW + vt;
    const int ch = 2 * ((tile & ~7) | ((tile & 7) ^ (tr_row & 7)));
    tr_addr[vt] = smem_base + tr_row * C::WPITCH + ch * 16 + 8 * (s16 & 3);
  }

  // one 32-row K block of a stage: the weights at LDS byte aoff (read
  // transposed), the wave's fragment (term t, row tile bt) at
  // bsrc + (t tstride + bt) KiB; tiles past ntile are skipped
  auto mma_block = [&](uint32_t aoff, const unsigned char* bsrc, int tstride, int ntile) {
    s16x4 alo[C::VTW], ahi[C::VTW];
#pragma unroll
    for (int vt = 0; vt < C::VTW; ++vt) {
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(alo[vt]) : "v"(tr_addr[vt] + aoff));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(ahi[vt])
                   : "v"(tr_addr[vt] + aoff), "i"(16 * C::WPITCH));
    }
    bf16x8 bfr[C::BTW][NT];
#pragma unroll
    for (int bt = 0; bt < C::BTW; ++bt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bfr[bt][t] =
            *reinterpret_cast<const bf16x8*>(bsrc + ((t * tstride + bt) * 64 + lane) * 16);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int vt = 0; vt < C::VTW; ++vt) asm volatile("" : "+v"(alo[vt]), "+v"(ahi[vt]));
#pragma unroll
    for (int vt = 0; vt < C::VTW; ++vt) {
      if (vt < ntile) {
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 av = {alo[vt][0], alo[vt][1], alo[vt][2], alo[vt][3],
                          ahi[vt][0], ahi[vt][1], ahi[vt][2], ahi[vt][3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int bt = 0; bt < C::BTW; ++bt)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[vt][bt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr[bt][t], acc[vt][bt], 0, 0, 0);
      }
    }
  };

  // the wave's finished tiles of columns [v0, vend): scaled logits, the
  // maxima of groups below gend, and cleared accumulators
  auto flush = [&](int v0, int vend, int gend) {
#pragma unroll
    for (int bt = 0; bt < C::BTW; ++bt) {
      const int b = b0 + (wb * C::BTW + bt) * 16 + s16;
      const float sc = scale[bt];
      uint32_t gm = 0;
#pragma unroll
      for (int vt = 0; vt < C::VTW; ++vt) {
        const int v = v0 + (wv * C::VTW + vt) * 16 + 4 * kg;
        const float4 o = make_float4(acc[vt][bt][0] * sc, acc[vt][bt][1] * sc,
                                     acc[vt][bt][2] * sc, acc[vt][bt][3] * sc);
        if (b < gbs && v < vend) {
          *reinterpret_cast<float4*>(logits + size_t(b) * V + v) = o;
          gm = max(gm, max(max(float_key(o.x), float_key(o.y)),
                           max(float_key(o.z), float_key(o.w))));
        }
        if (vt % 4 == 3) {
          gm = max(gm, (uint32_t)__shfl_xor((int)gm, 16, 64));
          gm = max(gm, (uint32_t)__shfl_xor((int)gm, 32, 64));
          const int g = (v0 + (wv * C::VTW + vt - 3) * 16) / kFusedGroup;
          if (gkey && kg == 0 && b < gbs && g < gend) gkey[size_t(b) * groups + g] = gm;
          gm = 0;
        }
        acc[vt][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  for (int p = 0; p < NS - 1 && p < total; ++p) issue(p);
  for (int q = 0; q < nmain; ++q) {
    // this wave's copies of step q are done once at most those of the steps
    // after it that are already issued are outstanding (copies complete in
    // issue order); the barrier extends that to every wave, and also retires
    // every wave's reads of step q - 1, whose stage step q + NS - 1 reuses
    wait_steps<C::WAIT, NS - 2>(min(NS - 2, total - 1 - q));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (q + NS - 1 < total) issue(q + NS - 1);

    const int j = q / nks, ks = q % nks;
    const int v0 = c0 + j * VT, vend = min(v0 + VT, c1);
    const int ntile = __builtin_amdgcn_readfirstlane((vend - v0 + 15) / 16 - wv * C::VTW);
    const uint32_t soff = uint32_t((q % NS) * C::STAGE);
    const unsigned char* st = smem + (q % NS) * C::STAGE;
    mma_block(soff, st + C::WBYTES + wb * C::BTW * 1024, NBT, ntile);
    asm volatile("" ::: "memory");
    if (ks == nks - 1) flush(v0, vend, g1);
  }

  // leftover item steps: only the item's row group computes, blocks kb and
  // kb + 1 in that order, so every element accumulates its K in order
  if constexpr (C::ITEMS) {
    for (int q = nmain; q < total; ++q) {
      wait_steps<C::WAIT, NS - 2>(min(NS - 2, total - 1 - q));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (q + NS - 1 < total) issue(q + NS - 1);
      int v0, kb;
      const int rg = item_at(q, v0, kb);
      if (wb != rg) continue;
      const int vend = min(v0 + VT, V);
      const int ntile = __builtin_amdgcn_readfirstlane((vend - v0 + 15) / 16 - wv * C::VTW);
      const uint32_t soff = uint32_t((q % NS) * C::STAGE);
      const unsigned char* st = smem + (q % NS) * C::STAGE + 2 * C::WBYTES;
#pragma nounroll
      for (int blk = 0; blk < 2; ++blk)
        mma_block(soff + blk * C::WBYTES, st + blk * NT * C::BTW * 1024, C::BTW, ntile);
      asm volatile("" ::: "memory");
      if (kb == nks - 2) flush(v0, vend, groups);
    }
  }
}

template <int VT, int WV, int WB, int NBT, int NT, int NS>
hipError_t launch_dma(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V, int K,
                      int pad_s, const float* row_scale, int gbs, int b0, float* logits,
                      uint32_t* gkey, hipStream_t st) {
  auto kern = dma_kernel<VT, WV, WB, NBT, NT, NS>;
  // resident workgroups of this kernel on the current device (once per device)
  static std::once_flag once[kMaxDevices];
  static int slots_cache[kMaxDevices];
  const int slots = per_device(once, slots_cache, [&](int dev) {
    int n = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, WV * WB * 64, 0) != hipSuccess ||
        n < 1)
      n = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    return n * cus;
  });
  const FastDiv pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  const int groups = (V + kFusedGroup - 1) / kFusedGroup;
  const int P = min(groups, slots);
  // groups dealt as whole ranges; the rest go out as leftover items
  const int gmain = DCfg<VT, WV, WB, NBT, NT, NS>::ITEMS ? groups / P * P : groups;
  hipLaunchKernelGGL(kern, dim3(P), dim3(WV * WB * 64), 0, st, act, rows_pad, Kp, w, V, K, pad_s,
                     pdiv, row_scale, gbs, b0, logits, gkey, groups, gmain);
  return hipGetLastError();
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
  // a split K runs every chunk on the per-tile kernel (128-row chunks); so
  // do two-term batches up to 192 rows, for which a 128-row chunk plus the
  // rest costs less than the persistent kernel's 256-row chunk (with one
  // term the persistent kernel stays ahead)
  const int chunk = kc_n > 1 || (NT == 2 && gbs <= 192) ? 128 : 256;
  for (int b0 = 0; b0 < gbs; b0 += chunk) {
    const int rows = gbs - b0 < chunk ? gbs - b0 : chunk;
    const int nbt = (rows + 15) / 16;
    hipError_t e;
    if (nbt <= 8) {
      // 512-column tiles (393 workgroups for GPT-OSS) and 32-row K-steps;
      // up to 64 rows two workgroups share a CU, so all are resident at once
      if (nbt <= 1) e = launch_cfg<512, 4, 1, 1, NT, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
      else if (nbt <= 2) e = launch_cfg<512, 4, 1, 2, NT, 32, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
      else if (nbt <= 4) e = launch_cfg<512, 4, 1, 4, NT, 32, 2>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
      else e = launch_cfg<512, 4, 2, 8, NT, 32>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, kc_n, part, st);
    } else {
      // persistent, direct-copy kernel; rows past the chunk are never stored.
      // One term leaves LDS for a fourth ring stage.
      e = launch_dma<256, 2, 4, 16, NT, NT == 1 ? 4 : 3>(act, rows_pad, Kp, w, V, H_u, pad_s, row_scale, gbs, b0, logits, gkey, st);
    }
    if (e != hipSuccess) return e;
  }
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
