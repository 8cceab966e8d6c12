// lm_head contraction for batches of more than 64 rows (from 65 to 128 only
// over a vocabulary wide enough to fill the chip without splitting K), on
// the bf16 matrix cores with v_mfma_f32_32x32x16_bf16 (GPT-OSS tail API page, parameter
// "lm_head_weight_t": [H, V] bf16, already transposed and C-contiguous).
//
// logits[b, v] = row_scale[b] * sum_h (sum_t A_t[b, h]) * W[h, v]
//
// The activations arrive as NT bf16 terms (two by default, each the bf16
// rounding of what the earlier terms left, so every MFMA product is exact;
// one in the page-precision mode), stored by the activation producer as
// ready B-operand fragments: one 1 KB fragment per (16-lane K block, term,
// 32-row tile), lane 32 h + n holding row n at K lanes 8 h .. 8 h + 7.
//
// One launch covers a chunk of batch rows for the whole vocabulary, with one
// persistent workgroup per CU of 8 waves, two per SIMD, each wave owning one
// 32-row tile of the chunk and a column part of every tile, in accumulators
// of 32 x 32 (at most 13 blocks: 208 of the wave's 256 registers).  Two
// shapes: CPN = 2 column parts (a 128-row chunk; wave w owns rows
// 32 (w % 4) .. + 31 and the first (w < 4) or second half of the tile's
// blocks), used up to 128 rows, and CPN = 1 (a 256-row chunk; wave w owns
// rows 32 w .. + 31 and all of the tile's blocks, except that a two-term
// chunk of 5 or 6 real tiles halves some of them, see below), used above.
// Either way the tiles hold up to MB = 13 blocks, so GPT-OSS's vocabulary
// takes 2 passes over the activations instead of the 3 that 9-block tiles
// need (a third fewer activation bytes re-read from L2).  The vocabulary is cut
// into 32-column blocks and the blocks into npass * P tiles of equal width
// (to within one block, at most MB blocks); workgroup w takes tiles w,
// w + P, w + 2P, ..., so at any time the P workgroups read one contiguous
// column range of every weight row (whole DRAM pages together: measured
// 6.9 TB/s for the weight stream alone against 5.3 TB/s with contiguous
// per-workgroup ranges).
//
// A wave whose rows are all padding (a short last chunk) skips its reads and
// MFMAs and only takes part in the copies and barriers.  Per K-step of 16
// hidden lanes the tile's weight [16 x 32 W] goes to an LDS ring of NSW
// stages, NSW - 1 steps ahead, and the step's activation fragments (one per
// 32-row tile and term) to a ring of NSA stages, NSA - 1 steps ahead, by
// direct global-to-LDS copies: waves 0-3 copy the weight, waves 4-7 the
// activations, so each wave waits only on one stream (vector memory
// operations complete in issue order per wave: one wave carrying both the
// slow weight stream and the fast activation stream made the fast one wait
// for the slow one, 320 us against 227 us for the data movement of one
// gbs-256 call).  One barrier per step publishes the stage and retires the
// reads of the stage the next copies overwrite; it is the bare s_barrier,
// since a workgroup fence before it would drain every copy in flight.  The
// copies are issued as inline assembly: a compiler that sees them would make
// every LDS read of the wave wait for every copy in flight.  They write only
// LDS, so no register of the wave is pending.
//
// In the two-part shape the two waves of a SIMD are staggered by half a
// step: between two barriers waves 0-3 read the step's operands and then run
// its MFMAs, while waves 4-7 first run the MFMAs of the operands they read
// before the barrier and then read the step's, so one wave's LDS reads
// overlap the other's MFMAs.  The one-part shape cannot hold a whole step's
// operands across a barrier next to 208 accumulators, so every wave reads
// and multiplies block by block, the reads a few blocks ahead.
//
// LDS layouts: a weight stage holds 16 rows of 32 MB columns at a row pitch
// of 64 MB bytes padded to 64 mod 256, so the 8 row segments that 32 lanes of
// a transposing read touch fall in distinct 32-byte bank groups.  The weight
// operand of a block comes from two ds_read_b64_tr_b16: in each 16-lane group
// g of the wave, lane s supplies row 8 (g / 2) + s / 4 (+4 for the second
// read), columns 16 (g % 2) + 4 (s % 4) .. + 3 of the block, and receives
// column 16 (g % 2) + s at K lanes 8 (g / 2) .. + 7: the natural K order of
// the activation fragments, which an activation stage holds as copied (1 KB
// each, read back linearly).
//
// Epilogue (after a tile's last K-step): accumulator register 4 i + e of lane
// l holds column 8 i + 4 (l / 32) + e of the block for row l % 32, so each
// lane stores float4s; the 64-column key groups' maxima go to gkey (a plain
// store when both 32-column blocks of the group belong to the wave, an atomic
// maximum into the cleared entry when the group straddles two parts or two
// tiles).
//
// Determinism: every output element is one fixed sequence of MFMAs (K-steps
// in order, terms in order), the same for every column and row and in both
// shapes.
//
// Fused top-k and sampler (optional, FusedSelect): the page's tail is one
// kernel from the RMSNorm to the sampled token (GPT-OSS tail API page,
// Background).  Here the workgroups of a launch, one per CU and normally all
// resident at once, finish their tiles, then meet at a grid barrier (their
// logit and group-maximum stores written back device-wide, one lane per
// workgroup counts the workgroup in on an arrival counter and polls it until
// all have arrived, as in the leader-follower barrier of the Triton
// megakernel page), and then take the launch's rows one at a time from a
// second counter and run the select of select_row.h on each with all 512
// threads, the rings' LDS reused for its lists.  The poll is bounded: a
// workgroup that stops polling leaves the rows to the others, and the last
// one to arrive never polls, so every row is selected whether or not the
// workgroups were resident together, and every workgroup ends.  The results
// are bitwise those of the separate select launch.
#include "lds_copy.h"
#include "select_row.h"

namespace tail {
namespace {

using namespace mfma32;

template <int NT, int MB, int NSW, int NSA, int CPN>
struct RCfg {
  static constexpr int RT = 8 / CPN;                     // 32-row tiles per chunk (one per row group)
  static constexpr int CHUNK = 32 * RT;                  // 128 or 256 rows
  static constexpr int WPITCH = weight_pitch(MB);
  static constexpr int WCH = WPITCH / 16;                // 16-byte chunks per weight row
  static constexpr int WSTAGE = 16 * WPITCH;
  static constexpr int WCOP = WSTAGE / 1024;             // weight copies per step
  static constexpr int WPER = (WCOP + 3) / 4;            // most weight copies of a wave
  static constexpr int AFR = NT * RT;                    // activation fragments per step
  static constexpr int APER = AFR / 4;                   // activation copies per wave
  static constexpr int ASTAGE = AFR * 1024;
  static constexpr int LDS = NSW * WSTAGE + NSA * ASTAGE;
  static constexpr int HB = (MB + CPN - 1) / CPN;        // most blocks of a column part
  static_assert((CPN == 1 || CPN == 2) && WSTAGE % 1024 == 0 && WPITCH % 256 == 64 &&
                    WCH <= 64 && AFR % 4 == 0 && NSW >= 2 && NSA >= 2 &&
                    WPER * (NSW - 2) < 64 && APER * (NSA - 2) < 64 && LDS <= 160 * 1024,
                "tile");
};

// The copies of one wave: the weight (waves 0-3) or the activations (4-7).
template <typename C, int NT, int NSW, int NSA>
struct Copier {
  const TileGeom& G;
  uint32_t wring, aring;  // LDS byte addresses of the rings
  int wave, lane;
  const uint16_t* __restrict__ act;
  int nrt;
  const uint16_t* __restrict__ w;
  int V, K, pad_s;
  FastDiv pdiv;
  int b0;

  // this wave's copies of step q (of all the wave's steps)
  __device__ __forceinline__ void issue(int q) const {
    const int j = q / G.nks, ks = q % G.nks;
    if (wave < 4) {
      int start, width;
      G.tile(j, start, width);
      const uint32_t st = wring + uint32_t((q % NSW) * C::WSTAGE);
#pragma unroll
      for (int c = 0; c < C::WPER; ++c) {
        const int ci = wave + 4 * c;  // copies wave, wave + 4, ...
        if (ci < C::WCOP) {
          const int i = ci * 64 + lane;  // 16-byte chunk of the stage
          const int r = i / C::WCH, cc = i % C::WCH;
          const int u = min(ks * 16 + r, K - 1);
          const int h = pad_s ? u + int(fastdiv(uint32_t(u), pdiv)) : u;
          const int col = min(start * 32 + cc * 8, V - 8);
          // lanes past the tile's width stay idle (every copy of 64 chunks
          // spans a whole row, so some of its lanes always copy)
          if (cc < 4 * width) copy_to_lds<true>(w + size_t(h) * V + col, st + uint32_t(ci * 1024));
        }
      }
    } else {
      const uint32_t st = aring + uint32_t((q % NSA) * C::ASTAGE);
#pragma unroll
      for (int c = 0; c < C::APER; ++c) {
        const int f = (wave - 4) * C::APER + c;  // fragment (term f / RT, row tile f % RT)
        const int t = f / C::RT, rt = min(b0 / 32 + f % C::RT, nrt - 1);
        copy_to_lds<false>(act + (((size_t(ks) * NT + t) * nrt + rt) * 64 + lane) * 8,
                           st + uint32_t(f * 1024));
      }
    }
  }
  __device__ __forceinline__ int ahead() const { return wave < 4 ? NSW - 1 : NSA - 1; }
  // this wave's copies of step q have landed once at most those of the steps
  // issued after it are outstanding
  __device__ __forceinline__ void wait(int q) const {
    if (wave < 4) {
      // waves whose last copy slot is empty issue one copy fewer per step
      if (wave + 4 * (C::WPER - 1) < C::WCOP)
        wait_copies<C::WPER, NSW - 2>(min(NSW - 2, G.total - 1 - q));
      else
        wait_copies<C::WPER - 1, NSW - 2>(min(NSW - 2, G.total - 1 - q));
    } else {
      wait_copies<C::APER, NSA - 2>(min(NSA - 2, G.total - 1 - q));
    }
  }
  // the start of a step: this wave's copies of it landed and its reads of the
  // previous one done, then the barrier
  __device__ __forceinline__ void step(int q) const {
    wait(q);
    wait_lds();
    step_barrier();
  }
  // the end of a step's work: the copies NS - 1 steps ahead.  Issued after
  // the step's reads and MFMAs, since an issue that the memory pipeline does
  // not accept at once stalls the wave's next instructions (measured: 4.5%
  // faster than issuing right after the barrier).
  __device__ __forceinline__ void refill(int q) const {
    if (q + ahead() < G.total) issue(q + ahead());
  }
};

// One wave's part of one tile (steps q0 .. q0 + nks - 1): WC blocks starting
// at block cb0 of the tile, row tile rg of the chunk.  LAG: the wave runs each
// step's MFMAs after the next barrier (see above).
template <typename C, typename CP, int NT, int NSW, int NSA, int WC, bool LAG>
__device__ __forceinline__ void tile_part(const CP& cp, const lds_u8* wring, const lds_u8* aring,
                                          int rg, int lane, int q0, int blk0, int cb0,
                                          float scale, int b0, int gbs, int V,
                                          float* __restrict__ logits,
                                          uint32_t* __restrict__ gkey, int groups) {
  const int tr_off = tr_lane_offset<C::WPITCH>(lane) + cb0 * 64;
  const int b_off = (rg * 64 + lane) * 16;
  const int nks = cp.G.nks;

  f32x16 acc[WC];
#pragma unroll
  for (int c = 0; c < WC; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;

  bf16x8 bop[NT], aop[WC];
  auto read = [&](int q) {
    int tro = tr_off, bo = b_off;
    // with 208 accumulators, the compiler would otherwise keep every
    // block's LDS address in a register of its own (hoisted out of the K
    // loop) and spill; opaque per-step offsets make it fold the block
    // offsets into the reads' immediate fields
    if constexpr (WC > 7) asm volatile("" : "+v"(tro), "+v"(bo));
    const lds_u8* wst = wring + (q % NSW) * C::WSTAGE + tro;
    const lds_u8* ast = aring + (q % NSA) * C::ASTAGE + bo;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bop[t] = *reinterpret_cast<const lds_bf16x8*>(ast + t * C::RT * 1024);
#pragma unroll
    for (int c = 0; c < WC; ++c) aop[c] = weight_operand<C::WPITCH>(wst + c * 64);
  };
  auto mma = [&]() {
#pragma unroll
    for (int c = 0; c < WC; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[c], bop[t], acc[c], 0, 0, 0);
  };

  for (int ks = 0; ks < nks; ++ks) {
    const int q = q0 + ks;
    cp.step(q);
    if constexpr (LAG) {
      if (ks > 0) mma();
      read(q);
    } else {
      read(q);
      mma();
    }
    cp.refill(q);
  }
  if constexpr (LAG) mma();

  // epilogue: scaled logits, key-group maxima
  const int b = b0 + rg * 32 + (lane & 31);
  store_tile<WC>(acc, scale, b, b < gbs, blk0, cp.G.nblk, lane, V, logits, gkey, groups);
}

// The grid barrier and the select phase (see above) over rows b0 .. b0 +
// nrows - 1; smem holds at least a SelShared and one more word.  MIRROR: the
// page-precision mode's bf16 ranking.  tid = 64 wave + lane, the lane
// recomputed from the execution mask (carrying the work-item id through the
// tile phase would cost a register there).
template <bool MIRROR>
__device__ __forceinline__ void fused_select(unsigned char* smem, int tid, const FusedSelect& fs,
                                             uint32_t* sync, const float* logits,
                                             const uint32_t* gkey, int V, int b0, int nrows) {
  SelShared& s = *reinterpret_cast<SelShared*>(smem);
  int* const word = reinterpret_cast<int*>(smem + sizeof(SelShared));
  // arrival: every wave waits until its stores have reached the L2, then one
  // lane writes the L2 back device-wide (one release per workgroup: a release
  // in every wave, each writing the whole L2 back, cost about 35 us at 256
  // rows) and counts the workgroup in.  Leaving, that lane invalidates the
  // caches its CU and L2 hold for the other workgroups' results (once for
  // all waves of the CU).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    // the explicit waits after the write-back and after the invalidation
    // make each complete before the arrival, and before the other waves
    // read (the compiler adds none there when no store or load of this wave
    // is outstanding)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t n = __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) + 1u;
    for (int i = 0; n < gridDim.x && i < fs.spin; ++i) {
      __builtin_amdgcn_s_sleep(8);
      n = __hip_atomic_load(&sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *word = n >= gridDim.x;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*word)) return;  // the rows are left to the others
  // the sampler's candidates per lane, as the standalone select launches it
  const int pc = fs.k <= 64 ? 1 : fs.k <= 128 ? 2 : fs.k <= 256 ? 4 : fs.k <= 512 ? 8 : 16;
  auto sample = [&](SelShared& sh, const RowParams& prm, int lane) -> int32_t {
#define TAIL_FUSED_SAMPLE(PC) \
  return sample_row_wave<PC>(sh.top_v, sh.top_i, fs.k, prm.top_k, prm.top_p, prm.temp, prm.u, lane)
    switch (pc) {
      case 1: TAIL_FUSED_SAMPLE(1);
      case 2: TAIL_FUSED_SAMPLE(2);
      case 4: TAIL_FUSED_SAMPLE(4);
      case 8: TAIL_FUSED_SAMPLE(8);
      default: TAIL_FUSED_SAMPLE(16);
    }
#undef TAIL_FUSED_SAMPLE
  };
  for (;;) {
    __syncthreads();  // the previous row's lists have been read
    if (tid == 0)
      *word = int(__hip_atomic_fetch_add(&sync[1], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    const int r = __builtin_amdgcn_readfirstlane(*word);
    if (r >= nrows) break;
    select_row<512, MIRROR>(s, tid, b0 + r, logits, V, fs.gs, fs.groups, fs.k, gkey, 0, fs.vals, fs.idx,
                            nullptr, fs.params, fs.ncols, fs.tokens, sample);
  }
}

template <int NT, int MB, int NSW, int NSA, int CPN>
__global__ __launch_bounds__(512, 1) void rows_kernel(
    const uint16_t* __restrict__ act, int nrt, int Kp, const uint16_t* __restrict__ w, int V, int K,
    int pad_s, FastDiv pdiv, const float* __restrict__ row_scale, int gbs, int b0,
    float* __restrict__ logits, uint32_t* __restrict__ gkey, int groups, int npass,
    const FusedSelect* __restrict__ fsp) {
  using C = RCfg<NT, MB, NSW, NSA, CPN>;
  using CP = Copier<C, NT, NSW, NSA>;
  static_assert(sizeof(SelShared) + 4 <= C::LDS, "select lists in the rings' LDS");
  __shared__ __align__(1024) unsigned char smem[C::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TileGeom G(V, Kp, npass);
  if (G.total == 0 && fsp == nullptr) return;  // the whole workgroup
  lds_u8* const wring = (lds_u8*)smem;
  lds_u8* const aring = wring + NSW * C::WSTAGE;
  const uint32_t wring_addr = uint32_t(reinterpret_cast<uintptr_t>(wring));
  const CP cp{G, wring_addr, wring_addr + uint32_t(NSW * C::WSTAGE), wave, lane, act, nrt, w, V,
              K, pad_s, pdiv, b0};

  // row tile and column part of this wave (part 0: the tile's first half, 1:
  // its second half, 2: the whole tile)
  int rg = CPN == 2 ? (wave & 3) : wave, part = CPN == 2 ? (wave >> 2) : 2;
  if constexpr (CPN == 1 && NT == 2) {
    // 5 or 6 real tiles in a 256-row chunk: whole-tile waves would leave two
    // SIMDs running two whole tiles each while others idle.  So 8 - nreal
    // tiles are halved instead: waves 0 .. 2 nreal - 9 take the whole tiles
    // 8 - nreal .., and each of the others a half, the SIMD partners (w,
    // w + 4) of the whole-tile waves first, so no SIMD runs more than one
    // whole tile and one half.  (Not in the one-term kernel, whose
    // registers it would overrun by a few.)
    const int nreal = min(C::RT, nrt - b0 / 32);
    if (nreal == 5 || nreal == 6) {
      const int nwhole = 2 * nreal - 8;  // 2 or 4
      if (wave < nwhole) {
        rg = 8 - nreal + wave;
      } else {
        // half-tile waves in the order 4, 5, 6, 7, then nwhole .. 3
        const int order = wave >= 4 ? wave - 4 : wave - nwhole + 4;
        rg = order >> 1;
        part = order & 1;
      }
    }
  }
  // a 32-row tile that holds no row of the batch is padding: its reads and
  // MFMAs are skipped
  const bool real = b0 + rg * 32 < gbs;
  const int b = b0 + rg * 32 + (lane & 31);
  const float scale = (b < gbs && row_scale) ? row_scale[b] : 1.0f;
  // the scale has arrived before the first copy is issued
  wait_vm<0>();
  for (int p = 0; p < cp.ahead() && p < G.total; ++p) cp.issue(p);

  for (int j = 0; j < G.ntl; ++j) {
    int start, width;
    G.tile(j, start, width);
    const int w0 = part == 2 ? width : (width + 1) / 2;
    const int cb0 = part == 1 ? w0 : 0, wc = part == 1 ? width - w0 : w0;
    const int q0 = j * G.nks;
#define TAIL_ROWS_PART(WW)                                                                     \
  case WW:                                                                                     \
    if constexpr (WW <= C::HB) {                                                               \
      if (CPN == 2 && part)                                                                    \
        tile_part<C, CP, NT, NSW, NSA, WW, CPN == 2>(cp, wring, aring, rg, lane, q0,           \
                                                     start + cb0, cb0, scale, b0, gbs, V,      \
                                                     logits, gkey, groups);                    \
      else                                                                                     \
        tile_part<C, CP, NT, NSW, NSA, WW, false>(cp, wring, aring, rg, lane, q0, start + cb0, \
                                                  cb0, scale, b0, gbs, V, logits, gkey,        \
                                                  groups);                                     \
    }                                                                                          \
    break;
    // a one-block tile leaves the second part empty, and a short last chunk
    // leaves the waves of its all-padding 32-row tiles idle: barriers (and
    // their share of the copies) only
    switch (real ? wc : 0) {
      case 0:
        for (int ks = 0; ks < G.nks; ++ks) {
          cp.step(q0 + ks);
          cp.refill(q0 + ks);
        }
        break;
      TAIL_ROWS_PART(1) TAIL_ROWS_PART(2) TAIL_ROWS_PART(3) TAIL_ROWS_PART(4) TAIL_ROWS_PART(5)
      TAIL_ROWS_PART(6) TAIL_ROWS_PART(7) TAIL_ROWS_PART(8) TAIL_ROWS_PART(9) TAIL_ROWS_PART(10)
      TAIL_ROWS_PART(11) TAIL_ROWS_PART(12) TAIL_ROWS_PART(13)
      default: break;
    }
#undef TAIL_ROWS_PART
  }
  // not in the one-term one-part kernel, which uses all 256 registers and
  // spills with any code after its tiles (rows_fuse_select)
  if constexpr (NT == 2 || CPN == 2) {
    if (fsp != nullptr) {
      const FusedSelect fs = *fsp;
      // each launch of a multi-launch batch has its own two counters
      fused_select<NT == 1>(smem, wave * 64 + int(__lane_id()), fs, fs.sync + 2 * (b0 / C::CHUNK),
                            logits, gkey, V, b0, min(gbs - b0, C::CHUNK));
    }
  }
}

template <int NT, int MB, int NSW, int NSA, int CPN>
hipError_t launch_rows_cfg(const uint16_t* act, int rows_pad, int Kp, const uint16_t* w, int V,
                           int K, int pad_s, const float* row_scale, int gbs, float* logits,
                           uint32_t* gkey, const FusedSelect* fs, hipStream_t st) {
  auto kern = rows_kernel<NT, MB, NSW, NSA, CPN>;
  static std::once_flag once[kMaxDevices];
  static int cus_cache[kMaxDevices];
  const int cus = per_device(once, cus_cache, [&](int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    return n;
  });
  const FastDiv pdiv = make_fastdiv(pad_s > 1 ? uint32_t(pad_s - 1) : 1u);
  const int nblk = (V + 31) / 32;
  const int P = nblk < cus ? nblk : cus;
  const int npass = (nblk + P * MB - 1) / (P * MB);
  const int groups = (V + kFusedGroup - 1) / kFusedGroup;
  for (int b0 = 0; b0 < gbs; b0 += RCfg<NT, MB, NSW, NSA, CPN>::CHUNK) {
    hipLaunchKernelGGL(kern, dim3(P), dim3(512), 0, st, act, rows_pad / 32, Kp, w, V, K, pad_s,
                       pdiv, row_scale, gbs, b0, logits, gkey, groups, npass, fs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_lm_head_rows(const uint16_t* act, int nt, int rows_pad, int Kp, const uint16_t* w,
                               int V, int K, int pad_s, const float* row_scale, int gbs,
                               float* logits, uint32_t* gkey, const FusedSelect* fs,
                               hipStream_t st) {
  // up to 128 rows: one 128-row chunk in two column parts; above: 256-row
  // chunks in one part.  Tiles of up to 13 blocks either way (2 passes for
  // GPT-OSS); ring depths from sweeps.
  if (gbs <= 128) {
    if (nt == 2)
      return launch_rows_cfg<2, 13, 8, 4, 2>(act, rows_pad, Kp, w, V, K, pad_s, row_scale, gbs,
                                             logits, gkey, fs, st);
    if (nt == 1)
      return launch_rows_cfg<1, 13, 8, 6, 2>(act, rows_pad, Kp, w, V, K, pad_s, row_scale, gbs,
                                             logits, gkey, fs, st);
    return hipErrorInvalidValue;
  }
  if (nt == 2)
    return launch_rows_cfg<2, 13, 8, 3, 1>(act, rows_pad, Kp, w, V, K, pad_s, row_scale, gbs,
                                           logits, gkey, fs, st);
  if (nt == 1)
    return launch_rows_cfg<1, 13, 8, 5, 1>(act, rows_pad, Kp, w, V, K, pad_s, row_scale, gbs,
                                           logits, gkey, fs, st);
  return hipErrorInvalidValue;
}

}  // namespace tail
