// Exact top-k of one logit row over the full vocabulary (GPT-OSS tail API
// page: Background -- the global top-k is computed locally over the full
// vocabulary -- and parameter "k"), optionally followed by the row's sampler,
// by one workgroup of NTHR threads.  The standalone select kernel (1024
// threads, topk.hip) and the phase after the grid barrier of the large-batch
// lm_head (512 threads, lm_head_rows.hip) run this same code, so a row gives
// the same bytes either way.
//
// Input: the logits and, per row, the largest order-preserving key of every
// group of gs consecutive columns (gs a power of two with at least k groups).
//
// select_row:
//  a. t0 = a lower bound of the k-th largest group maximum (one histogram of
//     the maxima in power-of-two bins).  At least k groups have a maximum >=
//     t0 and each maximum is an element, so every top-k member is >= t0, and
//     only groups whose maximum is >= t0 can hold one.
//  b. Those groups are scanned (loads batched five deep per thread) and every
//     element >= t0 is appended to an LDS list as the composite key
//     (value key << 32) | ~index: larger value first, lower index first.
//  c. Lists longer than 2k are cut to the k-th largest value v* (radix select)
//     and, when ties at v* would still leave more than 2k, to the lowest
//     indices among the elements equal to v* (radix select on ~index).
//  d. Survivors are counting-sorted into 256 bins of their value key; a
//     survivor's rank is its bin's start plus the number of larger composite
//     keys in its own bin (about one entry on typical rows); ranks below k
//     are written out (and kept in LDS for the sampler).
//  e. More than kCap elements >= t0 (massive ties): the same two cuts are
//     found by radix passes that re-read the candidate groups, then only the
//     k winners are collected.  Exact for any input, slow only for such rows.
//  f. With sampling parameters, wave 0 samples the row from the sorted list.
//
// Values are copied from the logits, so -0.0 keeps its sign while ranking
// equal to +0.0.
//
// Mirror mode (parameter "emit_logits": the page's top-k ranks the bf16
// mirror of the fp32 logits): every element is rounded to bf16 (nearest,
// ties to even) as it is read, and the rounded value is what is ranked and
// returned.  The group maxima may come from the unrounded logits: rounding
// is monotone, so the rounded maximum of a group is the maximum of its
// rounded elements, and step a's bound holds unchanged.
//
// NaN fold (parameter "skip_nan_fold" off): a NaN logit (either sign) ranks
// and is returned as -inf; the group maxima must then come from
// group_max_kernel with the same fold (a NaN in the lm_head epilogue's
// maxima would hide its group's real maximum).  Without the fold, NaN
// ordering is unspecified; infinities always order as numbers.
//
// Taps (optional, per row, 4 x u32): the bound t0 as an order-preserving key,
// the number of candidate groups, the number of elements with key >= t0 (all
// of them, also past the LDS capacity), and 1 when that number exceeded the
// capacity (the radix path of step e ran), else 0.
#pragma once

#include "sampler_row.h"
#include "../../include/tail.h"

namespace tail {
namespace {

constexpr int kCap = 4096;  // LDS candidate capacity
// the final ranking keeps 2k composites and 2k value bits in the group list's space
static_assert(kMaxGroups >= 6 * TAIL_K_MAX, "group list too small for the sorted copy");
constexpr int kBatch = 4;      // float4 loads in flight per thread
constexpr int kScanBatch = 5;  // the same in the candidate scan (step b)
static_assert(kScanBatch * 4 <= 32, "the scan's per-thread hit mask is 32 bits");

// Wave-wide integer reductions and prefix sums through lane moves inside the
// register file (DPP): quad permutations and row mirrors combine the 16 lanes
// of a row, row shifts build a row's prefix, and the row broadcasts of lanes
// 15 and 31 carry it across rows.  Integer results do not depend on the
// order, and each step costs a few cycles where an LDS-routed shuffle costs
// a round trip.  Every lane of the wave must be active.  A lane that
// receives nothing from a move keeps `old`.
template <int CTRL, int ROWS = 0xf, int BANKS = 0xf>
__device__ inline uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), CTRL, ROWS, BANKS, false));
}
template <typename Op>
__device__ inline uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_mov<0xb1>(v, v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4e>(v, v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141>(v, v));  // row_half_mirror
  v = op(v, dpp_mov<0x140>(v, v));  // row_mirror: every lane holds its row's result
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
// inclusive prefix sum in lane order
__device__ inline uint32_t wave_incl_sum_u32(uint32_t v) {
  v += dpp_mov<0x111>(0u, v);        // row_shr:1
  v += dpp_mov<0x112>(0u, v);        // row_shr:2
  v += dpp_mov<0x114>(0u, v);        // row_shr:4
  v += dpp_mov<0x118>(0u, v);        // row_shr:8: prefix within each row
  v += dpp_mov<0x142, 0xa>(0u, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_mov<0x143, 0xc>(0u, v);  // row_bcast:31 into rows 2 and 3
  return v;
}

struct SelShared {
  uint32_t act[kMaxGroups];  // candidate groups of the row
  uint64_t c[kCap];          // candidate composite keys
  uint32_t cb[kCap];         // their original value bits (keeps the sign of -0.0)
  float top_v[TAIL_K_MAX];   // the sorted result, for the sampler
  int32_t top_i[TAIL_K_MAX];
  uint32_t hist[256];
  uint32_t bstart[257];     // bin starts of the final ranking
  uint32_t bc[4];
  uint32_t cnt, nact;
};

__device__ inline uint64_t composite(uint32_t key, int e) {
  return (uint64_t(key) << 32) | uint64_t(~uint32_t(e));
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Block-wide radix select: the k-th largest (k >= 1) 32-bit key among those
// visit(f) enumerates (f(key) once per key of the calling thread; every
// thread calls visit).  Returns the key; *above = keys strictly greater,
// *equal = keys equal to it.  The visited set must hold at least k keys.
// A first pass takes the keys' minimum and maximum, so the digit passes
// (8 bits each, most significant first) start at the highest bit on which
// the keys differ: no pass spends its histogram on one crowded bin.
template <typename Visit>
__device__ uint32_t radix_kth(SelShared& s, int tid, uint32_t k, Visit&& visit, uint32_t* above,
                              uint32_t* equal) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0, cnt = 0;
  visit([&](uint32_t key) {
    lo = min(lo, key);
    hi = max(hi, key);
    ++cnt;
  });
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  cnt = wave_sum_u32(cnt);
  if (tid == 0) {
    s.bc[0] = 0xFFFFFFFFu;
    s.bc[1] = 0u;
    s.bc[2] = 0u;
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    atomicMin(&s.bc[0], lo);
    atomicMax(&s.bc[1], hi);
    atomicAdd(&s.bc[2], cnt);
  }
  __syncthreads();
  lo = s.bc[0];
  hi = s.bc[1];
  cnt = s.bc[2];
  __syncthreads();
  if (lo == hi) {  // all keys equal
    *above = 0;
    *equal = cnt;
    return lo;
  }
  int top = 31 - __clz(int(lo ^ hi));  // highest bit on which keys differ
  uint32_t prefix = top == 31 ? 0u : (hi & ~((2u << top) - 1u));
  uint32_t need = k, eq = 0;
  while (top >= 0) {
    const int w = top + 1 < 8 ? top + 1 : 8;
    const int shift = top - w + 1;
    const uint32_t amask = top == 31 ? 0u : ~((2u << top) - 1u);  // bits above the digit
    const uint32_t dmask = (1u << w) - 1u;
    if (tid < 256) s.hist[tid] = 0;
    __syncthreads();
    visit([&](uint32_t key) {
      if ((key & amask) == prefix) atomicAdd(&s.hist[(key >> shift) & dmask], 1u);
    });
    __syncthreads();
    if (tid < 64) {  // wave 0: bins in descending digit order, lane l holds 255-4l .. 252-4l
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s.hist[255 - 4 * tid - j];
        loc += c[j];
      }
      const uint32_t incl = wave_incl_sum_u32(loc);
      uint32_t run = incl - loc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < need && run + c[j] >= need) {
          s.bc[0] = 255 - 4 * tid - j;
          s.bc[1] = need - run;
          s.bc[2] = c[j];
        }
        run += c[j];
      }
    }
    __syncthreads();
    prefix |= s.bc[0] << shift;
    need = s.bc[1];
    eq = s.bc[2];
    top = shift - 1;
    __syncthreads();
  }
  *above = k - need;
  *equal = eq;
  return prefix;
}

// Append (key, e) of the lanes where pred holds; slots past kCap are counted
// but not stored.  Must be called by all lanes of the wave.
__device__ inline void wave_append(SelShared& s, bool pred, uint32_t key, int e, uint32_t bits,
                                   int lane) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&s.cnt, (uint32_t)__popcll(mask));
  base = __builtin_amdgcn_readlane(base, 0);
  if (pred) {
    const uint32_t pos = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (pos < kCap) {
      s.c[pos] = composite(key, e);
      s.cb[pos] = bits;
    }
  }
}

// The bits an element is ranked and returned by: its own, or (mirror) its
// bf16 rounding.
template <bool MIRROR>
__device__ inline uint32_t rank_bits(float x, bool fold) {
  uint32_t u = __float_as_uint(x);
  if (fold && (u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN -> -inf
  if constexpr (MIRROR) return bf16_rne_bits(u) << 16;
  else return u;
}

// Order-preserving key -> the key of the value's bf16 rounding.
__device__ inline uint32_t mirror_key(uint32_t key) {
  const uint32_t bits = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return float_key(__uint_as_float(bf16_rne_bits(bits) << 16));
}

// One batch of candidate float4 slots f0 + u * NTHR (gs >= 4, per =
// gs / 4 = 2^lg slots a group, total slots): every group id is read from LDS
// first, then every load is issued, from a clamped slot, through a global
// pointer, with no branch between the loads.  (The helpers that call this
// are not always inlined; through the generic row pointer they issued
// generic loads, which count in the LDS wait counter too.  Timing did not
// change.)  in[u] tells the slots that exist and lie below V.
template <int NTHR, int NB>
__device__ inline void load_candidates(const SelShared& s, const float* row, int V, int gs, int lg,
                                       int total, int f0, float4 (&v)[NB], int (&e)[NB],
                                       bool (&in)[NB]) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) f32x4v gf32x4;
  const int per = gs >> 2;
  int grp[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int fi = f0 + u * NTHR;
    grp[u] = int(s.act[(fi < total ? fi : total - 1) >> lg]);
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int fi = f0 + u * NTHR;
    const int fc = fi < total ? fi : total - 1;
    e[u] = grp[u] * gs + (fc & (per - 1)) * 4;
    in[u] = fi < total && e[u] < V;
    const f32x4v x = *(gf32x4*)(row + min(e[u], V - 4));  // V is a multiple of 8
    v[u] = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// Visit every element of the candidate groups, kBatch float4 loads in flight
// per thread.  f(in, key, e, bits) is called by all lanes of a wave the same
// number of times (out-of-range slots have in == false).
template <int NTHR, bool MIRROR, typename F>
__device__ inline void for_candidates(const SelShared& s, const float* row, int V, int gs, int nact,
                                      int tid, bool fold, F&& f) {
  const int wave_first = tid & ~63;
  if (gs >= 4) {
    const int per = gs >> 2;  // float4 items per group (a power of two)
    const int lg = __ffs(per) - 1;
    const int total = nact * per;
    for (int w0 = wave_first; w0 < total; w0 += kBatch * NTHR) {
      float4 v[kBatch];
      int e[kBatch];
      bool in[kBatch];
      load_candidates<NTHR>(s, row, V, gs, lg, total, w0 + (tid & 63), v, e, in);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t bx = rank_bits<MIRROR>(v[u].x, fold), by = rank_bits<MIRROR>(v[u].y, fold);
        const uint32_t bz = rank_bits<MIRROR>(v[u].z, fold), bw = rank_bits<MIRROR>(v[u].w, fold);
        f(in[u], float_key(__uint_as_float(bx)), e[u], bx);
        f(in[u], float_key(__uint_as_float(by)), e[u] + 1, by);
        f(in[u], float_key(__uint_as_float(bz)), e[u] + 2, bz);
        f(in[u], float_key(__uint_as_float(bw)), e[u] + 3, bw);
      }
    }
  } else {
    const int total = nact * gs;
    for (int w0 = wave_first; w0 < total; w0 += NTHR) {
      const int fi = w0 + (tid & 63);
      const int fc = fi < total ? fi : total - 1;
      const int e = int(s.act[fc / gs]) * gs + fc % gs;
      const bool in = fi < total && e < V;
      const float x = *(const __attribute__((address_space(1))) float*)(row + min(e, V - 1));
      const uint32_t bx = rank_bits<MIRROR>(in ? x : 0.0f, fold);
      f(in, float_key(__uint_as_float(bx)), e, bx);
    }
  }
}

// Step b: append every element with key >= t0 to the LDS list.  Each thread
// issues kScanBatch float4 loads at once and checks them together (a bit
// mask).  With 1024 threads, five per thread cover up to 320 candidate groups
// of 64 in one pass (k = 256 rows of GPT-OSS hold about 265): the scan then
// took 4.6-5.1 us against 5.1-5.8 us with four (two passes) and 6.1-6.5 us
// with eight (one pass, but every thread checks 32 mostly empty slots); 512
// threads take two passes.  The wave
// prefix-sums the counts with shuffles, and one LDS atomic per wave and batch
// reserves the slots (none when the wave found nothing, the common case);
// positions past kCap are counted but not stored.  Same elements, keys and
// bits as for_candidates.
template <int NTHR, bool MIRROR>
__device__ inline void scan_candidates(SelShared& s, const float* row, int V, int gs, int nact,
                                       int tid, bool fold, uint32_t t0) {
  const int lane = tid & 63;
  if (gs < 4) {
    for_candidates<NTHR, MIRROR>(s, row, V, gs, nact, tid, fold,
                           [&](bool in, uint32_t key, int e, uint32_t bits) {
                             wave_append(s, in && key >= t0, key, e, bits, lane);
                           });
    return;
  }
  const int wave_first = tid & ~63;
  const int per = gs >> 2;  // float4 items per group (a power of two)
  const int lg = __ffs(per) - 1;
  const int total = nact * per;
  for (int w0 = wave_first; w0 < total; w0 += kScanBatch * NTHR) {
    float4 v[kScanBatch];
    int e[kScanBatch];
    bool in[kScanBatch];
    load_candidates<NTHR>(s, row, V, gs, lg, total, w0 + lane, v, e, in);
    uint32_t bits[kScanBatch * 4], mask = 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      bits[4 * u] = rank_bits<MIRROR>(v[u].x, fold);
      bits[4 * u + 1] = rank_bits<MIRROR>(v[u].y, fold);
      bits[4 * u + 2] = rank_bits<MIRROR>(v[u].z, fold);
      bits[4 * u + 3] = rank_bits<MIRROR>(v[u].w, fold);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (in[u] && float_key(__uint_as_float(bits[4 * u + c])) >= t0) mask |= 1u << (4 * u + c);
    }
    if (__ballot(mask != 0) == 0) continue;  // nothing in the whole wave
    const uint32_t cnt = __popc(mask);  // kScanBatch * 4 <= 32 bits
    const uint32_t incl = wave_incl_sum_u32(cnt);
    const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&s.cnt, wtot);
    base = __builtin_amdgcn_readlane(base, 0);
    uint32_t pos = base + incl - cnt;
#pragma unroll
    for (int j = 0; j < kScanBatch * 4; ++j) {
      if (mask & (1u << j)) {
        if (pos < uint32_t(kCap)) {
          s.c[pos] = composite(float_key(__uint_as_float(bits[j])), e[j >> 2] + (j & 3));
          s.cb[pos] = bits[j];
        }
        ++pos;
      }
    }
  }
}

// The top-k of row row_id (steps a-f), run by all NTHR threads of the
// workgroup (tid: the thread's index in it) with s in its LDS.
// sample(s, prm, lane) returns the row's token on wave 0 (only called with
// params).
template <int NTHR, bool MIRROR, typename Sample>
__device__ inline void select_row(SelShared& s, int tid, int row_id, const float* __restrict__ logits, int V,
                                  int gs, int groups, int k, const uint32_t* __restrict__ gkey,
                                  int fold, float* __restrict__ vals, int32_t* __restrict__ idx,
                                  uint32_t* __restrict__ taps, const float* __restrict__ params,
                                  int ncols, int32_t* __restrict__ tokens, Sample&& sample) {
  static_assert(NTHR >= 256 && NTHR % 64 == 0 && kMaxGroups % NTHR == 0 && kCap % NTHR == 0,
                "select workgroup");
  constexpr int kGPer = kMaxGroups / NTHR;  // group keys per thread in registers
  constexpr int kPerThread = kCap / NTHR;   // candidates per thread in registers
  const int lane = tid & 63;
  const float* row = logits + size_t(row_id) * V;
  uint32_t above, equal;

  RowParams prm{0.f, 0.f, 0.f, 0.f};
  if (params != nullptr && tid < 64) prm = load_params(params, ncols, row_id);

  // a. t0: a lower bound of the k-th largest group maximum from one histogram
  // of the group maxima over [lo, hi] in power-of-two bins: the bin where the
  // count from the top first reaches k starts at t0, so at least k group
  // maxima (hence k elements) are >= t0.
  // every slot is loaded (past the row's groups from its last group) before
  // any is used: a load inside the bounds branch with its use folded in
  // waited for each key in turn
  uint32_t gk[kGPer];
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int j = 0; j < kGPer; ++j) {
    const int g = tid + j * NTHR;
    gk[j] = gkey[size_t(row_id) * groups + (g < groups ? g : groups - 1)];
  }
#pragma unroll
  for (int j = 0; j < kGPer; ++j) {
    if (tid + j * NTHR < groups) {
      if constexpr (MIRROR) gk[j] = mirror_key(gk[j]);
      lo = min(lo, gk[j]);
      hi = max(hi, gk[j]);
    } else {
      gk[j] = 0u;
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (tid < 256) s.hist[tid] = 0;
  if (tid == 0) {
    s.cnt = s.nact = 0;
    s.bc[0] = 0xFFFFFFFFu;
    s.bc[1] = 0u;
  }
  __syncthreads();
  if (lane == 0) {
    atomicMin(&s.bc[0], lo);
    atomicMax(&s.bc[1], hi);
  }
  __syncthreads();
  lo = s.bc[0];
  hi = s.bc[1];
  const uint32_t span = hi - lo;
  const int bshift = span < 256u ? 0 : 32 - __clz(int(span >> 8));  // (span >> bshift) < 256
#pragma unroll
  for (int j = 0; j < kGPer; ++j)
    if (tid + j * NTHR < groups) atomicAdd(&s.hist[(gk[j] - lo) >> bshift], 1u);
  __syncthreads();
  if (tid < 64) {  // wave 0: bins in descending order, lane l holds 255-4l .. 252-4l
    uint32_t c[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = s.hist[255 - 4 * tid - j];
      loc += c[j];
    }
    const uint32_t incl = wave_incl_sum_u32(loc);
    uint32_t run = incl - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run < uint32_t(k) && run + c[j] >= uint32_t(k)) s.bc[2] = 255 - 4 * tid - j;
      run += c[j];
    }
  }
  __syncthreads();
  const uint32_t t0 = lo + (s.bc[2] << bshift);

  // list the candidate groups
#pragma unroll
  for (int j = 0; j < kGPer; ++j) {
    const bool a = tid + j * NTHR < groups && gk[j] >= t0;
    const uint64_t m = __ballot(a);
    if (m) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s.nact, (uint32_t)__popcll(m));
      base = __builtin_amdgcn_readlane(base, 0);
      if (a) s.act[base + __popcll(m & ((1ull << lane) - 1ull))] = uint32_t(tid + j * NTHR);
    }
  }
  __syncthreads();
  const int nact = int(s.nact);

  // b. every element >= t0
  scan_candidates<NTHR, MIRROR>(s, row, V, gs, nact, tid, fold != 0, t0);
  __syncthreads();
  uint32_t n = s.cnt;
  if (taps != nullptr && tid == 0) {
    uint32_t* tp = taps + size_t(row_id) * 4;
    tp[0] = t0;
    tp[1] = uint32_t(nact);
    tp[2] = n;
    tp[3] = n > uint32_t(kCap) ? 1u : 0u;
  }

  // e. too many: find the cut by radix passes over the candidate groups
  if (n > uint32_t(kCap)) {
    auto visit_all = [&](auto&& f) {
      for_candidates<NTHR, MIRROR>(s, row, V, gs, nact, tid, fold != 0, [&](bool in, uint32_t key, int, uint32_t) {
        if (in && key >= t0) f(key);
      });
    };
    const uint32_t vstar = radix_kth(s, tid, uint32_t(k), visit_all, &above, &equal);
    int ecut = V;  // keep key > v*, and key == v* with index <= ecut
    if (above + equal > uint32_t(kCap)) {
      uint32_t a2, e2;
      const uint32_t nk = radix_kth(s, tid, uint32_t(k) - above, [&](auto&& f) {
        for_candidates<NTHR, MIRROR>(s, row, V, gs, nact, tid, fold != 0, [&](bool in, uint32_t key, int e, uint32_t) {
          if (in && key == vstar) f(~uint32_t(e));
        });
      }, &a2, &e2);
      ecut = int(~nk);
    }
    __syncthreads();
    if (tid == 0) s.cnt = 0;
    __syncthreads();
    for_candidates<NTHR, MIRROR>(s, row, V, gs, nact, tid, fold != 0, [&](bool in, uint32_t key, int e, uint32_t bits) {
      wave_append(s, in && (key > vstar || (key == vstar && e <= ecut)), key, e, bits, lane);
    });
    __syncthreads();
    n = s.cnt;
  }

  // c. cut long lists to the k best (value, then lowest index among ties)
  if (n > uint32_t(2 * k)) {
    uint64_t mine[kPerThread];
    uint32_t mbits[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = tid + j * NTHR;
      mine[j] = i < int(n) ? s.c[i] : 0ull;
      mbits[j] = i < int(n) ? s.cb[i] : 0u;
    }
    const uint32_t vstar = radix_kth(s, tid, uint32_t(k), [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (tid + j * NTHR < int(n)) f(uint32_t(mine[j] >> 32));
    }, &above, &equal);
    uint32_t lowcut = 0;  // smallest ~index kept among keys == v*
    if (above + equal > uint32_t(2 * k)) {
      uint32_t a2, e2;
      lowcut = radix_kth(s, tid, uint32_t(k) - above, [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
          if (tid + j * NTHR < int(n) && uint32_t(mine[j] >> 32) == vstar) f(uint32_t(mine[j]));
      }, &a2, &e2);
    }
    if (tid == 0) s.cnt = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint32_t key = uint32_t(mine[j] >> 32);
      const bool keep = tid + j * NTHR < int(n) &&
                        (key > vstar || (key == vstar && uint32_t(mine[j]) >= lowcut));
      const uint64_t m = __ballot(keep);
      if (m) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&s.cnt, (uint32_t)__popcll(m));
        base = __builtin_amdgcn_readlane(base, 0);
        if (keep) {
          const uint32_t pos = base + __popcll(m & ((1ull << lane) - 1ull));
          s.c[pos] = mine[j];
          s.cb[pos] = mbits[j];
        }
      }
    }
    __syncthreads();
    n = s.cnt;
  }

  // d. exact ranks by a counting sort on the value keys: the survivors are
  // binned by (khi - key) >> bsh into 256 bins (bin 0 holds the largest
  // keys), the bins are laid out in order by an exclusive prefix sum, and a
  // survivor's rank is its bin's start plus the number of entries of its own
  // bin with a larger composite key (larger value, then lower index).  A bin
  // holds about one survivor on typical rows; equal keys share a bin.
  {
    uint32_t klo = 0xFFFFFFFFu, khi = 0;
    for (int i = tid; i < int(n); i += NTHR) {
      const uint32_t v = uint32_t(s.c[i] >> 32);
      klo = min(klo, v);
      khi = max(khi, v);
    }
    klo = wave_min_u32(klo);
    khi = wave_max_u32(khi);
    if (tid < 256) s.hist[tid] = 0;
    if (tid == 0) {
      s.bc[0] = 0xFFFFFFFFu;
      s.bc[1] = 0u;
    }
    __syncthreads();
    if (lane == 0) {
      atomicMin(&s.bc[0], klo);
      atomicMax(&s.bc[1], khi);
    }
    __syncthreads();
    klo = s.bc[0];
    khi = s.bc[1];
    const uint32_t kspan = khi - klo;
    const int bsh = kspan < 256u ? 0 : 32 - __clz(int(kspan >> 8));  // (kspan >> bsh) < 256
    for (int i = tid; i < int(n); i += NTHR)
      atomicAdd(&s.hist[(khi - uint32_t(s.c[i] >> 32)) >> bsh], 1u);
    __syncthreads();
    if (tid < 64) {  // exclusive prefix over the bins, 4 per lane; hist becomes the fill cursor
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s.hist[4 * tid + j];
        loc += c[j];
      }
      const uint32_t incl = wave_incl_sum_u32(loc);
      uint32_t run = incl - loc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s.bstart[4 * tid + j] = run;
        s.hist[4 * tid + j] = run;
        run += c[j];
      }
      if (tid == 63) s.bstart[256] = run;
    }
    __syncthreads();
    // the candidate-group list is no longer needed: it holds the sorted copy
    uint64_t* sc = reinterpret_cast<uint64_t*>(s.act);  // n <= 2k composites
    uint32_t* sbits = s.act + 2 * (2 * TAIL_K_MAX);     // and their value bits
    for (int i = tid; i < int(n); i += NTHR) {
      const uint64_t ci = s.c[i];
      const uint32_t pos = atomicAdd(&s.hist[(khi - uint32_t(ci >> 32)) >> bsh], 1u);
      sc[pos] = ci;
      sbits[pos] = s.cb[i];
    }
    __syncthreads();
    for (int i = tid; i < int(n); i += NTHR) {
      const uint64_t ci = sc[i];
      const int bin = int((khi - uint32_t(ci >> 32)) >> bsh);
      const int j0 = int(s.bstart[bin]), j1 = int(s.bstart[bin + 1]);
      uint32_t rank = uint32_t(j0);
      for (int j = j0; j < j1; ++j) rank += sc[j] > ci;
      if (rank < uint32_t(k)) {
        s.top_v[rank] = __uint_as_float(sbits[i]);
        s.top_i[rank] = int(~uint32_t(ci));
      }
    }
  }
  __syncthreads();

  // f. the row's sampler (wave 0) while the other waves write the list out
  if (params != nullptr && tid < 64) {
    const int32_t t = sample(s, prm, lane);
    if (lane == 0) tokens[row_id] = t;
  }
  for (int i = params != nullptr ? tid - 64 : tid; i < k; i += NTHR) {
    if (i >= 0) {
      vals[size_t(row_id) * k + i] = s.top_v[i];
      idx[size_t(row_id) * k + i] = s.top_i[i];
    }
  }
}

}  // namespace
}  // namespace tail
