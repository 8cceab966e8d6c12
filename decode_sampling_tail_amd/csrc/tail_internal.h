// Internal declarations shared by the host API and the kernel translation
// units of the decode-tail library (gfx950 only).  Not part of the ABI.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace tail {

// ------------------------------------------------------------ small helpers
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Unpadded lane u -> physical hidden lane h, when every group of s lanes ends
// with one pad lane (s = 0: no padding).
__host__ __device__ inline int phys_lane(int u, int s) { return s ? u + u / (s - 1) : u; }

// Exact unsigned division by a run-time constant d >= 1 for n < 2^31
// (multiply-high and shift, Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, section 4):
// q = (mulhi(n, mul) + n) >> shift with shift = ceil(log2 d) and
// mul = floor(2^32 * (2^shift - d) / d) + 1.
struct FastDiv {
  uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t shift = 0;
  while ((uint64_t(1) << shift) < d) ++shift;
  uint64_t mul = ((uint64_t(1) << 32) * ((uint64_t(1) << shift) - d)) / d + 1;
  return FastDiv{uint32_t(mul), shift};
}
__host__ __device__ inline uint32_t fastdiv(uint32_t n, FastDiv f) {
#ifdef __HIP_DEVICE_COMPILE__
  const uint32_t hi = __umulhi(n, f.mul);
#else
  const uint32_t hi = uint32_t((uint64_t(n) * f.mul) >> 32);
#endif
  return (hi + n) >> f.shift;
}

// Streamed weight loads: each weight byte is read once per call and never
// reused, so non-temporal 16-byte loads keep it from displacing useful lines
// (and measurably raise the achieved bandwidth on gfx950).
typedef unsigned tail_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_stream(const uint16_t* p) {
  const tail_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const tail_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// float32 -> bfloat16, round to nearest, ties to even (the bf16 is the upper
// 16 bits of the result; adding 0x7FFF plus the lowest kept bit carries
// exactly when the dropped half is above, or at and odd, the midpoint).  A NaN
// stays a quiet NaN; values past the largest bf16 become infinities.
__device__ inline uint32_t bf16_rne_bits(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u | 0x00400000u) >> 16;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_round(float f) {
  return __uint_as_float(bf16_rne_bits(__float_as_uint(f)) << 16);
}

// Once-per-device host initialization: init(dev) runs the first time a
// device (the current one) needs it, thread-safely; later calls return its
// cached value.  T must be default-constructible.
constexpr int kMaxDevices = 64;
template <typename T, typename F>
T per_device(std::once_flag (&once)[kMaxDevices], T (&value)[kMaxDevices], F&& init) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return init(dev);
  std::call_once(once[dev], [&] { value[dev] = init(dev); });
  return value[dev];
}

// A hidden element's raw bits (the fp32 pattern, or the 16-bit pattern
// zero-extended) from element i of a row-major hidden array of dtype DT
// (0 fp32, 1 fp16, 2 bf16), and their exact widening to fp32.
template <int DT>
__device__ inline uint32_t load_bits(const void* p, size_t i) {
  if constexpr (DT == 0) return __float_as_uint(static_cast<const float*>(p)[i]);
  else return static_cast<const uint16_t*>(p)[i];
}
template <int DT>
__device__ inline float widen_bits(uint32_t b) {
  if constexpr (DT == 0) return __uint_as_float(b);
  else if constexpr (DT == 1) return __half2float(__ushort_as_half(uint16_t(b)));
  else return __uint_as_float(b << 16);
}

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
constexpr int kFusedGroup = 64;  // group size the lm_head epilogues emit maxima for
struct TopkGeom {
  int gs;      // group size (columns)
  int groups;  // ceil(V / gs)
};
inline bool topk_geometry(int V, int k, TopkGeom* g) {
  int gs = kFusedGroup;
  while (gs > 1 && (V + gs - 1) / gs < k) gs >>= 1;
  while ((V + gs - 1) / gs > kMaxGroups) gs <<= 1;
  g->gs = gs;
  g->groups = (V + gs - 1) / gs;
  return g->groups >= k && g->groups <= kMaxGroups;
}

// Launchers (each defined next to its kernels).  They assume validated
// arguments and return the launch status.
// page: round every output to bf16 (the GEMM input of the page-precision mode)
hipError_t launch_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H, int H_u,
                          int pad_s, float eps, bool deferred, bool page, float* y, float* r,
                          hipStream_t st);

// Weight-streaming lm_head over K contraction lanes (pad lanes skipped when
// pad_s > 0).  gkey (may be NULL): per row, the largest order-preserving key
// of each group of kFusedGroup columns, [gbs, ceil(V / kFusedGroup)].  page:
// the activations are rounded to bf16 before the contraction.  part_ws:
// gemv_part_bytes(gbs, K, V) bytes (256-byte aligned) for the split-K
// partials when the vocabulary is too narrow to fill the chip.
int gemv_ksplit(int V, int K);
size_t gemv_part_bytes(int gbs, int K, int V);
hipError_t launch_lm_head_gemv(const float* y, int ldy, const uint16_t* w, const float* row_scale,
                               int gbs, int K, int pad_s, int V, bool page, float* logits,
                               uint32_t* gkey, void* part_ws, hipStream_t st);

// The same with the RMSNorm fused into the prologue (hidden rows in their
// storage dtype); r_out (may be NULL) receives the per-row rms scale.
bool gemv_fusable(int gbs, int K);
hipError_t launch_norm_gemv(const void* hidden, int dtype, const float* gamma, int gbs, int H,
                            int H_u, int K, int pad_s, float eps, bool deferred, bool page,
                            const uint16_t* w, int V, float* logits, float* r_out, uint32_t* gkey,
                            void* part_ws, hipStream_t st);

// Batches above this size run the lm_head on the matrix cores (at 4 rows
// the matrix-core step measured 188 us against 194 us for weight streaming,
// at 3 rows 186 us for weight streaming).
constexpr int kGemvMaxBatch = 3;
constexpr int kKStep = 64;  // K granularity of the matrix-core path
int mfma_terms(int gbs, bool page);  // bf16 terms per activation (1 in the page-precision mode)

// Batches of kRowsMinBatch rows and more run the lm_head on the 32x32x16
// large-batch kernel (lm_head_rows.hip), and so do batches from
// kRowsMidBatch rows over a vocabulary whose 512-column tiles fill the chip
// (where the 16x16x32 kernel would not split K); they read their
// activations in fragment layout 1, the others in layout 0
// (lm_head_mfma.hip), which splits K for narrow vocabularies.
constexpr int kRowsMinBatch = 129;
constexpr int kRowsMidBatch = 65;
int mfma_ksplit(int V, int Kp);
inline int mfma_layout(int gbs, int V, int Kp) {
  return (gbs >= kRowsMinBatch || (gbs >= kRowsMidBatch && mfma_ksplit(V, Kp) == 1)) ? 1 : 0;
}
inline int mfma_row_tile(int layout) { return layout ? 32 : 16; }

// The top-k and sampler of every row, run by the large-batch lm_head after a
// grid barrier (lm_head_rows.hip) instead of by a launch of their own.
// Group size gs must be kFusedGroup (the epilogue's key groups), without the
// NaN fold; mirror ranking follows the one-term (page-precision) kernels.
// The producer (launch_split) stores it in device memory, where that kernel
// reads it after its tiles (as kernel arguments it would hold registers
// through the whole contraction), and clears the counters.
struct FusedSelect {
  float* vals;          // [gbs, k]
  int32_t* idx;         // [gbs, k]
  const float* params;  // [gbs, ncols] or NULL (no sampling)
  int ncols;
  int32_t* tokens;      // [gbs] (with params)
  int k, gs, groups;
  uint32_t* sync;       // 2 words per launch of 128 or 256 rows (fused_sync_words)
  int nsync;            // fused_sync_words(gbs)
  int spin;             // polls of the arrival counter before a workgroup leaves the rows to others
};
inline int fused_sync_words(int gbs) { return 2 * ((gbs + 127) / 128); }
// whether the large-batch kernel that takes gbs rows of nt terms has the
// select phase (not the one-term kernel above 128 rows)
inline bool rows_fuse_select(int nt, int gbs) { return nt == 2 || gbs <= 128; }

// Split (and, with norm, RMS-normalize) activations for the matrix-core path:
// act holds nt * rows_pad * Kp bf16 bits over the K contraction lanes as 1 KB
// MFMA operand fragments ordered (term, row tile, K block) in the given layout
// (0: 16-row tiles and 32-lane K blocks for v_mfma_f32_16x16x32_bf16, 1:
// 32-row tiles and 16-lane K blocks for v_mfma_f32_32x32x16_bf16); r [gbs]
// (norm only, may be NULL); gz [gbs, groups] (may be NULL) is cleared; fs_out
// (may be NULL, device memory): receives fs, and fs.sync [fs.nsync] is cleared.
hipError_t launch_split(const void* src, int dtype, bool norm, const float* gamma, int gbs, int H,
                        int H_u, int K, int pad_s, float eps, bool deferred, int nt, int layout,
                        int rows_pad, int Kp, uint16_t* act, float* r, uint32_t* gz, int groups,
                        const FusedSelect& fs, FusedSelect* fs_out, hipStream_t st);

// Matrix-core lm_head; part_ws: mfma_part_bytes(gbs, Kp, V) bytes (256-byte
// aligned) for the split-K partials of a narrow vocabulary.
size_t mfma_part_bytes(int gbs, int Kp, int V);
hipError_t launch_lm_head_mfma(const uint16_t* act, int nt, int rows_pad, int Kp, const uint16_t* w,
                               int V, int H_u, int pad_s, const float* row_scale, int gbs,
                               float* logits, uint32_t* gkey, void* part_ws, hipStream_t st);

// The large-batch lm_head (layout 1 batches, see mfma_layout): act in layout 1 with
// rows_pad a multiple of 32; gkey (may be NULL) must hold zeros where the
// producer cleared it; fs (may be NULL; device memory the producer wrote):
// also the rows' top-k and sampler.
hipError_t launch_lm_head_rows(const uint16_t* act, int nt, int rows_pad, int Kp, const uint16_t* w,
                               int V, int K, int pad_s, const float* row_scale, int gbs,
                               float* logits, uint32_t* gkey, const FusedSelect* fs,
                               hipStream_t st);

// Split-K finish shared by the lm_head paths: logits[b, v] = row_scale[b] (or
// 1) * sum over kc in order of part[kc][b][v]; gkey (may be NULL) as above.
hipError_t launch_part_reduce(const float* part, int kc_n, int gbs, int V, const float* row_scale,
                              float* logits, uint32_t* gkey, hipStream_t st);

// fold: NaN counts as -inf (the page's stage-1 NaN fold)
hipError_t launch_group_max(const float* logits, int gbs, int V, const TopkGeom& geom, bool fold,
                            uint32_t* gkey, hipStream_t st);

// params NULL: no sampling (ncols and tokens unused).  mirror: rank the bf16
// rounding of every logit and return the rounded values (gkey may hold the
// unrounded group maxima: rounding is monotone, so the rounded maximum is the
// maximum of the rounded values).  fold: NaN ranks and is returned as -inf
// (gkey must then be computed with the same fold).  taps (may be NULL): 4 u32
// stage-1 diagnostics per row.
hipError_t launch_select(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                         const uint32_t* gkey, bool mirror, bool fold, float* vals, int32_t* idx,
                         uint32_t* taps, const float* params, int ncols, int32_t* tokens,
                         hipStream_t st);

hipError_t launch_topk(const float* logits, int gbs, int V, int k, const TopkGeom& geom,
                       uint32_t* gkey_ws, bool mirror, bool fold, float* vals, int32_t* idx,
                       uint32_t* taps, hipStream_t st);

hipError_t launch_sample(const float* vals, const int32_t* idx, int gbs, int k,
                         const float* params, int ncols, int32_t* tokens, hipStream_t st);

}  // namespace tail
