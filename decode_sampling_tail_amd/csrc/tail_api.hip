// Host side of the decode-tail C ABI: argument validation (pure host logic,
// run before any HIP call), workspace layout and kernel dispatch.  The entry
// points and their contracts are declared in include/tail.h.
#include "../../include/tail.h"
#include "tail_internal.h"

#include <math.h>
#include <stdlib.h>

#define TAIL_API extern "C" __attribute__((visibility("default")))

namespace {

using tail::align256;

// flags each entry accepts (any other bit is TAIL_ERR_INVALID_ARG)
constexpr unsigned kNormFlags =
    TAIL_EMIT_LOGITS | TAIL_ZERO_PAD | TAIL_DEFERRED_RMS | TAIL_PAGE_PRECISION;
constexpr unsigned kAllFlags = kNormFlags | TAIL_NAN_FOLD;
constexpr unsigned kTopkFlags = TAIL_PAGE_PRECISION | TAIL_NAN_FOLD;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_bytes(int dtype) { return dtype == TAIL_F32 ? 4 : 2; }

// Stride s of the interleaved pad lanes (0 when there are none to skip), or
// -1 when the padding geometry is invalid.
int pad_stride(int H, int H_u, unsigned flags) {
  if (!(flags & TAIL_ZERO_PAD) || H == H_u) return 0;
  int npad = H - H_u;
  if (H % npad != 0) return -1;
  int s = H / npad;
  return s >= 2 ? s : -1;
}

int check_shape(int gbs, int H, int H_u) {
  if (gbs < 1 || H < 1 || H_u < 1 || H_u > H) return TAIL_ERR_INVALID_ARG;
  if (gbs > TAIL_GBS_MAX || H > TAIL_H_MAX) return TAIL_ERR_UNSUPPORTED;
  return TAIL_OK;
}

int check_vocab(int V) {
  if (V < 1) return TAIL_ERR_INVALID_ARG;
  if (V % 8 != 0) return TAIL_ERR_UNSUPPORTED;  // 16-byte weight rows
  return TAIL_OK;
}

int check_k(int V, int k) {
  if (k < 1 || k > V) return TAIL_ERR_INVALID_ARG;
  if (k > TAIL_K_MAX) return TAIL_ERR_UNSUPPORTED;
  tail::TopkGeom g;
  if (!tail::topk_geometry(V, k, &g)) return TAIL_ERR_UNSUPPORTED;
  return TAIL_OK;
}

// Geometry of the matrix-core path's split activations: [nt][rows_pad][Kp] bf16
// (nt = 1 in the page-precision mode).
struct SplitGeom {
  int K, Kp, rows_pad, nt, layout;
  size_t bytes;
};
SplitGeom split_geom(int gbs, int H, int H_u, int pad_s, int V, unsigned flags) {
  SplitGeom g;
  g.K = pad_s ? H_u : H;
  g.Kp = (g.K + tail::kKStep - 1) / tail::kKStep * tail::kKStep;
  g.layout = tail::mfma_layout(gbs, V, g.Kp);
  const int rt = tail::mfma_row_tile(g.layout);
  g.rows_pad = (gbs + rt - 1) / rt * rt;
  g.nt = tail::mfma_terms(gbs, flags & TAIL_PAGE_PRECISION);
  g.bytes = gbs > tail::kGemvMaxBatch ? size_t(g.nt) * g.rows_pad * g.Kp * 2 : 0;
  return g;
}

struct FwdLayout {
  size_t y, r, act, part, logits, gkey, sync, total;
};

// split-K partials of the lm_head path this batch takes (narrow vocabularies)
size_t gemv_part(int gbs, int H, int H_u, int pad_s, int V) {
  const int K = pad_s ? H_u : H;
  if (gbs <= tail::kGemvMaxBatch) return tail::gemv_part_bytes(gbs, K, V);
  const int Kp = (K + tail::kKStep - 1) / tail::kKStep * tail::kKStep;
  if (tail::mfma_layout(gbs, V, Kp)) return 0;  // the large-batch kernel never splits K
  return tail::mfma_part_bytes(gbs, Kp, V);
}

FwdLayout forward_layout(int gbs, int H, int H_u, int pad_s, int V, int k, unsigned flags) {
  tail::TopkGeom g;
  tail::topk_geometry(V, k, &g);
  FwdLayout L;
  size_t off = 0;
  L.y = off;
  off = align256(off + size_t(gbs) * H * 4);
  L.r = off;
  off = align256(off + size_t(gbs) * 4);
  L.act = off;
  off = align256(off + split_geom(gbs, H, H_u, pad_s, V, flags).bytes);
  L.part = off;
  off = align256(off + gemv_part(gbs, H, H_u, pad_s, V));
  L.logits = off;
  if (!(flags & TAIL_EMIT_LOGITS)) off = align256(off + size_t(gbs) * V * 4);
  L.gkey = off;
  off = align256(off + size_t(gbs) * g.groups * 4);
  L.sync = off;  // the fused select's arguments, then its counters
  off = align256(off + sizeof(tail::FusedSelect) + size_t(tail::fused_sync_words(gbs)) * 4);
  L.total = off;
  return L;
}

size_t topk_ws_bytes(int gbs, int V, int k) {
  tail::TopkGeom g;
  tail::topk_geometry(V, k, &g);
  return align256(size_t(gbs) * g.groups * 4);
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return TAIL_OK;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < need) return TAIL_ERR_WORKSPACE;
  return TAIL_OK;
}

// RMSNorm + lm_head: fused weight-streaming kernel, or RMSNorm then the
// weight-streaming kernel, or the bf16-split producer then the matrix cores.
// y (gbs*H floats) and act (split_geom bytes) are workspace.  fs (may be
// NULL, large-batch kernel only): that kernel also runs the top-k and sampler,
// with the arguments fs stored by the producer at fs_dev (workspace).
hipError_t norm_lm_head(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t,
                        int gbs, int H, int H_u, int V, float eps, int ps, unsigned flags, float* y,
                        float* r, uint16_t* act, void* part, float* logits, uint32_t* gkey,
                        const tail::FusedSelect* fs, tail::FusedSelect* fs_dev, hipStream_t st) {
  const bool deferred = flags & TAIL_DEFERRED_RMS, page = flags & TAIL_PAGE_PRECISION;
  const SplitGeom sg = split_geom(gbs, H, H_u, ps, V, flags);
  if (tail::gemv_fusable(gbs, sg.K))
    return tail::launch_norm_gemv(hidden, dtype, gamma, gbs, H, H_u, sg.K, ps, eps, deferred, page,
                                  w_t, V, logits, r, gkey, part, st);
  hipError_t e;
  if (gbs <= tail::kGemvMaxBatch) {
    e = tail::launch_rmsnorm(hidden, dtype, gamma, gbs, H, H_u, ps, eps, deferred, page, y, r, st);
    if (e == hipSuccess)  // y is already rounded in the page mode
      e = tail::launch_lm_head_gemv(y, H, w_t, deferred ? r : nullptr, gbs, sg.K, ps, V, false,
                                    logits, gkey, part, st);
    return e;
  }
  const int layout = sg.layout;
  // the large-batch kernel combines straddling key groups into cleared entries
  uint32_t* gz = layout ? gkey : nullptr;
  const bool fused = layout && fs && fs_dev;
  e = tail::launch_split(hidden, dtype, true, gamma, gbs, H, H_u, sg.K, ps, eps, deferred, sg.nt,
                         layout, sg.rows_pad, sg.Kp, act, r, gz,
                         (V + tail::kFusedGroup - 1) / tail::kFusedGroup,
                         fused ? *fs : tail::FusedSelect{}, fused ? fs_dev : nullptr, st);
  if (e != hipSuccess) return e;
  if (layout)
    return tail::launch_lm_head_rows(act, sg.nt, sg.rows_pad, sg.Kp, w_t, V, sg.K, ps,
                                     deferred ? r : nullptr, gbs, logits, gkey,
                                     fused ? fs_dev : nullptr, st);
  return tail::launch_lm_head_mfma(act, sg.nt, sg.rows_pad, sg.Kp, w_t, V, sg.K, ps,
                                   deferred ? r : nullptr, gbs, logits, gkey, part, st);
}

int hip_status(hipError_t e) { return e == hipSuccess ? TAIL_OK : TAIL_ERR_HIP; }

}  // namespace

TAIL_API const char* tail_status_string(int status) {
  switch (status) {
    case TAIL_OK: return "ok";
    case TAIL_ERR_INVALID_ARG: return "invalid argument";
    case TAIL_ERR_UNSUPPORTED: return "unsupported by this library";
    case TAIL_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TAIL_ERR_HIP: return "HIP launch error";
    case TAIL_ERR_SCRATCH_LIMIT:
      return "the call needs more than the library's static scratch (TAIL_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

TAIL_API size_t tail_workspace_size(int gbs, int H, int H_u, int V, int k, unsigned flags) {
  if (check_shape(gbs, H, H_u) || check_vocab(V) || check_k(V, k)) return 0;
  if (pad_stride(H, H_u, flags) < 0) return 0;
  const int ps = pad_stride(H, H_u, flags);
  size_t fwd = forward_layout(gbs, H, H_u, ps, V, k, flags).total;
  size_t tk = topk_ws_bytes(gbs, V, k);
  // tail_lm_head: the split-K partials, after the split activations on the
  // matrix-core path
  const size_t lm = align256(split_geom(gbs, H, H_u, ps, V, flags).bytes) +
                    align256(gemv_part(gbs, H, H_u, ps, V));
  size_t m = fwd > tk ? fwd : tk;
  return m > lm ? m : lm;
}

TAIL_API int tail_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H,
                          int H_u, float eps, unsigned flags, float* out_y, float* out_r,
                          void* stream) {
  if (int s = check_shape(gbs, H, H_u)) return s;
  if (dtype != TAIL_F32 && dtype != TAIL_F16 && dtype != TAIL_BF16) return TAIL_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return TAIL_ERR_INVALID_ARG;
  if (flags & ~kNormFlags) return TAIL_ERR_INVALID_ARG;
  int ps = pad_stride(H, H_u, flags);
  if (ps < 0) return TAIL_ERR_INVALID_ARG;
  bool deferred = flags & TAIL_DEFERRED_RMS;
  if (!hidden || !gamma || !out_y || (deferred && !out_r)) return TAIL_ERR_INVALID_ARG;
  if (!aligned(hidden, dtype_bytes(dtype)) || !aligned(gamma, 4) || !aligned(out_y, 4) ||
      (out_r && !aligned(out_r, 4)))
    return TAIL_ERR_INVALID_ARG;
  return hip_status(tail::launch_rmsnorm(hidden, dtype, gamma, gbs, H, H_u, ps, eps, deferred,
                                         flags & TAIL_PAGE_PRECISION, out_y, out_r,
                                         (hipStream_t)stream));
}

TAIL_API int tail_lm_head(const float* y, const uint16_t* w_t, const float* row_scale, int gbs,
                          int H, int H_u, int V, unsigned flags, float* logits, void* ws,
                          size_t ws_bytes, void* stream) {
  if (int s = check_shape(gbs, H, H_u)) return s;
  if (int s = check_vocab(V)) return s;
  if (flags & ~kNormFlags) return TAIL_ERR_INVALID_ARG;
  int ps = pad_stride(H, H_u, flags);
  if (ps < 0) return TAIL_ERR_INVALID_ARG;
  if (!y || !w_t || !logits) return TAIL_ERR_INVALID_ARG;
  if (!aligned(y, 4) || !aligned(w_t, 16) || !aligned(logits, 16) ||
      (row_scale && !aligned(row_scale, 4)))
    return TAIL_ERR_INVALID_ARG;
  const SplitGeom sg = split_geom(gbs, H, H_u, ps, V, flags);
  hipStream_t st = (hipStream_t)stream;
  if (gbs <= tail::kGemvMaxBatch) {
    if (int s = check_ws(ws, ws_bytes, gemv_part(gbs, H, H_u, ps, V))) return s;
    return hip_status(tail::launch_lm_head_gemv(y, H, w_t, row_scale, gbs, sg.K, ps, V,
                                                flags & TAIL_PAGE_PRECISION, logits, nullptr, ws,
                                                st));
  }
  // matrix-core path: the split activations, then the split-K partials
  if (int s = check_ws(ws, ws_bytes, align256(sg.bytes) + gemv_part(gbs, H, H_u, ps, V))) return s;
  uint16_t* act = (uint16_t*)ws;
  const int layout = sg.layout;
  hipError_t e = tail::launch_split(y, TAIL_F32, false, nullptr, gbs, H, H_u, sg.K, ps, 0.0f, false,
                                    sg.nt, layout, sg.rows_pad, sg.Kp, act, nullptr, nullptr, 0,
                                    tail::FusedSelect{}, nullptr, st);
  if (e == hipSuccess)
    e = layout ? tail::launch_lm_head_rows(act, sg.nt, sg.rows_pad, sg.Kp, w_t, V, sg.K, ps,
                                           row_scale, gbs, logits, nullptr, nullptr, st)
               : tail::launch_lm_head_mfma(act, sg.nt, sg.rows_pad, sg.Kp, w_t, V, sg.K, ps,
                                           row_scale, gbs, logits, nullptr,
                                           (char*)ws + align256(sg.bytes), st);
  return hip_status(e);
}

TAIL_API int tail_rmsnorm_lm_head(const void* hidden, int dtype, const float* gamma,
                                  const uint16_t* w_t, int gbs, int H, int H_u, int V, float eps,
                                  unsigned flags, float* logits, float* out_r, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (int s = check_shape(gbs, H, H_u)) return s;
  if (int s = check_vocab(V)) return s;
  if (dtype != TAIL_F32 && dtype != TAIL_F16 && dtype != TAIL_BF16) return TAIL_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return TAIL_ERR_INVALID_ARG;
  if (flags & ~kNormFlags) return TAIL_ERR_INVALID_ARG;
  const int ps = pad_stride(H, H_u, flags);
  if (ps < 0) return TAIL_ERR_INVALID_ARG;
  if (!hidden || !gamma || !w_t || !logits) return TAIL_ERR_INVALID_ARG;
  if (!aligned(hidden, dtype_bytes(dtype)) || !aligned(gamma, 4) || !aligned(w_t, 16) ||
      !aligned(logits, 16) || (out_r && !aligned(out_r, 4)))
    return TAIL_ERR_INVALID_ARG;
  // the same workspace layout as tail_forward (its y, r and act regions)
  const FwdLayout L = forward_layout(gbs, H, H_u, ps, V, 1, flags | TAIL_EMIT_LOGITS);
  if (int s = check_ws(ws, ws_bytes, L.gkey)) return s;
  char* base = (char*)ws;
  float* r = out_r ? out_r : (float*)(base + L.r);
  return hip_status(norm_lm_head(hidden, dtype, gamma, w_t, gbs, H, H_u, V, eps, ps, flags,
                                 (float*)(base + L.y), r, (uint16_t*)(base + L.act),
                                 base + L.part, logits, nullptr, nullptr, nullptr,
                                 (hipStream_t)stream));
}

namespace {
int topk_call(const float* logits, int gbs, int V, int k, unsigned flags, float* vals, int32_t* idx,
              uint32_t* taps, void* ws, size_t ws_bytes, void* stream) {
  if (flags & ~kTopkFlags) return TAIL_ERR_INVALID_ARG;
  if (gbs < 1) return TAIL_ERR_INVALID_ARG;
  if (gbs > TAIL_GBS_MAX) return TAIL_ERR_UNSUPPORTED;
  if (int s = check_vocab(V)) return s;
  if (int s = check_k(V, k)) return s;
  if (!logits || !vals || !idx) return TAIL_ERR_INVALID_ARG;
  if (!aligned(logits, 16) || !aligned(vals, 4) || !aligned(idx, 4) || (taps && !aligned(taps, 4)))
    return TAIL_ERR_INVALID_ARG;
  if (int s = check_ws(ws, ws_bytes, topk_ws_bytes(gbs, V, k))) return s;
  tail::TopkGeom g;
  tail::topk_geometry(V, k, &g);
  return hip_status(tail::launch_topk(logits, gbs, V, k, g, (uint32_t*)ws,
                                      flags & TAIL_PAGE_PRECISION, flags & TAIL_NAN_FOLD, vals, idx,
                                      taps, (hipStream_t)stream));
}
}  // namespace

TAIL_API int tail_topk(const float* logits, int gbs, int V, int k, float* vals, int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream) {
  return topk_call(logits, gbs, V, k, 0u, vals, idx, nullptr, ws, ws_bytes, stream);
}

TAIL_API int tail_topk_ex(const float* logits, int gbs, int V, int k, unsigned flags, float* vals,
                          int32_t* idx, uint32_t* taps, void* ws, size_t ws_bytes, void* stream) {
  return topk_call(logits, gbs, V, k, flags, vals, idx, taps, ws, ws_bytes, stream);
}

TAIL_API int tail_sample(const float* vals, const int32_t* idx, int gbs, int k,
                         const float* params, int ncols, int32_t* tokens, void* stream) {
  if (gbs < 1 || k < 1) return TAIL_ERR_INVALID_ARG;
  if (gbs > TAIL_GBS_MAX || k > TAIL_K_MAX) return TAIL_ERR_UNSUPPORTED;
  if (ncols != 3 && ncols != 4) return TAIL_ERR_INVALID_ARG;
  if (!vals || !idx || !params || !tokens) return TAIL_ERR_INVALID_ARG;
  if (!aligned(vals, 4) || !aligned(idx, 4) || !aligned(params, 4) || !aligned(tokens, 4))
    return TAIL_ERR_INVALID_ARG;
  return hip_status(
      tail::launch_sample(vals, idx, gbs, k, params, ncols, tokens, (hipStream_t)stream));
}

namespace {
// Argument checks of tail_forward (pure host logic); the workspace is checked
// by the caller.  ps receives the pad stride, L the workspace layout.
int check_forward(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t, int gbs,
                  int H, int H_u, int V, int k, float eps, unsigned flags, const float* params,
                  int ncols, float* logits, float* vals, int32_t* idx, int32_t* tokens, int* ps,
                  FwdLayout* L) {
  if (int s = check_shape(gbs, H, H_u)) return s;
  if (int s = check_vocab(V)) return s;
  if (int s = check_k(V, k)) return s;
  if (dtype != TAIL_F32 && dtype != TAIL_F16 && dtype != TAIL_BF16) return TAIL_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return TAIL_ERR_INVALID_ARG;
  if (flags & ~kAllFlags) return TAIL_ERR_INVALID_ARG;
  *ps = pad_stride(H, H_u, flags);
  if (*ps < 0) return TAIL_ERR_INVALID_ARG;
  const bool emit = flags & TAIL_EMIT_LOGITS;
  if (!hidden || !gamma || !w_t || !vals || !idx) return TAIL_ERR_INVALID_ARG;
  if (emit && !logits) return TAIL_ERR_INVALID_ARG;
  if (params && (ncols != 3 && ncols != 4)) return TAIL_ERR_INVALID_ARG;
  if (params && !tokens) return TAIL_ERR_INVALID_ARG;
  if (!aligned(hidden, dtype_bytes(dtype)) || !aligned(gamma, 4) || !aligned(w_t, 16) ||
      !aligned(vals, 4) || !aligned(idx, 4) || (emit && !aligned(logits, 16)) ||
      (params && (!aligned(params, 4) || !aligned(tokens, 4))))
    return TAIL_ERR_INVALID_ARG;
  *L = forward_layout(gbs, H, H_u, *ps, V, k, flags);
  return TAIL_OK;
}

// The top-k and sampler run in a launch of their own unless the environment
// sets TAIL_FUSED_SELECT=1: then the large-batch lm_head kernel runs them
// after a grid barrier (bitwise the same results, but measured slower: the
// barrier costs what the kernel boundary does, and the select on 512 threads
// takes longer than on 1024).  TAIL_FUSED_SPIN sets how often a workgroup
// polls that barrier before it leaves the rows to the others (tests set it to
// 0, so that the last workgroup to arrive selects every row).  Read at every
// call.
bool fused_select_enabled() {
  const char* e = getenv("TAIL_FUSED_SELECT");
  return e && e[0] == '1' && e[1] == '\0';
}
int fused_select_spin() {
  constexpr int kDefaultSpin = 4096;  // a few ms of polling; the normal wait is tens of us
  const char* e = getenv("TAIL_FUSED_SPIN");
  if (!e || !*e) return kDefaultSpin;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? 0 : v > (1 << 24) ? (1 << 24) : int(v);
}

// The launches of tail_forward on a checked workspace of L.total bytes at ws.
hipError_t forward_launch(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t,
                          int gbs, int H, int H_u, int V, int k, float eps, unsigned flags, int ps,
                          const float* params, int ncols, float* logits, float* vals, int32_t* idx,
                          int32_t* tokens, const FwdLayout& L, void* ws, hipStream_t st) {
  const bool emit = flags & TAIL_EMIT_LOGITS;
  char* base = (char*)ws;
  float* y = (float*)(base + L.y);
  float* r = (float*)(base + L.r);
  uint16_t* act = (uint16_t*)(base + L.act);
  float* lg = emit ? logits : (float*)(base + L.logits);
  uint32_t* gk = (uint32_t*)(base + L.gkey);
  tail::TopkGeom g;
  tail::topk_geometry(V, k, &g);
  // group maxima come from the lm_head epilogue when the top-k groups are its
  // 64-column groups; otherwise (or with the NaN fold) from a separate pass
  // over the logits
  const bool fold = flags & TAIL_NAN_FOLD;
  const bool fused_groups = g.gs == tail::kFusedGroup && !fold;
  uint32_t* gk_fused = fused_groups ? gk : nullptr;
  // on the large-batch path with the epilogue's key groups, the lm_head
  // kernel runs the top-k and sampler itself
  const SplitGeom sg = split_geom(gbs, H, H_u, ps, V, flags);
  const bool fused = fused_groups && gbs > tail::kGemvMaxBatch && sg.layout == 1 &&
                     tail::rows_fuse_select(sg.nt, gbs) && fused_select_enabled();
  tail::FusedSelect* fs_dev = (tail::FusedSelect*)(base + L.sync);
  const tail::FusedSelect fs{vals,     idx,      params,
                             ncols,    tokens,   k,
                             g.gs,     g.groups, (uint32_t*)(base + L.sync + sizeof(tail::FusedSelect)),
                             tail::fused_sync_words(gbs), fused_select_spin()};
  hipError_t e = norm_lm_head(hidden, dtype, gamma, w_t, gbs, H, H_u, V, eps, ps, flags, y, r, act,
                              base + L.part, lg, gk_fused, fused ? &fs : nullptr,
                              fused ? fs_dev : nullptr, st);
  if (fused) return e;
  if (e == hipSuccess && !fused_groups) e = tail::launch_group_max(lg, gbs, V, g, fold, gk, st);
  if (e == hipSuccess)
    e = tail::launch_select(lg, gbs, V, k, g, gk, flags & TAIL_PAGE_PRECISION, fold, vals, idx,
                            nullptr, params, ncols, tokens, st);
  return e;
}

// The static scratch of tail_forward_noalloc: one array per device, which
// every call on that device shares.  Its device address comes from
// hipGetSymbolAddress, once per device with that device current (the name
// itself is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(TAIL_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_address() {
  static std::once_flag once[tail::kMaxDevices];
  static void* addr[tail::kMaxDevices];
  return tail::per_device(once, addr, [](int) -> void* {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    return p;
  });
}
}  // namespace

TAIL_API int tail_forward(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t,
                          int gbs, int H, int H_u, int V, int k, float eps, unsigned flags,
                          const float* params, int ncols, float* logits, float* vals, int32_t* idx,
                          int32_t* tokens, void* ws, size_t ws_bytes, void* stream) {
  int ps;
  FwdLayout L;
  if (int s = check_forward(hidden, dtype, gamma, w_t, gbs, H, H_u, V, k, eps, flags, params, ncols,
                            logits, vals, idx, tokens, &ps, &L))
    return s;
  if (int s = check_ws(ws, ws_bytes, L.total)) return s;
  return hip_status(forward_launch(hidden, dtype, gamma, w_t, gbs, H, H_u, V, k, eps, flags, ps,
                                   params, ncols, logits, vals, idx, tokens, L, ws,
                                   (hipStream_t)stream));
}

TAIL_API int tail_forward_noalloc(const void* hidden, int dtype, const float* gamma,
                                  const uint16_t* w_t, int gbs, int H, int H_u, int V, int k,
                                  float eps, unsigned flags, const float* params, int ncols,
                                  float* logits, float* vals, int32_t* idx, int32_t* tokens,
                                  void* stream) {
  int ps;
  FwdLayout L;
  if (int s = check_forward(hidden, dtype, gamma, w_t, gbs, H, H_u, V, k, eps, flags, params, ncols,
                            logits, vals, idx, tokens, &ps, &L))
    return s;
  if (L.total > kScratchBytes) return TAIL_ERR_SCRATCH_LIMIT;
  void* ws = scratch_address();
  if (!ws) return TAIL_ERR_HIP;
  return hip_status(forward_launch(hidden, dtype, gamma, w_t, gbs, H, H_u, V, k, eps, flags, ps,
                                   params, ncols, logits, vals, idx, tokens, L, ws,
                                   (hipStream_t)stream));
}
