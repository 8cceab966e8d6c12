// Building blocks of the 32x32x16 matrix-core lm_head (lm_head_rows.hip):
// direct global-to-LDS copies and the waits on them, the transposing read
// of a weight operand, the tile geometry and the epilogue.  gfx950 only.
#pragma once

#include "tail_internal.h"

namespace tail {
namespace mfma32 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// Row pitch (bytes) of an LDS weight stage holding mb 32-column bf16 blocks:
// 64 mb padded up to 64 mod 256, so the 8 row segments that 32 lanes of a
// transposing read touch fall in distinct 32-byte bank groups.
constexpr int weight_pitch(int mb) { return mb * 64 + ((64 - (mb * 64) % 256) + 256) % 256; }

template <int N>
__device__ inline void wait_vm() {
  // vmcnt field split over bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most PER * n of this wave's vector memory operations are
// outstanding (0 <= n <= N, wave-uniform).
template <int PER, int N>
__device__ inline void wait_copies(int n) {
  if constexpr (N <= 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<PER * N>();
    else wait_copies<PER, N - 1>(n);
  }
}

// lgkmcnt(0) only (vmcnt and expcnt left at their maximum)
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// The bare s_barrier: a workgroup fence before it (as __syncthreads emits)
// would drain every copy in flight.
__device__ inline void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct copy of 16 bytes per lane from global memory into LDS at
// lds_addr + 16 lane (lds_addr wave-uniform).  The copy takes its LDS address
// from m0, which the statement sets itself; no other code of the kernel
// uses m0 (it is a reserved register, so the clobber only documents the
// write).  It is inline assembly so that the compiler, which would otherwise
// make every LDS read of the wave wait for every copy in flight, does not see
// it; it writes only LDS, so no register of the wave is left pending.  The
// callers issue every copy with at least one lane active (an instruction
// that a branch skipped would not count), so the per-wave count of
// outstanding copies that the waits assume is exact.
template <bool NONTEMPORAL>
__device__ inline void copy_to_lds(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (NONTEMPORAL)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(gptr), "s"(m0) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(m0) : "memory", "m0");
}

// The weight operand of one 32-column block for one K-step of 16 lanes, from
// a stage of row pitch PITCH: two ds_read_b64_tr_b16.  In each 16-lane group
// g, lane s supplies row 8 (g / 2) + s / 4 (+4 for the second read), columns
// 16 (g % 2) + 4 (s % 4) .. + 3 of the block, and receives column
// 16 (g % 2) + s at K lanes 8 (g / 2) .. + 7 (the A operand of
// v_mfma_f32_32x32x16_bf16).  tr_lane_offset gives the per-lane part.
template <int PITCH>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int g = lane >> 4, s = lane & 15;
  return (8 * (g >> 1) + (s >> 2)) * PITCH + 32 * (g & 1) + 8 * (s & 3);
}
template <int PITCH>
__device__ __forceinline__ bf16x8 weight_operand(const lds_u8* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * PITCH));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The tiles of one workgroup.  The vocabulary is cut into 32-column blocks
// and the blocks into npass * P tiles of equal width (to within one block);
// workgroup wg of P takes tiles wg, wg + P, ..., so at any time the P
// workgroups read one contiguous column range of every weight row.
struct TileGeom {
  int P, wg, nblk, tbase, textra, ntl, nks, total;
  __device__ __forceinline__ TileGeom(int V, int Kp, int npass) {
    P = gridDim.x;
    wg = blockIdx.x;
    nblk = (V + 31) / 32;
    const int ntiles = P * npass;
    tbase = nblk / ntiles;
    textra = nblk % ntiles;
    // tiles j = 0 .. ntl - 1 are tiles j P + wg (widths do not grow with the
    // tile index, so the non-empty ones come first)
    ntl = 0;
    while (ntl < npass && tbase + ((ntl * P + wg) < textra ? 1 : 0) > 0) ++ntl;
    nks = Kp / 16;
    total = ntl * nks;
  }
  __device__ __forceinline__ void tile(int j, int& start, int& width) const {
    const int t = j * P + wg;
    width = tbase + (t < textra ? 1 : 0);
    start = t * tbase + (t < textra ? t : textra);
  }
};

// Epilogue of one wave's accumulators for one 32-row tile: WC blocks from
// block blk0, rows b .. (lane l: row b + l % 32).  Accumulator register
// 4 i + e of lane l holds column 8 i + 4 (l / 32) + e of the block, so each
// lane stores float4s; the 64-column key groups' maxima go to gkey (a plain
// store when both 32-column blocks of the group belong to the wave, an atomic
// maximum into the cleared entry when the group straddles two waves or two
// tiles).
template <int WC>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[WC], float scale, int b, bool row_ok,
                                           int blk0, int nblk, int lane, int V,
                                           float* __restrict__ logits, uint32_t* __restrict__ gkey,
                                           int groups) {
  uint32_t prev = 0;  // maximum of the previous block
#pragma unroll
  for (int c = 0; c < WC; ++c) {
    const int blk = blk0 + c;
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = blk * 32 + 8 * i + 4 * (lane >> 5);
      const float4 o = make_float4(acc[c][4 * i] * scale, acc[c][4 * i + 1] * scale,
                                   acc[c][4 * i + 2] * scale, acc[c][4 * i + 3] * scale);
      if (row_ok && v < V) {
        *reinterpret_cast<float4*>(logits + size_t(b) * V + v) = o;
        mx = max(mx, max(max(float_key(o.x), float_key(o.y)), max(float_key(o.z), float_key(o.w))));
      }
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
    if (gkey && row_ok && lane < 32) {
      uint32_t* dst = gkey + size_t(b) * groups + blk / 2;
      const bool even = (blk & 1) == 0;
      // a one-block last group has no partner
      const bool partner_here = even ? (c + 1 < WC || blk + 1 >= nblk) : (c > 0);
      if (!partner_here) atomicMax(dst, mx);  // the group straddles two waves
      else if (!even) *dst = max(prev, mx);   // both blocks here: one store
      else if (blk + 1 >= nblk) *dst = mx;
    }
    prev = mx;
  }
}

}  // namespace mfma32
}  // namespace tail
