// Device helpers shared by the prefill kernels: lane-pair reductions, scalar
// buffer resources, loads that land directly in LDS, and barriers with
// explicit wait counts.
#pragma once

#include "common.h"

namespace pkv {
namespace prefill_detail {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The running max is raised only when a tile's max exceeds it by more than
// this many log2 units, so p <= 2^kRescaleSlack and rescales are rare.
constexpr float kRescaleSlack = 8.0f;

// max / sum of a value over lanes l and l^32 (v_permlane32_swap: no LDS trip)
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource (SGPR quad) over [p, p + bytes): stride 0, raw offsets,
// lanes whose offset falls past `bytes` read zeros.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* p, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xffffu), bytes, 0x00020000};
}

// 16 bytes per lane from rs + voff + soff into LDS at m0 + 16*lane.  Issued
// as inline assembly so that the compiler neither counts it nor guards the
// kernel's LDS reads against it: every wait for these loads is explicit.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(i32x4 rs, uint32_t m0, int voff, int soff) {
  // the operands are wave-uniform; readfirstlane only tells the compiler so
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                   __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r),
                  "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}
// the same with the streaming policy (nt): data read once
__device__ __forceinline__ void load_lds16_nt(i32x4 rs, uint32_t m0, int voff, int soff) {
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                   __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r),
                  "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// S^T = K Q^T with the accumulator in VGPRs.  The compiler gives every MFMA
// of a kernel the AGPR-accumulator form; at head_dim 512 the O accumulators
// of 32 rows take all 256 AGPRs, so the score tile is accumulated through
// these instead.  An MFMA may take the previous one's result as its
// accumulator input directly (the hardware forwards it); vector
// instructions may read the result only after mfma_settle, which covers
// the longest latency of a 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma32_v_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_v_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_settle(f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}
// t *= alpha for an accumulator tile held in AGPRs, element by element in
// place (written out so that the compiler cannot move copies of the tile
// into VGPRs out of the rare rescale branch).  The tile's last MFMA must
// have been issued at least mfma_settle's wait earlier.
__device__ __forceinline__ void scale_agpr(f32x16& t, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = t[r], tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp) : "v"(alpha));
    t[r] = x;
  }
}
#pragma clang diagnostic pop

// barrier that first waits for LDS reads and for all but VM of this wave's
// memory loads (LDS-destination loads included); no cache maintenance
template <int VM>
__device__ __forceinline__ void phase_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | 0x70 | ((VM >> 4) << 14));  // vmcnt(VM) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Key splits of the split entry.  A work block -- the key tiles a prefill
// workgroup's rows may see, or the pages of a one-row sequence -- is cut
// into S runs of whole units, S = min(nsplit, units / min_units) (no split
// below 2 * min_units), run s being units [units*s/S, units*(s+1)/S).  The
// prefill kernel and the merge both derive S from the same device values.
__device__ __forceinline__ int split_count(int units, int nsplit, int min_units) {
  if (nsplit <= 1 || units < 2 * min_units) return 1;
  return min(nsplit, units / min_units);
}
__device__ __forceinline__ int split_begin(int units, int S, int s) {
  return (int)(((int64_t)units * s) / S);
}
// Keys [kstart, kend) that rows q0..last (positions shift + r) may attend.
__device__ __forceinline__ int2 block_keys(int q0, int last, int shift, int Lk, int window) {
  const int pmin = shift + q0, pmax = shift + last;
  return make_int2(window > 0 ? max(0, pmin - window + 1) : 0, min(pmax + 1, Lk));
}
__device__ __forceinline__ int block_tiles(int2 kr, int bn) {
  return kr.y > kr.x ? (kr.y - 1) / bn - kr.x / bn + 1 : 0;
}
// Pages [p0, pend) holding the keys a one-row sequence of L keys attends.
__device__ __forceinline__ int2 row_pages(int L, int window, int ps) {
  const int first = window > 0 ? max(0, L - window) : 0;
  return make_int2(first / ps, (L + ps - 1) / ps);
}
// minimum units per run: 128 keys of a prefill block, two pages per wave
// of a one-row sequence
__device__ __forceinline__ int min_split_tiles(int bn) { return bn >= 128 ? 1 : 128 / bn; }
__device__ __forceinline__ int min_split_pages(int nw) { return 2 * nw; }

}  // namespace prefill_detail
}  // namespace pkv
