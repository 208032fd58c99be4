// Shared device helpers for the gfx950 kernels (bf16 bit handling, MFMA
// operand types, wave-level broadcasts) and the internal launcher interface.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include <type_traits>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 pattern in the low / high half of a 32-bit word -> float (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane SRC of this lane's 16-lane row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(SRC >= 0 && SRC < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + SRC, 0xf, 0xf, false));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(static_cast<F&&>(f));
  }
}

// Wait for every vector memory access of this wave (vmcnt(0), other counters
// untouched).  Placed at the end of a rarely taken branch that issues loads
// (a block-table fetch, a query load), it keeps the compiler's per-register
// wait bookkeeping exact on the paths that skip the branch: without it the
// join of the two paths counts those loads as possibly pending, and every
// later use of their registers waits for all loads in flight, including the
// next step's prefetch.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// A wave-uniform 64-bit value, stated as such (kept in scalar registers).
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Buffer resource over [p, p + bytes): loads through it are bounds-checked by
// the hardware (out-of-range lanes read 0) and take a uniform base in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // cache-policy bits: nt (streaming data)
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16 bytes at lane offset + a wave-uniform (scalar) offset, with the
// streaming policy (data read once) or the default one (data that other
// workgroups read again, which should stay in L2).
template <bool STREAM = true>
__device__ __forceinline__ uint4 buffer_load16_s(__amdgpu_buffer_rsrc_t r, int byte_off, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, soff, STREAM ? kNonTemporal : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kNonTemporal);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void buffer_load(uint4& d, __amdgpu_buffer_rsrc_t r, int off) { d = buffer_load16(r, off); }
__device__ __forceinline__ void buffer_load(uint2& d, __amdgpu_buffer_rsrc_t r, int off) { d = buffer_load8(r, off); }

// Vector stores through a buffer resource (lanes past its range write nothing).
__device__ __forceinline__ void buffer_store(__amdgpu_buffer_rsrc_t r, int byte_off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, byte_off, 0, 0);
}
__device__ __forceinline__ void buffer_store(__amdgpu_buffer_rsrc_t r, int byte_off, const uint2& v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, byte_off, 0, 0);
}

// Streaming loads (read once, not kept in cache): 16 and 8 bytes.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// launchers (host side; arguments already validated by the C ABI layer)
// ---------------------------------------------------------------------------

// Raise a kernel's dynamic LDS limit (64 KB by default) once per device;
// thread-safe, and a no-op after the first call on a device.
inline hipError_t raise_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* part_m;      // split mode
  float* part_l;
  float* part_acc;
  uint16_t* out;      // direct mode
  int64_t head_stride;  // elements per KV head in a pool = num_pages*page_size*D
  int max_pages;
  int num_pages;
  int num_q_heads;
  int num_kv_heads;
  int group;          // Hq / Hkv (per virtual KV head, see kv_shift)
  int kv_shift;       // stream-K: KV head = virtual KV head >> kv_shift
  int num_splits;
  int pages_per_split;
  int window;
  float scale_log2;   // scale * log2(e)
  // fused append (k_new != NULL): row b's new token, at position
  // seq_lens[b] - 1, is attended from k_new / v_new [num_seqs, Hkv, D]
  // instead of the pool, and the wave that attends it (for its first
  // virtual KV head) also writes it to its pool slot
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool_w;  // the same pools, writable
  uint16_t* v_pool_w;
};

hipError_t launch_slot_mapping(const int32_t* bt, int max_pages, const int32_t* cu_q,
                               const int32_t* cu_k, int num_seqs, int total, int page_size,
                               int num_pages, int32_t* slots, hipStream_t st);
hipError_t launch_append_mapped(const uint16_t* k_new, const uint16_t* v_new, const int32_t* bt,
                                int max_pages, const int32_t* cu_q, const int32_t* cu_k,
                                int num_seqs, int total, int max_q, int page_size, int num_pages,
                                int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                                int64_t num_slots, int32_t* slots_out, hipStream_t st);
hipError_t launch_page_alloc(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int32_t* bt,
                             int max_pages, int page_size, const int32_t* free_pages,
                             int32_t* free_count, int num_pages, int32_t* status, hipStream_t st);
hipError_t launch_page_free(const int32_t* seq_lens, const int32_t* release, int num_seqs,
                            int32_t* bt, int max_pages, int page_size, int32_t* free_pages,
                            int32_t* free_count, int num_pages, int32_t* status, hipStream_t st);
hipError_t launch_append_last(const uint16_t* k_new, const uint16_t* v_new, const int32_t* bt,
                              int max_pages, const int32_t* seq_lens, int num_seqs, int page_size,
                              int num_pages, int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                              hipStream_t st);
int stream_read_sink_words(int workgroups);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t st);
hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slots,
                         int num_tokens, int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                         int64_t num_slots, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int num_seqs, int head_dim, int page_size,
                         bool split, hipStream_t st);
hipError_t launch_combine(const float* m, const float* l, const float* acc, int num_seqs,
                          int hq, int d, int splits, uint16_t* out, hipStream_t st);

// Stream-K decode: per persistent wave two partial slots of g*(D+2) floats
// (accumulator, then max and sum per head) and two merge descriptors.
constexpr int kDescInts = 8;  // valid, sequence, KV head, last wave, total units
struct StreamArgs {
  DecodeArgs base;
  int num_seqs;
  int num_waves;
  float* part;  // [2*num_waves][g*(D+2)]
  int* desc;    // [2*num_waves][kDescInts]
};
hipError_t launch_decode_stream(const StreamArgs& sa, int head_dim, int page_size, hipStream_t st);
hipError_t launch_stream_merge(const StreamArgs& sa, int head_dim, hipStream_t st);

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* out;
  int64_t head_stride;
  int max_pages;
  int num_pages;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int total_q;
  int window;
  float scale_log2;
  // key splits (head_dim <= 256): with nsplit > 1 a work block whose keys
  // are cut into S > 1 runs writes one partial per (row, head, run) (max in
  // log2 units, sum, unnormalised accumulator) to part_m/part_l [Tq, Hq,
  // nsplit] and part_acc [Tq, Hq, nsplit, D], and a merge launch writes out
  int nsplit;
  float* part_m;
  float* part_l;
  float* part_acc;
  int* part_S;  // [Tq] split count of each row's work block (written when nsplit > 1)
};
hipError_t launch_prefill(const PrefillArgs& a, int num_seqs, int max_seqlen_q, int head_dim,
                          int page_size, hipStream_t st);

// head_dim 512: one kernel for varlen rows (cu_q/cu_k set) and decode rows
// (cu_q NULL: row j is the last position of seq_lens[j]); with num_splits
// > 1 (decode) it writes split partials in the combine kernel's layout.
struct Attn512Args {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* cu_q;      // varlen rows, or NULL
  const int32_t* cu_k;
  const int32_t* seq_lens;  // decode rows when cu_q is NULL
  uint16_t* out;            // num_splits == 1
  float* part_m;            // num_splits > 1
  float* part_l;
  float* part_acc;
  int64_t head_stride;
  int max_pages;
  int num_pages;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int window;
  int num_splits;
  int pages_per_split;
  int one_row_only;         // varlen rows: attend only the one-row sequences
  int total_q;              // varlen rows: packed query rows (cu_q is clamped to it)
  float scale_log2;
};
hipError_t launch_attn512(const Attn512Args& a, int num_seqs, int max_rows, int page_size,
                          hipStream_t st);
// head_dim 512 decode as a stream-K partition over workgroups (num_waves
// counts workgroups of four waves, one per compute unit), merged by the
// stream-K merge kernel
hipError_t launch_attn512_stream(const StreamArgs& sa, int page_size, hipStream_t st);

}  // namespace pkv
