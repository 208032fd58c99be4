// Paged attention for head_dim 512: the full-attention layers of the
// dual-regime model, next to its head_dim-256 sliding layers (benchmarks
// commit log 1847125, the Gemma-4-E2B-it engine entry, "Dual attention
// regimes": full_attention with head_dim 512, sliding_attention with
// head_dim 256 and window 512).
//
// At 512 dims the register and LDS budgets of the head_dim <= 256 kernels
// do not hold: one wave's K/V step buffers alone would need 256 registers,
// and the prefill kernel's Q operands and 32-row accumulators twice as
// many.  Here the head dimension is split over the four waves of a
// workgroup: wave w owns dims [128w, 128w + 128) of Q, K, V and O.
//   S^T = K Q^T   each wave multiplies its 128-dim slices on
//                 v_mfma_f32_32x32x16_bf16 (K rows as A, the query columns
//                 as B) and the four partial score tiles are summed through
//                 LDS (one barrier per 32-key tile);
//   softmax       every wave runs the same online softmax on the full tile;
//   O^T += V^T P^T each wave on its own 128 dims: V is staged row-major in
//                 LDS and read transposed (ds_read_b64_tr_b16), and the
//                 probabilities already sit in B-operand order because the
//                 K rows are loaded in a permuted order.
// For decode rows K and V are read from the pool with coalesced loads (each
// instruction covers four rows of the wave's 256-byte slice) and staged in
// LDS; the K operands of S^T are read back in MFMA order.  Loading K
// straight in operand order makes every instruction touch 32 rows, 32 bytes
// each, whose cache-line requests fill the compute unit's miss queue (twice
// the decode time); varlen rows, with more MFMA work per tile, keep the
// direct operand loads.
// The 32 MFMA columns are (row, head) pairs of one KV group: R = 32/g rows
// times the g query heads, so every K/V tile is read once for the whole
// group.  A decode row is one row (g columns), a prefill workgroup R rows.
// Rows come through cu_seq_lens_q/k (varlen prefill, decode rows as
// one-row sequences) or through seq_lens (decode), and decode may cut the
// keys into splits whose partials go to the common combine kernel.
#include <math.h>

#include "common.h"
#include "prefill_common.h"

namespace pkv {
namespace {

using prefill_detail::bf16x2;
using prefill_detail::half_max;
using prefill_detail::kRescaleSlack;
using prefill_detail::half_sum;
using prefill_detail::lds_s16x4;
using prefill_detail::s16x4;
using prefill_detail::i32x4;
using prefill_detail::lds_void;
using prefill_detail::load_lds16_nt;
using prefill_detail::sgpr_rsrc;

constexpr int D5 = 512;
constexpr int kWaves5 = 4;                  // waves per workgroup, 128 dims each
constexpr int kSlice = D5 / kWaves5;         // dims per wave
constexpr int kTile = 32;                    // keys per tile
// LDS bytes per staged V row: 256 + 64, so that the four rows and two dim
// groups one transposed read touches fall in eight disjoint 8-bank windows
constexpr int kVStride = kSlice * 2 + 64;
constexpr int kVBytes = kTile * kVStride;    // one wave's staged V tile
constexpr int kSBytes = 64 * 16 * 4;         // one wave's partial score tile
// LDS bytes per staged K row: 256 + 16, so that the 16 rows one quarter of
// an operand read touches start in 16 disjoint 4-bank groups
constexpr int kKStride = kSlice * 2 + 16;
constexpr int kKBytes = kTile * kKStride;    // one wave's staged K tile
// LDS: [2 tiles][4 waves] partial scores, [2 tiles][4 waves] V slices, then
// [4 waves] K slices (a wave reads back only its own K, in program order)
constexpr int kLds5 = 2 * kWaves5 * kSBytes + 2 * kWaves5 * kVBytes + kWaves5 * kKBytes;

// Key (relative to its tile) that lane row i of the K operand loads.  With
// this order, score register r of lane half h holds key 16(r/8) + 8h + r%8,
// which is the B-operand order of the O^T += V^T P^T step.
__device__ __forceinline__ int key_of_row(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// The key-tile pipeline of one pass: tiles covering keys [k_lo, k_hi) of
// the sequence whose block-table row is row j, for KV head hk, with the 32
// MFMA columns this workgroup's lanes describe (column position pos, valid
// when col_ok; pmin / pmax the least and greatest position of the valid
// columns).  Folds the tiles into this lane's (acc, m_run, l_run); m_run
// is in log2 units.  Every wave of the workgroup calls it with the same
// tile range (the tiles exchange partial scores through LDS).
template <int PS, bool KLDS>
__device__ __forceinline__ void tile_loop(const Attn512Args& a, int hk, int j, int w, int lane,
                                          int k_lo, int k_hi, int pmin, int pmax, int pos,
                                          bool col_ok, const bf16x8 (&qop)[8],
                                          unsigned char* smem5, f32x16 (&acc)[4], float& m_run,
                                          float& l_run) {
  const int h = lane >> 5;
  const float c = a.scale_log2;
  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride + kSlice * w;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride + kSlice * w;
  // block-table row read through the scalar cache (never written here), so
  // that waiting for an entry does not wait for the K/V loads in flight
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)j * a.max_pages);
  const int krel = key_of_row(lane & 31);  // key this lane loads as K operand row

  // A 32-key tile spans one page (page_size 32) or two (16): their table
  // entries, or -1 for an unusable entry.
  constexpr int NPG = kTile / PS;
  struct TileRegs {
    uint4 k[8];       // K slice rows staged to LDS before use, or (no
                      // staging) the K operands of the 8 k-steps
    uint4 v[8];       // V slice rows, staged to LDS before use
    uint32_t usable;  // bit kr: key kb + kr is in [k_lo, k_hi) on a usable page
  };
  // Load addresses: K and V chunk i is key 4i + lane/16 of the tile, dims
  // 8 * (lane % 16) .. +7 of the wave's slice: a page resource (scalar
  // registers), one lane offset and a scalar row offset per chunk.  A tile
  // starts on a page boundary.
  const int lane_off = ((lane >> 4) * D5 + 8 * (lane & 15)) * 2;  // bytes
  // without staging, lane row i loads the K operand of key key_of_row(i)
  const int k_off = ((krel % PS) * D5 + 8 * h) * 2;                // bytes
  auto load_tile = [&](TileRegs& tr, int t) {
    const int kb = t * kTile;
    // pages of the tile (wave-uniform); an unusable entry reads page 0
    int ph[NPG];
    uint32_t usable = 0;
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) {
      // entries past the last page holding a key below k_hi are not read
      const int e = bt_row[max(0, min(kb / PS + pg, (k_hi - 1) / PS))];
      const bool ok = e >= 0 && e < a.num_pages;
      ph[pg] = ok ? e : 0;
      // keys of this page inside [k_lo, k_hi)
      const int lo = max(k_lo - kb - pg * PS, 0), hi = min(k_hi - kb - pg * PS, PS);
      if (ok && hi > lo)
        usable |= (hi - lo >= 32 ? 0xffffffffu : ((1u << (hi - lo)) - 1u)) << (pg * PS + lo);
    }
    tr.usable = usable;
    // Loads are issued unconditionally (unusable keys read their page base
    // or page 0, which always exists) so that the compiler can count them
    // exactly and keep the next tile in flight; K rows of such keys only
    // meet masked scores, and V rows are zeroed when staged.
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) {
      const int64_t pb = (int64_t)ph[pg] * PS * D5;
      const auto kr = make_rsrc(kh + pb, PS * D5 * 2);
      const auto vr = make_rsrc(vh + pb, PS * D5 * 2);
#pragma unroll
      for (int i = pg * (8 / NPG); i < (pg + 1) * (8 / NPG); ++i) {
        const int row_off = ((4 * i) % PS) * D5 * 2;
        if constexpr (KLDS) tr.k[i] = buffer_load16_s<KLDS>(kr, lane_off, row_off);
        tr.v[i] = buffer_load16_s<KLDS>(vr, lane_off, row_off);
      }
    }
    if constexpr (!KLDS) {
      // the operand rows straight from the pool: lane row i holds key
      // key_of_row(i), which lies on page ph[0] or (page 16) ph[1]
      const int pgk = (NPG == 1 || krel < PS) ? 0 : NPG - 1;
      const auto kr = make_rsrc(kh + (int64_t)ph[pgk] * PS * D5, PS * D5 * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) tr.k[ks] = buffer_load16_s<false>(kr, k_off, 32 * ks);
    }
  };

  float* sbuf = reinterpret_cast<float*>(smem5);
  unsigned char* vbuf = smem5 + 2 * kWaves5 * kSBytes;
  unsigned char* kw = smem5 + 2 * kWaves5 * kSBytes + 2 * kWaves5 * kVBytes + w * kKBytes;
  // this lane's K operand row in the staged tile (lane row i is key key_of_row(i))
  const unsigned char* ka = kw + krel * kKStride + 16 * h;

  auto process = [&](const TileRegs& tr, int t) {
    const int kb = t * kTile;
    const int par = t & 1;
    // partial scores of this wave's 128 dims
    f32x16 sp = {};
    if constexpr (KLDS) {
      // stage this wave's K rows, then read them back in operand order: lane
      // (row i, half h) takes K[key_of_row(i)][16ks + 8h .. +7] for k-step ks
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int chunk = lane + 64 * i;
        *reinterpret_cast<uint4*>(kw + (chunk >> 4) * kKStride + 16 * (chunk & 15)) = tr.k[i];
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sp = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(ka + 32 * ks)), qop[ks], sp);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sp = mfma32(as_bf16x8(tr.k[ks]), qop[ks], sp);
    }
    // partial tile as [4 quads][64 lanes] float4s: each store and load
    // instruction covers 1 KB contiguous (no bank conflicts)
    float* my = sbuf + (par * kWaves5 + w) * 64 * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(my + (q * 64 + lane) * 4) =
          make_float4(sp[4 * q], sp[4 * q + 1], sp[4 * q + 2], sp[4 * q + 3]);
    // this wave's V rows, row-major with a padded stride
    unsigned char* vw = vbuf + (par * kWaves5 + w) * kVBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int chunk = lane + 64 * i, key = chunk >> 4, part = chunk & 15;
      *reinterpret_cast<uint4*>(vw + key * kVStride + 16 * part) =
          ((tr.usable >> key) & 1u) ? tr.v[i] : make_uint4(0, 0, 0, 0);
    }
    // LDS writes done, then the barrier; no wait for the next tile's global
    // loads (a __syncthreads would drain them and serialise the prefetch)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    // full scores: the four partials of this lane's (column, keys)
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves5; ++ww) {
      const float* src = sbuf + (par * kWaves5 + ww) * 64 * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(src + (q * 64 + lane) * 4);
        x[4 * q] += v.x;
        x[4 * q + 1] += v.y;
        x[4 * q + 2] += v.z;
        x[4 * q + 3] += v.w;
      }
    }
    // mask: register r holds key kb + 16(r/8) + 8h + r%8 of this lane's
    // column.  A tile whose keys are all usable and visible to every row of
    // the workgroup needs no per-key test (columns past the rows are never
    // written, whatever their scores).
    const bool full = tr.usable == 0xffffffffu && kb + kTile - 1 <= pmin &&
                      (a.window <= 0 || pmax - kb < a.window);
    float mt = -INFINITY;
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] *= c;
        mt = fmaxf(mt, x[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + 8 * h + (r & 7), k = kb + kr;
        bool ok = col_ok && k <= pos && ((tr.usable >> kr) & 1u);
        if (a.window > 0) ok = ok && pos - k < a.window;
        x[r] = ok ? x[r] * c : -INFINITY;
        mt = fmaxf(mt, x[r]);
      }
    }
    mt = half_max(mt);
    // the running max moves only when a tile exceeds it by more than the
    // slack, so p <= 2^slack and the accumulators are rarely rescaled
    const bool raise = mt > m_run + kRescaleSlack;
    float alpha = 1.f;
    if (raise) {
      alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mt);
      m_run = mt;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = fast_exp2(x[r] - m_use);
      psum += x[r];
    }
    l_run = l_run * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    // O^T += V^T P^T on this wave's dims
    const int gi = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // p in [0, 2^slack]: the hardware round-to-nearest conversion suffices
      const bf16x2 p01 = {(__bf16)x[8 * ks + 0], (__bf16)x[8 * ks + 1]};
      const bf16x2 p23 = {(__bf16)x[8 * ks + 2], (__bf16)x[8 * ks + 3]};
      const bf16x2 p45 = {(__bf16)x[8 * ks + 4], (__bf16)x[8 * ks + 5]};
      const bf16x2 p67 = {(__bf16)x[8 * ks + 6], (__bf16)x[8 * ks + 7]};
      uint4 pk;
      pk.x = __builtin_bit_cast(uint32_t, p01);
      pk.y = __builtin_bit_cast(uint32_t, p23);
      pk.z = __builtin_bit_cast(uint32_t, p45);
      pk.w = __builtin_bit_cast(uint32_t, p67);
      const bf16x8 pop = as_bf16x8(pk);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        // transposed reads: source lane 4r'+a' of a 16-lane group points at
        // V[key0 + r'][d0 + 4a']; output lane i gets V[key0 .. key0+3][d0 + i]
        const int d0 = 32 * dt + 16 * (gi & 1) + 4 * (sl & 3);
        uint2 part[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int key = 16 * ks + 8 * (gi >> 1) + 4 * q + (sl >> 2);
          const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) unsigned char*)(vw + key * kVStride + 2 * d0));
          part[q] = __builtin_bit_cast(uint2, v4);
        }
        const bf16x8 vop = as_bf16x8(make_uint4(part[0].x, part[0].y, part[1].x, part[1].y));
        acc[dt] = mfma32(vop, pop, acc[dt]);
      }
    }
  };

  // Two register sets, one tile ahead.  The prefetch is issued on every
  // step, also past the last tile (those keys are all unusable: row-0 reads,
  // masked), so every path issues the same loads and the compiler waits for
  // exactly the tile being processed.
  const int t0 = k_lo / kTile, t1 = k_hi > k_lo ? (k_hi + kTile - 1) / kTile : t0;
  // The scheduling barriers keep each prefetch ahead of the processing of
  // the tile before it: without them the compiler hoists the first MFMA of
  // process(t) above the loads of tile t+1, so that the wait for tile t
  // finds nothing else in flight.
  TileRegs ta, tb;
  if (t0 < t1) load_tile(ta, t0);
  for (int t = t0; t < t1; t += 2) {
    load_tile(tb, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    process(ta, t);
    if (t + 1 >= t1) break;
    load_tile(ta, t + 2);
    __builtin_amdgcn_sched_barrier(0);
    process(tb, t + 1);
  }

}

// ---------------------------------------------------------------------------
// Key tiles of a decode row in the stream-K kernel.  A decode row fills at
// most 8 MFMA columns (its query-head group), so the matrix steps here use
// v_mfma_f32_16x16x32_bf16 (16 columns) instead of the 32-column tiles of
// tile_loop, which halves the MFMA issue and the softmax work per tile.
// Lane (q, n) = (lane / 16, lane % 16):
//   S^T = K Q^T     this wave's 128 dims, two 16-key blocks; A row n of
//                   block b is key 8(n/4) + 4b + n%4, so score register
//                   4b + j of lane (q, n) is key 8q + 4b + j of head n: the
//                   lane holds keys 8q .. 8q+7, the B-operand order of PV;
//   O^T += V^T P^T  eight 16-dim tiles, V^T read transposed from LDS.
// K and V go to LDS with LDS-destination buffer loads, without passing
// through registers: one instruction moves the wave's 256-byte slices of 4
// key rows into 1 KB of LDS, lane l's 16 bytes at 16 l, and lane l loads
// chunk (l % 16) ^ swz(row) of its row, which makes the MFMA-order reads of
// K and the transposed reads of V free of bank conflicts.  Each wave owns
// two K/V slots (the tile it processes and the next one, whose loads are in
// flight meanwhile); only the partial scores cross waves.  A page's buffer
// resource ends at the tile's last allowed key, and an unusable page has an
// empty one, so those rows arrive as zeros.
constexpr int kScBytes = 2 * kWaves5 * 2048;                  // [2 tiles][4 waves] partial scores
constexpr int kKVSlot = 2 * kTile * kSlice * 2;               // a wave's K and V slices of a tile
constexpr int kLdsStream = kScBytes + kWaves5 * 2 * kKVSlot;  // 144 KB

// staged row r holds, at 16-byte position p, chunk p ^ swz(r) of its slice
__device__ __forceinline__ int swz_k(int r) { return (r & 3) | ((r >> 1) & 12); }
__device__ __forceinline__ int swz_v(int r) { return 2 * ((r & 3) | ((r >> 1) & 4)); }

// wait until at most N of this wave's vector memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0f70 | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// max / sum over lanes l, l^16, l^32 and l^48 (the four k-groups of a column)
__device__ __forceinline__ float quad_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return half_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return half_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Folds the tiles of keys [k_lo, k_hi) of the row at position pos (block
// table row j, KV head hk) into this lane's (acc, m_run, l_run); m_run is
// in log2 units and l_run this lane's share of the sum (summed over the
// four k-groups by the caller).  qp points at this lane's query slice (head
// n of the group, dims 128w + 8q ..), read when col_ok.  When kn is set,
// key pos is the step's new token: its K/V rows (kn, vn: this KV head's new
// rows) are written to the pool (kw, vw: this KV head's pools), and into
// the staged tile that holds the key once that tile has landed in LDS (no
// other workgroup reads that pool row).  Every wave calls it with the same
// range.
template <int PS>
__device__ __forceinline__ void stream_tiles(const Attn512Args& a, int hk, int j, int w, int lane,
                                             int k_lo, int k_hi, int pos, bool col_ok,
                                             const uint16_t* qp, unsigned char* smem,
                                             f32x4 (&acc)[8], float& m_run, float& l_run,
                                             const uint16_t* kn = nullptr,
                                             const uint16_t* vn = nullptr, uint16_t* kw = nullptr,
                                             uint16_t* vw = nullptr) {
  constexpr int NPG = kTile / PS;  // pages per tile
  constexpr int LPP = 8 / NPG;     // loads per page and tensor
  const int t0 = k_lo / kTile, t1 = k_hi > k_lo ? (k_hi + kTile - 1) / kTile : t0;
  if (t0 >= t1) return;
  const int q = lane >> 4, n = lane & 15;
  const float c = a.scale_log2;
  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride + kSlice * w;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride + kSlice * w;
  const int32_t* bt_row = a.block_tables + (int64_t)j * a.max_pages;
  const int last_page = (k_hi - 1) / PS;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
  const int kv0 = kScBytes + w * 2 * kKVSlot;  // this wave's slots (byte offsets in LDS)

  // load i of a tensor: tile row 4i + q, source chunk n ^ swz(row)
  int vo_k[8], vo_v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + q;
    vo_k[i] = (r % PS) * D5 * 2 + 16 * (n ^ swz_k(r));
    vo_v[i] = (r % PS) * D5 * 2 + 16 * (n ^ swz_v(r));
  }
  // K operand of k-step ks, block b: key 8(n/4) + 4b + n%4 (whose swizzle is
  // n), chunk 4ks + q
  int ka[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka[ks] = (8 * (n >> 2) + (n & 3)) * 256 + 16 * ((4 * ks + q) ^ n);
  // transposed V reads: lane (q, n) points at key 8q + 4hh + n/4, dims
  // 16dt + 4(n%4) .. +3, i.e. 16-byte pair dt ^ s2 of the row
  const int s2 = (n >> 2) + 4 * (q & 1);
  int va[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) va[dt] = (8 * q + (n >> 2)) * 256 + 8 * (n & 3) + 32 * (dt ^ s2);

  // Table entries 64 pages at a time, lane l holding page pbase + l: a
  // scalar load per tile would be waited for by every LDS wait of the tile
  // (one counter covers both), a full memory round trip per tile.
  int pbase = t0 * NPG, ent = 0;
  auto fetch_entries = [&]() {
    ent = bt_row[min(pbase + lane, last_page)];
  };
  auto entries = [&](int t, int (&e)[NPG]) {
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg)
      e[pg] = __builtin_amdgcn_readlane(ent, min(t * NPG + pg, last_page) - pbase);
  };
  // makes the pages of tile t readable from ent (a refill drains the loads
  // in flight: once per 64 pages)
  auto cover = [&](int t) {
    if (min(t * NPG + NPG - 1, last_page) - pbase >= 64) {
      pbase = t * NPG;
      fetch_entries();
      wait_vm<0>();
    }
  };
  // keys of tile t inside [k_lo, k_hi) on a usable page
  auto usable_of = [&](int t, const int (&e)[NPG]) {
    uint32_t u = 0;
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) {
      const int kb = t * kTile + pg * PS;
      const bool ok = e[pg] >= 0 && e[pg] < a.num_pages;
      const int lo = max(k_lo - kb, 0), hi = min(k_hi - kb, PS);
      if (ok && hi > lo)
        u |= (hi - lo >= 32 ? 0xffffffffu : ((1u << (hi - lo)) - 1u)) << (pg * PS + lo);
    }
    return u;
  };
  // page pg of tile t, cut at k_hi (an unusable page or one past k_hi is empty)
  auto rsrc = [&](const uint16_t* base, int t, int pg, int e) {
    const int kb = t * kTile + pg * PS;
    const bool ok = e >= 0 && e < a.num_pages && kb < k_hi;
    const int hi = ok ? min(k_hi - kb, PS) : 0;
    return sgpr_rsrc(base + (ok ? (int64_t)e * PS * D5 : 0), hi * D5 * 2);
  };
  auto issue_k = [&](int t, const int (&e)[NPG], int slot) {
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) {
      const i32x4 rs = rsrc(kh, t, pg, e[pg]);
#pragma unroll
      for (int i = pg * LPP; i < (pg + 1) * LPP; ++i) load_lds16_nt(rs, lds0 + slot + i * 1024, vo_k[i], 0);
    }
  };

  // Q^T as the B operand: lane (q, n) holds q[head n][128w + 32ks + 8q .. +7];
  // read with the table entries and waited for here, so that no wait in the
  // tile loop has to cover these loads
  fetch_entries();
  bf16x8 qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col_ok) v = *reinterpret_cast<const uint4*>(qp + 32 * ks);
    qop[ks] = as_bf16x8(v);
  }
  // the new token: this wave's 256-byte slices of its K and V rows, one
  // dword per lane, and its page's table entry
  uint32_t nk = 0, nv = 0;
  int e_new = -1;
  if (kn != nullptr) {
    nk = reinterpret_cast<const uint32_t*>(kn + kSlice * w)[lane];
    nv = reinterpret_cast<const uint32_t*>(vn + kSlice * w)[lane];
    e_new = bt_row[pos / PS];
  }
  wait_vm<0>();
  // staged position of the new token's dword of this lane: row pos % 32 of
  // the last tile, chunk lane / 4 at its swizzled position
  const int r_new = pos % kTile;
  const int lk_new = r_new * 256 + 16 * ((lane >> 2) ^ swz_k(r_new)) + 4 * (lane & 3);
  const int lv_new = kTile * kSlice * 2 + r_new * 256 + 16 * ((lane >> 2) ^ swz_v(r_new)) + 4 * (lane & 3);
  if (kn != nullptr) {
    e_new = __builtin_amdgcn_readfirstlane(e_new);
    if (e_new >= 0 && e_new < a.num_pages) {  // an unusable entry takes no write
      const int64_t off = ((int64_t)e_new * PS + pos % PS) * D5 + kSlice * w;
      reinterpret_cast<uint32_t*>(kw + off)[lane] = nk;
      reinterpret_cast<uint32_t*>(vw + off)[lane] = nv;
    }
  }

  int e_cur[NPG], e_nxt[NPG];
  entries(t0, e_cur);
  uint32_t use_cur = usable_of(t0, e_cur);
  issue_k(t0, e_cur, kv0);
#pragma unroll
  for (int pg = 0; pg < NPG; ++pg) {
    const i32x4 rs = rsrc(vh, t0, pg, e_cur[pg]);
#pragma unroll
    for (int i = pg * LPP; i < (pg + 1) * LPP; ++i)
      load_lds16_nt(rs, lds0 + kv0 + kTile * kSlice * 2 + i * 1024, vo_v[i], 0);
  }

  for (int t = t0; t < t1; ++t) {
    const int par = (t - t0) & 1;
    const int cur = kv0 + par * kKVSlot, nxt = kv0 + (par ^ 1) * kKVSlot;
    // the next tile's K goes to the free slot first (a tile past the range
    // has empty resources: it moves zeros and reads no memory)
    cover(t + 1);
    entries(t + 1, e_nxt);
    issue_k(t + 1, e_nxt, nxt);
    const uint32_t use_nxt = usable_of(t + 1, e_nxt);
    i32x4 rv[NPG];
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) rv[pg] = rsrc(vh, t + 1, pg, e_nxt[pg]);
    wait_vm<8>();  // this tile's K and V are in LDS
    if (kn != nullptr && t == t1 - 1) {
      // the new token over the row the tile read from the pool (the pool
      // write above may not have landed when the tile was requested)
      *reinterpret_cast<uint32_t*>(smem + cur + lk_new) = nk;
      *reinterpret_cast<uint32_t*>(smem + cur + lv_new) = nv;
    }

    // partial S^T of this wave's dims (all K operands requested first), the
    // next tile's V loads in between
    uint4 kop[8];
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
      kop[jb] = *reinterpret_cast<const uint4*>(smem + cur + ka[jb >> 1] + (jb & 1) * 1024);
    f32x4 sp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) sp[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      sp[jb & 1] = mfma16(as_bf16x8(kop[jb]), qop[jb >> 1], sp[jb & 1]);
      load_lds16_nt(rv[jb / LPP], lds0 + nxt + kTile * kSlice * 2 + jb * 1024, vo_v[jb], 0);
    }
    float* my = reinterpret_cast<float*>(smem) + (par * kWaves5 + w) * 512;
    *reinterpret_cast<f32x4*>(my + 4 * lane) = sp[0];
    *reinterpret_cast<f32x4*>(my + 256 + 4 * lane) = sp[1];
    // LDS writes done, then the barrier; the loads in flight stay in flight
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    // full scores of this lane's column: register r is key 8q + r
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = 0.f;
    if (col_ok) {
#pragma unroll
      for (int ww = 0; ww < kWaves5; ++ww) {
        const float* src = reinterpret_cast<const float*>(smem) + (par * kWaves5 + ww) * 512;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + 4 * lane);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 256 + 4 * lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] += v0[r];
          x[4 + r] += v1[r];
        }
      }
    }
    const int kb = t * kTile;
    const bool full = use_cur == 0xffffffffu && kb + kTile - 1 <= pos &&
                      (a.window <= 0 || pos - kb < a.window);
    float mt = -INFINITY;
    if (full) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        x[r] *= c;
        mt = fmaxf(mt, x[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kr = 8 * q + r, k = kb + kr;
        bool ok = col_ok && k <= pos && ((use_cur >> kr) & 1u);
        if (a.window > 0) ok = ok && pos - k < a.window;
        x[r] = ok ? x[r] * c : -INFINITY;
        mt = fmaxf(mt, x[r]);
      }
    }
    mt = quad_max(mt);
    const bool raise = mt > m_run + kRescaleSlack;
    float alpha = 1.f;
    if (raise) {
      alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mt);
      m_run = mt;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = fast_exp2(x[r] - m_use);
      psum += x[r];
    }
    l_run = l_run * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] *= alpha;
    }
    // P^T as the B operand (p <= 2^slack: the hardware conversion suffices)
    uint4 pk;
    pk.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[0], (__bf16)x[1]});
    pk.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[2], (__bf16)x[3]});
    pk.z = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[4], (__bf16)x[5]});
    pk.w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[6], (__bf16)x[7]});
    const bf16x8 pop = as_bf16x8(pk);
    const unsigned char* vs = smem + cur + kTile * kSlice * 2;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 part[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) unsigned char*)(vs + va[dt] + hh * 1024));
        part[hh] = __builtin_bit_cast(uint2, v4);
      }
      acc[dt] = mfma16(as_bf16x8(make_uint4(part[0].x, part[0].y, part[1].x, part[1].y)), pop, acc[dt]);
    }
    use_cur = use_nxt;
  }
  // the loads past the range are done before the slots are reused
  wait_vm<0>();
}

template <int PS, bool KLDS>
__global__ __launch_bounds__(kWaves5 * 64, 1) void attn512_kernel(Attn512Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem5[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;     // lane half: k-group of the operands
  const int col = lane & 31;   // MFMA column: (row, head) pair
  const int g = a.group;
  const int R = 32 / g;        // rows per workgroup
  const int nsplit = a.num_splits;
  const int s = blockIdx.x % nsplit;
  const int rb = blockIdx.x / nsplit;
  const int hk = blockIdx.y;
  const int j = blockIdx.z;

  int q_start, Lq, Lk;
  if (a.cu_q != nullptr) {
    // clamped to the packed rows [0, total_q), so that no q read or out
    // write leaves its buffer whatever cu_seq_lens_q holds
    q_start = min(max(a.cu_q[j], 0), a.total_q);
    Lq = min(max(a.cu_q[j + 1], q_start), a.total_q) - q_start;
    Lk = a.cu_k[j + 1] - a.cu_k[j];
  } else {
    q_start = j;
    Lq = 1;
    Lk = a.seq_lens[j];
  }
  Lk = max(0, min(Lk, a.max_pages * PS));
  if (a.one_row_only && Lq != 1) return;
  const int row0 = rb * R;
  if (row0 >= Lq) return;
  const int nrows = min(R, Lq - row0);
  const int shift = Lk - Lq;

  // this lane's column
  const int crow = col / g, chead = col - crow * g;
  const bool col_ok = crow < nrows;
  const int head = hk * g + chead;
  const int pos = shift + row0 + crow;  // position of the column's row
  const int qrow = q_start + row0 + (col_ok ? crow : 0);

  // keys this workgroup may need: the rows' causal/window band, cut to the split
  const int pmin = shift + row0, pmax = shift + row0 + nrows - 1;
  int k_lo = a.window > 0 ? max(0, pmin - a.window + 1) : 0;
  int k_hi = min(pmax + 1, Lk);
  if (nsplit > 1) {
    const int first_key = a.window > 0 ? max(0, Lk - a.window) : 0;
    const int p0 = first_key / PS;
    k_lo = max(k_lo, (p0 + s * a.pages_per_split) * PS);
    k_hi = min(k_hi, (p0 + (s + 1) * a.pages_per_split) * PS);
  }

  // Q slice as the B operand: lane holds q[column][128w + 16ks + 8h .. +7]
  bf16x8 qop[8];
  {
    const uint16_t* qp = a.q + ((int64_t)qrow * a.num_q_heads + head) * D5 + kSlice * w + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col_ok) v = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      qop[ks] = as_bf16x8(v);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  tile_loop<PS, KLDS>(a, hk, j, w, lane, k_lo, k_hi, pmin, pmax, pos, col_ok, qop, smem5, acc,
                      m_run, l_run);

  // ---- write: lane holds dims 32dt + 8(r/4) + 4h + r%4 of its column ----
  const float lt = half_sum(l_run);
  if (!col_ok) return;
  const int dbase = kSlice * w + 4 * h;
  if (nsplit == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = a.out + ((int64_t)qrow * a.num_q_heads + head) * D5 + dbase;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[dt][4 * rq] * inv, acc[dt][4 * rq + 1] * inv);
        pk.y = pack_bf16x2(acc[dt][4 * rq + 2] * inv, acc[dt][4 * rq + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * rq) = pk;
      }
  } else {
    const int64_t cell = ((int64_t)qrow * a.num_q_heads + head) * nsplit + s;
    float* pa = a.part_acc + cell * D5 + dbase;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(pa + 32 * dt + 8 * rq) =
            make_float4(acc[dt][4 * rq], acc[dt][4 * rq + 1], acc[dt][4 * rq + 2], acc[dt][4 * rq + 3]);
    if (w == 0 && h == 0) {
      a.part_m[cell] = m_run;
      a.part_l[cell] = lt;
    }
  }
}

// Decode rows as a stream-K partition over workgroups.  The units of the
// batch -- every 32-key tile that holds an allowed key, for every KV head of
// every row, ordered by row, then KV head, then tile -- are cut into one
// contiguous range of equal size per workgroup (one workgroup per compute
// unit), so that every compute unit streams the same number of tiles
// whatever the length mix.  A (row, KV head) segment inside one range is
// finished by its workgroup; a segment cut by range ends leaves one partial
// per piece (unnormalised accumulator, then max in log2 units and sum, for
// each of the g query heads) and, from the workgroup where it starts, a
// merge descriptor, in the layout the stream-K merge kernel combines in
// workgroup order.  The g query heads of a row are g of the 32 MFMA
// columns, so each K/V tile is read once for the whole group.
template <int PS>
__global__ __launch_bounds__(kWaves5 * 64, 1) void attn512_stream_kernel(StreamArgs sa) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem5[];
  const DecodeArgs& d = sa.base;
  const int B = sa.num_seqs, nw = sa.num_waves, wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int Hkv = d.num_kv_heads, g = d.group;
  int* pre = reinterpret_cast<int*>(smem5 + kLdsStream);  // pre[b] = first unit of row b; pre[B] = U
  // row lengths, read through the scalar cache (never written here)
  const __attribute__((address_space(4))) int32_t* sl =
      (const __attribute__((address_space(4))) int32_t*)d.seq_lens;
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };

  // ---- units per row (tiles of allowed keys) x KV heads, scanned by wave 0 ----
  if (w == 0) {
    int carry = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      int v = 0;
      if (b < B) {
        const int L = max(0, min(d.seq_lens[b], d.max_pages * PS));
        const int fk = d.window > 0 ? max(0, L - d.window) : 0;
        v = ((L + kTile - 1) / kTile - fk / kTile) * Hkv;
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off);
        if (lane >= off) v += t;
      }
      if (b < B) pre[b + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (lane == 0) pre[0] = 0;
  }
  if (tid < 2) sa.desc[(2 * wg + tid) * kDescInts] = 0;  // this launch's descriptors
  __syncthreads();
  const int U = uni(pre[B]);
  // rows of empty sequences are zero (a row with any key has a unit)
  for (int b = wg; b < B; b += nw) {
    if (pre[b + 1] != pre[b]) continue;
    uint16_t* o = d.out + (int64_t)b * d.num_q_heads * D5;
    for (int i = tid; i < d.num_q_heads * D5; i += kWaves5 * 64) o[i] = 0;
  }
  if (U == 0) return;
  const int u0 = (int)((int64_t)wg * U / nw), u1 = (int)((int64_t)(wg + 1) * U / nw);
  if (u0 >= u1) return;

  Attn512Args a = {};
  a.k_pool = d.k_pool;
  a.v_pool = d.v_pool;
  a.block_tables = d.block_tables;
  a.head_stride = d.head_stride;
  a.max_pages = d.max_pages;
  a.num_pages = d.num_pages;
  a.window = d.window;
  a.scale_log2 = d.scale_log2;

  // first segment: the largest row b with pre[b] <= u0 is non-empty (u0 < U)
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(pre[mid]) <= u0) lo = mid; else hi = mid;
  }
  int b = lo;
  int hk = (u0 - uni(pre[lo])) / ((uni(pre[lo + 1]) - uni(pre[lo])) / Hkv);
  const bool col_ok = col < g;
  const int dbase = kSlice * w + 4 * q;  // lane (q, col) holds dims 16dt + 4q .. +3 of head col
  for (int u = u0; u < u1;) {
    const int L = max(0, min(sl[b], d.max_pages * PS));
    const int E = (uni(pre[b + 1]) - uni(pre[b])) / Hkv;
    const int s0 = uni(pre[b]) + hk * E, s1 = s0 + E;
    const int first_key = a.window > 0 ? max(0, L - a.window) : 0;
    const int tf = first_key / kTile;
    const int ub = min(u1, s1);
    const int k_lo = max(first_key, (tf + (u - s0)) * kTile);
    const int k_hi = min(L, (tf + (ub - s0)) * kTile);
    const int head = hk * g + (col_ok ? col : 0);
    const uint16_t* qp = d.q + ((int64_t)b * d.num_q_heads + head) * D5 + kSlice * w + 8 * q;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // the previous segment's last tile is done with the LDS score slots,
    // whatever this segment's first tile parity
    __syncthreads();
    // the piece holding the row's last key appends the step's new token
    // (a row longer than its table appends nothing)
    const bool app = d.k_new != nullptr && k_hi == L && L >= 1 && sl[b] == L;
    const int64_t nrow = ((int64_t)b * Hkv + hk) * D5;
    const int64_t hoff = (int64_t)hk * d.head_stride;
    stream_tiles<PS>(a, hk, b, w, lane, k_lo, k_hi, L - 1, col_ok, qp, smem5, acc, m_run, l_run,
                     app ? d.k_new + nrow : nullptr, app ? d.v_new + nrow : nullptr,
                     d.k_pool_w + hoff, d.v_pool_w + hoff);
    const float lt = quad_sum(l_run);
    if (s0 >= u0 && s1 <= u1) {  // the whole segment is here: final rows
      if (col_ok) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t* op = d.out + ((int64_t)b * d.num_q_heads + head) * D5 + dbase;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
          pk.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * dt) = pk;
        }
      }
    } else {
      // a piece of a cut segment: slot 0 holds the piece at the start of
      // this workgroup's range, slot 1 the one at its end
      const int slot = 2 * wg + (s0 <= u0 ? 0 : 1);
      float* p = sa.part + (int64_t)slot * g * (D5 + 2);
      if (col_ok) {
        float* pa = p + col * D5 + dbase;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(pa + 16 * dt) = acc[dt];
        if (w == 0 && q == 0) {
          p[g * D5 + col] = m_run;
          p[g * D5 + g + col] = lt;
        }
      }
      if (s0 >= u0 && tid == 0) {  // the segment starts here: describe it for the merge
        int* dsc = sa.desc + slot * kDescInts;
        dsc[1] = b;
        dsc[2] = hk;
        dsc[3] = (int)(((int64_t)s1 * nw - 1) / U);  // workgroup holding the segment's last unit
        dsc[4] = U;
        dsc[0] = 1;
      }
    }
    u = ub;
    if (++hk == Hkv) {  // next row with any unit
      hk = 0;
      ++b;
      while (b < B - 1 && uni(pre[b + 1]) == uni(pre[b])) ++b;
    }
  }
}

template <int PS>
hipError_t launch_stream_ps(const StreamArgs& sa, hipStream_t st) {
  static std::atomic<uint64_t> lds_raised{0};
  constexpr int kMaxLds = kLdsStream + (2048 + 1) * 4;  // the scan of up to 2048 rows
  const hipError_t e = raise_lds_limit(
      reinterpret_cast<const void*>(&attn512_stream_kernel<PS>), kMaxLds, lds_raised);
  if (e != hipSuccess) return e;
  const size_t smem = kLdsStream + (size_t)(sa.num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL((attn512_stream_kernel<PS>), dim3(sa.num_waves), dim3(kWaves5 * 64), smem, st,
                     sa);
  return hipGetLastError();
}

// K staged through LDS and loads with the streaming policy for decode rows
// (a workgroup's columns are one row: the kernel is bound by the loads in
// flight, and each page is read once); straight operand loads with the
// default policy for varlen rows (the MFMA work per tile is larger, and the
// row blocks of a sequence read the same pages, which should stay in L2)
template <int PS, bool KLDS>
hipError_t launch_ps(const Attn512Args& a, int num_seqs, int row_blocks, hipStream_t st) {
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&attn512_kernel<PS, KLDS>),
                                       kLds5, lds_raised);
  if (e != hipSuccess) return e;
  const dim3 grid(row_blocks * a.num_splits, a.num_kv_heads, num_seqs);
  hipLaunchKernelGGL((attn512_kernel<PS, KLDS>), grid, dim3(kWaves5 * 64), kLds5, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn512_stream(const StreamArgs& sa, int page_size, hipStream_t st) {
  return page_size == 16 ? launch_stream_ps<16>(sa, st) : launch_stream_ps<32>(sa, st);
}

hipError_t launch_attn512(const Attn512Args& a, int num_seqs, int max_rows, int page_size,
                          hipStream_t st) {
  const int R = 32 / a.group;
  const int row_blocks = (max_rows + R - 1) / R;
  if (a.cu_q == nullptr)
    return page_size == 16 ? launch_ps<16, true>(a, num_seqs, row_blocks, st)
                           : launch_ps<32, true>(a, num_seqs, row_blocks, st);
  return page_size == 16 ? launch_ps<16, false>(a, num_seqs, row_blocks, st)
                         : launch_ps<32, false>(a, num_seqs, row_blocks, st);
}

}  // namespace pkv
