// Varlen causal prefill over the paged pool on bf16 MFMA.
//
// Rows of several sequences are packed and delimited by cu_seq_lens_q/k
// (CB sync-driver commit 5f3e1c9, "qwen3_grpo_unified.py fixes"; benchmarks
// README, "Flash Attention 4 on Blackwell (sm_100)" item 2).  Masks are the
// per-sequence causal mask, plus q_pos - kv_pos < window in the sliding
// regime (commit log 1847125, per-regime mask entry).  Because every
// workgroup belongs to one sequence, the document boundary costs nothing:
// no per-key document lookup is ever made (the same log reports that such
// per-kv lookups were the slow path of the packed prefill mask).
//
// Work decomposition.  A workgroup of NW waves owns BM query rows of one
// sequence for HW query heads of one KV group; each wave owns 32 rows of one
// head.  K/V tiles of BN keys are gathered page by page into LDS once per
// workgroup and shared by all its heads and rows.
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16: A = K rows straight from LDS,
//                B = Q rows held in registers; the result keeps one query
//                row per lane column, so the softmax row statistics are
//                lane-local plus one exchange with the lane 32 away.
//   O^T += V^T P^T: the probabilities already sit in B-operand order in the
//                score registers (only rounded to bf16); V stays row-major
//                in LDS and is read transposed with ds_read_b64_tr_b16.
// Softmax: p = 2^(s*c - m*c) with c = scale*log2(e) in one FMA; the running
// maximum is raised only when a tile's maximum exceeds it by more than
// kRescaleSlack (in log2 units), which keeps p <= 2^kRescaleSlack and skips
// most rescales of the accumulator.
//
// Ping-pong schedule.  Every key tile t costs each wave two phases: a
// vector phase V(t) (mask, max, exponentials, P packing, staging of the
// next tile) and a matrix phase M(t) (O += V(t) P(t), then S(t+1) =
// K(t+1) Q^T).  The waves form two groups, one wave of each on every SIMD;
// group B runs one phase behind group A, and a workgroup barrier closes
// every phase, so on each SIMD one wave's MFMAs overlap the other wave's
// softmax.  Group A stages K tiles and group B stages V tiles: K(t+1) is
// written during A's V(t) and V(t+1) during B's V(t), which is exactly when
// the tile two back is no longer read, so two LDS buffers per tensor
// suffice.  Global loads run two tiles ahead of those stores and
// block-table entries two tiles ahead of the loads.
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// Tuning knobs (fixed at build time) for head_dim <= 128: waves per
// workgroup, keys per tile, LDS row pads, wave priority in matrix phases.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_KEYS
#define PKV_PREFILL_KEYS 64
#endif
#ifndef PKV_PREFILL_KPAD
#define PKV_PREFILL_KPAD 8      // K row pad (elements)
#endif
#ifndef PKV_PREFILL_VPAD
#define PKV_PREFILL_VPAD 32     // V row pad (elements)
#endif
#ifndef PKV_PREFILL_SETPRIO
#define PKV_PREFILL_SETPRIO 1   // raise the matrix-phase wave's issue priority
#endif

template <int D, int HW>
struct PrefillCfg {
  static constexpr int NW = D == 256 ? 4 : PKV_PREFILL_WAVES;  // waves per workgroup
  static constexpr int NT = NW * 64;           // threads
  static constexpr int GT = NT / 2;            // threads per group
  static constexpr int QB = NW / HW;           // waves along the rows
  static constexpr int BM = 32 * QB;           // query rows per workgroup
  static constexpr int BN = D == 256 ? 32 : PKV_PREFILL_KEYS;  // keys per tile
  static constexpr int KT = BN / 32;           // 32-key tiles of S^T
  static constexpr int NU = BN / 16;           // 16-key steps of O^T
  static constexpr int KP = D + PKV_PREFILL_KPAD;  // LDS row pitch of K (elements)
  static constexpr int VP = D + PKV_PREFILL_VPAD;  // LDS row pitch of V (elements)
  static constexpr int KS = D / 16;            // k-steps of S^T
  static constexpr int DT = D / 32;            // 32-row tiles of O^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per token row
  static constexpr int WK = BN / (NW / 2);     // keys per wave per tile
  static constexpr int KPW = 64 / CPR;         // keys per wave per 16-byte chunk
  static constexpr int CH = WK / KPW;          // chunks per thread of its group's tensor
  static constexpr int KBUF = BN * KP;         // elements of one K buffer
  static constexpr int VBUF = BN * VP;         // elements of one V buffer
  static constexpr int LDS_BYTES = 2 * (KBUF + VBUF) * 2;
  static_assert(NW % 2 == 0 && NW >= 2, "two wave groups");
  static_assert(CH >= 1 && WK % KPW == 0 && BN % (NW / 2) == 0, "tile chunks must split evenly");
  static_assert(QB >= 1, "more heads than waves");
};

template <int D, int PS, int HW>
__global__ __launch_bounds__((PrefillCfg<D, HW>::NT), 1) void prefill_kernel(PrefillArgs a, int nqb) {
  using C = PrefillCfg<D, HW>;
  // [K buffer 0][K buffer 1][V buffer 0][V buffer 1]
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  // grid: x = (KV head, head group), y = sequence, z = query block counted
  // from the end, so the longest (latest) blocks of every sequence go first
  const int HG = a.group / HW;  // workgroups per KV head along the heads
  const int j = blockIdx.y;
  const int hk = blockIdx.x / HG;
  const int hg = blockIdx.x - hk * HG;
  const int qb = nqb - 1 - (int)blockIdx.z;

  const int q_start = a.cu_q[j];
  const int Lq = a.cu_q[j + 1] - q_start;
  int Lk = a.cu_k[j + 1] - a.cu_k[j];
  Lk = min(Lk, a.max_pages * PS);
  const int q0 = qb * C::BM;
  if (q0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query row within the wave's 32 rows
  const int hh = lane >> 5;   // k-group half
  const int hw = w % HW;
  const int head = hk * a.group + hg * HW + hw;
  const int r0 = q0 + 32 * (w / HW);  // first row of this wave
  const int qrow = r0 + col;
  const int shift = Lk - Lq;          // position of row r is shift + r
  const bool grp_b = w >= C::NW / 2;  // group B: one phase behind, stages V
  const int gw = w - (grp_b ? C::NW / 2 : 0);

  // Q rows as the B operand of S^T: lane holds q[qrow][16ks + 8hh .. +7].
  bf16x8 qop[C::KS];
  {
    const bool ok = qrow < Lq;
    const uint16_t* qp =
        a.q + ((int64_t)(q_start + (ok ? qrow : 0)) * a.num_q_heads + head) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      qop[ks] = as_bf16x8(v);
    }
  }

  // keys any row of this workgroup may see
  const int wg_last = min(q0 + C::BM, Lq) - 1;
  const int pmin = shift + q0, pmax = shift + wg_last;
  const int kstart = a.window > 0 ? max(0, pmin - a.window + 1) : 0;
  const int kend = min(pmax + 1, Lk);  // exclusive
  // this wave's rows
  const int w_last = min(r0 + 31, Lq - 1);
  const int wpmin = shift + r0, wpmax = shift + w_last;
  const int mypos = shift + qrow;
  const float c = a.scale_log2;

  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores (this lane's query row)
  float l_run = 0.f;        // this lane's partial sum of p

  // ---- staging: group A fetches K tiles, group B V tiles ----
  // Wave gw of a group fetches the WK keys t*BN + WK*gw .. +WK-1 of tile t,
  // which lie in one page: one table entry and one scalar buffer resource
  // per wave and tile, bounded to the page's keys below kend (the hardware
  // returns zeros past the bound, so keys past kend and unusable pages read
  // zeros).  Lane chunk `it` is key WK*gw + KPW*it + lane/CPR, 16-byte
  // column chunk lane%CPR; the chunks of one lane sit 1 KB apart in the page
  // (immediate offsets).
  const uint16_t* src = (grp_b ? a.v_pool : a.k_pool) + (int64_t)hk * a.head_stride;
  uint16_t* const kbuf = smem;
  uint16_t* const vbuf = smem + 2 * C::KBUF;
  const int dbuf = grp_b ? C::VBUF : C::KBUF;   // elements per buffer of own tensor
  const int dpitch = grp_b ? C::VP : C::KP;     // row pitch of own tensor
  const auto bt_rsrc = make_rsrc(a.block_tables + (int64_t)j * a.max_pages, a.max_pages * 4);
  const int lkey = lane / C::CPR;
  const int lcol = (lane % C::CPR) * 16;  // byte offset within the row
  static_assert(PS % C::WK == 0, "a wave's keys of a tile must share a page");
  // this lane's first element in its tensor's LDS buffer 0
  uint16_t* const dst = (grp_b ? vbuf : kbuf) + (C::WK * gw + lkey) * dpitch + lcol / 2;
  // Two staging sets alternate: tile s uses set (s - t_first) & 1.  A set's
  // loads are consumed two tiles after they are issued, and its table
  // entry two tiles before its loads, so no wait ever covers the loads of
  // the tile in between (memory loads complete in issue order).
  int pg[2];              // block-table entry (same in every lane)
  uint4 stage[2][C::CH];  // K or V rows on their way to LDS
  auto bt_load = [&](int t, int& pgs) {
    const int kb = t * C::BN + C::WK * gw;
    pgs = __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, kb < kend ? (kb / PS) * 4 : -1, 0, 0);
  };
  auto load_tile = [&](int t, uint4 (&stg)[C::CH], int pgs) {
    const int kb = t * C::BN + C::WK * gw;
    const int phys = __builtin_amdgcn_readfirstlane(pgs);
    const int page0 = kb - kb % PS;
    const bool ok = kb < kend && phys >= 0 && phys < a.num_pages;
    const int valid = ok ? min(kend - page0, PS) : 0;  // keys of the page below kend
    const auto r = make_rsrc(src + (ok ? (int64_t)phys * PS * D : 0), valid * D * 2);
    const int off = ((kb - page0) + lkey) * (D * 2) + lcol;
#pragma unroll
    for (int it = 0; it < C::CH; ++it) stg[it] = buffer_load16(r, off + it * C::KPW * D * 2);
  };
  auto store_tile = [&](int t, const uint4 (&stg)[C::CH]) {
    uint16_t* d = dst + (t & 1) * dbuf;
#pragma unroll
    for (int it = 0; it < C::CH; ++it) *reinterpret_cast<uint4*>(d + it * C::KPW * dpitch) = stg[it];
  };

  // transposed-read geometry (ds_read_b64_tr_b16, 16-lane groups): source
  // lane 4r+a of a group reads V[key0 + r][d0 + 4a .. +3]; output lane i of
  // the group then holds V[key0 .. key0+3][d0 + i].
  const int grp = lane >> 4, gi = lane & 15;
  const int tr_key = 4 * (grp >> 1) + (gi >> 2);       // + 16u (+8 for the second half)
  const int tr_d = 16 * (grp & 1) + 4 * (gi & 3);      // + 32dt

  // S^T of key tile t: the K operands of a 32-key tile are all read before
  // its MFMAs start
  auto qk = [&](f32x16 (&st)[C::KT], int t) {
    const uint16_t* kl = kbuf + (t & 1) * C::KBUF;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      const uint16_t* krow = kl + (32 * kt + col) * C::KP + 8 * hh;
      bf16x8 kop[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        kop[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * ks));
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) s = mfma32(kop[ks], qop[ks], s);
      st[kt] = s;
    }
  };
  // O^T += V(t)^T P^T, 16 keys per step
  auto pv = [&](const bf16x8 (&pop)[C::NU], int t) {
    const uint16_t* vl = vbuf + (t & 1) * C::VBUF;
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
      bf16x8 vop[C::DT];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint16_t* v0 = vl + (16 * u + tr_key) * C::VP + 32 * dt + tr_d;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)v0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(v0 + 8 * C::VP));
        const uint2 l2 = __builtin_bit_cast(uint2, lo);
        const uint2 h2 = __builtin_bit_cast(uint2, hi);
        vop[dt] = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[dt] = mfma32(vop[dt], pop[u], acc[dt]);
    }
  };

  // Every wave executes the same number of barriers: group B one extra
  // before its first phase, group A one extra after its last.
  if (kend > kstart) {
    const int t_first = kstart / C::BN, t_last = (kend - 1) / C::BN;
    // prologue: tile t_first of both tensors in LDS; tiles t_first+1 and
    // t_first+2 in flight; table entries of t_first+3 and t_first+4 too.
    // Loads are issued unconditionally (tiles past the end read zeros from
    // empty buffer ranges), so the number of loads in flight is the same on
    // every path and each wait covers exactly the loads it needs.
    bt_load(t_first, pg[0]);
    load_tile(t_first, stage[0], pg[0]);
    store_tile(t_first, stage[0]);
    bt_load(t_first + 1, pg[1]);
    bt_load(t_first + 2, pg[0]);
    // same issue order as a pair of steady-state tile steps
    load_tile(t_first + 1, stage[1], pg[1]);
    bt_load(t_first + 3, pg[1]);
    load_tile(t_first + 2, stage[0], pg[0]);
    bt_load(t_first + 4, pg[0]);
    __syncthreads();
    if (grp_b) __syncthreads();

    f32x16 st[C::KT];
    qk(st, t_first);
    __syncthreads();

    // one key tile: X is the staging set of tile t+1 (and t+3, t+5)
    auto tile_step = [&](int t, auto X) {
      constexpr int x = decltype(X)::value;
      // ======== V(t): staging and softmax of S(t) ========
#if PKV_PREFILL_SETPRIO
      __builtin_amdgcn_s_setprio(0);
#endif
      if (t + 1 <= t_last) store_tile(t + 1, stage[x]);  // fetched two tiles ago
      load_tile(t + 3, stage[x], pg[x]);
      bt_load(t + 5, pg[x]);
      const int k0 = t * C::BN;
      // register r of key tile kt is key k0 + 32kt + 8(r/4) + 4hh + r%4
      const bool need_mask = (k0 + C::BN - 1 > wpmin) ||
                             (a.window > 0 && wpmax - k0 >= a.window) || (k0 + C::BN > Lk);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kp = k0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = kp <= mypos && kp < Lk && (a.window <= 0 || mypos - kp < a.window);
            st[kt][r] = ok ? st[kt][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kt][r]);
      const float tmax = half_max(mx);
      // raise the running max only when this tile exceeds it by the slack
      const bool raise = (tmax - m_run) * c > kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? tmax : m_run;
        const float alpha = raise ? fast_exp2((m_run - m_new) * c) : 1.f;  // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      bf16x8 pop[C::NU];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(st[u >> 1][8 * (u & 1) + e], c, -mc));
          psum += p[e];
        }
        const bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]};
        const bf16x2 p23 = {(__bf16)p[2], (__bf16)p[3]};
        const bf16x2 p45 = {(__bf16)p[4], (__bf16)p[5]};
        const bf16x2 p67 = {(__bf16)p[6], (__bf16)p[7]};
        uint4 pp;
        pp.x = __builtin_bit_cast(uint32_t, p01);
        pp.y = __builtin_bit_cast(uint32_t, p23);
        pp.z = __builtin_bit_cast(uint32_t, p45);
        pp.w = __builtin_bit_cast(uint32_t, p67);
        pop[u] = as_bf16x8(pp);
      }
      l_run += psum;
      __syncthreads();

      // ======== M(t): O += V(t) P(t), S(t+1) = K(t+1) Q^T ========
#if PKV_PREFILL_SETPRIO
      __builtin_amdgcn_s_setprio(1);
#endif
      pv(pop, t);
      if (t + 1 <= t_last) qk(st, t + 1);
      __syncthreads();
    };
    // pairs of steps with no branch between them, so the loads in flight at
    // the loop head are the same on every path
    int t = t_first;
    for (; t + 1 <= t_last; t += 2) {
      tile_step(t, std::integral_constant<int, 1>{});
      tile_step(t + 1, std::integral_constant<int, 0>{});
    }
    if (t <= t_last) tile_step(t, std::integral_constant<int, 1>{});
#if PKV_PREFILL_SETPRIO
    __builtin_amdgcn_s_setprio(0);
#endif
    if (!grp_b) __syncthreads();
  }

  // ---- normalise and write: lane holds d = 32dt + 8(r/4) + 4hh + r%4 ----
  const float lt = half_sum(l_run);
  if (qrow < Lq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = a.out + ((int64_t)(q_start + qrow) * a.num_q_heads + head) * D + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[dt][4 * rb] * inv, acc[dt][4 * rb + 1] * inv);
        pk.y = pack_bf16x2(acc[dt][4 * rb + 2] * inv, acc[dt][4 * rb + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * rb) = pk;
      }
  }
}

template <int D, int PS, int HW>
hipError_t launch_p3(const PrefillArgs& a, int num_seqs, int max_q, hipStream_t st) {
  using C = PrefillCfg<D, HW>;
  const int nqb = (max_q + C::BM - 1) / C::BM;
  dim3 grid(a.num_kv_heads * (a.group / HW), num_seqs, nqb);
  const size_t smem = C::LDS_BYTES;
  static bool attr_set = false;  // raise the dynamic LDS limit once (above 64 KB)
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_kernel<D, PS, HW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((prefill_kernel<D, PS, HW>), grid, dim3(C::NT), smem, st, a, nqb);
  return hipGetLastError();
}

template <int D, int PS>
hipError_t launch_p2(const PrefillArgs& a, int num_seqs, int max_q, hipStream_t st) {
  constexpr int NW = PrefillCfg<D, 1>::NW;
  if constexpr (NW >= 8) {
    if (a.group % 8 == 0) return launch_p3<D, PS, 8>(a, num_seqs, max_q, st);
  }
  if (a.group % 4 == 0) return launch_p3<D, PS, 4>(a, num_seqs, max_q, st);
  if (a.group % 2 == 0) return launch_p3<D, PS, 2>(a, num_seqs, max_q, st);
  return launch_p3<D, PS, 1>(a, num_seqs, max_q, st);
}

template <int D>
hipError_t launch_p1(const PrefillArgs& a, int num_seqs, int max_q, int ps, hipStream_t st) {
  return ps == 16 ? launch_p2<D, 16>(a, num_seqs, max_q, st) : launch_p2<D, 32>(a, num_seqs, max_q, st);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int num_seqs, int max_seqlen_q, int head_dim,
                          int page_size, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_p1<64>(a, num_seqs, max_seqlen_q, page_size, st);
    case 128: return launch_p1<128>(a, num_seqs, max_seqlen_q, page_size, st);
    default: return launch_p1<256>(a, num_seqs, max_seqlen_q, page_size, st);
  }
}

}  // namespace pkv
