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
// Work decomposition.  A workgroup of eight waves owns up to 32*QB query
// rows of one sequence for HW query heads of one KV group (HW*QB = 8); each
// wave owns 32 rows of one head.  K/V tiles of BN keys are gathered page by
// page into LDS once per workgroup (three buffers) and shared by all its
// heads and rows.  The key loop is software-pipelined: while the vector
// ALUs turn tile t's scores into probabilities, the matrix cores already
// compute tile t+1's scores, and tile t+3's global loads are in flight;
// one barrier per tile.
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
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kRescaleSlack = 8.0f;

// Tuning knobs (fixed at build time): waves per workgroup for D <= 128 and
// keys per tile.
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

template <int D, int HW>
struct PrefillCfg {
  static constexpr int NW = D == 256 ? 4 : PKV_PREFILL_WAVES;  // waves per workgroup
  static constexpr int NT = NW * 64;           // threads
  static constexpr int QB = NW / HW;           // 32-row query blocks per workgroup
  static constexpr int BM = 32 * QB;           // query rows per workgroup
  static constexpr int BN = D == 256 ? 32 : PKV_PREFILL_KEYS;  // keys per tile
  static constexpr int KT = BN / 32;           // 32-key tiles of S^T
  static constexpr int KP = D + PKV_PREFILL_KPAD;  // LDS row pitch of K (elements)
  static constexpr int VP = D + PKV_PREFILL_VPAD;  // LDS row pitch of V (elements)
  static constexpr int KS = D / 16;            // k-steps of S^T
  static constexpr int DT = D / 32;            // 32-row tiles of O^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per token row
  static constexpr int CH = BN * CPR / NT;     // K (and V) chunks per thread per tile
  static constexpr int TILE = BN * KP + BN * VP;  // elements of one LDS buffer
  static_assert(CH >= 1 && BN * CPR % NT == 0, "tile chunks must split evenly");
  static_assert(QB >= 1, "more heads than waves");
};

template <int D, int PS, int HW>
__global__ __launch_bounds__((PrefillCfg<D, HW>::NT), 1) void prefill_kernel(PrefillArgs a, int nqb) {
  using C = PrefillCfg<D, HW>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // 3 x (K tile, V tile)

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

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31;  // query row within the wave's block
  const int hh = lane >> 5;   // k-group half
  const int hw = w % HW;
  const int head = hk * a.group + hg * HW + hw;
  const int r0 = q0 + 32 * (w / HW);
  const int qrow = r0 + col;
  const int shift = Lk - Lq;  // position of row r is shift + r

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

  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride;
  const int32_t* bt_row = a.block_tables + (int64_t)j * a.max_pages;

  uint4 kreg[C::CH], vreg[C::CH];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < C::CH; ++it) {
      const int ci = tid + C::NT * it;
      const int key = ci / C::CPR, cc = ci - key * C::CPR;
      const int kpos = k0 + key;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kpos < kend) {
        const int phys = bt_row[kpos / PS];
        if (phys >= 0 && phys < a.num_pages) {
          const int64_t off = ((int64_t)phys * PS + (kpos % PS)) * D + 8 * cc;
          kv = *reinterpret_cast<const uint4*>(kh + off);
          vv = *reinterpret_cast<const uint4*>(vh + off);
        }
      }
      kreg[it] = kv;
      vreg[it] = vv;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kl = smem + buf * C::TILE;
    uint16_t* vl = kl + C::BN * C::KP;
#pragma unroll
    for (int it = 0; it < C::CH; ++it) {
      const int ci = tid + C::NT * it;
      const int key = ci / C::CPR, cc = ci - key * C::CPR;
      *reinterpret_cast<uint4*>(kl + key * C::KP + 8 * cc) = kreg[it];
      *reinterpret_cast<uint4*>(vl + key * C::VP + 8 * cc) = vreg[it];
    }
  };

  // transposed-read geometry (ds_read_b64_tr_b16, 16-lane groups): source
  // lane 4r+a of a group reads V[key0 + r][d0 + 4a .. +3]; output lane i of
  // the group then holds V[key0 .. key0+3][d0 + i].
  const int grp = lane >> 4, gi = lane & 15;
  const int tr_key = 4 * (grp >> 1) + (gi >> 2);       // + 16u (+8 for the second half)
  const int tr_d = 16 * (grp & 1) + 4 * (gi & 3);      // + 32dt

  // S^T tile of keys k0.. from the LDS buffer of that tile
  auto qk = [&](f32x16* st, int buf) {
    const uint16_t* kl = smem + buf * C::TILE;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      const uint16_t* krow = kl + (32 * kt + col) * C::KP + 8 * hh;
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + 16 * ks);
        s = mfma32(as_bf16x8(kv), qop[ks], s);
      }
      st[kt] = s;
    }
  };

  if (kend > kstart) {
    // Pipeline over key tiles t (three LDS buffers, tile t in buffer t % 3):
    //   iteration t: store tile t+2 (fetched during iteration t-1) into the
    //   buffer tile t-1 used, issue the global loads of tile t+3; S(t+1) =
    //   K(t+1) Q^T on the matrix cores while the vector ALUs turn S(t) into
    //   probabilities; O += V(t) P(t); one barrier.
    const int t_first = kstart / C::BN, t_last = (kend - 1) / C::BN;
    auto bufof = [&](int t) { return (t - t_first) % 3; };
    load_tile(t_first * C::BN);
    store_tile(0);
    if (t_first + 1 <= t_last) {
      load_tile((t_first + 1) * C::BN);
      store_tile(1);
    }
    __syncthreads();
    if (t_first + 2 <= t_last) load_tile((t_first + 2) * C::BN);
    f32x16 st[C::KT], sn[C::KT];
    qk(st, 0);
    for (int t = t_first; t <= t_last; ++t) {
      const int k0 = t * C::BN;
      if (t + 2 <= t_last) store_tile(bufof(t + 2));  // loads issued one iteration ago
      if (t + 3 <= t_last) load_tile((t + 3) * C::BN);  // in flight for a whole iteration

      // register r of tile kt is key k0 + 32kt + 8(r/4) + 4hh + r%4
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
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[kt][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
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

      // next tile's scores on the matrix cores, this tile's probabilities on
      // the VALU (unconditional, so both sit in one block the scheduler can
      // interleave; after the last tile the result is simply unused)
      qk(sn, bufof(t + 1));
      float psum = 0.f;
      bf16x8 pop[C::BN / 16];
#pragma unroll
      for (int u = 0; u < C::BN / 16; ++u) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(st[u >> 1][8 * (u & 1) + e], c, -mc));
          psum += p[e];
        }
        bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]};
        bf16x2 p23 = {(__bf16)p[2], (__bf16)p[3]};
        bf16x2 p45 = {(__bf16)p[4], (__bf16)p[5]};
        bf16x2 p67 = {(__bf16)p[6], (__bf16)p[7]};
        uint4 pp;
        pp.x = __builtin_bit_cast(uint32_t, p01);
        pp.y = __builtin_bit_cast(uint32_t, p23);
        pp.z = __builtin_bit_cast(uint32_t, p45);
        pp.w = __builtin_bit_cast(uint32_t, p67);
        pop[u] = as_bf16x8(pp);
      }
      l_run += psum;

      // ---- O^T += V^T P^T, 16 keys per step ----
      const uint16_t* vl = smem + bufof(t) * C::TILE + C::BN * C::KP;
#pragma unroll
      for (int u = 0; u < C::BN / 16; ++u) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const uint16_t* v0 = vl + (16 * u + tr_key) * C::VP + 32 * dt + tr_d;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)v0);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(v0 + 8 * C::VP));
          const uint2 l2 = __builtin_bit_cast(uint2, lo);
          const uint2 h2 = __builtin_bit_cast(uint2, hi);
          const uint4 vv = make_uint4(l2.x, l2.y, h2.x, h2.y);
          acc[dt] = mfma32(as_bf16x8(vv), pop[u], acc[dt]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) st[kt] = sn[kt];
    }
  }

  // ---- normalise and write: lane holds d = 32dt + 8(r/4) + 4hh + r%4 ----
  const float lt = l_run + __shfl_xor(l_run, 32);
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
  const size_t smem = 3 * (size_t)C::TILE * sizeof(uint16_t);
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
  if constexpr (D != 256 && PKV_PREFILL_WAVES >= 8) {
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
