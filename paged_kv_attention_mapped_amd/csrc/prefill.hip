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
// Work decomposition.  A workgroup owns up to 128 query rows of one
// sequence for up to four query heads of one KV group; its waves each own
// 32 rows of one head.  K/V tiles of 64 keys are gathered page by page
// into LDS once per workgroup and shared by all its heads.
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16: A = K rows straight from LDS,
//                B = Q rows held in registers; the result keeps one query
//                row per lane column, so the softmax row statistics are
//                lane-local plus one exchange with the lane 32 away.
//   O^T += V^T P^T: the probabilities already sit in B-operand order in the
//                score registers (only rounded to bf16); V is stored
//                transposed in LDS while it is being staged.
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

template <int D, int HW>
struct PrefillCfg {
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int QB = NW / HW;           // 32-row query blocks per workgroup
  static constexpr int BM = 32 * QB;           // query rows per workgroup
  static constexpr int BN = 64;                // keys per tile
  static constexpr int KPAD = D + 8;           // LDS row stride of K (elements)
  static constexpr int VPAD = BN + 4;          // LDS row stride of V^T (elements)
  static constexpr int KS = D / 16;            // k-steps of S^T
  static constexpr int DT = D / 32;            // 32-row tiles of O^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per token row
  static constexpr int KCH = BN * CPR / 256;   // K chunks per thread per tile
  static constexpr int VTASK = (BN / 4) * CPR; // (4 keys x 1 chunk) V tasks per tile
  static constexpr int VPT = (VTASK + 255) / 256;
};

template <int D, int PS, int HW>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a, int nqb) {
  using C = PrefillCfg<D, HW>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[C::BN * C::KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * C::VPAD];

  const int HG = a.group / HW;  // workgroups per KV head along the heads
  const int j = blockIdx.z;
  const int hk = blockIdx.y / HG;
  const int hg = blockIdx.y - hk * HG;
  const int qb = nqb - 1 - (int)blockIdx.x;  // late (long) query blocks first

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
    const uint16_t* qp = a.q + ((int64_t)(q_start + (ok ? qrow : 0)) * a.num_q_heads + head) * D + 8 * hh;
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

  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride;
  const int32_t* bt_row = a.block_tables + (int64_t)j * a.max_pages;

  uint4 kreg[C::KCH];
  uint4 vreg[C::VPT][4];

  auto row_addr = [&](int kpos, int64_t& off) -> bool {
    if (kpos >= kend) return false;
    const int phys = bt_row[kpos / PS];
    if (phys < 0 || phys >= a.num_pages) return false;
    off = ((int64_t)phys * PS + (kpos % PS)) * D;
    return true;
  };
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int ci = tid + 256 * it;
      const int key = ci / C::CPR, c = ci - key * C::CPR;
      int64_t off;
      kreg[it] = row_addr(k0 + key, off) ? *reinterpret_cast<const uint4*>(kh + off + 8 * c)
                                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int vt = tid + 256 * it;
      const int kg = vt / C::CPR, c = vt - kg * C::CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t off;
        vreg[it][i] = (vt < C::VTASK && row_addr(k0 + 4 * kg + i, off))
                          ? *reinterpret_cast<const uint4*>(vh + off + 8 * c)
                          : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int ci = tid + 256 * it;
      const int key = ci / C::CPR, c = ci - key * C::CPR;
      *reinterpret_cast<uint4*>(&k_lds[key * C::KPAD + 8 * c]) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int vt = tid + 256 * it;
      if (vt >= C::VTASK) continue;
      const int kg = vt / C::CPR, c = vt - kg * C::CPR;
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[it][0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[it][1]);
      const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vreg[it][2]);
      const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vreg[it][3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint2 t;
        if (e & 1) {
          t.x = (v0[wd] >> 16) | (v1[wd] & 0xffff0000u);
          t.y = (v2[wd] >> 16) | (v3[wd] & 0xffff0000u);
        } else {
          t.x = (v0[wd] & 0xffffu) | (v1[wd] << 16);
          t.y = (v2[wd] & 0xffffu) | (v3[wd] << 16);
        }
        *reinterpret_cast<uint2*>(&vt_lds[(8 * c + e) * C::VPAD + 4 * kg]) = t;
      }
    }
  };

  if (kend > kstart) {
    const int t_first = kstart / C::BN, t_last = (kend - 1) / C::BN;
    load_tile(t_first * C::BN);
    for (int t = t_first; t <= t_last; ++t) {
      const int k0 = t * C::BN;
      __syncthreads();
      store_tile();
      __syncthreads();
      if (t < t_last) load_tile(k0 + C::BN);

      // ---- S^T = K Q^T for 64 keys x 32 rows ----
      f32x16 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
        const uint16_t* krow = &k_lds[(32 * kt + col) * C::KPAD + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const uint4 kv = *reinterpret_cast<const uint4*>(krow + 16 * ks);
          st[kt] = mfma32(as_bf16x8(kv), qop[ks], st[kt]);
        }
      }
      // register r of tile kt is key k0 + 32kt + 8(r/4) + 4hh + r%4
      float x[2][16];
      const bool need_mask = (k0 + C::BN - 1 > wpmin) ||
                             (a.window > 0 && wpmax - k0 >= a.window) || (k0 + C::BN > Lk);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = st[kt][r] * a.scale_log2;
          if (need_mask) {
            const int kp = k0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = kp <= mypos && kp < Lk && (a.window <= 0 || mypos - kp < a.window);
            v = ok ? v : -INFINITY;
          }
          x[kt][r] = v;
        }
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, x[kt][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[kt][r] = fast_exp2(x[kt][r] - m_use);
          psum += x[kt][r];
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

      // ---- O^T += V^T P^T, 16 keys per step ----
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pu = &x[u >> 1][8 * (u & 1)];
        uint4 pp;
        pp.x = pack_bf16x2(pu[0], pu[1]);
        pp.y = pack_bf16x2(pu[2], pu[3]);
        pp.z = pack_bf16x2(pu[4], pu[5]);
        pp.w = pack_bf16x2(pu[6], pu[7]);
        const bf16x8 pop = as_bf16x8(pp);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const uint16_t* vrow = &vt_lds[(32 * dt + col) * C::VPAD + 16 * u + 4 * hh];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
          acc[dt] = mfma32(as_bf16x8(vv), pop, acc[dt]);
        }
      }
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
  dim3 grid(nqb, a.num_kv_heads * (a.group / HW), num_seqs);
  hipLaunchKernelGGL((prefill_kernel<D, PS, HW>), grid, dim3(256), 0, st, a, nqb);
  return hipGetLastError();
}

template <int D, int PS>
hipError_t launch_p2(const PrefillArgs& a, int num_seqs, int max_q, hipStream_t st) {
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
