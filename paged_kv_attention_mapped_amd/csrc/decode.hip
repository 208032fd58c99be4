// GQA decode attention over the paged pool, with split-K partitions and a
// combine kernel.
//
// One query row per sequence attends its cached keys through the block
// table (scripts/benchmarks commit log 1847125, flex_attention paged-KV
// engine entry, "Why this works" items 1-2); the sliding regime adds
// q_pos - kv_pos < window (same log, per-regime mask entry).
//
// Work decomposition.  A workgroup owns one (sequence, KV head, split): the
// whole query-head group shares every K/V page it streams, so each page is
// read from HBM once per group.  Its four waves take the split's pages
// round-robin.  Per page a wave
//   * loads K in the A-operand layout of v_mfma_f32_16x16x32_bf16 (rows =
//     16 tokens, k = 32 head-dim elements) and computes the scores of all
//     query heads of the group at once (columns = heads);
//   * loads V row-major, 16 lanes per token (16 B per lane for D=128), so
//     every load instruction reads whole contiguous token rows;
//   * keeps an online softmax per (16-lane row, head): the A rows are
//     permuted so that lane row j of the score tile holds exactly the tokens
//     j, j+4, j+8, ... whose V rows lane row j loaded, and each lane gets
//     its probabilities from lane h of its own row with a DPP broadcast.
// K needs no transpose (the contraction runs over head_dim, its contiguous
// axis); V would, so PV runs on the vector ALUs in fp32.
#include <limits.h>
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

// Tuning knobs (fixed at build time): tokens processed per step of a wave
// (a whole page or half of one), register buffers per wave (1, or 2 to keep
// the next step's loads in flight while the current one is processed),
// waves per workgroup and the occupancy the register budget is sized for.
#ifndef PKV_DECODE_UNIT
#define PKV_DECODE_UNIT 16
#endif
#ifndef PKV_DECODE_BUFFERS
#define PKV_DECODE_BUFFERS 2
#endif
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
#ifndef PKV_DECODE_OCCUPANCY
#define PKV_DECODE_OCCUPANCY 2
#endif

template <int D, int PS, int G>
struct DecodeCfg {
  static constexpr int NW = PKV_DECODE_WAVES;  // waves per workgroup
  static constexpr int UT = PKV_DECODE_UNIT < PS ? PKV_DECODE_UNIT : PS;  // tokens per step
  static constexpr int UPP = PS / UT;          // steps per page
  static constexpr int EPL = D / 16;           // head-dim elements per lane (PV side)
  static constexpr int CH = EPL < 8 ? EPL : 8; // elements per V load (8 B or 16 B)
  static constexpr int NCH = EPL / CH;         // V loads per token per lane
  static constexpr int KT = UT / 16;           // 16-token MFMA tiles per step
  static constexpr int KB = D / 32;            // MFMA k-steps over head_dim
  static constexpr int TPR = UT / 4;           // tokens per lane row per step
  static constexpr int OCC = D == 256 ? 1 : PKV_DECODE_OCCUPANCY;
  static_assert(G <= 16, "group larger than one MFMA column tile");
  static_assert(UT % 16 == 0 && PS % UT == 0, "step must be whole MFMA tiles of a page");
};

template <int CH>
struct VChunkT;
template <>
struct VChunkT<8> { using type = uint4; };
template <>
struct VChunkT<4> { using type = uint2; };

__device__ __forceinline__ void unpack(const uint4& v, float* f) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ void unpack(const uint2& v, float* f) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
}

template <int D, int PS, int G, bool SPLIT>
__global__ __launch_bounds__(PKV_DECODE_WAVES * 64, (DecodeCfg<D, PS, G>::OCC))
void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<D, PS, G>;
  using VChunk = typename VChunkT<C::CH>::type;
  __shared__ float sm_m[C::NW][G];
  __shared__ float sm_l[C::NW][G];
  __shared__ float sm_acc[C::NW][G][D];

  const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int jj = lane >> 4;  // lane row
  const int n = lane & 15;   // column within the row (= head slot on the score side)
  const int g = a.group;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * PS));
  const int first_key = a.window > 0 ? max(0, L - a.window) : 0;
  const int p0 = first_key / PS;
  const int pend = (L + PS - 1) / PS;
  const int pa = min(pend, p0 + s * a.pages_per_split);
  const int pb = min(pend, pa + a.pages_per_split);

  // Q^T as the B operand: lane (jj, n) holds q[head n][32kb + 8jj .. +7].
  bf16x8 qop[C::KB];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.num_q_heads + hk * g + n) * D + 8 * jj;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < g) v = *reinterpret_cast<const uint4*>(qrow + 32 * kb);
      qop[kb] = as_bf16x8(v);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  float acc[G][C::EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) acc[h][e] = 0.f;

  const uint16_t* kh_base = a.k_pool + (int64_t)hk * a.head_stride;
  const uint16_t* vh_base = a.v_pool + (int64_t)hk * a.head_stride;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.max_pages;
  // A-operand row n holds token 4*(n%4) + n/4 of each 16-token tile, so score
  // register r of lane row jj is token 4r + jj.
  const int tok_a = 4 * (n & 3) + (n >> 2);

  // This wave's pages are pa + w, pa + w + NW, ...; their table entries are
  // fetched 64 at a time (one per lane) and read back with readlane, so no
  // page load waits on a table load.
  const int npw = pb - pa > w ? (pb - pa - w + C::NW - 1) / C::NW : 0;
  const int nsteps = npw * C::UPP;
  int phys_lane = 0;

  struct Buf {
    uint4 k[C::KT][C::KB];
    VChunk v[C::TPR][C::NCH];
    int tok0;
    bool valid;
  };
  auto load = [&](Buf& bf, int j) {
    const int i = j / C::UPP;            // page of this wave
    const int half = j - i * C::UPP;     // step within the page
    if ((i & 63) == 0 && half == 0) {
      const int pl = pa + w + C::NW * (i + lane);
      phys_lane = (i + lane < npw) ? bt_row[pl] : -1;
    }
    int phys = __builtin_amdgcn_readlane(phys_lane, i & 63);
    bf.valid = phys >= 0 && phys < a.num_pages;
    phys = bf.valid ? phys : 0;  // an unusable entry reads page 0 and is masked out
    bf.tok0 = (pa + w + C::NW * i) * PS + half * C::UT;
    const int64_t row0 = (int64_t)phys * PS + half * C::UT;
    const auto kr = make_rsrc(kh_base + row0 * D, C::UT * D * 2);
    const auto vr = make_rsrc(vh_base + row0 * D, C::UT * D * 2);
#pragma unroll
    for (int ti = 0; ti < C::KT; ++ti)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        bf.k[ti][kb] = buffer_load16(kr, 2 * ((ti * 16 + tok_a) * D + 32 * kb + 8 * jj));
#pragma unroll
    for (int i2 = 0; i2 < C::TPR; ++i2)
#pragma unroll
      for (int ch = 0; ch < C::NCH; ++ch)
        buffer_load(bf.v[i2][ch], vr, 2 * ((4 * i2 + jj) * D + C::CH * n + 16 * C::CH * ch));
  };
  auto process = [&](const Buf& bf) {
    // scores, in log2 units: x[i] belongs to token 4i + jj of the step
    float x[C::TPR];
#pragma unroll
    for (int ti = 0; ti < C::KT; ++ti) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) c = mfma16(as_bf16x8(bf.k[ti][kb]), qop[kb], c);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * ti + r] = c[r] * a.scale_log2;
    }
    // rows outside [first_key, L) (tail, window start, unusable page) are
    // selected away: their scores become -inf and their V rows 0
    const int lo = bf.valid ? first_key : INT_MAX;
    const bool partial = (bf.tok0 < lo) || (bf.tok0 + C::UT > L);
    uint32_t keep = 0xffffffffu;
    if (partial) {
      keep = 0;
#pragma unroll
      for (int i = 0; i < C::TPR; ++i) {
        const int t = bf.tok0 + 4 * i + jj;
        const bool ok = t >= lo && t < L;
        keep |= (ok ? 1u : 0u) << i;
        x[i] = ok ? x[i] : -INFINITY;
      }
    }
    float pmax = x[0];
#pragma unroll
    for (int i = 1; i < C::TPR; ++i) pmax = fmaxf(pmax, x[i]);
    const float m_new = fmaxf(m_run, pmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < C::TPR; ++i) {
      x[i] = fast_exp2(x[i] - m_use);
      psum += x[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    static_for<0, G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ah = row_bcast<h>(alpha);
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) acc[h][e] *= ah;
    });
#pragma unroll
    for (int i = 0; i < C::TPR; ++i) {
      float vf[C::EPL];
#pragma unroll
      for (int ch = 0; ch < C::NCH; ++ch) unpack(bf.v[i][ch], vf + ch * C::CH);
      if (partial) {
        const bool ok = (keep >> i) & 1u;
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
      static_for<0, G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float ph = row_bcast<h>(x[i]);
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      });
    }
  };

  if constexpr (PKV_DECODE_BUFFERS >= 2) {
    // ping-pong: step j+1 is in flight while step j is processed
    Buf b0, b1;
    if (nsteps > 0) load(b0, 0);
    for (int j = 0; j < nsteps; j += 2) {
      if (j + 1 < nsteps) load(b1, j + 1);
      process(b0);
      if (j + 1 >= nsteps) break;
      if (j + 2 < nsteps) load(b0, j + 2);
      process(b1);
    }
  } else {
    for (int j = 0; j < nsteps; ++j) {
      Buf b0;
      load(b0, j);
      process(b0);
    }
  }

  // ---- merge the four lane rows of this wave ----------------------------
  float M = m_run;
  M = fmaxf(M, __shfl_xor(M, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  const float f = (M == -INFINITY) ? 0.f : fast_exp2(m_run - M);
  float lw = l_run * f;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  static_for<0, G>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    const float fh = row_bcast<h>(f);
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) {
      float v = acc[h][e] * fh;
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[h][e] = v;
    }
  });
  if (jj == 0) {
    if (n < G) {
      sm_m[w][n] = M;
      sm_l[w][n] = lw;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < C::EPL; ++e)
        sm_acc[w][h][C::CH * n + (e % C::CH) + 16 * C::CH * (e / C::CH)] = acc[h][e];
  }
  __syncthreads();

  // ---- merge the waves and write ----------------------------------------
  for (int idx = tid; idx < g * D; idx += 64 * C::NW) {
    const int h = idx / D, d = idx - h * D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < C::NW; ++ww) Mx = fmaxf(Mx, sm_m[ww][h]);
    float o = 0.f, lsum = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < C::NW; ++ww) {
        const float mw = sm_m[ww][h];
        if (mw == -INFINITY) continue;
        const float wt = fast_exp2(mw - Mx);
        o = fmaf(wt, sm_acc[ww][h][d], o);
        lsum = fmaf(wt, sm_l[ww][h], lsum);
      }
    }
    const int64_t row = (int64_t)b * a.num_q_heads + hk * g + h;
    if constexpr (SPLIT) {
      const int64_t cell = row * a.num_splits + s;
      a.part_acc[cell * D + d] = o;
      if (d == 0) {
        a.part_m[cell] = Mx;
        a.part_l[cell] = lsum;
      }
    } else {
      const float val = lsum > 0.f ? o / lsum : 0.f;
      a.out[row * D + d] = (uint16_t)f32_to_bf16(val);
    }
  }
}

// Combine: one thread per 4 head-dim elements of a (sequence, head) row;
// splits are merged in index order, so the result does not depend on timing.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ m,
                                                      const float* __restrict__ l,
                                                      const float* __restrict__ acc, int rows,
                                                      int S, uint16_t* __restrict__ out) {
  constexpr int TPRW = D / 4;
  constexpr int RPB = 256 / TPRW;
  const int row = blockIdx.x * RPB + threadIdx.x / TPRW;
  const int d0 = (threadIdx.x % TPRW) * 4;
  if (row >= rows) return;
  const float* mr = m + (int64_t)row * S;
  const float* lr = l + (int64_t)row * S;
  float Mx = -INFINITY;
  for (int s = 0; s < S; ++s) Mx = fmaxf(Mx, mr[s]);
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f, lsum = 0.f;
  if (Mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = mr[s];
      if (ms == -INFINITY) continue;
      const float wt = fast_exp2(ms - Mx);
      lsum = fmaf(wt, lr[s], lsum);
      const float4 av = *reinterpret_cast<const float4*>(acc + ((int64_t)row * S + s) * D + d0);
      o0 = fmaf(wt, av.x, o0);
      o1 = fmaf(wt, av.y, o1);
      o2 = fmaf(wt, av.z, o2);
      o3 = fmaf(wt, av.w, o3);
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint2 pk;
  pk.x = pack_bf16x2(o0 * inv, o1 * inv);
  pk.y = pack_bf16x2(o2 * inv, o3 * inv);
  *reinterpret_cast<uint2*>(out + (int64_t)row * D + d0) = pk;
}

template <int D, int PS, int G>
hipError_t launch_dpg(const DecodeArgs& a, int num_seqs, bool split, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_kv_heads, num_seqs);
  if (split)
    hipLaunchKernelGGL((decode_kernel<D, PS, G, true>), grid, dim3(64 * PKV_DECODE_WAVES), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, PS, G, false>), grid, dim3(64 * PKV_DECODE_WAVES), 0, st, a);
  return hipGetLastError();
}

template <int D, int PS>
hipError_t launch_dp(const DecodeArgs& a, int num_seqs, bool split, hipStream_t st) {
  if (a.group <= 2) return launch_dpg<D, PS, 2>(a, num_seqs, split, st);
  if (a.group <= 4) return launch_dpg<D, PS, 4>(a, num_seqs, split, st);
  return launch_dpg<D, PS, 8>(a, num_seqs, split, st);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int num_seqs, int ps, bool split, hipStream_t st) {
  return ps == 16 ? launch_dp<D, 16>(a, num_seqs, split, st)
                  : launch_dp<D, 32>(a, num_seqs, split, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int num_seqs, int head_dim, int page_size,
                         bool split, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_d<64>(a, num_seqs, page_size, split, st);
    case 128: return launch_d<128>(a, num_seqs, page_size, split, st);
    default: return launch_d<256>(a, num_seqs, page_size, split, st);
  }
}

hipError_t launch_combine(const float* m, const float* l, const float* acc, int num_seqs, int hq,
                          int d, int splits, uint16_t* out, hipStream_t st) {
  const int rows = num_seqs * hq;
  const int rpb = 256 / (d / 4);
  dim3 grid((rows + rpb - 1) / rpb);
  switch (d) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, st, m, l, acc, rows, splits, out); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, st, m, l, acc, rows, splits, out); break;
    default: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(256), 0, st, m, l, acc, rows, splits, out); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
