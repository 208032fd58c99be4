// The per-wave decode machinery of the stream-K decode kernel (WaveDecoder)
// and of the direct decode kernel and the varlen kernel's one-row sequences
// (RowDecoder, at the end): one wave attends the query-head group of one KV
// head over a run of page steps and keeps an online softmax in registers.
//
// Layout of the work inside a wave.  A step is UT tokens of one page.
//   * K is loaded in the A-operand layout of v_mfma_f32_16x16x32_bf16
//     (rows = 16 tokens, k = 32 head-dim elements), and the scores of all
//     query heads of the group come out of one MFMA per 32 head-dim
//     elements (columns = heads).  K needs no transpose: the contraction
//     runs over head_dim, its contiguous axis.
//   * V is loaded row-major, 16 lanes per token row (16 B per lane for
//     D=128), so every load instruction reads whole contiguous rows.
//   * The A rows are permuted so that lane row j (lanes 16j..16j+15) of the
//     score tile holds tokens j, j+4, j+8, ... of the step -- exactly the
//     tokens whose V rows lane row j loaded.  Each lane row therefore runs
//     its own online softmax per head, lane-locally, and a lane gets the
//     probability of head h from lane h of its own row with a DPP
//     row_newbcast.  PV accumulates in fp32 on the vector ALUs.
//   * Rows outside [first_key, L) (sequence tail, window start, unusable
//     page) are selected away -- score -inf, V row 0 -- so stale data in a
//     page (NaN in tests) never reaches the result.
#pragma once

#include <limits.h>
#include <math.h>

#include "common.h"
#include "prefill_common.h"

namespace pkv {

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

template <int D, int PS, int G, int UT_>
struct WaveDecoder {
  static constexpr int UT = UT_ < PS ? UT_ : PS;  // tokens per step
  static constexpr int UPP = PS / UT;             // steps per page
  static constexpr int EPL = D / 16;              // head-dim elements per lane (PV side)
  static constexpr int CH = EPL < 8 ? EPL : 8;    // elements per V load (8 B or 16 B)
  static constexpr int NCH = EPL / CH;            // V loads per token per lane
  static constexpr int KT = UT / 16;              // 16-token MFMA tiles per step
  static constexpr int KB = D / 32;               // MFMA k-steps over head_dim
  static constexpr int TPR = UT / 4;              // tokens per lane row per step
  static_assert(G <= 16, "group larger than one MFMA column tile");
  static_assert(UT % 16 == 0 && PS % UT == 0, "a step is whole MFMA tiles of a page");
  using VChunk = typename VChunkT<CH>::type;

  struct Buf {
    uint4 k[KT][KB];
    VChunk v[TPR][NCH];
  };
  int jj, n, tok_a;
  float m_run, l_run;
  float acc[G][EPL];
  bf16x8 qop[KB];

  __device__ __forceinline__ void init(int lane) {
    jj = lane >> 4;
    n = lane & 15;
    // A-operand row n holds token 4*(n%4) + n/4 of each 16-token tile, so
    // score register r of lane row jj is token 4r + jj.
    tok_a = 4 * (n & 3) + (n >> 2);
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // Q^T as the B operand: lane (jj, n) holds q[head n][32kb + 8jj .. +7];
  // qg points at the group's first query head, heads >= g read as zero.
  __device__ __forceinline__ void load_q(const uint16_t* qg, int g) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < g) v = *reinterpret_cast<const uint4*>(qg + n * D + 32 * kb + 8 * jj);
      qop[kb] = as_bf16x8(v);
    }
  }

  // Issue the loads of one step; krow/vrow point at the step's first token
  // row.  A step past the end (live false) issues the same loads through an
  // empty range: they return zeros and read no memory, so that a loop can
  // request its next step unconditionally and the compiler's wait before a
  // step covers that step's loads only, not the next step's.
  __device__ __forceinline__ void load(Buf& bf, const uint16_t* krow, const uint16_t* vrow,
                                       bool live = true) const {
    const auto kr = make_rsrc(krow, live ? UT * D * 2 : 0);
    const auto vr = make_rsrc(vrow, live ? UT * D * 2 : 0);
#pragma unroll
    for (int ti = 0; ti < KT; ++ti)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bf.k[ti][kb] = buffer_load16(kr, 2 * ((ti * 16 + tok_a) * D + 32 * kb + 8 * jj));
#pragma unroll
    for (int i = 0; i < TPR; ++i)
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
        buffer_load(bf.v[i][ch], vr, 2 * ((4 * i + jj) * D + CH * n + 16 * CH * ch));
  }

  // Fold one step into the running state.  Tokens tok0 .. tok0+UT-1 of the
  // sequence; the ones outside [lo, hi) are masked.
  __device__ __forceinline__ void process(const Buf& bf, int tok0, int lo, int hi,
                                          float scale_log2) {
    float x[TPR];
#pragma unroll
    for (int ti = 0; ti < KT; ++ti) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) c = mfma16(as_bf16x8(bf.k[ti][kb]), qop[kb], c);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * ti + r] = c[r] * scale_log2;
    }
    const bool partial = (tok0 < lo) || (tok0 + UT > hi);
    uint32_t keep = 0xffffffffu;
    if (partial) {
      keep = 0;
#pragma unroll
      for (int i = 0; i < TPR; ++i) {
        const int t = tok0 + 4 * i + jj;
        const bool ok = t >= lo && t < hi;
        keep |= (ok ? 1u : 0u) << i;
        x[i] = ok ? x[i] : -INFINITY;
      }
    }
    float pmax = x[0];
#pragma unroll
    for (int i = 1; i < TPR; ++i) pmax = fmaxf(pmax, x[i]);
    const float m_new = fmaxf(m_run, pmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < TPR; ++i) {
      x[i] = fast_exp2(x[i] - m_use);
      psum += x[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    static_for<0, G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ah = row_bcast<h>(alpha);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= ah;
    });
#pragma unroll
    for (int i = 0; i < TPR; ++i) {
      float vf[EPL];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) unpack(bf.v[i][ch], vf + ch * CH);
      if (partial) {
        const bool ok = (keep >> i) & 1u;
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
      static_for<0, G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float ph = row_bcast<h>(x[i]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      });
    }
  }

  // Fused append: token tn of a loaded step (0 <= tn < UT, wave-uniform)
  // is the row's new token, whose K/V rows are read from knew / vnew (one
  // KV head's D elements) instead of the pool.  The lanes whose operand
  // slots hold that token reload them from there: four lanes for K (lane
  // row n of tile ti is token 16ti + tok_a), one lane row for V (value i of
  // lane row jj is token 4i + jj).
  // Loads and stores go through buffer resources (a wave-uniform base in
  // SGPRs, 32-bit lane offsets), so that no 64-bit lane address is kept
  // live across the streaming loop.
  __device__ __forceinline__ void inject(Buf& bf, int tn, const uint16_t* knew,
                                         const uint16_t* vnew) const {
    const auto kr = make_rsrc(knew, D * 2);
    const auto vr = make_rsrc(vnew, D * 2);
#pragma unroll
    for (int ti = 0; ti < KT; ++ti)
      if (16 * ti + tok_a == tn)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bf.k[ti][kb] = buffer_load16(kr, 2 * (32 * kb + 8 * jj));
#pragma unroll
    for (int i = 0; i < TPR; ++i)
      if (4 * i + jj == tn)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) buffer_load(bf.v[i][ch], vr, 2 * (CH * n + 16 * CH * ch));
  }

  // After inject: the same lanes write token tn's rows to its pool slot
  // (kdst / vdst = the slot's row in the K / V pool).
  __device__ __forceinline__ void store_new(const Buf& bf, int tn, uint16_t* kdst,
                                            uint16_t* vdst) const {
    const auto kr = make_rsrc(kdst, D * 2);
    const auto vr = make_rsrc(vdst, D * 2);
#pragma unroll
    for (int ti = 0; ti < KT; ++ti)
      if (16 * ti + tok_a == tn)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) buffer_store(kr, 2 * (32 * kb + 8 * jj), bf.k[ti][kb]);
#pragma unroll
    for (int i = 0; i < TPR; ++i)
      if (4 * i + jj == tn)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) buffer_store(vr, 2 * (CH * n + 16 * CH * ch), bf.v[i][ch]);
  }

  // Merge the four lane-row streams.  Afterwards every lane (jj, n) holds
  // the wave maximum M (log2 units) and sum of head n, and every lane row
  // holds the merged accumulator (relative to M).
  __device__ __forceinline__ void merge_rows(float& M, float& lsum) {
    M = m_run;
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(m_run - M);
    lsum = l_run * f;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    static_for<0, G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float fh = row_bcast<h>(f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float v = acc[h][e] * fh;
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[h][e] = v;
      }
    });
  }

  // Row h of the merged accumulator (lane row 0 after merge_rows), times
  // inv, rounded to bf16 and stored at element h*D of the buffer: each lane
  // writes its CH consecutive dims as one 16- or 8-byte store.
  template <int H>
  __device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, float inv) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int off = 2 * (H * D + CH * n + 16 * CH * c);
      const float* x = acc[H] + c * CH;
      if constexpr (CH == 8) {
        buffer_store(r, off, make_uint4(pack_bf16x2(x[0] * inv, x[1] * inv),
                                        pack_bf16x2(x[2] * inv, x[3] * inv),
                                        pack_bf16x2(x[4] * inv, x[5] * inv),
                                        pack_bf16x2(x[6] * inv, x[7] * inv)));
      } else {
        buffer_store(r, off, make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv),
                                        pack_bf16x2(x[2] * inv, x[3] * inv)));
      }
    }
  }

  // Row h of the merged accumulator as float32 at element h*D of the buffer.
  template <int H>
  __device__ __forceinline__ void store_acc(__amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int off = 4 * (H * D + CH * n + 16 * CH * c);
      const float* x = acc[H] + c * CH;
#pragma unroll
      for (int q = 0; q < CH / 4; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(x[4 * q]), __float_as_uint(x[4 * q + 1]),
                  __float_as_uint(x[4 * q + 2]), __float_as_uint(x[4 * q + 3])},
            r, off + 16 * q, 0, 0);
    }
  }

  // Head-dim index of accumulator element e of this lane.
  __device__ __forceinline__ int dim_of(int e) const {
    return CH * n + (e % CH) + 16 * CH * (e / CH);
  }
};

// RowDecoder: the wave decoder of the direct decode kernel and of the one-row
// sequences of the varlen kernel.  A step is 16 tokens of a page:
//   S = K Q^T     v_mfma_f32_16x16x32_bf16 with K rows as A (read back from
//                 LDS in operand order, row n of the tile being token
//                 4(n%4) + n/4, so that score register r of lane row jj is
//                 token 4r + jj) and the NH heads as columns;
//   softmax       one running max and sum per head, the max taken over the
//                 four lane rows (two exchanges per step);
//   O^T += V^T P  v_mfma_f32_16x16x16_bf16 per 16 dims: lane (jj, n) holds
//                 the probabilities of tokens jj, 4+jj, 8+jj, 12+jj for head
//                 n, which is the B operand when k = 4jj + r stands for
//                 token 4r + jj; V is staged row-major with token 4r + jj at
//                 row 4jj + r, so one transposed read (ds_read_b64_tr_b16)
//                 per 16 dims yields the matching A operand.
// K and V arrive with whole-line loads (RPI rows per instruction) and go
// through a per-wave LDS area, 16-byte chunks XOR-swizzled by row.  The
// matrix cores take the PV products that would otherwise cost NH fused
// multiply-adds per token and dim on the vector ALUs.
template <int D, int PS, int NH>
struct RowDecoder {
  static constexpr int UT = 16;               // tokens per step
  static constexpr int UPP = PS / UT;         // steps per page
  static constexpr int KB = D / 32;           // k-steps of S
  static constexpr int DB = D / 16;           // 16-dim blocks of O^T
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;        // rows per load instruction
  static constexpr int NL = UT / RPI;         // load instructions per tensor per step
  static constexpr int SWZ = CPR < 16 ? CPR - 1 : 15;
  static constexpr int STAGE = 2 * UT * D * 2;  // LDS bytes per wave (K rows, V rows)
  static_assert(NH <= 16 && PS % UT == 0 && UT % RPI == 0, "decoder shape");
  struct Buf {
    uint4 k[NL];
    uint4 v[NL];
  };

  int jj, n, tok_a;
  unsigned char* kst;
  unsigned char* vst;
  float m_run, l_run;
  f32x4 oacc[DB];  // O^T: dims 16b + 4jj + r of head n
  bf16x8 qop[KB];

  __device__ __forceinline__ void init(int lane, unsigned char* stage) {
    jj = lane >> 4;
    n = lane & 15;
    tok_a = 4 * (n & 3) + (n >> 2);
    kst = stage;
    vst = stage + UT * D * 2;
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Q^T as the B operand of S: lane (jj, n) holds q[head n][32kb + 8jj ..
  // +7]; qg points at the first of nh <= NH heads, columns n >= nh are zero.
  __device__ __forceinline__ void load_q(const uint16_t* qg, int nh) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < nh) v = *reinterpret_cast<const uint4*>(qg + n * D + 32 * kb + 8 * jj);
      qop[kb] = as_bf16x8(v);
    }
  }

  // The loads of one step (krow / vrow: its first token row).  With live
  // false they go through an empty range: zeros, no memory read.
  __device__ __forceinline__ void load(Buf& bf, const uint16_t* krow, const uint16_t* vrow,
                                       bool live) const {
    const auto kr = make_rsrc(krow, live ? UT * D * 2 : 0);
    const auto vr = make_rsrc(vrow, live ? UT * D * 2 : 0);
    const int lane = 16 * jj + n;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int off = 2 * ((RPI * i + lane / CPR) * D + 8 * (lane % CPR));
      bf.k[i] = buffer_load16(kr, off);
      bf.v[i] = buffer_load16(vr, off);
    }
  }

  // Fold one step (tokens tok0 .. tok0+15; those outside [lo, hi) masked).
  __device__ __forceinline__ void process(const Buf& bf, int tok0, int lo, int hi,
                                          float scale_log2) {
    const int lane = 16 * jj + n, c = lane % CPR;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int r = RPI * i + lane / CPR;
      *reinterpret_cast<uint4*>(kst + r * (2 * D) + 16 * (c ^ (r & SWZ))) = bf.k[i];
      const int pr = 4 * (r & 3) + (r >> 2);
      *reinterpret_cast<uint4*>(vst + pr * (2 * D) + 16 * (c ^ (pr & SWZ))) = bf.v[i];
    }
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 kop =
          *reinterpret_cast<const uint4*>(kst + tok_a * (2 * D) + 16 * ((4 * kb + jj) ^ (tok_a & SWZ)));
      sc = mfma16(as_bf16x8(kop), qop[kb], sc);
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = sc[r] * scale_log2;
    const bool partial = (tok0 < lo) || (tok0 + UT > hi);
    uint32_t keep = 0xfu;
    if (partial) {
      keep = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + 4 * r + jj;
        const bool ok = t >= lo && t < hi;
        keep |= (ok ? 1u : 0u) << r;
        x[r] = ok ? x[r] : -INFINITY;
      }
    }
    float pmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 16));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 32));
    const float m_new = fmaxf(m_run, pmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = fast_exp2(x[r] - m_use);
      psum += x[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // p in [0, 1]: the hardware round-to-nearest conversion suffices
    const prefill_detail::bf16x2 p01 = {(__bf16)x[0], (__bf16)x[1]};
    const prefill_detail::bf16x2 p23 = {(__bf16)x[2], (__bf16)x[3]};
    const prefill_detail::s16x4 pop = __builtin_bit_cast(prefill_detail::s16x4, make_uint2(__builtin_bit_cast(uint32_t, p01),
                                                            __builtin_bit_cast(uint32_t, p23)));
    // transposed reads: source lane n of lane row jj points at row
    // 4jj + n/4, dims 16b + 4(n%4); lane n receives rows 4jj .. 4jj+3
    // (tokens jj, 4+jj, 8+jj, 12+jj) of dim 16b + n
    const int prow = 4 * jj + (n >> 2), a4 = n & 3;
    unsigned char* vrow = vst + prow * (2 * D) + 8 * (a4 & 1);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      prefill_detail::s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (prefill_detail::lds_s16x4*)(__attribute__((address_space(3))) unsigned char*)(
              vrow + 16 * ((2 * b + (a4 >> 1)) ^ (prow & SWZ))));
      if (partial) {  // masked tokens' V rows may hold anything (NaN)
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = ((keep >> r) & 1u) ? v4[r] : (short)0;
      }
      oacc[b] *= alpha;
      oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v4, pop, oacc[b], 0, 0, 0);
    }
  }

  // Fused append: token tn of a loaded step (0 <= tn < 16, wave-uniform) is
  // the row's new token; the lanes that loaded its K and V chunks reload
  // them from knew / vnew (one KV head's D elements), and after the loads
  // have landed store_new writes them to the token's pool slot.
  __device__ __forceinline__ void inject(Buf& bf, int tn, const uint16_t* knew,
                                         const uint16_t* vnew) const {
    const auto kr = make_rsrc(knew, D * 2);
    const auto vr = make_rsrc(vnew, D * 2);
    const int lane = 16 * jj + n;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (RPI * i + lane / CPR == tn) {
        bf.k[i] = buffer_load16(kr, 16 * (lane % CPR));
        bf.v[i] = buffer_load16(vr, 16 * (lane % CPR));
      }
  }
  __device__ __forceinline__ void store_new(const Buf& bf, int tn, uint16_t* kdst,
                                            uint16_t* vdst) const {
    const auto kr = make_rsrc(kdst, D * 2);
    const auto vr = make_rsrc(vdst, D * 2);
    const int lane = 16 * jj + n;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (RPI * i + lane / CPR == tn) {
        buffer_store(kr, 16 * (lane % CPR), bf.k[i]);
        buffer_store(vr, 16 * (lane % CPR), bf.v[i]);
      }
  }

  // The step state after the last step: M (log2 units) and the sum of head
  // n, the same in every lane row.
  __device__ __forceinline__ void finish(float& M, float& lsum) const {
    M = m_run;
    lsum = l_run + __shfl_xor(l_run, 16);
    lsum += __shfl_xor(lsum, 32);
  }
};

}  // namespace pkv
