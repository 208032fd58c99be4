// GQA decode attention over the paged pool: split-K partitions with a
// combine kernel, and a persistent stream-K partition with a merge kernel.
//
// One query row per sequence attends its cached keys through the block
// table (scripts/benchmarks commit log 1847125, flex_attention paged-KV
// engine entry, "Why this works" items 1-2); the sliding regime adds
// q_pos - kv_pos < window (same log, per-regime mask entry).  In both
// decompositions the whole query-head group of a KV head shares every page
// it streams, so each page crosses HBM once; the per-wave work is in
// decode_core.h.
//
// Split-K: a workgroup owns one (sequence, KV head, split of pages); its
// waves take the split's pages round-robin and are merged through LDS.
//
// Stream-K: the (sequence, KV head, page) units of the whole batch are
// flattened in that order and cut into one contiguous, equal range per
// persistent wave, so every wave streams the same number of pages whatever
// the length mix.  A (sequence, KV head) segment that lies inside one
// wave's range is finished by that wave; a segment cut by range boundaries
// leaves one partial per piece (at most two per wave), and a small merge
// kernel combines the pieces in wave order.
#include "decode_core.h"

namespace pkv {
namespace {

// Tuning knobs (fixed at build time).
#ifndef PKV_DECODE_UNIT
#define PKV_DECODE_UNIT 16          // tokens per step (half a 32-token page)
#endif
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 8          // waves per split-K workgroup
#endif
#ifndef PKV_DECODE_OCCUPANCY
#define PKV_DECODE_OCCUPANCY 2      // waves per SIMD the split-K registers are sized for
#endif
#ifndef PKV_STREAM_OCCUPANCY
#define PKV_STREAM_OCCUPANCY 2      // waves per SIMD for the stream-K kernel
#endif

template <int D>
constexpr int occ(int o) { return D == 256 ? 1 : o; }

// ---------------------------------------------------------------------------
// split-K
// ---------------------------------------------------------------------------
template <int D, int PS, int G, bool SPLIT>
__global__ __launch_bounds__(PKV_DECODE_WAVES * 64, occ<D>(PKV_DECODE_OCCUPANCY))
void decode_kernel(DecodeArgs a) {
  using W = RowDecoder<D, PS, G>;
  constexpr int NW = PKV_DECODE_WAVES;
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  // each wave's K and V rows pass through LDS (RowDecoder); after its last
  // step the wave's accumulator goes there, [G][D] floats
  static_assert(G * D * 4 <= W::STAGE, "accumulator fits the stage");
  __shared__ __attribute__((aligned(16))) unsigned char sm_st[NW][W::STAGE];

  const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = a.group;
  W wd;
  wd.init(lane, sm_st[w]);
  wd.load_q(a.q + ((int64_t)b * a.num_q_heads + hk * g) * D, g);

  const int Lraw = a.seq_lens[b];
  const int L = max(0, min(Lraw, a.max_pages * PS));
  // fused append only for a row inside its table (a length past it writes nothing)
  const bool fuse = a.k_new != nullptr && Lraw == L;
  const int first_key = a.window > 0 ? max(0, L - a.window) : 0;
  const int p0 = first_key / PS;
  const int pend = (L + PS - 1) / PS;
  const int pa = min(pend, p0 + s * a.pages_per_split);
  const int pb = min(pend, pa + a.pages_per_split);

  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.max_pages;

  // This wave's pages are pa + w, pa + w + NW, ...; their table entries are
  // fetched 64 at a time (one per lane) and read back with readlane.
  const int npw = pb - pa > w ? (pb - pa - w + NW - 1) / NW : 0;
  const int nsteps = npw * W::UPP;
  int phys_lane = 0;
  int tok_of[2] = {0, 0};
  bool ok_of[2] = {false, false};
  int tn_of[2] = {-1, -1};       // fused append: the new token's index in the step, or -1
  int64_t row_of[2] = {0, 0};    // pool row of the step's first token (within the head)
  auto load = [&](typename W::Buf& bf, int j, int slot) {
    const int i = j / W::UPP, part = j - i * W::UPP;
    if ((i & 63) == 0 && part == 0) {
      phys_lane = (i + lane < npw) ? bt_row[pa + w + NW * (i + lane)] : -1;
      wait_vm_all();
    }
    int phys = __builtin_amdgcn_readlane(phys_lane, i & 63);
    ok_of[slot] = phys >= 0 && phys < a.num_pages;
    phys = ok_of[slot] ? phys : 0;  // an unusable entry reads page 0 and is masked out
    tok_of[slot] = (pa + w + NW * i) * PS + part * W::UT;
    const int64_t row = (int64_t)phys * PS + part * W::UT;
    row_of[slot] = row;
    const int t = L - 1 - tok_of[slot];
    tn_of[slot] = (fuse && ok_of[slot] && t >= 0 && t < W::UT) ? t : -1;
    wd.load(bf, kh + row * D, vh + row * D, true);
    // the row's new token: its lanes reload it from k_new / v_new (loads
    // return in issue order, so these land after the pool's)
    if (tn_of[slot] >= 0) {
      const int64_t nrow = ((int64_t)b * a.num_kv_heads + hk) * D;
      wd.inject(bf, tn_of[slot], a.k_new + nrow, a.v_new + nrow);
      wait_vm_all();
    }
  };
  auto process = [&](typename W::Buf& bf, int slot) {
    if (tn_of[slot] >= 0) {  // ... and is written to the pool
      const int tn = tn_of[slot];
      const int64_t prow = (int64_t)hk * a.head_stride + (row_of[slot] + tn) * D;
      wd.store_new(bf, tn, a.k_pool_w + prow, a.v_pool_w + prow);
    }
    wd.process(bf, tok_of[slot], ok_of[slot] ? first_key : INT_MAX, L, a.scale_log2);
  };
  typename W::Buf b0, b1;
  if (nsteps > 0) load(b0, 0, 0);
  for (int j = 0; j < nsteps; j += 2) {
    if (j + 1 < nsteps) load(b1, j + 1, 1);
    process(b0, 0);
    if (j + 1 >= nsteps) break;
    if (j + 2 < nsteps) load(b0, j + 2, 0);
    process(b1, 1);
  }

  float M, lw;
  wd.finish(M, lw);
  if (wd.n < G) {
    if (wd.jj == 0) {
      sm_m[w][wd.n] = M;
      sm_l[w][wd.n] = lw;
    }
    float* acc_w = reinterpret_cast<float*>(sm_st[w]);  // the wave is done with its stage
#pragma unroll
    for (int bb = 0; bb < W::DB; ++bb)
      *reinterpret_cast<f32x4*>(acc_w + wd.n * D + 16 * bb + 4 * wd.jj) = wd.oacc[bb];
  }
  __syncthreads();

  for (int idx = tid; idx < g * D; idx += 64 * NW) {
    const int h = idx / D, d = idx - h * D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, sm_m[ww][h]);
    float o = 0.f, lsum = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = sm_m[ww][h];
        if (mw == -INFINITY) continue;
        const float wt = fast_exp2(mw - Mx);
        o = fmaf(wt, reinterpret_cast<const float*>(sm_st[ww])[h * D + d], o);
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

// ---------------------------------------------------------------------------
// stream-K
// ---------------------------------------------------------------------------
// Wave whose range [w*U/nw, (w+1)*U/nw) contains unit u.
__device__ __forceinline__ int wave_of(int64_t u, int64_t U, int nw) {
  return (int)(((u + 1) * nw - 1) / U);
}

template <int D, int PS, int G>
__global__ __launch_bounds__(64, occ<D>(PKV_STREAM_OCCUPANCY))
void decode_stream_kernel(StreamArgs sa) {
  using W = WaveDecoder<D, PS, G, PKV_DECODE_UNIT>;
  extern __shared__ int smem[];
  const DecodeArgs& a = sa.base;
  const int B = sa.num_seqs, nw = sa.num_waves, w = blockIdx.x;
  const int lane = threadIdx.x;
  const int Hkv = a.num_kv_heads, g = a.group;
  int* pre = smem;           // pre[b] = first unit of sequence b; pre[B] = U
  // clamped lengths, negated when seq_lens[b] ran past the table (the fused
  // append then writes nothing for that row)
  int* lens = smem + B + 1;

  // ---- flattened unit counts: E_b pages per KV head, units = E_b * Hkv ----
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int v = 0;
    if (b < B) {
      const int raw = a.seq_lens[b];
      const int L = max(0, min(raw, a.max_pages * PS));
      const int fk = a.window > 0 ? max(0, L - a.window) : 0;
      const int E = (L + PS - 1) / PS - fk / PS;
      lens[b] = raw > L ? -L : L;
      v = E * Hkv;
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
  __syncthreads();
  const int U = __builtin_amdgcn_readfirstlane(pre[B]);

  // every wave clears its two merge descriptors for this launch
  if (lane < 2) sa.desc[(2 * w + lane) * kDescInts] = 0;
  // rows of empty sequences are zero
  for (int b = w; b < B; b += nw) {
    if (lens[b] != 0) continue;  // (a negated length is not 0 either)
    uint16_t* o = a.out + (int64_t)b * a.num_q_heads * D;
    for (int i = lane; i < a.num_q_heads * D; i += 64) o[i] = 0;
  }
  if (U == 0) return;
  const int64_t u0 = (int64_t)w * U / nw, u1 = (int64_t)(w + 1) * U / nw;
  if (u0 >= u1) return;

  W wd;
  wd.init(lane);

  // ---- segments: (b, hk) with units [s0, s1) = its pages p0 .. ----------
  struct Seg {
    int b, hk, L, fk, p0, s0, s1;
    bool fuse;  // the fused append may write this row's new token
  };
  // values read from LDS are per-lane registers; readfirstlane keeps the
  // (wave-uniform) segment bookkeeping in scalar registers
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  auto seg_at = [&](int b, int hk) -> Seg {
    Seg sg;
    sg.b = b;
    sg.hk = hk;
    const int lv = uni(lens[b]);
    sg.L = lv < 0 ? -lv : lv;
    sg.fuse = lv >= 0;
    sg.fk = a.window > 0 ? max(0, sg.L - a.window) : 0;
    sg.p0 = sg.fk / PS;
    const int pb0 = uni(pre[b]);
    const int E = (uni(pre[b + 1]) - pb0) / Hkv;
    sg.s0 = pb0 + hk * E;
    sg.s1 = sg.s0 + E;
    return sg;
  };
  auto seg_next = [&](const Seg& sg) -> Seg {
    int b = sg.b, hk = sg.hk + 1;
    if (hk == Hkv) {
      hk = 0;
      ++b;
      while (b < B - 1 && uni(pre[b + 1]) == uni(pre[b])) ++b;  // skip empty sequences
    }
    return seg_at(b, hk);
  };
  // first segment: the largest b with pre[b] <= u0 is non-empty (u0 < U)
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(pre[mid]) <= u0) lo = mid; else hi = mid;
  }
  const int hk_first = (int)((u0 - uni(pre[lo])) / ((uni(pre[lo + 1]) - uni(pre[lo])) / Hkv));

  // load cursor (runs one step ahead of the process cursor)
  Seg ls = seg_at(lo, hk_first);
  int tab_base = -1;  // unit of the first table entry held in phys_lane
  int phys_lane = 0;
  struct StepInfo {
    Seg sg;
    int u, part, tok0;
    bool ok;
    int tn;        // fused append: the row's new token's index in the step, or -1
    int64_t hoff;  // pool element offset of the step's first token row
  };
  const int nsteps = (int)(u1 - u0) * W::UPP;
  auto load = [&](typename W::Buf& bf, StepInfo& si, int j) {
    const int u = (int)u0 + j / W::UPP, part = j % W::UPP;
    while (u >= ls.s1) {
      ls = seg_next(ls);
      tab_base = -1;
    }
    if (tab_base < 0 || u - tab_base >= 64) {
      tab_base = u;
      const int page = ls.p0 + (u - ls.s0) + lane;
      phys_lane = (u + lane < ls.s1) ? a.block_tables[(int64_t)ls.b * a.max_pages + page] : -1;
      wait_vm_all();
    }
    int phys = __builtin_amdgcn_readlane(phys_lane, u - tab_base);
    si.ok = phys >= 0 && phys < a.num_pages;
    phys = si.ok ? phys : 0;  // an unusable entry reads page 0 and is masked out
    si.sg = ls;
    si.u = u;
    si.part = part;
    si.tok0 = (ls.p0 + (u - ls.s0)) * PS + part * W::UT;
    const int64_t hoff =
        (int64_t)(ls.hk >> a.kv_shift) * a.head_stride + ((int64_t)phys * PS + part * W::UT) * D;
    si.hoff = hoff;
    const int t = ls.L - 1 - si.tok0;
    si.tn = (a.k_new != nullptr && si.ok && t >= 0 && t < W::UT) ? t : -1;
    wd.load(bf, a.k_pool + hoff, a.v_pool + hoff);
    // the row's new token (only for a row inside its table: a length past
    // it writes nothing): its lanes reload it from k_new / v_new, after the
    // pool loads (loads return in issue order)
    if (si.tn >= 0 && ls.fuse) {
      const int64_t nrow =
          uni64(((int64_t)ls.b * (a.num_kv_heads >> a.kv_shift) + (ls.hk >> a.kv_shift)) * D);
      wd.inject(bf, si.tn, a.k_new + nrow, a.v_new + nrow);
      wait_vm_all();
    } else {
      si.tn = -1;
    }
  };

  // stores go through buffer resources with wave-uniform bases, so that no
  // 64-bit lane address stays live across the streaming loop
  auto finish = [&](const Seg& sg) {
    float M, lsum;
    wd.merge_rows(M, lsum);
    if (sg.s0 >= u0 && sg.s1 <= u1) {  // the whole segment is here: final rows
      if (wd.jj == 0) {
        const auto orr = make_rsrc(
            a.out + uni64(((int64_t)sg.b * a.num_q_heads + sg.hk * g) * D), g * D * 2);
        static_for<0, G>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float ls_h = row_bcast<h>(lsum);
          if (h < g) wd.template store_out<h>(orr, ls_h > 0.f ? 1.f / ls_h : 0.f);
        });
      }
      return;
    }
    const int slot = 2 * w + (sg.s0 <= u0 ? 0 : 1);
    const auto pr = make_rsrc(sa.part + (int64_t)slot * g * (D + 2), g * (D + 2) * 4);
    if (wd.jj == 0) {
      static_for<0, G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        if (h < g) wd.template store_acc<h>(pr);
      });
      if (wd.n < g) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), pr, 4 * (g * D + wd.n), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lsum), pr, 4 * (g * D + g + wd.n), 0, 0);
      }
    }
    if (sg.s0 >= u0 && lane == 0) {  // first piece: describe the segment for the merge
      int* dsc = sa.desc + slot * kDescInts;
      dsc[1] = sg.b;
      dsc[2] = sg.hk;
      dsc[3] = wave_of(sg.s1 - 1, U, nw);
      dsc[4] = U;
      dsc[0] = 1;
    }
  };

  auto process = [&](typename W::Buf& bf, const StepInfo& si) {
    const Seg& sg = si.sg;
    if (si.part == 0 && (si.u == sg.s0 || si.u == u0)) {  // first step of the segment here
      wd.reset();
      wd.load_q(a.q + ((int64_t)sg.b * a.num_q_heads + sg.hk * g) * D, g);
      wait_vm_all();
    }
    // the row's new token, injected at load time, is written to the pool by
    // the first of the virtual heads that share its KV head
    if (si.tn >= 0 && (sg.hk & ((1 << a.kv_shift) - 1)) == 0) {
      const int64_t prow = uni64(si.hoff + (int64_t)si.tn * D);
      wd.store_new(bf, si.tn, a.k_pool_w + prow, a.v_pool_w + prow);
    }
    wd.process(bf, si.tok0, si.ok ? sg.fk : INT_MAX, sg.L, a.scale_log2);
    if (si.part == W::UPP - 1 && (si.u == sg.s1 - 1 || si.u == u1 - 1)) finish(sg);
  };
  StepInfo i0, i1;
  typename W::Buf b0, b1;
  load(b0, i0, 0);
  for (int j = 0; j < nsteps; j += 2) {
    if (j + 1 < nsteps) load(b1, i1, j + 1);
    process(b0, i0);
    if (j + 1 >= nsteps) break;
    if (j + 2 < nsteps) load(b0, i0, j + 2);
    process(b1, i1);
  }
}

// Merge of cut segments: one workgroup per merge descriptor, one wave per
// query head (fewer, larger workgroups: most descriptors are empty).  The
// pieces are taken in wave order, kMergeBatch at a time with all their loads
// issued together, and folded into a running (max, sum, accumulator), so the
// result does not depend on timing and a segment cut into n pieces costs
// about n / kMergeBatch memory round trips.  Lane l holds D/64 consecutive
// dims (one store of its bf16 dims).
constexpr int kMergeBatch = 8;

// N consecutive floats of a piece; pieces are g*(D+2) floats apart, so only
// 8-byte alignment holds and the loads are float2
template <int N>
__device__ __forceinline__ void load_floats(float* d, const float* p) {
  if constexpr (N == 1) {
    d[0] = p[0];
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const float2 v = *reinterpret_cast<const float2*>(p + i);
      d[i] = v.x;
      d[i + 1] = v.y;
    }
  }
}

template <int D>
__global__ __launch_bounds__(512) void stream_merge_kernel(StreamArgs sa) {
  constexpr int EPL = D / 64;
  constexpr int MB = kMergeBatch;
  const int slot = blockIdx.x, h = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const DecodeArgs& a = sa.base;
  const int g = a.group, nw = sa.num_waves;
  // descriptor: [valid, sequence, KV head, last wave, total units]
  const int dv = lane < 5 ? sa.desc[slot * kDescInts + lane] : 0;
  if (__builtin_amdgcn_readfirstlane(dv) == 0) return;
  const int b = __builtin_amdgcn_readlane(dv, 1);
  const int hk = __builtin_amdgcn_readlane(dv, 2);
  const int w1 = __builtin_amdgcn_readlane(dv, 3);
  const int64_t U = __builtin_amdgcn_readlane(dv, 4);
  const int w0 = slot >> 1;
  const int64_t stride = (int64_t)g * (D + 2);
  // waves with an empty range (possible when there are fewer units than
  // waves) hold no piece
  auto holds = [&](int w) { return (int64_t)w * U / nw < (int64_t)(w + 1) * U / nw; };

  float Mr = -INFINITY, Lr = 0.f, o[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) o[i] = 0.f;
  for (int wb = w0; wb <= w1; wb += MB) {
    float mk[MB], lk[MB], pv[MB][EPL];
    // loads are unconditional (a wave past w1 re-reads w1's piece) so that
    // they all leave before the first one is used
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int w = min(wb + k, w1);
      const float* p = sa.part + (int64_t)(w == w0 ? slot : 2 * w) * stride;
      mk[k] = p[g * D + h];
      lk[k] = p[g * D + g + h];
      load_floats<EPL>(pv[k], p + h * D + EPL * lane);
    }
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int w = wb + k;
      if (w > w1 || !holds(w) || mk[k] == -INFINITY) continue;
      const float Mn = fmaxf(Mr, mk[k]);
      const float al = fast_exp2(Mr - Mn);
      const float be = fast_exp2(mk[k] - Mn);
      Lr = fmaf(Lr, al, lk[k] * be);
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] = fmaf(o[i], al, pv[k][i] * be);
      Mr = Mn;
    }
  }
  const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
  uint16_t* out = a.out + ((int64_t)b * a.num_q_heads + hk * g + h) * D + EPL * lane;
  if constexpr (EPL == 1) {
    *out = (uint16_t)f32_to_bf16(o[0] * inv);
  } else if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else if constexpr (EPL == 4) {
    *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv),
                                                pack_bf16x2(o[2] * inv, o[3] * inv));
  } else {
    *reinterpret_cast<uint4*>(out) = make_uint4(
        pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
        pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv));
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
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

template <int D, int PS, int G>
hipError_t launch_sg(const StreamArgs& sa, hipStream_t st) {
  const size_t smem = (size_t)(2 * sa.num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL((decode_stream_kernel<D, PS, G>), dim3(sa.num_waves), dim3(64), smem, st, sa);
  return hipGetLastError();
}

template <int D, int PS>
hipError_t launch_sp(const StreamArgs& sa, hipStream_t st) {
  if (sa.base.group <= 2) return launch_sg<D, PS, 2>(sa, st);
  if (sa.base.group <= 4) return launch_sg<D, PS, 4>(sa, st);
  return launch_sg<D, PS, 8>(sa, st);
}

template <int D>
hipError_t launch_s(const StreamArgs& sa, int ps, hipStream_t st) {
  return ps == 16 ? launch_sp<D, 16>(sa, st) : launch_sp<D, 32>(sa, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int num_seqs, int head_dim, int page_size,
                         bool split, hipStream_t st) {
  if (head_dim == 512) {  // the head-dim-split kernel, decode rows
    Attn512Args b = {};
    b.q = a.q;
    b.k_pool = a.k_pool;
    b.v_pool = a.v_pool;
    b.block_tables = a.block_tables;
    b.seq_lens = a.seq_lens;
    b.out = a.out;
    b.part_m = a.part_m;
    b.part_l = a.part_l;
    b.part_acc = a.part_acc;
    b.head_stride = a.head_stride;
    b.max_pages = a.max_pages;
    b.num_pages = a.num_pages;
    b.num_q_heads = a.num_q_heads;
    b.num_kv_heads = a.num_kv_heads;
    b.group = a.group;
    b.window = a.window;
    b.num_splits = split ? a.num_splits : 1;
    b.pages_per_split = a.pages_per_split;
    b.scale_log2 = a.scale_log2;
    return launch_attn512(b, num_seqs, 1, page_size, st);
  }
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
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(256), 0, st, m, l, acc, rows, splits, out); break;
    default: hipLaunchKernelGGL(combine_kernel<512>, grid, dim3(256), 0, st, m, l, acc, rows, splits, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_stream(const StreamArgs& sa, int head_dim, int page_size, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_s<64>(sa, page_size, st);
    case 128: return launch_s<128>(sa, page_size, st);
    case 256: return launch_s<256>(sa, page_size, st);
    default: return launch_attn512_stream(sa, page_size, st);  // workgroup-level stream-K
  }
}

template <int D>
void launch_merge_d(const StreamArgs& sa, hipStream_t st) {
  // one wave per query head of the (virtual) group, at most 8
  hipLaunchKernelGGL((stream_merge_kernel<D>), dim3(2 * sa.num_waves), dim3(64 * sa.base.group), 0,
                     st, sa);
}

hipError_t launch_stream_merge(const StreamArgs& sa, int head_dim, hipStream_t st) {
  switch (head_dim) {
    case 64: launch_merge_d<64>(sa, st); break;
    case 128: launch_merge_d<128>(sa, st); break;
    case 256: launch_merge_d<256>(sa, st); break;
    default: launch_merge_d<512>(sa, st); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
