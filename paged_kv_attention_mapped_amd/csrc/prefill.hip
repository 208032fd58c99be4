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
// vector phase V(t) (mask, max, exponentials, P packing, staging) and a
// matrix phase M(t) (O += V(t) P(t), then S(t+1) = K(t+1) Q^T).  The waves
// form two groups, one wave of each on every SIMD; group B runs one phase
// behind group A, and a workgroup barrier closes every phase, so on each
// SIMD one wave's MFMAs overlap the other wave's softmax.
//
// Staging.  Group A fetches K tiles and group B V tiles, straight from the
// pool into LDS (buffer loads with the LDS destination; no registers, no
// LDS store instructions) into four-deep rings.  Tiles are laid out in LDS
// in the order the MFMAs consume them: a K tile as 1 KB blocks that each
// hold one 32x16 A operand with lane l's 16 bytes at 16*l, a V tile as
// 512-byte blocks that each feed one transposed read with lane l's 8 bytes
// at 8*l.  Every LDS read of the loop is therefore one contiguous,
// conflict-free block with a compile-time offset.  Tile t+3 is requested
// in V(t) and waited for at the end of V(t+2); block-table entries are
// read through the scalar cache one tile before their tile.
//
// Head dim 512.  Four waves of 32 rows, one per SIMD: O^T of 32 rows takes
// all 256 AGPRs and the Q operands half the VGPRs, so the score tile is
// accumulated in VGPRs by inline-assembly MFMAs and the rare rescale of O
// is written out per AGPR.  Tiles are staged in whole 128-byte lines into
// two K and three V ring slots (160 KB of LDS), and a key tile is one MFMA
// stream that carries the next tile's softmax and loads (co_loop).
#include <math.h>

#include "common.h"
#include "decode_core.h"
#include "prefill_common.h"

namespace pkv {
namespace {

using namespace prefill_detail;

// Tuning knobs (fixed at build time): waves per workgroup for head_dim
// <= 128 (a tile holds 8 keys per wave), wave priority in matrix phases.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_LOOKAHEAD
#define PKV_PREFILL_LOOKAHEAD 6  // MFMA jobs between an operand request and its use
#endif
#ifndef PKV_PREFILL_SETPRIO
#define PKV_PREFILL_SETPRIO 0   // raise the matrix-phase wave's issue priority
#endif
#ifndef PKV_PREFILL_ZGROUP
#define PKV_PREFILL_ZGROUP 8    // consecutive query blocks of one sequence dispatched together
#endif
// launches with at most this many sequences (and few query blocks each) walk
// a compact work list; each workgroup scans the sequence lengths once
constexpr int kCompactMaxSeqs = 1024;


template <int D, int HW>
struct PrefillCfg {
  static constexpr int NW = D >= 256 ? 4 : PKV_PREFILL_WAVES;  // waves per workgroup
  static constexpr int NT = NW * 64;           // threads
  static constexpr int G = NW / 2;             // waves per group
  static constexpr int QB = NW / HW;           // waves along the rows
  static constexpr int BM = 32 * QB;           // query rows per workgroup
  static constexpr int BN = 8 * NW;            // keys per tile: one 16-key V step per group-B wave
  static constexpr int KT = BN / 32;           // 32-key tiles of S^T
  static constexpr int NU = BN / 16;           // 16-key steps of O^T
  static constexpr int KS = D / 16;            // k-steps of S^T
  static constexpr int DT = D / 32;            // 32-row tiles of O^T
  // ring depth (tiles) of K (NB) and V (NBV); at head_dim 512 a tile is
  // 32 KB: two K and three V tiles (160 KB, the whole LDS)
  static constexpr int NB = D == 512 ? 2 : 4;
  static constexpr int NBV = D == 512 ? 3 : NB;
  static constexpr int TILE = BN * D * 2;      // bytes of one K (or V) tile
  static constexpr int LDS_BYTES = (NB + NBV) * TILE;
  // each wave moves DT 1 KB blocks per tile: K blocks gw*DT .. +DT-1 (one
  // 32-key row tile), or V step u = gw for all DT column tiles
  static_assert(NW % 2 == 0 && NU == G && KS % DT == 0, "staging split");
  static_assert(QB >= 1, "more heads than waves");
};

// A sequence with a single query row (a decode row packed into the varlen
// batch, or a one-token prompt): the workgroup's NW waves take the allowed
// pages round-robin with RowDecoder (decode_core.h; NH heads of one KV
// head) and merge
// their softmax states through LDS, instead of running 32-row MFMA tiles
// for one row.  A mixed batch of decode rows and prompts is thereby one
// launch.
template <int D, int PS, int NH, int NW>
__device__ __forceinline__ void decode_row(const PrefillArgs& a, int j, int hk, int head0,
                                           int q_row, int L, int split, float* sm,
                                           bool mark, unsigned char* kstage) {
  // with key splits the row's pages are cut into S runs (split_count); split
  // s takes run s and writes its partial (max in log2 units, sum,
  // unnormalised accumulator) for the merge, and a row that is not cut
  // (S = 1) is written whole by split 0
  constexpr int G = NH;
  const int2 pr = row_pages(L, a.window, PS);
  const int S = split_count(pr.y - pr.x, a.nsplit, min_split_pages(NW));
  if (split >= S) return;
  if (mark && split == 0 && threadIdx.x == 0 && a.nsplit > 1) a.part_S[q_row] = S;
  using W = RowDecoder<D, PS, NH>;
  float* sm_m = sm;                 // [NW][G]
  float* sm_l = sm + NW * G;        // [NW][G]
  float* sm_acc = sm + 2 * NW * G;  // [NW][G][D]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  W wd;
  wd.init(lane, kstage + w * W::STAGE);
  wd.load_q(a.q + ((int64_t)q_row * a.num_q_heads + head0) * D, NH);
  const int first_key = a.window > 0 ? max(0, L - a.window) : 0;
  int p0 = pr.x, pend = pr.y;
  if (S > 1) {
    p0 = pr.x + split_begin(pr.y - pr.x, S, split);
    pend = pr.x + split_begin(pr.y - pr.x, S, split + 1);
  }
  const uint16_t* kh = a.k_pool + (int64_t)hk * a.head_stride;
  const uint16_t* vh = a.v_pool + (int64_t)hk * a.head_stride;
  const int32_t* bt_row = a.block_tables + (int64_t)j * a.max_pages;
  // this wave's pages: p0 + w, p0 + w + NW, ...; table entries 64 at a time
  const int npw = pend - p0 > w ? (pend - p0 - w + NW - 1) / NW : 0;
  const int nsteps = npw * W::UPP;
  int phys_lane = 0;
  int tok_of[2] = {0, 0};
  bool ok_of[2] = {false, false};
  auto load = [&](typename W::Buf& bf, int i_step, int slot) {
    const bool live = i_step < nsteps;  // a step past the end loads nothing
    const int i = i_step / W::UPP, part = i_step - i * W::UPP;
    if (live && (i & 63) == 0 && part == 0) {
      phys_lane = (i + lane < npw) ? bt_row[p0 + w + NW * (i + lane)] : -1;
      wait_vm_all();
    }
    int phys = __builtin_amdgcn_readlane(phys_lane, i & 63);
    ok_of[slot] = live && phys >= 0 && phys < a.num_pages;
    phys = ok_of[slot] ? phys : 0;  // an unusable entry reads page 0 and is masked out
    tok_of[slot] = (p0 + w + NW * i) * PS + part * W::UT;
    const int64_t row = (int64_t)phys * PS + part * W::UT;
    wd.load(bf, kh + row * D, vh + row * D, live);
  };
  auto process = [&](const typename W::Buf& bf, int slot) {
    wd.process(bf, tok_of[slot], ok_of[slot] ? first_key : INT_MAX, L, a.scale_log2);
  };
  // the next step is requested unconditionally (past the end it loads
  // nothing), so the wait before a step leaves the next one in flight
  typename W::Buf b0, b1;
  if (nsteps > 0) load(b0, 0, 0);
  for (int i = 0; i < nsteps; i += 2) {
    load(b1, i + 1, 1);
    process(b0, 0);
    if (i + 1 >= nsteps) break;
    load(b0, i + 2, 0);
    process(b1, 1);
  }

  float M, lw;
  wd.finish(M, lw);
  if (wd.n < G) {
    if (wd.jj == 0) {
      sm_m[w * G + wd.n] = M;
      sm_l[w * G + wd.n] = lw;
    }
#pragma unroll
    for (int b = 0; b < W::DB; ++b)
      *reinterpret_cast<f32x4*>(sm_acc + (w * G + wd.n) * D + 16 * b + 4 * wd.jj) = wd.oacc[b];
  }
  __syncthreads();
  for (int idx = tid; idx < NH * D; idx += 64 * NW) {
    const int h = idx / D, d = idx - h * D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, sm_m[ww * G + h]);
    float o = 0.f, lsum = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = sm_m[ww * G + h];
        if (mw == -INFINITY) continue;
        const float wt = fast_exp2(mw - Mx);
        o = fmaf(wt, sm_acc[(ww * G + h) * D + d], o);
        lsum = fmaf(wt, sm_l[ww * G + h], lsum);
      }
    }
    if (S > 1) {
      const int64_t cell = ((int64_t)q_row * a.num_q_heads + head0 + h) * a.nsplit + split;
      a.part_acc[cell * D + d] = o;
      if (d == 0) {
        a.part_m[cell] = Mx;
        a.part_l[cell] = lsum;
      }
      continue;
    }
    const float val = lsum > 0.f ? o / lsum : 0.f;
    a.out[((int64_t)q_row * a.num_q_heads + head0 + h) * D + d] = (uint16_t)f32_to_bf16(val);
  }
}

// Rows and keys of sequence j, clamped to the packed rows [0, total_q) and
// to the block table, so that no q read, out write or partial write leaves
// its buffer whatever cu_seq_lens_q/k hold.
struct SeqGeo {
  int q_start, Lq, Lk;
};
template <int PS>
__device__ __forceinline__ SeqGeo seq_geo(const PrefillArgs& a, int j) {
  SeqGeo g;
  g.q_start = min(max(a.cu_q[j], 0), a.total_q);
  g.Lq = min(max(a.cu_q[j + 1], g.q_start), a.total_q) - g.q_start;
  g.Lk = max(0, min(a.cu_k[j + 1] - a.cu_k[j], a.max_pages * PS));
  return g;
}

// Key splits of a sequence's work under the split entry: every query block
// of a prompt or chunk is cut into the same S runs, S set by its last block
// (the one that sees the most keys); a one-row sequence by its pages.
template <int BM, int BN, int PS, int NW>
__device__ __forceinline__ int seq_splits(const PrefillArgs& a, const SeqGeo& g) {
  if (a.nsplit <= 1 || g.Lq <= 0) return 1;
  if (g.Lq == 1) {
    const int2 pr = row_pages(g.Lk, a.window, PS);
    return split_count(pr.y - pr.x, a.nsplit, min_split_pages(NW));
  }
  const int q0 = ((g.Lq - 1) / BM) * BM;
  return split_count(block_tiles(block_keys(q0, g.Lq - 1, g.Lk - g.Lq, g.Lk, a.window), BN),
                     a.nsplit, min_split_tiles(BN));
}

// Compact work list: the launch's work items are, sequence by sequence, its
// query blocks from the last (longest) to the first, each cut into S runs,
// each run for every (KV head, head group) -- X0 items per run; a one-row
// sequence has one block and X1 items per run (X1 = the KV heads when one
// workgroup takes a KV head's whole group of heads).  Workgroup `item`
// scans the sequences' item counts, NT at a time with a workgroup prefix
// sum, and finds its sequence j, j's geometry and its index k among j's
// items; false past the end of the list.  Without ONE_ROW one-row
// sequences have no items (another launch takes them).  lds: NT/64 + 5
// ints.
template <int NT, int BM, int BN, int PS, int NW, bool ONE_ROW>
__device__ bool find_item(const PrefillArgs& a, int num_seqs, int X0, int X1, int item, int* lds,
                          int& j, int& k, SeqGeo& geo) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) lds[NWV] = -1;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += NT) {
    const int t = c0 + tid;
    int cnt = 0;
    SeqGeo g = {0, 0, 0};
    if (t < num_seqs) {
      g = seq_geo<PS>(a, t);
      if (g.Lq > (ONE_ROW ? 0 : 1))
        cnt = (g.Lq == 1 ? X1 : (g.Lq + BM - 1) / BM * X0) * seq_splits<BM, BN, PS, NW>(a, g);
    }
    int v = cnt;  // inclusive prefix within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane == 63) lds[wv] = v;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < NWV; ++w2) {
      const int x = lds[w2];
      pre += w2 < wv ? x : 0;
      tot += x;
    }
    const int hi = base + pre + v, lo = hi - cnt;
    if (cnt > 0 && item >= lo && item < hi) {
      lds[NWV] = t;
      lds[NWV + 1] = item - lo;
      lds[NWV + 2] = g.q_start;
      lds[NWV + 3] = g.Lq;
      lds[NWV + 4] = g.Lk;
    }
    __syncthreads();
    if (lds[NWV] >= 0) {
      j = lds[NWV];
      k = lds[NWV + 1];
      geo = SeqGeo{__builtin_amdgcn_readfirstlane(lds[NWV + 2]),
                   __builtin_amdgcn_readfirstlane(lds[NWV + 3]),
                   __builtin_amdgcn_readfirstlane(lds[NWV + 4])};
      return true;
    }
    base += tot;
  }
  return false;
}

template <int D, int PS, int HW>
__global__ __launch_bounds__((PrefillCfg<D, HW>::NT), 1) void prefill_kernel(PrefillArgs a, int nqb, int zg,
                                                                           int num_seqs) {
  using C = PrefillCfg<D, HW>;
  // one-row sequences run decode_row here, except at head_dim 512, where a
  // wave-level decoder does not fit the registers (launch_prefill sends
  // them to the head-dim-split kernel)
  constexpr bool kOneRow = D != 512;
  // [K ring: NB tiles][V ring: NB tiles]
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int HG = a.group / HW;       // workgroups per KV head along the heads
  const int X0 = a.num_kv_heads * HG;
  // at head_dim 256 (four waves, HW = 4) a group of 8 heads takes two
  // workgroups per prompt block; a one-row sequence then runs its whole group
  // in one workgroup (the 8 heads are 8 of the decoder's 16 MFMA columns),
  // so its pages are read once, not once per head group
  constexpr bool kPairRow = kOneRow && D == 256 && 2 * HW <= 8;
  const bool pair_row = kPairRow && HG == 2;
  int bx, j, b, split;               // (KV head, head group), sequence, block from the end, run
  SeqGeo geo;                        // sequence j's rows and keys
  if (zg == 0) {
    // compact work list (few query blocks per sequence): the workgroups
    // that find nothing are all at the end of the dispatch order
    int k;
    if (!find_item<C::NT, C::BM, C::BN, PS, C::NW, kOneRow>(
            a, num_seqs, X0, pair_row ? a.num_kv_heads : X0, (int)blockIdx.x,
            reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + C::LDS_BYTES - 256), j, k, geo))
      return;
    const int Sj = seq_splits<C::BM, C::BN, PS, C::NW>(a, geo);
    const bool pr1 = pair_row && geo.Lq == 1;
    const int Xj = pr1 ? a.num_kv_heads : X0;
    bx = k % Xj;
    if (pr1) bx *= HG;  // head group 0 of KV head bx
    k /= Xj;
    split = k % Sj;
    b = k / Sj;
  } else {
    // grid: x = (KV head, head group, run), y = sequence, z = query block
    // counted from the end, so the longest (latest) blocks of every sequence
    // go first; a one-row sequence runs in the z = 0 block
    bx = blockIdx.x;
    j = blockIdx.y;
    b = blockIdx.z;
    if (zg > 1) {
      // dispatch order: groups of zg query blocks (largest first), and within
      // a group every sequence's zg blocks back to back, so the workgroups
      // that run together on one XCD (the same KV head when the x extent is a
      // multiple of 8) stream the same K/V pages through its L2
      const uint32_t X = gridDim.x, Y = gridDim.y, Z = (uint32_t)zg;
      const uint32_t lin = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
      const uint32_t r = lin / X, rest = r / Z;
      bx = (int)(lin - r * X);
      j = (int)(rest % Y);
      b = (int)((rest / Y) * Z + (r - rest * Z));
      if (b >= nqb) return;  // padding of the last group
    }
    split = bx / X0;
    bx -= split * X0;
  }
  const int hk = bx / HG;
  const int hg = bx - hk * HG;

  if (zg != 0) geo = seq_geo<PS>(a, j);
  const int q_start = geo.q_start, Lq = geo.Lq, Lk = geo.Lk;
  if (Lq <= 1) {
    if constexpr (kOneRow) {
      if (Lq == 1 && b == 0) {
        float* sm = reinterpret_cast<float*>(smem);
        unsigned char* ks = reinterpret_cast<unsigned char*>(smem) + C::LDS_BYTES / 2;
        if constexpr (kPairRow) {
          if (pair_row) {  // head group 0 takes both; the other one has nothing
            if (hg == 0)
              decode_row<D, PS, 2 * HW, C::NW>(a, j, hk, hk * a.group, q_start, Lk, split, sm,
                                               bx == 0, ks);
            return;
          }
        }
        decode_row<D, PS, HW, C::NW>(a, j, hk, hk * a.group + hg * HW, q_start, Lk, split, sm,
                                     bx == 0, ks);
      }
    }
    return;
  }
  const int qb = (zg == 0 ? (Lq + C::BM - 1) / C::BM : nqb) - 1 - b;
  const int q0 = qb * C::BM;
  if (q0 >= Lq) return;
  const int shift = Lk - Lq;          // position of row r is shift + r
  // keys any row of this workgroup may see, and with key splits this
  // split's run of their tiles (split_count; a block that is not cut is
  // written whole by split 0)
  const int wg_last = min(q0 + C::BM, Lq) - 1;
  int2 kr = block_keys(q0, wg_last, shift, Lk, a.window);
  const int S = seq_splits<C::BM, C::BN, PS, C::NW>(a, geo);
  if (split >= S) return;
  if (S > 1) {  // this run of the block's tiles (a block with fewer tiles than runs has empty runs)
    const int nt = block_tiles(kr, C::BN);
    const int tf = kr.x / C::BN;
    kr.x = max(kr.x, (tf + split_begin(nt, S, split)) * C::BN);
    kr.y = min(kr.y, (tf + split_begin(nt, S, split + 1)) * C::BN);
  }
  const int kstart = kr.x, kend = kr.y;
  if (a.nsplit > 1 && split == 0 && bx == 0)  // the rows' split count, for the merge
    for (int r = q0 + (int)threadIdx.x; r <= wg_last; r += C::NT) a.part_S[q_start + r] = S;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query row within the wave's 32 rows
  const int hh = lane >> 5;   // k-group half
  const int hw = w % HW;
  const int head = hk * a.group + hg * HW + hw;
  const int r0 = q0 + 32 * (w / HW);  // first row of this wave
  const int qrow = r0 + col;
  const bool grp_b = w >= C::NW / 2;  // group B: one phase behind, stages V
  const int gw = w - (grp_b ? C::NW / 2 : 0);

  // Q rows as the B operand of S^T: lane holds q[qrow][16ks + 8hh .. +7].
  bf16x8 qop[C::KS];
  if constexpr (D != 512) {  // (head_dim 512 stages Q through LDS: co_loop)
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
  // Wave gw's rows of tile s start at key s*BN + w0 (32 rows for K, 16 for
  // V) and are fetched as NR page runs of RR rows (two 16-row runs for K
  // when pages hold 16 keys).  Each run is one scalar buffer resource
  // bounded to its keys below kend: the hardware writes zeros for lanes past
  // the bound, so keys past kend and unusable pages read as zeros.
  //
  // At head_dim 512 (CO) every load reads whole 128-byte lines: 8 rows x
  // 128 bytes per instruction instead of 32 rows x 32 bytes (K) or 16 rows x
  // 64 bytes (V), which cuts the time the vector memory path spends on a
  // tile's loads fourfold.  Wave w stages rows 8w..8w+7 of both tensors (one
  // page run, one table entry), with the loads spread through the MFMA
  // stream (co_loop below).
  //   K: block (rg, cg) (rows 8rg.., 16-byte chunks 8cg..) at (4cg + rg) KB,
  //      lane 8i+x's 16 bytes = row 8rg+i, chunk 8cg + (x ^ i ^ (rg&1)); the
  //      XOR keeps the MFMA operand reads free of bank conflicts.
  //   V: block (u, p, h) (keys 16u+8h.., dims 64p..) at ((u*DT/2 + p)*2 + h)
  //      KB; its halves are the lo/hi 512-byte pieces of the transposed-read
  //      layout below for dt = 2p and 2p+1.
  constexpr bool CO = D == 512;
  constexpr int NR = (CO || PS >= 32) ? 1 : 2;   // page runs per wave and tile
  constexpr int NDMA = C::DT * NR;               // LDS-destination loads per wave and tile
  constexpr int VM_AHEAD = 2 * NDMA;             // loads of the two tiles requested after
  static_assert(!CO || C::KT == 1, "whole-line staging layout");
  const uint16_t* src = (grp_b ? a.v_pool : a.k_pool) + (int64_t)hk * a.head_stride;
  const int w0 = CO ? 8 * w : grp_b ? 16 * gw : 32 * ((gw * C::DT) / C::KS);
  const int rr_all = CO ? 8 : grp_b ? 16 : 32;   // rows of this wave
  const int RR = NR == 2 ? 16 : rr_all;          // rows per run
  const int roff = (NR == 2 && !grp_b) ? 16 : 0; // first row of run 1
  const int sstride = grp_b ? 64 : 32;           // global bytes between the wave's blocks
  // lane's row (relative to its run) and 16-byte chunk within the row
  int lrow, lchunk;
  if (!grp_b) {  // K block (kt, ks): lane l holds row l%32, d-chunk 2ks + l/32
    lrow = lane & 31;
    lchunk = 2 * ((gw * C::DT) % C::KS) + (lane >> 5);
  } else {       // V: lane l covers transposed-read lanes 2(l%32), +1 of half l/32
    const int s5 = lane & 31, g = s5 >> 3;
    lrow = 8 * (lane >> 5) + 4 * (g >> 1) + ((s5 >> 1) & 3);
    lchunk = 2 * (g & 1) + (s5 & 1);
  }
  // with two runs, lanes 16-31 and 48-63 take run 1 (K rows 16-31; for V
  // both runs are the same page run, so both groups issue the same loads)
  const bool run1 = NR == 2 && (lane & 16) != 0;
  const int loff = ((run1 && !grp_b ? lrow - 16 : lrow) * D + 8 * lchunk) * 2;  // bytes from the run base
  // CO: lane offsets from the run base of the wave's K and V loads, and the
  // K operand reads' lane offsets for k-steps ks = 4cg + m
  int coff_k = 0, coff_v = 0, kaddr[4] = {0, 0, 0, 0};
  if constexpr (CO) {
    {
      const int i = lane >> 3, x = lane & 7;
      coff_k = (i * D + 8 * (x ^ i ^ (w & 1))) * 2;
    }
    {
      const int s5 = lane & 31;
      const int kk = 4 * (s5 >> 4) + ((s5 >> 1) & 3), cc = 2 * ((s5 >> 3) & 1) + (s5 & 1);
      coff_v = (kk * D + 32 * (lane >> 5) + 8 * cc) * 2;
    }
    const int r = lane & 31, rg = r >> 3, i = r & 7, h = lane >> 5;
#pragma unroll
    for (int m = 0; m < 4; ++m) kaddr[m] = rg * 1024 + 16 * (8 * i + ((2 * m + h) ^ i ^ (rg & 1)));
  }
  // block-table row, read through the scalar cache (it is never written here)
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)j * a.max_pages);
  // LDS rings: K tiles at [0, NB*TILE), V tiles at [NB*TILE, 2*NB*TILE)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
  const uint32_t ring = lds0 + (grp_b ? C::NB * C::TILE : 0) + gw * C::DT * 1024;

  // block-table entries of tile s (scalar loads; a clamped index keeps the
  // read inside the row, entries past kend are not used)
  auto bt_load = [&](int s, int (&pgs)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int kb = s * C::BN + w0 + roff * r;
      pgs[r] = bt_row[min(kb / PS, a.max_pages - 1)];
    }
  };
  // request this wave's blocks of tile s into ring slot s % NB
  auto dma_tile = [&](int s, const int (&pgs)[NR]) {
    i32x4 rs[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int kb = s * C::BN + w0 + roff * r;
      const int phys = pgs[r];
      const bool ok = kb < kend && phys >= 0 && phys < a.num_pages;
      const int valid = ok ? min(kend - kb, RR) : 0;
      rs[r] = sgpr_rsrc(src + (ok ? ((int64_t)phys * PS + kb % PS) * D : 0), valid * D * 2);
    }
    const uint32_t m0 = ring + (s & (C::NB - 1)) * C::TILE;
#pragma unroll
    for (int i = 0; i < C::DT; ++i) {
      if constexpr (NR == 1) {
        load_lds16(rs[0], m0 + i * 1024, loff, sstride * i);
      } else {
        // both halves issue on every wave (exec-masked), so the load count
        // is the same for all waves
        if (run1) load_lds16(rs[1], m0 + i * 1024, loff, sstride * i);
        else      load_lds16(rs[0], m0 + i * 1024, loff, sstride * i);
      }
    }
  };

  // CO staging: the run of wave w in tile s of a pool, and its loads
  constexpr int NCG = C::DT / 2;  // 128-byte column groups of a row
  auto co_rsrc = [&](int s, int phys, const uint16_t* pool) {
    const int kb = s * C::BN + w0;
    const bool ok = kb < kend && phys >= 0 && phys < a.num_pages;
    const int valid = ok ? min(kend - kb, 8) : 0;
    return sgpr_rsrc(pool + (int64_t)hk * a.head_stride + (ok ? ((int64_t)phys * PS + kb % PS) * D : 0),
                     valid * D * 2);
  };
  // K blocks (w, cg) of tile s into the 32 KB slot at lds byte `slot`
  auto co_dma_k = [&](uint32_t slot, int s, int phys) {
    const i32x4 rs = co_rsrc(s, phys, a.k_pool);
    const uint32_t m0 = slot + w * 1024;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) load_lds16(rs, m0 + cg * 4096, coff_k, 128 * cg);
  };
  // V block (w/2, p, w%2) of a tile into V ring slot vslot
  auto co_dma_v = [&](const i32x4& rs, int vslot, int p) {
    const uint32_t m0 = lds0 + (C::NB + vslot) * C::TILE + ((w >> 1) * C::DT + (w & 1)) * 1024;
    load_lds16(rs, m0 + p * 2048, coff_v, 128 * p);
  };

  // Matrix phase M(t): O^T += V(t)^T P(t)^T, then S(t+1)^T = K(t+1) Q^T, as
  // one stream of MFMA jobs whose LDS operands are requested LA jobs ahead
  // (the scheduling barriers keep that order).  A V job (u, dt) takes the
  // two transposed reads of blocks (u, dt, half): lane l's 8 bytes at 8*l,
  // after which lane l of 16-lane group g holds
  // V[16u + 8half + 4(g/2) .. +3][32dt + 16(g%2) + l%16].  A K job (kt, ks)
  // takes block (kt, ks), lane l's 16 bytes at 16*l: the A operand
  // K[32kt + l%32][16ks + 8(l/32) .. +7].  K jobs alternate between the two
  // 32-key halves so that consecutive MFMAs do not depend on each other.
  auto mphase = [&](const bf16x8 (&pop)[C::NU], int t, f32x16 (&st)[C::KT]) {
    constexpr int NPV = C::NU * C::DT, NJ = NPV + C::KT * C::KS, LA = PKV_PREFILL_LOOKAHEAD;
    const char* vl = (const char*)smem + (C::NB + (t & (C::NB - 1))) * C::TILE + 8 * lane;
    const char* kl = (const char*)smem + ((t + 1) & (C::NB - 1)) * C::TILE + 16 * lane;
    bf16x8 opnd[LA + 1];
    f32x16 s[C::KT];
    auto fetch = [&](auto J) {
      constexpr int jj = decltype(J)::value, slot = jj % (LA + 1);
      if constexpr (jj < NPV) {
        constexpr int u = jj / C::DT, dt = jj % C::DT;
        const char* v0 = vl + (u * C::DT + dt) * 1024;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)v0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(v0 + 512));
        const uint2 l2 = __builtin_bit_cast(uint2, lo);
        const uint2 h2 = __builtin_bit_cast(uint2, hi);
        opnd[slot] = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
      } else {
        constexpr int q = jj - NPV, kt = q % C::KT, ks = q / C::KT;
        opnd[slot] = as_bf16x8(*reinterpret_cast<const uint4*>(kl + (kt * C::KS + ks) * 1024));
      }
    };
    static_for<0, LA>(fetch);
    static_for<0, NJ>([&](auto J) {
      constexpr int jj = decltype(J)::value, slot = jj % (LA + 1);
      if constexpr (jj + LA < NJ) fetch(std::integral_constant<int, jj + LA>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (jj < NPV) {
        constexpr int u = jj / C::DT, dt = jj % C::DT;
        acc[dt] = mfma32(opnd[slot], pop[u], acc[dt]);
      } else {
        constexpr int q = jj - NPV, kt = q % C::KT, ks = q / C::KT;
        s[kt] = mfma32(opnd[slot], qop[ks], ks == 0 ? f32x16{} : s[kt]);
      }
    });
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) st[kt] = s[kt];
  };
  // S^T of key tile t_first (prologue), same block layout
  auto qk_first = [&](f32x16 (&st)[C::KT], int t) {
    const char* kl = (const char*)smem + (t & (C::NB - 1)) * C::TILE + 16 * lane;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      f32x16 sacc = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        sacc = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(kl + (kt * C::KS + ks) * 1024)),
                      qop[ks], sacc);
      st[kt] = sacc;
    }
  };

  // ---- head_dim 512: one phase per key tile ----
  // Step t runs one MFMA stream: S(t+1) = K(t+1) Q^T (32 jobs, with the
  // loads of K(t+2) among them), then O += V(t) P(t) (32 jobs, with the
  // loads of V(t+2) and the softmax of S(t+1) among them), so that the
  // vector work and the loads run under the MFMAs.  P(t) was formed with
  // the maximum before S(t+1); a rescale that S(t+1) asks for is applied
  // to O at the start of step t+1.  One barrier closes the step: K(t+2) (needed
  // first thing in step t+1) and V(t+1) have landed by then, V(t+2) may
  // still be in flight.  K ring: slot (t-t_first)%2; V ring: (t-t_first)%3.
  auto co_loop = [&]() {
    if (kend <= kstart) return;
    constexpr int LA = PKV_PREFILL_LOOKAHEAD, NK = C::KS, NJ = NK + C::NU * C::DT;
    static_assert(!CO || (C::NBV == 3 && C::NB == 2 && NK == 32 && NJ == 64), "head_dim 512 stream");
    const int t_first = kstart / C::BN, t_last = (kend - 1) / C::BN;
    auto bt1 = [&](int s) { return bt_row[min((s * C::BN + w0) / PS, a.max_pages - 1)]; };
    // softmax of one 32-key tile in stages (fed a score tile whose MFMAs
    // have settled); `live` = false computes without committing anything
    f32x16 sc;  // the scores, then (from stage 3) their probabilities
    float mx = -INFINITY, alpha = 1.f, mc = 0.f;
    bool any_raise = false;
    // Stage q of NSOFT, one per O job: a few independent vector operations
    // per stage, each consuming what an earlier stage produced, so that the
    // stage issues under its MFMA without waiting on its own results.
    bool need_mask = false, raise = false;
    int mlo = 0, mhi = 0;
    float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f, m_new = 0.f, rarg = 0.f, psum = 0.f;
    auto soft = [&](auto Q, int k0, bool live, bf16x8 (&pn)[C::NU]) {
      constexpr int q = decltype(Q)::value;
      // register r holds key k0 + 8(r/4) + 4hh + r%4
      if constexpr (q == 0) {
        need_mask = (k0 + C::BN - 1 > wpmin) || (a.window > 0 && wpmax - k0 >= a.window) ||
                    (k0 + C::BN > Lk);
        // usable keys of this lane's row: mlo <= key - k0 - 4hh <= mhi
        mhi = min(mypos, Lk - 1) - k0 - 4 * hh;
        mlo = (a.window > 0 ? mypos - a.window + 1 : INT_MIN / 2) - k0 - 4 * hh;
      } else if constexpr (q == 1 || q == 2) {
        if (need_mask) {
#pragma unroll
          for (int r = 8 * (q - 1); r < 8 * q; ++r) {
            const int kr = 8 * (r >> 2) + (r & 3);
            sc[r] = (kr <= mhi) & (kr >= mlo) ? sc[r] : -INFINITY;
          }
        }
      } else if constexpr (q == 3) {
        x0 = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
        x1 = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
        x2 = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
        x3 = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
      } else if constexpr (q == 4) {
        x0 = fmaxf(fmaxf(x0, x1), sc[15]);
        x1 = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
        x2 = fmaxf(x2, x3);
      } else if constexpr (q == 5) {
        mx = fmaxf(fmaxf(x0, x1), x2);
      } else if constexpr (q == 6) {
        mx = half_max(mx);
      } else if constexpr (q == 7) {
        raise = live && (mx - m_run) * c > kRescaleSlack;
        any_raise = __builtin_amdgcn_ballot_w64(raise) != 0;
      } else if constexpr (q == 8) {
        m_new = raise ? mx : m_run;
      } else if constexpr (q == 9) {
        rarg = (m_run - m_new) * c;
        mc = (m_new == -INFINITY) ? 0.f : m_new * c;
      } else if constexpr (q == 10) {
        alpha = raise ? fast_exp2(rarg) : 1.f;  // 0 from -inf
        m_run = m_new;
        sc[0] = fmaf(sc[0], c, -mc);
        sc[1] = fmaf(sc[1], c, -mc);
      } else if constexpr (q >= 11 && q < 19) {
        // exponentials of pair q-11, arguments of pair q-10
        constexpr int e = 2 * (q - 11);
        if constexpr (q == 11) l_run *= alpha;
        sc[e] = fast_exp2(sc[e]);
        sc[e + 1] = fast_exp2(sc[e + 1]);
        if constexpr (e + 2 < 16) {
          sc[e + 2] = fmaf(sc[e + 2], c, -mc);
          sc[e + 3] = fmaf(sc[e + 3], c, -mc);
        }
      } else if constexpr (q == 19) {
        x0 = sc[0] + sc[1];
        x1 = sc[2] + sc[3];
        x2 = sc[4] + sc[5];
        x3 = sc[6] + sc[7];
      } else if constexpr (q == 20) {
        x0 += x1;
        x2 += x3;
        x1 = sc[8] + sc[9];
        x3 = sc[10] + sc[11];
      } else if constexpr (q == 21) {
        x0 += x2;
        x1 += x3;
        x2 = sc[12] + sc[13];
        x3 = sc[14] + sc[15];
      } else if constexpr (q == 22 || q == 23) {
        constexpr int u = q - 22;
        uint4 pp;
        pp.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)sc[8 * u], (__bf16)sc[8 * u + 1]});
        pp.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)sc[8 * u + 2], (__bf16)sc[8 * u + 3]});
        pp.z = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)sc[8 * u + 4], (__bf16)sc[8 * u + 5]});
        pp.w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)sc[8 * u + 6], (__bf16)sc[8 * u + 7]});
        pn[u] = as_bf16x8(pp);
        if constexpr (q == 22) {
          x0 += x1;
          x2 += x3;
        } else {
          psum = x0 + x2;
        }
      } else if constexpr (q == 24) {
        if (live) l_run += psum;
      }
    };
    constexpr int NSOFT = 25;
    auto rescale = [&]() {  // O *= alpha, once the last MFMA on O has settled
      if (!any_raise) return;
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) scale_agpr(acc[dt], alpha);
    };

    // Prologue.  Q is staged like a K tile, each wave's 32 rows of its head
    // in whole lines into its own 32 KB of the rings (the B-operand layout
    // read back as the K operands are), beside K(t_first) in the fifth slot;
    // once Q is in registers, the rings take K(t_first+1), V(t_first) and
    // V(t_first+1) while S(t_first) and P(t_first) are computed.  Ring slots
    // count from t_first.
    {
      const int nvalid = min(32, Lq - r0);
      const int rstride = a.num_q_heads * D * 2;  // bytes between packed rows
      const i32x4 rq = sgpr_rsrc(a.q + ((int64_t)(q_start + r0) * a.num_q_heads + head) * D,
                                 nvalid > 0 ? (nvalid - 1) * rstride + D * 2 : 0);
      const int i = lane >> 3, x = lane & 7;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int vo = (8 * rg + i) * rstride + 16 * (x ^ i ^ (rg & 1));
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          load_lds16(rq, lds0 + w * C::TILE + (cg * 4 + rg) * 1024, vo, 128 * cg);
      }
    }
    const uint32_t slot5 = lds0 + (C::NB + 2) * C::TILE;
    co_dma_k(slot5, t_first, bt1(t_first));
    phase_barrier<0>();  // Q and K(t_first) in LDS
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qop[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(
          (const char*)smem + w * C::TILE + (ks >> 2) * 4096 + kaddr[ks & 3]));
    phase_barrier<63>();  // every wave holds its Q: the rings are free
    int vslot = 0;
    int pe = bt1(t_first + 2);
    {
      const int p1 = bt1(t_first + 1);
      co_dma_k(lds0 + C::TILE, t_first + 1, p1);
      const i32x4 r0 = co_rsrc(t_first, bt1(t_first), a.v_pool), r1 = co_rsrc(t_first + 1, p1, a.v_pool);
#pragma unroll
      for (int q = 0; q < NCG; ++q) co_dma_v(r0, 0, q);
#pragma unroll
      for (int q = 0; q < NCG; ++q) co_dma_v(r1, 1, q);
    }
    bf16x8 pop[C::NU];
    {
      const char* k5 = (const char*)smem + (C::NB + 2) * C::TILE;
      f32x16 sacc;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 kop = as_bf16x8(*reinterpret_cast<const uint4*>(k5 + (ks >> 2) * 4096 + kaddr[ks & 3]));
        if (ks == 0)
          sacc = mfma32_v_first(kop, qop[ks]);
        else
          mfma32_v_acc(sacc, kop, qop[ks]);
      }
      mfma_settle(sacc);
      sc = sacc;
      static_for<0, NSOFT>([&](auto Q) { soft(Q, t_first * C::BN, true, pop); });
      // O is still zero: nothing to rescale
    }
    // K(t_first+1) and V(t_first) have landed (V(t_first+1) may still fly),
    // and every wave has read the fifth slot before V(t_first+2) lands there
    phase_barrier<NCG>();

    for (int t = t_first; t <= t_last; ++t) {
      // the rescale the previous step's softmax asked for, before O += V(t) P(t)
      if (t > t_first) rescale();
      const bool live = t < t_last;
      const int pnext = bt1(t + 3);
      const i32x4 rk = co_rsrc(t + 2, pe, a.k_pool), rv = co_rsrc(t + 2, pe, a.v_pool);
      const int rt = t - t_first;                                       // ring position
      const uint32_t kdst = lds0 + (rt & 1) * C::TILE + w * 1024;      // K(t+2)
      const int vs2 = vslot == 0 ? C::NBV - 1 : vslot - 1;             // V(t+2)
      const char* kl = (const char*)smem + ((rt + 1) & 1) * C::TILE;   // K(t+1)
      const char* vl = (const char*)smem + (C::NB + vslot) * C::TILE + 8 * lane;
      const int k1 = (t + 1) * C::BN;
      bf16x8 opnd[LA + 1], pn[C::NU];
      f32x16 s;
      auto fetch = [&](auto J) {
        constexpr int jj = decltype(J)::value, slot = jj % (LA + 1);
        if constexpr (jj < NK) {
          opnd[slot] = as_bf16x8(*reinterpret_cast<const uint4*>(kl + (jj >> 2) * 4096 + kaddr[jj & 3]));
        } else {
          constexpr int q = jj - NK, u = q / C::DT, dt = q % C::DT;
          const char* v0 = vl + u * C::DT * 1024 + (dt >> 1) * 2048 + (dt & 1) * 512;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) char*)v0);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) char*)(v0 + 1024));
          const uint2 l2 = __builtin_bit_cast(uint2, lo);
          const uint2 h2 = __builtin_bit_cast(uint2, hi);
          opnd[slot] = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
      };
      static_for<0, LA>(fetch);
      static_for<0, NJ>([&](auto J) {
        constexpr int jj = decltype(J)::value, slot = jj % (LA + 1);
        if constexpr (jj + LA < NJ) fetch(std::integral_constant<int, jj + LA>{});
        // K(t+2): one block per odd job of the first 16; V(t+2): one block
        // every fourth job of the second half
        if constexpr (jj < 2 * NCG && (jj & 1))
          load_lds16(rk, kdst + (jj >> 1) * 4096, coff_k, 128 * (jj >> 1));
        if constexpr (jj >= NK && (jj - NK) % 4 == 1 && (jj - NK) / 4 < NCG)
          co_dma_v(rv, vs2, (jj - NK) / 4);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (jj < NK) {
          if constexpr (jj == 0)
            s = mfma32_v_first(opnd[slot], qop[jj]);
          else
            mfma32_v_acc(s, opnd[slot], qop[jj]);
          if constexpr (jj == NK - 1) {  // the score chain's latency, under its last MFMA
            mfma_settle(s);
            sc = s;
          }
        } else {
          constexpr int q = jj - NK, u = q / C::DT, dt = q % C::DT;
          acc[dt] = mfma32(opnd[slot], pop[u], acc[dt]);
          // softmax of S(t+1) under the O MFMAs, one stage per job
          if constexpr (q < NSOFT) soft(std::integral_constant<int, q>{}, k1, live, pn);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int u = 0; u < C::NU; ++u) pop[u] = pn[u];
      pe = pnext;
      vslot = vslot == C::NBV - 1 ? 0 : vslot + 1;
      phase_barrier<NCG>();  // K(t+2) and V(t+1) landed; V(t+2)'s loads may still fly
    }
    // drain the loads of tiles past the end before the workgroup exits
    __builtin_amdgcn_s_waitcnt(0x0070);
  };

  if constexpr (CO) {
    co_loop();
  } else if (kend > kstart) {
    // Every wave executes the same number of barriers: group B one extra
    // before its first phase, group A one extra after its last.  Tile loads
    // are issued unconditionally (tiles past the end read zeros), so every
    // wave issues the same sequence and each wait count below is exact.
    const int t_first = kstart / C::BN, t_last = (kend - 1) / C::BN;
    int pg[2][NR];  // table entries of tile t+3 (slot (t+3-t_first)&1) and t+4
    {
      int p0[NR], p1[NR], p2[NR];
      bt_load(t_first, p0);
      bt_load(t_first + 1, p1);
      bt_load(t_first + 2, p2);
      bt_load(t_first + 3, pg[1]);
      dma_tile(t_first, p0);
      dma_tile(t_first + 1, p1);
      dma_tile(t_first + 2, p2);
    }
    // the Q loads and the first three tiles travel together; waiting for all
    // of them costs about one memory latency (the tiles were requested at
    // once) and leaves no load that the compiler's own waits do not count
    phase_barrier<0>();                // Q, and tile t_first of both tensors in LDS
    if (grp_b) phase_barrier<63>();

    f32x16 st[C::KT];
    qk_first(st, t_first);
    phase_barrier<63>();

    // one key tile; X is the table slot of tile t+3, the other slot takes t+4
    auto tile_step = [&](int t, auto X) {
      constexpr int x = decltype(X)::value;
      // ======== V(t): staging and softmax of S(t) ========
#if PKV_PREFILL_SETPRIO
      __builtin_amdgcn_s_setprio(0);
#endif
      dma_tile(t + 3, pg[x]);
      bt_load(t + 4, pg[x ^ 1]);
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
      phase_barrier<VM_AHEAD>();       // this wave's part of tile t+1 has landed

      // ======== M(t): O += V(t) P(t), S(t+1) = K(t+1) Q^T ========
#if PKV_PREFILL_SETPRIO
      __builtin_amdgcn_s_setprio(1);
#endif
      // (after the last tile the S result is unused: its ring slot holds
      // zeros or an older tile, both finite)
      mphase(pop, t, st);
      phase_barrier<63>();
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
    if (!grp_b) phase_barrier<63>();
    // drain the loads of tiles past the end before the workgroup exits
    __builtin_amdgcn_s_waitcnt(0x0070);
  }

  // ---- normalise and write: lane holds d = 32dt + 8(r/4) + 4hh + r%4 ----
  // The rows go out through LDS: each wave stages its 32 rows x D (16-byte
  // chunks XOR-swizzled by row, so the column-order writes spread over the
  // banks) and stores whole consecutive chunks of a row per lane group, in
  // place of 8- or 16-byte pieces of 32 different rows per instruction.
  const float lt = half_sum(l_run);
  // every wave is past its last read of the K/V rings
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  const int rows = min(32, Lq - r0);  // this wave's rows that exist
  // (key runs are not offered at head_dim 512, whose fp32 rows would not
  // fit the staging area)
  if (D <= 256 && S > 1) {
    // the split's partial (max in log2 units, sum, unnormalised accumulator),
    // merged by split_merge_kernel
    constexpr int CPR = D / 4;                      // 16-byte chunks per fp32 row
    constexpr int SW = CPR < 16 ? CPR - 1 : 15;
    unsigned char* stg = reinterpret_cast<unsigned char*>(smem) + w * 32 * D * 4;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<float4*>(stg + col * D * 4 + 16 * ((8 * dt + 2 * rb + hh) ^ (col & SW))) =
            make_float4(acc[dt][4 * rb], acc[dt][4 * rb + 1], acc[dt][4 * rb + 2], acc[dt][4 * rb + 3]);
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int cr = (64 * i + lane) / CPR, k = (64 * i + lane) % CPR;
      const float4 v = *reinterpret_cast<const float4*>(stg + cr * D * 4 + 16 * (k ^ (cr & SW)));
      if (cr < rows) {
        const int64_t cell = ((int64_t)(q_start + r0 + cr) * a.num_q_heads + head) * a.nsplit + split;
        *reinterpret_cast<float4*>(a.part_acc + cell * D + 4 * k) = v;
      }
    }
    if (qrow < Lq && hh == 0) {
      const int64_t cell = ((int64_t)(q_start + qrow) * a.num_q_heads + head) * a.nsplit + split;
      a.part_m[cell] = m_run == -INFINITY ? -INFINITY : m_run * c;
      a.part_l[cell] = lt;
    }
    return;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  constexpr int CPR = D / 8;                        // 16-byte chunks per bf16 row
  constexpr int SW = CPR < 16 ? CPR - 1 : 15;
  unsigned char* stg = reinterpret_cast<unsigned char*>(smem) + w * 32 * D * 2;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[dt][4 * rb] * inv, acc[dt][4 * rb + 1] * inv);
      pk.y = pack_bf16x2(acc[dt][4 * rb + 2] * inv, acc[dt][4 * rb + 3] * inv);
      *reinterpret_cast<uint2*>(stg + col * D * 2 + 16 * ((4 * dt + rb) ^ (col & SW)) + 8 * hh) = pk;
    }
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int cr = (64 * i + lane) / CPR, k = (64 * i + lane) % CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(stg + cr * D * 2 + 16 * (k ^ (cr & SW)));
    if (cr < rows)
      *reinterpret_cast<uint4*>(a.out + ((int64_t)(q_start + r0 + cr) * a.num_q_heads + head) * D + 8 * k) = v;
  }
}

// Merge of the key-split entry: workgroups (packed query row, chunk of
// its heads x dims).  The prefill launch recorded the run count S of every
// row it owns (part_S); a row with S > 1 gets its S partials merged in run
// order, four at a time with all their loads in flight, into a running
// (max, sum, accumulator).  Rows outside [cu_q[0], cu_q[N]) belong to no
// sequence and are left alone.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(PrefillArgs a, int num_seqs) {
  const int row = blockIdx.x;
  const int lo = min(max(a.cu_q[0], 0), a.total_q);
  const int hi = min(max(a.cu_q[num_seqs], lo), a.total_q);
  const int S = min(a.part_S[row], a.nsplit);
  if (row < lo || row >= hi || S <= 1) return;
  constexpr int TPC = D / 4;  // threads per (row, head), 4 dims each
  const int H = a.num_q_heads;
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (idx >= H * TPC) return;
  const int h = idx / TPC, d0 = 4 * (idx - h * TPC);
  const int64_t c0 = ((int64_t)row * H + h) * a.nsplit;
  float Mr = -INFINITY, Lr = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  for (int s0 = 0; s0 < S; s0 += 4) {
    float m[4], l[4];
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // unconditional loads (past S: run S-1 again, unused)
      const int64_t c = c0 + min(s0 + k, S - 1);
      m[k] = a.part_m[c];
      l[k] = a.part_l[c];
      v[k] = *reinterpret_cast<const float4*>(a.part_acc + c * D + d0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (s0 + k >= S || m[k] == -INFINITY) continue;
      const float Mn = fmaxf(Mr, m[k]);
      const float al = fast_exp2(Mr - Mn), be = fast_exp2(m[k] - Mn);
      Lr = fmaf(Lr, al, l[k] * be);
      o0 = fmaf(o0, al, v[k].x * be);
      o1 = fmaf(o1, al, v[k].y * be);
      o2 = fmaf(o2, al, v[k].z * be);
      o3 = fmaf(o3, al, v[k].w * be);
      Mr = Mn;
    }
  }
  const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
  uint2 pk;
  pk.x = pack_bf16x2(o0 * inv, o1 * inv);
  pk.y = pack_bf16x2(o2 * inv, o3 * inv);
  *reinterpret_cast<uint2*>(a.out + ((int64_t)row * H + h) * D + d0) = pk;
}

template <int D, int PS, int HW>
hipError_t launch_p3(const PrefillArgs& a, int num_seqs, int max_q, hipStream_t st) {
  using C = PrefillCfg<D, HW>;
  const int nqb = (max_q + C::BM - 1) / C::BM;
  // grouping pays where a sequence has many query blocks; with few blocks
  // (mixed decode/prefill steps, chunks) the launch walks a compact list of
  // its work items instead of a grid padded to the longest sequence
  const int X0 = a.num_kv_heads * (a.group / HW);
  const bool compact = nqb < 2 * PKV_PREFILL_ZGROUP && num_seqs <= kCompactMaxSeqs;
  const int zg = compact ? 0 : nqb >= 2 * PKV_PREFILL_ZGROUP ? PKV_PREFILL_ZGROUP : 1;
  dim3 grid;
  if (compact) {
    // items <= X0 * nsplit * sum_j ceil(Lq_j / BM) <= X0 * nsplit * (total_q / BM + num_seqs)
    const int64_t items = (int64_t)X0 * a.nsplit * ((int64_t)a.total_q / C::BM + num_seqs);
    if (items > INT32_MAX) return hipErrorInvalidConfiguration;
    grid = dim3((unsigned)items);
  } else {
    grid = dim3(X0 * a.nsplit, num_seqs, (nqb + zg - 1) / zg * zg);
  }
  const size_t smem = C::LDS_BYTES;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&prefill_kernel<D, PS, HW>),
                                       (int)smem, lds_raised);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<D, PS, HW>), grid, dim3(C::NT), smem, st, a, nqb, zg, num_seqs);
  if (a.nsplit <= 1) return hipGetLastError();
  const hipError_t e2 = hipGetLastError();
  if (e2 != hipSuccess) return e2;
  const unsigned chunks = (unsigned)((a.num_q_heads * (D / 4) + 255) / 256);
  hipLaunchKernelGGL(split_merge_kernel<D>, dim3(a.total_q, chunks), dim3(256), 0, st, a, num_seqs);
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
  if (head_dim == 512) {
    // prompts and chunks on the MFMA prefill kernel; one-row sequences (it
    // skips them) on the head-dim-split kernel, whose group of heads forms
    // the MFMA columns of one row
    if (max_seqlen_q > 1) {
      const hipError_t e = launch_p1<512>(a, num_seqs, max_seqlen_q, page_size, st);
      if (e != hipSuccess) return e;
    }
    Attn512Args b = {};
    b.q = a.q;
    b.k_pool = a.k_pool;
    b.v_pool = a.v_pool;
    b.block_tables = a.block_tables;
    b.cu_q = a.cu_q;
    b.cu_k = a.cu_k;
    b.out = a.out;
    b.head_stride = a.head_stride;
    b.max_pages = a.max_pages;
    b.num_pages = a.num_pages;
    b.num_q_heads = a.num_q_heads;
    b.num_kv_heads = a.num_kv_heads;
    b.group = a.group;
    b.window = a.window;
    b.num_splits = 1;
    b.one_row_only = 1;
    b.total_q = a.total_q;
    b.scale_log2 = a.scale_log2;
    return launch_attn512(b, num_seqs, 1, page_size, st);
  }
  switch (head_dim) {
    case 64: return launch_p1<64>(a, num_seqs, max_seqlen_q, page_size, st);
    case 128: return launch_p1<128>(a, num_seqs, max_seqlen_q, page_size, st);
    default: return launch_p1<256>(a, num_seqs, max_seqlen_q, page_size, st);
  }
}

}  // namespace pkv
