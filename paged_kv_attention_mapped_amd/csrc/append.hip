// Slot addressing and the slot-mapped K/V append.
//
// The engine writes each new token's K/V row straight into the shared page
// pool at a physical row address (scripts/benchmarks commit log 1847125,
// flex_attention paged-KV engine entry, "Files": k_cache[addr] = k_val).
// The address comes from the sequence's block table (same entry, "Why this
// works" item 1).
#include "common.h"

namespace pkv {
namespace {

// One workgroup per sequence; threads stride over its new tokens.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ bt, int max_pages, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int total, int page_size, int num_pages,
    int32_t* __restrict__ slots) {
  const int j = blockIdx.x;
  const int q0 = cu_q[j], q1 = cu_q[j + 1];
  const int lk = cu_k[j + 1] - cu_k[j];
  const int lq = q1 - q0;
  for (int r = threadIdx.x; r < lq; r += blockDim.x) {
    const int t = q0 + r;
    if (t < 0 || t >= total) continue;
    const int pos = lk - lq + r;
    int slot = -1;
    if (pos >= 0) {
      const int lp = pos / page_size;
      if (lp < max_pages) {
        const int phys = bt[(int64_t)j * max_pages + lp];
        if (phys >= 0 && phys < num_pages) slot = phys * page_size + pos % page_size;
      }
    }
    slots[t] = slot;
  }
}

// One thread per 16-byte chunk of a (token, head) row: consecutive lanes
// read consecutive bytes of k_new and write consecutive bytes of the pool
// row, so both sides are fully coalesced.
__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t total_chunks, int hkv, int chunks_per_row,
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, int64_t num_slots) {
  const int64_t per_token = (int64_t)hkv * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int64_t rem = i - t * per_token;
    const int64_t h = rem / chunks_per_row;
    const int64_t c = rem - h * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t dst = (h * num_slots + slot) * chunks_per_row + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

// Slot addressing and append in one launch.  Workgroup (j, y) copies the
// 16-byte chunks kAppendChunks*y .. kAppendChunks*(y+1)-1 of sequence j's new
// rows (token-major, then KV head, then chunk), resolving each token's slot
// from the block table as slot_mapping_kernel does and copying as
// append_kernel does; the host sizes y from its bound on the rows per
// sequence, so a long prompt gets many workgroups and a decode row one.
#ifndef PKV_APPEND_PER_THREAD
#define PKV_APPEND_PER_THREAD 2
#endif
constexpr int kAppendChunks = 256 * PKV_APPEND_PER_THREAD;  // chunks per workgroup

__global__ __launch_bounds__(256) void append_mapped_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ bt, int max_pages, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int total, int max_q, int page_size, int num_pages,
    unsigned per_token, unsigned chunks_per_row, uint4* __restrict__ k_pool,
    uint4* __restrict__ v_pool, int64_t num_slots, int32_t* __restrict__ slots_out) {
  constexpr int NC = kAppendChunks / 256;
  const int j = blockIdx.x;
  const int q0 = cu_q[j];
  const int lq = cu_q[j + 1] - q0;
  const int lk = cu_k[j + 1] - cu_k[j];
  const int rows = min(lq, max_q);  // rows past the host bound are not written
  if (rows <= 0) return;
  const unsigned n = (unsigned)rows * per_token;  // < 2^31 (checked on the host)
  for (unsigned base = blockIdx.y * (unsigned)kAppendChunks; base < n;
       base += gridDim.y * (unsigned)kAppendChunks) {
    int64_t src[NC], dst[NC];
    bool ok[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const unsigned k = base + c * 256u + threadIdx.x;
      const unsigned r = k / per_token;
      const unsigned rem = k - r * per_token;
      const int t = q0 + (int)r;
      const int pos = lk - lq + (int)r;
      int64_t slot = -1;
      if (k < n && pos >= 0 && pos / page_size < max_pages) {
        const int phys = bt[(int64_t)j * max_pages + pos / page_size];
        if (phys >= 0 && phys < num_pages) slot = (int64_t)phys * page_size + pos % page_size;
      }
      const bool tok_ok = k < n && t >= 0 && t < total;
      if (slots_out != nullptr && tok_ok && rem == 0) slots_out[t] = (int32_t)slot;
      ok[c] = tok_ok && slot >= 0 && slot < num_slots;
      const unsigned h = rem / chunks_per_row;
      src[c] = (int64_t)t * per_token + rem;
      dst[c] = ((int64_t)h * num_slots + slot) * chunks_per_row + (rem - h * chunks_per_row);
    }
    // all loads before the first store; a skipped chunk reads row 0 (the
    // token count is > 0 here) so that the arrays stay in registers
    uint4 kv[NC], vv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t sc = ok[c] ? src[c] : 0;
      kv[c] = k_new[sc];
      vv[c] = v_new[sc];
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (ok[c]) {
        k_pool[dst[c]] = kv[c];
        v_pool[dst[c]] = vv[c];
      }
  }
}

// The decode step's append on its own: row b's one new token, at position
// seq_lens[b] - 1, goes to its slot (what the fused decode does inside the
// attention launch, for the shapes whose decode kernel does not fuse it).
// One workgroup per row; threads stride over the 16-byte chunks of its
// KV heads' rows.  A row with length 0, or whose page is past its table or
// unusable, writes nothing.
__global__ __launch_bounds__(256) void append_last_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ bt, int max_pages, const int32_t* __restrict__ seq_lens,
    int page_size, int num_pages, unsigned per_token, unsigned chunks_per_row,
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, int64_t num_slots) {
  const int b = blockIdx.x;
  const int pos = seq_lens[b] - 1;
  if (pos < 0 || pos / page_size >= max_pages) return;
  const int phys = bt[(int64_t)b * max_pages + pos / page_size];
  if (phys < 0 || phys >= num_pages) return;
  const int64_t slot = (int64_t)phys * page_size + pos % page_size;
  for (unsigned k = threadIdx.x; k < per_token; k += blockDim.x) {
    const unsigned h = k / chunks_per_row;
    const int64_t src = (int64_t)b * per_token + k;
    const int64_t dst = ((int64_t)h * num_slots + slot) * chunks_per_row + (k - h * chunks_per_row);
    k_pool[dst] = k_new[src];
    v_pool[dst] = v_new[src];
  }
}

}  // namespace

hipError_t launch_append_last(const uint16_t* k_new, const uint16_t* v_new, const int32_t* bt,
                              int max_pages, const int32_t* seq_lens, int num_seqs, int page_size,
                              int num_pages, int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                              hipStream_t st) {
  const unsigned cpr = (unsigned)d / 8;
  hipLaunchKernelGGL(append_last_kernel, dim3(num_seqs), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     bt, max_pages, seq_lens, page_size, num_pages, (unsigned)hkv * cpr, cpr,
                     reinterpret_cast<uint4*>(k_pool), reinterpret_cast<uint4*>(v_pool),
                     (int64_t)num_pages * page_size);
  return hipGetLastError();
}

hipError_t launch_append_mapped(const uint16_t* k_new, const uint16_t* v_new, const int32_t* bt,
                                int max_pages, const int32_t* cu_q, const int32_t* cu_k,
                                int num_seqs, int total, int max_q, int page_size, int num_pages,
                                int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                                int64_t num_slots, int32_t* slots_out, hipStream_t st) {
  const unsigned cpr = (unsigned)d / 8;
  const unsigned per_token = (unsigned)hkv * cpr;
  int64_t y = ((int64_t)max_q * per_token + kAppendChunks - 1) / kAppendChunks;
  if (y > 65535) y = 65535;  // workgroups stride over the rest
  hipLaunchKernelGGL(append_mapped_kernel, dim3(num_seqs, (unsigned)y), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     bt, max_pages, cu_q, cu_k, total, max_q, page_size, num_pages, per_token, cpr,
                     reinterpret_cast<uint4*>(k_pool), reinterpret_cast<uint4*>(v_pool), num_slots,
                     slots_out);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* bt, int max_pages, const int32_t* cu_q,
                               const int32_t* cu_k, int num_seqs, int total, int page_size,
                               int num_pages, int32_t* slots, hipStream_t st) {
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, st, bt, max_pages, cu_q,
                     cu_k, total, page_size, num_pages, slots);
  return hipGetLastError();
}

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slots,
                         int num_tokens, int hkv, int d, uint16_t* k_pool, uint16_t* v_pool,
                         int64_t num_slots, hipStream_t st) {
  const int cpr = d / 8;
  const int64_t total = (int64_t)num_tokens * hkv * cpr;
  const int64_t want = (total + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     slots, total, hkv, cpr, reinterpret_cast<uint4*>(k_pool),
                     reinterpret_cast<uint4*>(v_pool), num_slots);
  return hipGetLastError();
}

}  // namespace pkv
