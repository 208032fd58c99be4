// Device page allocator for the block tables of a paged pool.
//
// The pool is one set of pages and a page table maps (sequence, logical
// page) to a physical page, pages being handed out as sequences grow
// (scripts/benchmarks commit log 1847125, flex_attention paged-KV engine
// entry, "Why this works" item 1 and "Files").  Here the free pages are a
// stack in device memory and both operations run on the device, so they can
// sit inside a captured step graph next to the append and the attention
// that read the tables they write.
//
// Policy: sequences are served in batch order and, within a sequence, its
// logical pages in increasing order, each taking the next page from the top
// of the stack; a request is all or nothing.  One workgroup does the work:
// an exclusive scan of the per-sequence page counts gives every sequence its
// range of stack positions, so the result is deterministic.
#include "common.h"

namespace pkv {
namespace {

constexpr int kAllocThreads = 1024;
constexpr int kAllocWaves = kAllocThreads / 64;

__device__ __forceinline__ int ceil_div_pos(int x, int d) { return x > 0 ? (x + d - 1) / d : 0; }

// Exclusive prefix sum of v over the workgroup, in thread order; *total gets
// the sum.  Every thread must call it.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(x, off);
    if (lane >= off) x += t;
  }
  if (lane == 63) lds[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kAllocWaves; ++i) {
    const int s = lds[i];
    before += i < w ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Largest c < n with first[c] <= k (first[] non-decreasing, first[0] = 0):
// the sequence of the chunk that owns the chunk's k-th page.
__device__ __forceinline__ int owner_of(const int* first, int n, int k) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (first[mid] <= k) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kAllocThreads) void page_alloc_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int num_seqs,
    int32_t* __restrict__ bt, int max_pages, int page_size, const int32_t* __restrict__ free_pages,
    int32_t* __restrict__ free_count, int num_pages, int32_t* __restrict__ status) {
  __shared__ int lds[kAllocWaves];
  __shared__ int table_full;
  const int F = min(max(*free_count, 0), num_pages);
  if (threadIdx.x == 0) table_full = 0;
  __syncthreads();
  // pages each sequence holds before the step and needs after it
  auto counts = [&](int j, int& held, int& need) {
    held = need = 0;
    if (j >= num_seqs) return;
    const int lq = cu_q[j + 1] - cu_q[j], lk = cu_k[j + 1] - cu_k[j];
    held = ceil_div_pos(lk - lq, page_size);
    const int want = ceil_div_pos(lk, page_size);
    if (want > max_pages) table_full = 1;
    need = max(0, want - held);
  };
  int total = 0;
  for (int base = 0; base < num_seqs; base += kAllocThreads) {
    int held, need, t;
    counts(base + threadIdx.x, held, need);
    block_exclusive_scan(need, lds, &t);
    total += t;
  }
  __syncthreads();
  const int st = table_full ? 1 : (total > F ? 2 : 0);
  if (st != 0) {
    if (threadIdx.x == 0 && status != nullptr) *status = st;
    return;
  }
  // second pass: the chunk's pages are spread over all threads, each finding
  // its sequence by a binary search of the scan, so one long prompt does not
  // serialise on one thread
  __shared__ int s_first[kAllocThreads], s_held[kAllocThreads];
  int taken = 0;
  for (int base = 0; base < num_seqs; base += kAllocThreads) {
    int held, need, t;
    counts(base + threadIdx.x, held, need);
    s_first[threadIdx.x] = block_exclusive_scan(need, lds, &t);
    s_held[threadIdx.x] = held;
    __syncthreads();
    const int n_chunk = min(kAllocThreads, num_seqs - base);
    for (int k = threadIdx.x; k < t; k += kAllocThreads) {
      const int c = owner_of(s_first, n_chunk, k);
      bt[(int64_t)(base + c) * max_pages + s_held[c] + (k - s_first[c])] =
          free_pages[F - 1 - (taken + k)];
    }
    __syncthreads();
    taken += t;
  }
  if (threadIdx.x == 0) {
    *free_count = F - total;
    if (status != nullptr) *status = 0;
  }
}

__global__ __launch_bounds__(kAllocThreads) void page_free_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ release, int num_seqs,
    int32_t* __restrict__ bt, int max_pages, int page_size, int32_t* __restrict__ free_pages,
    int32_t* __restrict__ free_count, int num_pages, int32_t* __restrict__ status) {
  __shared__ int lds[kAllocWaves];
  const int F = min(max(*free_count, 0), num_pages);
  __syncthreads();  // every thread has read the count before thread 0 rewrites it
  auto count = [&](int j) {
    if (j >= num_seqs || release[j] == 0) return 0;
    return min(ceil_div_pos(seq_lens[j], page_size), max_pages);
  };
  int total = 0;
  for (int base = 0; base < num_seqs; base += kAllocThreads) {
    int t;
    block_exclusive_scan(count(base + threadIdx.x), lds, &t);
    total += t;
  }
  if (F + total > num_pages) {
    if (threadIdx.x == 0 && status != nullptr) *status = 3;
    return;
  }
  // second pass: the chunk's pages spread over all threads (as in alloc)
  __shared__ int s_first[kAllocThreads];
  int pushed = 0;
  for (int base = 0; base < num_seqs; base += kAllocThreads) {
    int t;
    s_first[threadIdx.x] = block_exclusive_scan(count(base + threadIdx.x), lds, &t);
    __syncthreads();
    const int n_chunk = min(kAllocThreads, num_seqs - base);
    for (int k = threadIdx.x; k < t; k += kAllocThreads) {
      const int c = owner_of(s_first, n_chunk, k);
      int32_t* e = bt + (int64_t)(base + c) * max_pages + (k - s_first[c]);
      free_pages[F + pushed + k] = *e;
      *e = -1;
    }
    __syncthreads();
    pushed += t;
  }
  if (threadIdx.x == 0) {
    *free_count = F + total;
    if (status != nullptr) *status = 0;
  }
}

}  // namespace

hipError_t launch_page_alloc(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int32_t* bt,
                             int max_pages, int page_size, const int32_t* free_pages,
                             int32_t* free_count, int num_pages, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(page_alloc_kernel, dim3(1), dim3(kAllocThreads), 0, st, cu_q, cu_k, num_seqs,
                     bt, max_pages, page_size, free_pages, free_count, num_pages, status);
  return hipGetLastError();
}

hipError_t launch_page_free(const int32_t* seq_lens, const int32_t* release, int num_seqs,
                            int32_t* bt, int max_pages, int page_size, int32_t* free_pages,
                            int32_t* free_count, int num_pages, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(page_free_kernel, dim3(1), dim3(kAllocThreads), 0, st, seq_lens, release,
                     num_seqs, bt, max_pages, page_size, free_pages, free_count, num_pages, status);
  return hipGetLastError();
}

}  // namespace pkv
