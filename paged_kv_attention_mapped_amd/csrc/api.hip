// C ABI: host-side validation, split-K planning and kernel dispatch.
// Every check here runs before anything is enqueued, and nothing here
// touches device memory from the host or synchronises.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/pkv.h"
#include "common.h"

using namespace pkv;

namespace {

bool supported_dim(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }
bool stream_dim(int d) { return supported_dim(d); }  // stream-K decode (512: per workgroup)
bool supported_ps(int ps) { return ps == 16 || ps == 32; }

pkv_status check_heads(int hq, int hkv) {
  if (hq <= 0 || hkv <= 0) return PKV_ERR_BAD_SHAPE;
  if (hq % hkv != 0) return PKV_ERR_BAD_SHAPE;
  if (hq / hkv > 8) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

constexpr int kTargetWorkgroups = 1024;  // enough to fill 256 CUs several times over
constexpr int kMaxPagesPerSplit = 32;
constexpr int kMinPagesPerSplit = 4;

// Pages a row's allowed keys can span.
int64_t key_pages(int page_size, int max_seq_len, int window) {
  int64_t pages = (max_seq_len + (int64_t)page_size - 1) / page_size;
  if (window > 0) {
    const int64_t wp = (window - 1 + (int64_t)page_size - 1) / page_size + 1;
    if (wp < pages) pages = wp;
  }
  return pages < 1 ? 1 : pages;
}

constexpr int kStreamMaxSeqs = 2048;     // row lengths are scanned in LDS
// A batch of at most this many (sequence, KV head) rows is decoded by one
// workgroup per row with no second kernel: at that size a stream-K launch
// is no faster and its merge launch costs more than the balance it buys.
constexpr int kDirectMaxRows = 256;
constexpr int kMaxPrefillSplits = 64;      // key splits per prefill workgroup
constexpr int kStreamMinUnitsPerWave = 4;
constexpr int kStreamWavesPerSimd = 2;   // matches the stream kernel's register budget

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Stream-K works on virtual KV heads: a group of more than four query heads
// with head_dim >= 128 is split in two halves that each see every page of
// their KV head (the second read of a page hits L2), so one wave's
// accumulators and PV work stay within its register budget.  Query and
// output addressing is unchanged (virtual head v, half-group g' covers query
// heads v*g' ..); only the pool addressing maps v back to KV head v >> 1.
int stream_kv_shift(int num_q_heads, int num_kv_heads, int head_dim) {
  const int g = num_q_heads / num_kv_heads;
  // head_dim 512 keeps the whole group: its heads are MFMA columns
  return (head_dim >= 128 && head_dim < 512 && g > 4 && g % 2 == 0) ? 1 : 0;
}
size_t stream_part_bytes(int num_waves, int group, int head_dim) {
  const size_t b = (size_t)2 * num_waves * group * (head_dim + 2) * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL_ARG: return "null argument";
    case PKV_ERR_BAD_SHAPE: return "bad shape";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

pkv_status pkv_stream_read(const void* buffer, size_t bytes, int32_t workgroups,
                           uint32_t* sink, hipStream_t stream) {
  if (workgroups <= 0 || workgroups > (1 << 20) || bytes % 16 != 0) return PKV_ERR_BAD_SHAPE;
  if (bytes == 0) return PKV_OK;
  if (!buffer || !sink) return PKV_ERR_NULL_ARG;
  return hip_status(launch_stream_read(buffer, (int64_t)bytes, sink, workgroups, stream));
}

pkv_status pkv_device_info(int32_t* compute_units, int32_t* max_clock_khz) {
  if (compute_units == nullptr || max_clock_khz == nullptr) return PKV_ERR_NULL_ARG;
  int dev = 0, cus = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev);
  if (e != hipSuccess) return PKV_ERR_HIP;
  *compute_units = cus;
  *max_clock_khz = khz;
  return PKV_OK;
}

pkv_status pkv_slot_mapping(const int32_t* block_tables, int32_t max_pages_per_seq,
                            const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                            int32_t num_seqs, int32_t total_tokens, int32_t page_size,
                            int32_t num_pages, int32_t* slot_mapping, hipStream_t stream) {
  if (num_seqs < 0 || total_tokens < 0 || max_pages_per_seq <= 0 || num_pages <= 0)
    return PKV_ERR_BAD_SHAPE;
  if (page_size <= 0) return PKV_ERR_BAD_SHAPE;
  if ((int64_t)num_pages * page_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0 || total_tokens == 0) return PKV_OK;
  if (!block_tables || !cu_seq_lens_q || !cu_seq_lens_k || !slot_mapping) return PKV_ERR_NULL_ARG;
  return hip_status(launch_slot_mapping(block_tables, max_pages_per_seq, cu_seq_lens_q,
                                        cu_seq_lens_k, num_seqs, total_tokens, page_size,
                                        num_pages, slot_mapping, stream));
}

pkv_status pkv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      uint16_t* k_pool, uint16_t* v_pool, int64_t num_slots,
                      hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_slots <= 0) return PKV_ERR_BAD_SHAPE;
  if (!supported_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool) return PKV_ERR_NULL_ARG;
  return hip_status(launch_append(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                  k_pool, v_pool, num_slots, stream));
}

pkv_status pkv_append_mapped(const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                             int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen_q,
                             int32_t page_size, int32_t num_pages, int32_t num_kv_heads,
                             int32_t head_dim, uint16_t* k_pool, uint16_t* v_pool,
                             int32_t* slot_mapping, hipStream_t stream) {
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen_q < 0 || max_pages_per_seq <= 0 ||
      num_pages <= 0 || num_kv_heads <= 0 || page_size <= 0)
    return PKV_ERR_BAD_SHAPE;
  if ((int64_t)num_pages * page_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  if (!supported_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  // chunk indices of one sequence's rows stay below 2^31
  if ((int64_t)max_seqlen_q * num_kv_heads * (head_dim / 8) > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0 || total_tokens == 0 || max_seqlen_q == 0) return PKV_OK;
  if (num_seqs > INT32_MAX / 2) return PKV_ERR_BAD_SHAPE;
  if (!k_new || !v_new || !block_tables || !cu_seq_lens_q || !cu_seq_lens_k || !k_pool ||
      !v_pool)
    return PKV_ERR_NULL_ARG;
  return hip_status(launch_append_mapped(
      k_new, v_new, block_tables, max_pages_per_seq, cu_seq_lens_q, cu_seq_lens_k, num_seqs,
      total_tokens, max_seqlen_q, page_size, num_pages, num_kv_heads, head_dim, k_pool, v_pool,
      (int64_t)num_pages * page_size, slot_mapping, stream));
}

pkv_status pkv_page_alloc(const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                          int32_t num_seqs, int32_t* block_tables, int32_t max_pages_per_seq,
                          int32_t page_size, int32_t* free_pages, int32_t* free_count,
                          int32_t num_pages, int32_t* status, hipStream_t stream) {
  if (num_seqs < 0 || max_pages_per_seq <= 0 || page_size <= 0 || num_pages <= 0)
    return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!cu_seq_lens_q || !cu_seq_lens_k || !block_tables || !free_pages || !free_count)
    return PKV_ERR_NULL_ARG;
  return hip_status(launch_page_alloc(cu_seq_lens_q, cu_seq_lens_k, num_seqs, block_tables,
                                      max_pages_per_seq, page_size, free_pages, free_count,
                                      num_pages, status, stream));
}

pkv_status pkv_page_free(const int32_t* seq_lens, const int32_t* release, int32_t num_seqs,
                         int32_t* block_tables, int32_t max_pages_per_seq, int32_t page_size,
                         int32_t* free_pages, int32_t* free_count, int32_t num_pages,
                         int32_t* status, hipStream_t stream) {
  if (num_seqs < 0 || max_pages_per_seq <= 0 || page_size <= 0 || num_pages <= 0)
    return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_lens || !release || !block_tables || !free_pages || !free_count)
    return PKV_ERR_NULL_ARG;
  return hip_status(launch_page_free(seq_lens, release, num_seqs, block_tables, max_pages_per_seq,
                                     page_size, free_pages, free_count, num_pages, status,
                                     stream));
}

pkv_status pkv_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t page_size,
                           int32_t max_seq_len, int32_t window, int32_t num_splits_requested,
                           int32_t* num_splits, int32_t* pages_per_split) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_splits_requested < 0)
    return PKV_ERR_BAD_SHAPE;
  if (!supported_ps(page_size)) return PKV_ERR_UNSUPPORTED;
  const int64_t pages = key_pages(page_size, max_seq_len, window);
  int64_t pps, s;
  if (num_splits_requested > 0) {
    s = num_splits_requested;
    pps = (pages + s - 1) / s;
  } else {
    pps = pages < kMaxPagesPerSplit ? pages : kMaxPagesPerSplit;
    const int64_t rows = (int64_t)num_seqs * num_kv_heads;
    while (pps > kMinPagesPerSplit && rows * ((pages + pps - 1) / pps) < kTargetWorkgroups) {
      pps = (pps + 1) / 2;
      if (pps < kMinPagesPerSplit) pps = kMinPagesPerSplit;
    }
    s = (pages + pps - 1) / pps;
  }
  if (s > 65535) return PKV_ERR_UNSUPPORTED;
  if (num_splits) *num_splits = (int32_t)s;
  if (pages_per_split) *pages_per_split = (int32_t)pps;
  return PKV_OK;
}

pkv_status pkv_decode_method(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                             int32_t window, int32_t num_splits_requested, int32_t* method,
                             int32_t* count) {
  if (num_seqs < 0 || max_seq_len < 0 || num_splits_requested < 0) return PKV_ERR_BAD_SHAPE;
  const pkv_status hs = check_heads(num_q_heads, num_kv_heads);
  if (hs != PKV_OK) return hs;
  if (!supported_dim(head_dim) || !supported_ps(page_size)) return PKV_ERR_UNSUPPORTED;
  int32_t m = PKV_DECODE_SPLIT, c = 0;
  if (num_splits_requested == 0 && num_seqs > 0 && num_seqs <= kStreamMaxSeqs &&
      stream_dim(head_dim)) {
    const int shift = stream_kv_shift(num_q_heads, num_kv_heads, head_dim);
    // (head_dim 512 always streams: its direct kernel runs one workgroup per
    // row, too few to fill the device for the batches it serves)
    if (shift == 0 && head_dim != 512 && (int64_t)num_seqs * num_kv_heads <= kDirectMaxRows) {
      m = PKV_DECODE_DIRECT;
      c = 1;
    } else {
      m = PKV_DECODE_STREAM;
      const pkv_status st = pkv_decode_stream_waves(num_seqs, num_q_heads, num_kv_heads,
                                                    head_dim, page_size, max_seq_len, window, &c);
      if (st != PKV_OK) return st;
    }
  } else {
    int32_t pps = 0;
    const pkv_status st = pkv_decode_plan(num_seqs, num_kv_heads, page_size, max_seq_len, window,
                                          num_splits_requested, &c, &pps);
    if (st != PKV_OK) return st;
    if (c <= 1) m = PKV_DECODE_DIRECT;
  }
  if (method) *method = m;
  if (count) *count = c;
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_kv_heads, int32_t page_size, int32_t max_seq_len,
                                  int32_t window, int32_t num_splits_requested) {
  int32_t method = 0, nw = 0;
  if (pkv_decode_method(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                        window, num_splits_requested, &method, &nw) != PKV_OK)
    return 0;
  if (method == PKV_DECODE_STREAM)
    return pkv_decode_stream_workspace_bytes(nw, num_q_heads, num_kv_heads, head_dim);
  if (method == PKV_DECODE_DIRECT) return 0;
  int32_t s = 0, pps = 0;
  if (pkv_decode_plan(num_seqs, num_kv_heads, page_size, max_seq_len, window,
                      num_splits_requested, &s, &pps) != PKV_OK)
    return 0;
  if (s <= 1 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const size_t cells = (size_t)num_seqs * num_q_heads * s;
  return cells * ((size_t)head_dim + 2) * sizeof(float);
}

static pkv_status check_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                               const int32_t* block_tables, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t num_pages, int32_t max_seq_len) {
  if (num_seqs < 0 || max_pages_per_seq <= 0 || num_pages <= 0 || max_seq_len < 0)
    return PKV_ERR_BAD_SHAPE;
  pkv_status st = check_heads(num_q_heads, num_kv_heads);
  if (st != PKV_OK) return st;
  if (!supported_dim(head_dim) || !supported_ps(page_size)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_pages_per_seq * page_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  if (num_seqs > 65535) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens) return PKV_ERR_NULL_ARG;
  return PKV_OK;
}

static DecodeArgs decode_args(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* seq_lens, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t num_pages,
                              float scale, int32_t window, int32_t splits, int32_t pps) {
  DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.part_m = a.part_l = a.part_acc = nullptr;
  a.out = nullptr;
  a.head_stride = (int64_t)num_pages * page_size * head_dim;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.kv_shift = 0;
  a.num_splits = splits;
  a.pages_per_split = pps;
  a.window = window;
  a.scale_log2 = scale * kLog2e;
  a.k_new = a.v_new = nullptr;
  a.k_pool_w = a.v_pool_w = nullptr;
  return a;
}

// The decode step's new rows, when the append is fused into the decode.
struct FusedAppend {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
};

static void set_fused(DecodeArgs& a, const FusedAppend* f) {
  if (f == nullptr) return;
  a.k_new = f->k_new;
  a.v_new = f->v_new;
  a.k_pool_w = f->k_pool;
  a.v_pool_w = f->v_pool;
}

// forward declarations of the stream-K helpers below
static void stream_heads(DecodeArgs& a, int head_dim);
static void stream_layout(StreamArgs& sa, void* workspace, int num_waves, int group, int head_dim);

pkv_status pkv_decode_split(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, int32_t max_pages_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_seq_len, float scale, int32_t window,
                            int32_t num_splits, int32_t pages_per_split, float* part_m,
                            float* part_l, float* part_acc, hipStream_t stream) {
  pkv_status st = check_decode(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                               num_pages, max_seq_len);
  if (st != PKV_OK) return st;
  if (num_splits <= 0 || num_splits > 65535 || pages_per_split <= 0) return PKV_ERR_BAD_SHAPE;
  if ((int64_t)num_splits * pages_per_split < key_pages(page_size, max_seq_len, window))
    return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!part_m || !part_l || !part_acc) return PKV_ERR_NULL_ARG;
  DecodeArgs a = decode_args(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                             num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale,
                             window, num_splits, pages_per_split);
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_acc = part_acc;
  return hip_status(launch_decode(a, num_seqs, head_dim, page_size, true, stream));
}

pkv_status pkv_decode_combine(const float* part_m, const float* part_l, const float* part_acc,
                              int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t num_splits, uint16_t* out, hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_splits <= 0) return PKV_ERR_BAD_SHAPE;
  if (!supported_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * num_q_heads > INT32_MAX / 4) return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!part_m || !part_l || !part_acc || !out) return PKV_ERR_NULL_ARG;
  return hip_status(launch_combine(part_m, part_l, part_acc, num_seqs, num_q_heads, head_dim,
                                   num_splits, out, stream));
}

// pkv_decode, and pkv_decode_append when `fused` is set.
static pkv_status decode_impl(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, int32_t max_seq_len, float scale, int32_t window,
                              int32_t num_splits, void* workspace, size_t workspace_bytes,
                              uint16_t* out, hipStream_t stream, const FusedAppend* fused) {
  pkv_status st = check_decode(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                               num_pages, max_seq_len);
  if (st != PKV_OK) return st;
  if (num_splits < 0) return PKV_ERR_BAD_SHAPE;
  int32_t method = 0, nw = 0;
  st = pkv_decode_method(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                         window, num_splits, &method, &nw);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!out) return PKV_ERR_NULL_ARG;
  int32_t s = 1, pps = 0;
  size_t need = 0;
  if (method == PKV_DECODE_STREAM) {
    need = pkv_decode_stream_workspace_bytes(nw, num_q_heads, num_kv_heads, head_dim);
  } else {
    st = pkv_decode_plan(num_seqs, num_kv_heads, page_size, max_seq_len, window,
                         method == PKV_DECODE_DIRECT ? 1 : num_splits, &s, &pps);
    if (st != PKV_OK) return st;
    if (s > 1)
      need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_kv_heads, page_size,
                                        max_seq_len, window, num_splits);
  }
  if (need > 0) {
    if (!workspace) return PKV_ERR_NULL_ARG;
    if (workspace_bytes < need) return PKV_ERR_WORKSPACE_TOO_SMALL;
  }
  // head_dim 512: the stream-K kernel appends the rows itself; explicit
  // splits append them by a launch of their own first (same result)
  if (fused != nullptr && head_dim == 512 && method != PKV_DECODE_STREAM) {
    const pkv_status ast = hip_status(launch_append_last(
        fused->k_new, fused->v_new, block_tables, max_pages_per_seq, seq_lens, num_seqs, page_size,
        num_pages, num_kv_heads, head_dim, fused->k_pool, fused->v_pool, stream));
    if (ast != PKV_OK) return ast;
    fused = nullptr;
  }
  DecodeArgs a = decode_args(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                             num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale,
                             window, s, pps);
  set_fused(a, fused);
  a.out = out;
  if (method == PKV_DECODE_STREAM) {
    StreamArgs sa;
    sa.base = a;
    sa.num_seqs = num_seqs;
    stream_heads(sa.base, head_dim);
    stream_layout(sa, workspace, nw, sa.base.group, head_dim);
    st = hip_status(launch_decode_stream(sa, head_dim, page_size, stream));
    if (st != PKV_OK) return st;
    return hip_status(launch_stream_merge(sa, head_dim, stream));
  }
  if (s <= 1) return hip_status(launch_decode(a, num_seqs, head_dim, page_size, false, stream));
  const size_t cells = (size_t)num_seqs * num_q_heads * s;
  float* ws = static_cast<float*>(workspace);
  a.part_acc = ws;
  a.part_m = ws + cells * head_dim;
  a.part_l = a.part_m + cells;
  pkv_status r = hip_status(launch_decode(a, num_seqs, head_dim, page_size, true, stream));
  if (r != PKV_OK) return r;
  return hip_status(launch_combine(a.part_m, a.part_l, a.part_acc, num_seqs, num_q_heads,
                                   head_dim, s, out, stream));
}

pkv_status pkv_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                      const int32_t* block_tables, int32_t max_pages_per_seq,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t num_pages, int32_t max_seq_len, float scale, int32_t window,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      uint16_t* out, hipStream_t stream) {
  return decode_impl(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_seq_len,
                     scale, window, num_splits, workspace, workspace_bytes, out, stream, nullptr);
}

// Scratch of pkv_decode_noalloc: the decode partials (split-K partials, or
// stream-K partials and merge descriptors) for callers that cannot allocate.
// 16 MiB holds the stream-K workspace of every supported shape on a device
// of up to 256 compute units (at most 15 MB, for a group of 7 at head_dim
// 128).  Each device holds its own copy until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (the name is only a host-side stand-in for it).
static pkv_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return PKV_OK;
}

pkv_status pkv_decode_noalloc(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_pages, int32_t max_seq_len, float scale,
                              int32_t window, int32_t num_splits, uint16_t* out,
                              hipStream_t stream) {
  pkv_status st = check_decode(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                               num_pages, max_seq_len);
  if (st != PKV_OK) return st;
  if (num_splits < 0) return PKV_ERR_BAD_SHAPE;
  // sizes beyond the scratch are refused before any HIP call
  const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_kv_heads,
                                                 page_size, max_seq_len, window, num_splits);
  if (need > kNoAllocScratchBytes) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (num_seqs == 0) return PKV_OK;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_seq_len,
                     scale, window, num_splits, ws, need > 0 ? kNoAllocScratchBytes : 0, out,
                     stream, nullptr);
}

pkv_status pkv_decode_append(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_tables,
                             int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                             float scale, int32_t window, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL_ARG;
  if ((int64_t)num_pages * page_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  const FusedAppend f = {k_new, v_new, k_pool, v_pool};
  return decode_impl(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_seq_len,
                     scale, window, num_splits, workspace, workspace_bytes, out, stream, &f);
}

pkv_status pkv_decode_stream_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                                   int32_t window, int32_t* num_waves) {
  if (num_seqs < 0 || max_seq_len < 0) return PKV_ERR_BAD_SHAPE;
  const pkv_status hs = check_heads(num_q_heads, num_kv_heads);
  if (hs != PKV_OK) return hs;
  if (!stream_dim(head_dim) || !supported_ps(page_size)) return PKV_ERR_UNSUPPORTED;
  const int64_t heads = (int64_t)num_kv_heads << stream_kv_shift(num_q_heads, num_kv_heads, head_dim);
  // units: pages (head_dim <= 256, one wave each) or 32-key tiles (head_dim
  // 512, one workgroup of four waves per compute unit)
  const int64_t units = (int64_t)num_seqs * heads *
                        (head_dim == 512 ? key_pages(32, max_seq_len, window)
                                         : key_pages(page_size, max_seq_len, window));
  const int per_simd = head_dim == 256 ? 1 : kStreamWavesPerSimd;
  int64_t nw = head_dim == 512 ? (int64_t)device_cus() : (int64_t)device_cus() * 4 * per_simd;
  const int64_t want = (units + kStreamMinUnitsPerWave - 1) / kStreamMinUnitsPerWave;
  if (want < nw) nw = want;
  if (nw < 1) nw = 1;
  if (num_waves) *num_waves = (int32_t)nw;
  return PKV_OK;
}

size_t pkv_decode_stream_workspace_bytes(int32_t num_waves, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim) {
  if (num_waves <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return 0;
  return stream_part_bytes(num_waves, num_q_heads / num_kv_heads, head_dim) +
         (size_t)2 * num_waves * kDescInts * sizeof(int);
}

// the virtual KV heads of stream-K (see stream_kv_shift)
static void stream_heads(DecodeArgs& a, int head_dim) {
  a.kv_shift = stream_kv_shift(a.num_q_heads, a.num_kv_heads, head_dim);
  a.num_kv_heads <<= a.kv_shift;
  a.group >>= a.kv_shift;
}

static void stream_layout(StreamArgs& sa, void* workspace, int num_waves, int group, int head_dim) {
  sa.num_waves = num_waves;
  sa.part = static_cast<float*>(workspace);
  sa.desc = reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                   stream_part_bytes(num_waves, group, head_dim));
}

pkv_status pkv_decode_stream(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t num_pages, float scale, int32_t window, int32_t num_waves,
                             void* workspace, size_t workspace_bytes, uint16_t* out,
                             hipStream_t stream) {
  pkv_status st = check_decode(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                               num_pages, 0);
  if (st != PKV_OK) return st;
  if (num_seqs > kStreamMaxSeqs || !stream_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_waves <= 0 || num_waves > (1 << 20)) return PKV_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !workspace) return PKV_ERR_NULL_ARG;
  if (workspace_bytes <
      pkv_decode_stream_workspace_bytes(num_waves, num_q_heads, num_kv_heads, head_dim))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  StreamArgs sa;
  sa.base = decode_args(q, k_pool, v_pool, block_tables, max_pages_per_seq, seq_lens,
                        num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale, window,
                        1, 1);
  sa.base.out = out;
  sa.num_seqs = num_seqs;
  stream_heads(sa.base, head_dim);
  stream_layout(sa, workspace, num_waves, sa.base.group, head_dim);
  return hip_status(launch_decode_stream(sa, head_dim, page_size, stream));
}

pkv_status pkv_decode_stream_merge(const void* workspace, size_t workspace_bytes,
                                   int32_t num_waves, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, uint16_t* out, hipStream_t stream) {
  pkv_status st = check_heads(num_q_heads, num_kv_heads);
  if (st != PKV_OK) return st;
  if (!stream_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_waves <= 0 || num_waves > (1 << 20)) return PKV_ERR_BAD_SHAPE;
  if (!workspace || !out) return PKV_ERR_NULL_ARG;
  if (workspace_bytes <
      pkv_decode_stream_workspace_bytes(num_waves, num_q_heads, num_kv_heads, head_dim))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  StreamArgs sa = {};
  sa.base.out = out;
  sa.base.num_q_heads = num_q_heads;
  sa.base.num_kv_heads = num_kv_heads;
  sa.base.group = num_q_heads / num_kv_heads;
  stream_heads(sa.base, head_dim);
  stream_layout(sa, const_cast<void*>(workspace), num_waves, sa.base.group, head_dim);
  return hip_status(launch_stream_merge(sa, head_dim, stream));
}

static size_t split_region(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

size_t pkv_prefill_split_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                         int32_t num_splits) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 1) return 0;
  const size_t cells = (size_t)total_q * num_q_heads * num_splits;
  return 2 * split_region(cells * sizeof(float)) +
         split_region(cells * (size_t)head_dim * sizeof(float)) + (size_t)total_q * sizeof(int32_t);
}

static pkv_status prefill_entry(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                                const int32_t* block_tables, int32_t max_pages_per_seq,
                                const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                                int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t page_size, int32_t num_pages,
                                float scale, int32_t window, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
      max_pages_per_seq <= 0 || num_pages <= 0 || num_splits < 1 || num_splits > kMaxPrefillSplits)
    return PKV_ERR_BAD_SHAPE;
  pkv_status st = check_heads(num_q_heads, num_kv_heads);
  if (st != PKV_OK) return st;
  if (!supported_dim(head_dim) || !supported_ps(page_size)) return PKV_ERR_UNSUPPORTED;
  if (num_splits > 1 && head_dim == 512) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_pages_per_seq * page_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
  if (num_seqs > 65535) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !cu_seq_lens_q || !cu_seq_lens_k || !out)
    return PKV_ERR_NULL_ARG;
  PrefillArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.cu_q = cu_seq_lens_q;
  a.cu_k = cu_seq_lens_k;
  a.out = out;
  a.head_stride = (int64_t)num_pages * page_size * head_dim;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.total_q = total_q;
  a.window = window;
  a.scale_log2 = scale * kLog2e;
  a.nsplit = num_splits;
  a.part_m = a.part_l = a.part_acc = nullptr;
  a.part_S = nullptr;
  if (num_splits > 1) {
    if (!workspace) return PKV_ERR_NULL_ARG;
    if (workspace_bytes < pkv_prefill_split_workspace_bytes(total_q, num_q_heads, head_dim, num_splits))
      return PKV_ERR_WORKSPACE_TOO_SMALL;
    const size_t cells = (size_t)total_q * num_q_heads * num_splits;
    char* w = static_cast<char*>(workspace);
    a.part_m = reinterpret_cast<float*>(w);
    a.part_l = reinterpret_cast<float*>(w + split_region(cells * sizeof(float)));
    a.part_acc = reinterpret_cast<float*>(w + 2 * split_region(cells * sizeof(float)));
    a.part_S = reinterpret_cast<int*>(w + 2 * split_region(cells * sizeof(float)) +
                                      split_region(cells * (size_t)head_dim * sizeof(float)));
  }
  return hip_status(launch_prefill(a, num_seqs, max_seqlen_q, head_dim, page_size, stream));
}

pkv_status pkv_prefill_varlen(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                              int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t num_pages,
                              float scale, int32_t window, uint16_t* out, hipStream_t stream) {
  return prefill_entry(q, k_pool, v_pool, block_tables, max_pages_per_seq, cu_seq_lens_q,
                       cu_seq_lens_k, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_q_heads,
                       num_kv_heads, head_dim, page_size, num_pages, scale, window, 1, nullptr, 0,
                       out, stream);
}

pkv_status pkv_prefill_varlen_split(const uint16_t* q, const uint16_t* k_pool,
                                    const uint16_t* v_pool, const int32_t* block_tables,
                                    int32_t max_pages_per_seq, const int32_t* cu_seq_lens_q,
                                    const int32_t* cu_seq_lens_k, int32_t num_seqs, int32_t total_q,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_size, int32_t num_pages, float scale,
                                    int32_t window, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return prefill_entry(q, k_pool, v_pool, block_tables, max_pages_per_seq, cu_seq_lens_q,
                       cu_seq_lens_k, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_q_heads,
                       num_kv_heads, head_dim, page_size, num_pages, scale, window, num_splits,
                       workspace, workspace_bytes, out, stream);
}

}  // extern "C"
