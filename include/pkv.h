/*
 * pkv.h -- paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A stateless C ABI.  Every buffer is caller-owned device memory on the
 * current HIP device; the library allocates no device memory (the only
 * objects it creates are the step graphs of pkv_graph_end, which the caller
 * frees with pkv_graph_destroy), never synchronises and never reads device
 * memory from the host.  All work is enqueued on the
 * caller's stream and is asynchronous.  Calls are thread-safe.
 *
 * Data types.  bf16 values travel as their 16-bit patterns (uint16_t).
 * Tables and lengths are int32.  Output rows are rounded to bf16 with
 * round-to-nearest-even.
 *
 * Pool layout.  K and V each live in one tensor [Hkv, num_pages*page_size, D]
 * (row-major): for every KV head, all pages back to back, a page being
 * page_size consecutive token rows of D elements.  This is the single
 * contiguous cache with a (sequence, logical block) -> physical page table
 * that the rollout-engine pages describe (scripts/benchmarks commit log
 * 1847125, flex_attention paged-KV engine entry, "Why this works" item 1).
 * Pool row ("slot") s of head h starts at element (h*num_slots + s)*D.
 *
 * Block tables.  int32 [num_seqs, max_pages_per_seq], row-major; entry
 * [b][j] is the physical page holding logical tokens j*page_size ..
 * (j+1)*page_size-1 of sequence b.  Entries past ceil(len/page_size) are
 * never read.
 *
 * Masks.  Attention is causal.  window > 0 adds the sliding rule
 * q_pos - kv_pos < window, a strict less-than; window <= 0 is pure causal
 * (commit log 1847125, the entry that builds one block mask per attention
 * regime).  Query head h reads KV head h / (Hq/Hkv).
 *
 * Supported shapes: head_dim in {64, 128, 256, 512} (512: the full-attention
 * layers of the dual-regime model, commit log 1847125, Gemma-4-E2B-it engine
 * entry, "Dual attention regimes"); page_size in {16, 32};
 * Hq a multiple of Hkv with Hq/Hkv <= 8.  Anything else returns
 * PKV_ERR_UNSUPPORTED before any HIP call.
 *
 * Errors.  Problems the host can see (null pointers, shapes, sizes) return
 * a status before anything is enqueued.  Contents of device arrays (slot
 * numbers, table entries, lengths) are the caller's contract and cannot be
 * checked without a synchronisation: kernels skip or clamp anything out of
 * range so that no access leaves the buffers, but the results for such rows
 * are unspecified.  A failed launch returns PKV_ERR_HIP.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;

enum {
  PKV_OK = 0,
  PKV_ERR_NULL_ARG = 1,             /* a required pointer is NULL                     */
  PKV_ERR_BAD_SHAPE = 2,            /* a size or count is out of range or inconsistent */
  PKV_ERR_UNSUPPORTED = 3,          /* head_dim / page_size / grouping not built       */
  PKV_ERR_WORKSPACE_TOO_SMALL = 4,  /* split-K workspace smaller than required         */
  PKV_ERR_HIP = 5                   /* a kernel launch failed                          */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* pkv_status_string(pkv_status s);

/*
 * Compute units and peak shader clock (kHz) of the current HIP device, as
 * the runtime reports them (what the MFMA and bandwidth peaks are quoted
 * against).  Both pointers are host memory written on success.  Returns
 * PKV_ERR_NULL_ARG for a NULL pointer, PKV_ERR_HIP if the runtime query
 * fails.
 */
pkv_status pkv_device_info(int32_t* compute_units, int32_t* max_clock_khz);

/*
 * Measurement aid: a plain streaming read of `bytes` bytes at `buffer`
 * (device memory, 16-byte aligned, bytes a multiple of 16) by `workgroups`
 * workgroups of 256 threads, each lane reading 16-byte chunks with the
 * streaming (nontemporal) cache policy of the decode kernels and folding
 * them into a checksum; workgroup w writes words 4w .. 4w+3 of `sink`
 * (device memory of 4*workgroups uint32).  The time it takes is the
 * device's practical HBM read ceiling, the context for the decode
 * kernels' fraction of the 8 TB/s peak.  BAD_SHAPE for a size that is not
 * a multiple of 16 or a workgroup count outside 1..2^20; bytes = 0
 * enqueues nothing.
 */
pkv_status pkv_stream_read(const void* buffer, size_t bytes, int32_t workgroups, uint32_t* sink,
                           hipStream_t stream);

/*
 * Slot addressing: the physical pool row of every new token.
 *
 * Sequence j contributes Lq_j = cu_seq_lens_q[j+1]-cu_seq_lens_q[j] new
 * tokens and holds Lk_j = cu_seq_lens_k[j+1]-cu_seq_lens_k[j] tokens once
 * they are cached; its token r is logical position p = Lk_j - Lq_j + r and
 * goes to slot block_tables[j][p/page_size]*page_size + p%page_size.  This
 * is the address of the engine's in-kernel cache write (commit log 1847125,
 * flex_attention paged-KV engine entry, "Files"); the packing follows the
 * varlen cu_seq_lens convention (CB sync-driver commit 5f3e1c9,
 * "qwen3_grpo_unified.py fixes").
 *
 *   block_tables   int32 [num_seqs, max_pages_per_seq]     (device, read)
 *   cu_seq_lens_q  int32 [num_seqs+1], [0] = 0              (device, read)
 *   cu_seq_lens_k  int32 [num_seqs+1], [0] = 0              (device, read)
 *   slot_mapping   int32 [total_tokens] = cu_seq_lens_q[num_seqs] (device, written)
 *
 * A token whose page index or table entry is out of range gets slot -1
 * (which pkv_append skips).  total_tokens may be 0 (nothing is enqueued).
 */
pkv_status pkv_slot_mapping(const int32_t* block_tables, int32_t max_pages_per_seq,
                            const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                            int32_t num_seqs, int32_t total_tokens,
                            int32_t page_size, int32_t num_pages,
                            int32_t* slot_mapping, hipStream_t stream);

/*
 * Append: bit-exact copy of new K/V rows into their pool slots,
 * k_pool[h, slot_mapping[t], :] = k_new[t, h, :] (and V), for every KV head.
 * This is the engine's cache write at a physical row address (commit log
 * 1847125, flex_attention paged-KV engine entry, "Files": k_cache[addr] =
 * k_val), into the one contiguous pool the page table indexes (same entry,
 * "Why this works" item 1).
 *
 *   k_new, v_new   bf16 [num_tokens, num_kv_heads, head_dim]   (device, read)
 *   slot_mapping   int32 [num_tokens]; a slot < 0 or >= num_slots is skipped
 *   k_pool, v_pool bf16 [num_kv_heads, num_slots, head_dim]    (device, written)
 *
 * Two tokens with the same slot in one call give an unspecified row.
 * num_tokens may be 0.
 */
pkv_status pkv_append(const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* slot_mapping, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t head_dim,
                      uint16_t* k_pool, uint16_t* v_pool, int64_t num_slots,
                      hipStream_t stream);

/*
 * Slot addressing and append fused in one launch: the slot of each new
 * token is resolved from the block table exactly as pkv_slot_mapping does
 * and its K/V rows are copied exactly as pkv_append does, without the
 * slot array making a round trip through HBM (the engine writes the cache
 * from inside its step, commit log 1847125, flex_attention paged-KV engine
 * entry, "Files").  The pool holds num_pages*page_size slots.
 *
 *   k_new, v_new   bf16 [total_tokens, num_kv_heads, head_dim] (device, read)
 *   block_tables, cu_seq_lens_q, cu_seq_lens_k: as pkv_slot_mapping
 *   max_seqlen_q   host bound on the new rows of any one sequence
 *                  (Lq_j <= max_seqlen_q; 1 for a decode step); it sizes the
 *                  grid, and rows of a sequence past it are not written
 *   k_pool, v_pool bf16 [num_kv_heads, num_pages*page_size, head_dim]
 *                  (device, written)
 *   slot_mapping   int32 [total_tokens] (device, written) or NULL; when given
 *                  it receives, for every written row, the value
 *                  pkv_slot_mapping writes
 *
 * Tokens with slot -1 are skipped.  Two tokens with the same slot give an
 * unspecified row.  num_seqs, total_tokens or max_seqlen_q may be 0
 * (nothing is enqueued).  max_seqlen_q*num_kv_heads*head_dim/8 must stay
 * below 2^31.
 */
pkv_status pkv_append_mapped(const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                             int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen_q,
                             int32_t page_size, int32_t num_pages, int32_t num_kv_heads,
                             int32_t head_dim, uint16_t* k_pool, uint16_t* v_pool,
                             int32_t* slot_mapping, hipStream_t stream);

/*
 * Device page allocator.  The pool is one set of pages and each sequence's
 * block-table row maps its logical pages to physical ones; pages are handed
 * out as sequences grow (commit log 1847125, flex_attention paged-KV engine
 * entry, "Why this works" item 1 and "Files").  The free pages are a stack
 * in device memory, free_pages[0 .. *free_count) with its top at
 * free_pages[*free_count - 1]; both calls run on the device (one
 * workgroup), read no host state and so can be captured in a step graph
 * ahead of the append and the attention that read the tables.
 *
 * pkv_page_alloc: sequence j, with Lq_j new and Lk_j total tokens (the
 * cu_seq_lens convention of pkv_slot_mapping), holds ceil((Lk_j-Lq_j)/
 * page_size) pages and needs ceil(Lk_j/page_size); its missing logical
 * pages, in increasing order, each take the page at the top of the stack,
 * sequences served in batch order.  All or nothing: if some row needs more
 * than max_pages_per_seq entries (*status = 1) or the stack holds fewer
 * pages than the batch needs (*status = 2), nothing is written but status.
 * On success *free_count drops by the pages taken and *status = 0.
 *
 * pkv_page_free: every sequence j with release[j] != 0 pushes its first
 * ceil(seq_lens[j]/page_size) table entries onto the stack (sequences in
 * batch order, logical order) and sets them to -1.  If the stack would
 * exceed num_pages entries, nothing is written but *status = 3.
 *
 *   cu_seq_lens_q/k int32 [num_seqs+1]; seq_lens, release int32 [num_seqs]
 *                   (device, read)
 *   block_tables    int32 [num_seqs, max_pages_per_seq] (device, read/written)
 *   free_pages      int32 [num_pages] (device; read by alloc, written by free)
 *   free_count      int32 [1] (device, read and written)
 *   status          int32 [1] (device, written) or NULL
 *
 * num_seqs = 0 enqueues nothing.  The stack's contents are the caller's
 * contract (page numbers in [0, num_pages), each page either free or owned
 * by one table row); *free_count is clamped to [0, num_pages] when read.
 * Calls that overlap on one stack race: keep them on one stream.
 */
pkv_status pkv_page_alloc(const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                          int32_t num_seqs, int32_t* block_tables, int32_t max_pages_per_seq,
                          int32_t page_size, int32_t* free_pages, int32_t* free_count,
                          int32_t num_pages, int32_t* status, hipStream_t stream);
pkv_status pkv_page_free(const int32_t* seq_lens, const int32_t* release, int32_t num_seqs,
                         int32_t* block_tables, int32_t max_pages_per_seq, int32_t page_size,
                         int32_t* free_pages, int32_t* free_count, int32_t num_pages,
                         int32_t* status, hipStream_t stream);

/*
 * Split-K planning.  Split-K cuts each row's keys into num_splits
 * partitions of pages_per_split logical pages: the flash-decoding split of
 * a long context's keys over more workgroups than the batch has rows, which
 * the decode path of the rollout engine needs at small batch (its decode
 * attention runs over the pages of a block table, commit log 1847125,
 * flex_attention paged-KV engine entry, "Why this works" items 1-2).  The
 * plan depends only on host scalars.  num_splits_requested = 0 picks a count from
 * the grid size; 1 disables splitting.  Writes the plan through the two
 * output pointers (either may be NULL).
 */
pkv_status pkv_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t page_size,
                           int32_t max_seq_len, int32_t window, int32_t num_splits_requested,
                           int32_t* num_splits, int32_t* pages_per_split);

/*
 * The decomposition pkv_decode uses for these host arguments:
 *   *method = PKV_DECODE_DIRECT  one workgroup per (sequence, KV head), one
 *                                kernel, no workspace (*count = 1);
 *             PKV_DECODE_SPLIT   split-K partials + combine (*count = splits);
 *             PKV_DECODE_STREAM  stream-K + merge (*count = persistent waves,
 *                                or at head_dim 512 persistent workgroups).
 * With num_splits_requested = 0 a batch of at most 256 (sequence, KV head)
 * rows whose query-head group is not split in two by stream-K goes direct
 * (not at head_dim 512, which always streams), up to 2048 sequences go
 * stream-K, larger batches split-K.  Either output pointer may be NULL.
 */
enum { PKV_DECODE_DIRECT = 0, PKV_DECODE_SPLIT = 1, PKV_DECODE_STREAM = 2 };
pkv_status pkv_decode_method(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                             int32_t window, int32_t num_splits_requested, int32_t* method,
                             int32_t* count);

/*
 * Bytes of device workspace pkv_decode (and pkv_decode_append) needs for
 * these arguments: the partials of the decomposition pkv_decode_method
 * picks (split-K partials, or stream-K partials and merge descriptors; the
 * flash-decoding split of the keys, sized from host scalars only as the
 * engine's capture-time reservation needs, commit log 1847125,
 * flex_attention paged-KV engine entry, "Why this works" item 3).  The
 * decomposition depends on the KV-head count (stream-K counts units per KV
 * head and splits wide query-head groups) and on the window (it bounds the
 * pages a row's keys span), so both are arguments.  Returns 0 when no
 * workspace is needed or an argument is invalid.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_kv_heads, int32_t page_size, int32_t max_seq_len,
                                  int32_t window, int32_t num_splits_requested);

/*
 * Decode attention: one query row per sequence, GQA over the paged pool.
 * Row b sits at position seq_lens[b]-1 and attends keys 0..seq_lens[b]-1
 * (its own new token included, appended beforehand), restricted by the
 * window when window > 0.  The engine's decode step runs this attention
 * over physical pages through the block table (commit log 1847125,
 * flex_attention paged-KV engine entry, "Why this works" items 1-2).
 *
 *   q              bf16 [num_seqs, num_q_heads, head_dim]       (device, read)
 *   k_pool, v_pool bf16 [num_kv_heads, num_pages*page_size, head_dim]
 *   block_tables   int32 [num_seqs, max_pages_per_seq]
 *   seq_lens       int32 [num_seqs]; 0 <= len <= min(max_seq_len, max_pages_per_seq*page_size)
 *   scale          score multiplier (typically 1/sqrt(head_dim))
 *   workspace      device scratch of pkv_decode_workspace_bytes(...) bytes;
 *                  may be NULL when that is 0
 *   out            bf16 [num_seqs, num_q_heads, head_dim]       (device, written)
 *
 * num_splits = 0 picks the decomposition with pkv_decode_method: one
 * kernel with one workgroup per (sequence, KV head) row for small batches,
 * the stream-K partition (pkv_decode_stream + pkv_decode_stream_merge) up
 * to 2048 sequences, else split-K with an automatic split count;
 * num_splits >= 1 forces split-K with that many splits (1 = no split, no
 * workspace).
 *
 * A row with no key (seq_lens[b] == 0) is written as zeros.  Results are
 * deterministic and independent of the physical page order.
 */
pkv_status pkv_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                      const int32_t* block_tables, int32_t max_pages_per_seq,
                      const int32_t* seq_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                      float scale, int32_t window, int32_t num_splits,
                      void* workspace, size_t workspace_bytes,
                      uint16_t* out, hipStream_t stream);

/*
 * pkv_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * caller passes inputs and outputs only; the decode partials (split-K
 * partials, or stream-K partials and merge descriptors) live in a scratch
 * array of 16 MiB in the library's device memory, one per GPU, held until
 * the process ends.  The call allocates nothing and frees nothing; its
 * first call on a device looks up that device's scratch address (make that
 * call outside a capture).  Same arguments and results as pkv_decode,
 * without the workspace: bit-identical to pkv_decode with a workspace of
 * its own.  Returns PKV_ERR_WORKSPACE_TOO_SMALL, before any HIP call, when
 * pkv_decode_workspace_bytes for these arguments exceeds 16 MiB (split-K
 * over very large batches; stream-K of every supported shape fits on a
 * device of up to 256 compute units).
 *
 * Every call on a GPU shares that GPU's scratch and rewrites what it reads,
 * so nothing needs clearing between calls; calls that overlap in time on
 * one GPU (several streams, or several threads) race on it and give
 * unspecified results: keep them on one stream.
 */
pkv_status pkv_decode_noalloc(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                              float scale, int32_t window, int32_t num_splits,
                              uint16_t* out, hipStream_t stream);

/*
 * Decode step with its append fused in: what pkv_append_mapped of one new
 * token per row followed by pkv_decode computes, in the decode launch.  The
 * engine writes the new token's K/V into the cache from inside its captured
 * decode step (commit log 1847125, flex_attention paged-KV engine entry,
 * "Files": the in-kernel k_cache[addr] = k_val write; "Why this works" item
 * 3: the step replayed as one graph per batch-size bucket), and here that
 * write happens in the decode kernel itself: the wave that attends a row's
 * last page takes the new token's K and V from k_new / v_new rather than from
 * the pool and writes them to the token's slot.  No other wave of the launch
 * reads that pool row, so no ordering inside the launch is needed.
 *
 *   k_new, v_new   bf16 [num_seqs, num_kv_heads, head_dim] (device, read):
 *                  row b's new token, at position seq_lens[b] - 1
 *   k_pool, v_pool bf16 [num_kv_heads, num_pages*page_size, head_dim]
 *                  (device, read, and the new rows written)
 * Other arguments, the workspace and the result: as pkv_decode.
 *
 * Row b's new token goes to slot block_tables[b][p/page_size]*page_size +
 * p%page_size with p = seq_lens[b] - 1, exactly as pkv_append_mapped with
 * cu_seq_lens_q = 0, 1, .., num_seqs and cu_seq_lens_k = the running sum of
 * seq_lens places it.  A row with seq_lens[b] == 0 (a padded graph-bucket
 * row) appends nothing and is written as zeros; a row whose table entry for
 * that page is unusable, or whose length exceeds its table, writes nothing
 * to the pool.  At head_dim 512 the stream-K decode has the workgroup that
 * reads a row's last tile write the new token to the pool before it
 * requests that tile (no other workgroup reads it); with explicit splits the
 * rows are appended by a launch of their own before the decode (same
 * result).  num_pages*page_size must stay below 2^31.
 */
pkv_status pkv_decode_append(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_tables,
                             int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                             float scale, int32_t window, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/*
 * Decode, split-K half (the partial pass of flash-decoding over the
 * block-table pages of each row, commit log 1847125, flex_attention
 * paged-KV engine entry, "Why this works" items 1-2): for split s of row b,
 * over the allowed keys on
 * logical pages [p0 + s*pages_per_split, p0 + (s+1)*pages_per_split) where
 * p0 is the page of the row's first allowed key (0 without a window),
 * writes in float32
 *   part_m[b, h, s]    = log2(e) * max_i x_i          (-inf if the split is empty)
 *   part_l[b, h, s]    = sum_i exp(x_i - max)         (0 if empty)
 *   part_acc[b, h, s, :] = sum_i exp(x_i - max) v_i   (0 if empty)
 * with x_i = scale * (k_i . q).  Arrays: part_m, part_l [num_seqs,
 * num_q_heads, num_splits]; part_acc [num_seqs, num_q_heads, num_splits,
 * head_dim].  Splits beyond a row's pages are written as empty.
 * num_splits * pages_per_split must cover the longest row's key pages.
 */
pkv_status pkv_decode_split(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, int32_t max_pages_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                            float scale, int32_t window,
                            int32_t num_splits, int32_t pages_per_split,
                            float* part_m, float* part_l, float* part_acc,
                            hipStream_t stream);

/*
 * Decode, combine half (the log-sum-exp merge of flash-decoding's
 * partials, in a fixed order so that reruns are bit-identical: the engine's
 * drift verification asserts deterministic inference, commit log 1847125,
 * Gemma-4-E2B-it engine entry):
 * merges the partials of pkv_decode_split in a fixed split order, out = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s with
 * M = max_s m_s; a row whose splits are all empty is written as zeros.
 *   out  bf16 [num_seqs, num_q_heads, head_dim]
 */
pkv_status pkv_decode_combine(const float* part_m, const float* part_l, const float* part_acc,
                              int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t num_splits, uint16_t* out, hipStream_t stream);

/*
 * Decode, stream-K half: the flash-decoding split of pkv_decode_split with
 * the split points chosen over the whole batch instead of per row, so that
 * a batch of mixed lengths (the continuous-batching decode step, commit log
 * 1847125, flex_attention paged-KV engine entry, "Why this works" items
 * 1-2) keeps every wave equally busy.  The units of the batch -- every logical page that
 * holds an allowed key, for every KV head of every row, ordered by row,
 * then KV head, then page -- are cut into num_waves contiguous ranges of
 * equal size (unit counts differ by at most one), one per persistent wave,
 * so the work per wave does not depend on the length mix.  A (row, KV head)
 * whose pages all fall in one range is finished by that wave and written to
 * out; one cut by range boundaries leaves a partial per piece in the
 * workspace for pkv_decode_stream_merge.  Rows with seq_lens[b] == 0 are
 * written as zeros.  The result depends on num_waves only through rounding
 * order and is deterministic for a given num_waves.  With head_dim >= 128
 * and an even query-head group larger than 4, each KV head counts as two
 * units per page (each half of the group is a unit of its own, reading the
 * page again from L2), which keeps one wave's accumulators in registers.
 *
 *   num_waves   >= 1; pkv_decode_stream_waves gives the count pkv_decode
 *               uses (a few waves per compute unit of the current device).
 *               At head_dim 512 the partition is over workgroups of four
 *               waves instead (each wave owns 128 dims of every key, the
 *               units are 32-key tiles, one workgroup per compute unit), and
 *               num_waves counts those workgroups.
 *   workspace   pkv_decode_stream_workspace_bytes(num_waves, ...) bytes;
 *               holds partials and merge descriptors, and is fully rewritten
 *               by every call (no initialisation needed)
 *   num_seqs    <= 2048 (the row lengths are scanned in LDS)
 * Other arguments as for pkv_decode.
 */
pkv_status pkv_decode_stream_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                                   int32_t window, int32_t* num_waves);
size_t pkv_decode_stream_workspace_bytes(int32_t num_waves, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim);
pkv_status pkv_decode_stream(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t page_size, int32_t num_pages,
                             float scale, int32_t window, int32_t num_waves,
                             void* workspace, size_t workspace_bytes,
                             uint16_t* out, hipStream_t stream);

/*
 * Decode, stream-K merge half (the same log-sum-exp merge as
 * pkv_decode_combine, in fixed wave order): combines the pieces of every
 * cut (row, KV head) left by pkv_decode_stream (same workspace, num_waves and shapes),
 * in wave order, into out.  Rows pkv_decode_stream finished are untouched.
 */
pkv_status pkv_decode_stream_merge(const void* workspace, size_t workspace_bytes,
                                   int32_t num_waves, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   uint16_t* out, hipStream_t stream);

/*
 * Varlen causal prefill over the paged pool.  Query rows of num_seqs
 * sequences are packed back to back: rows cu_seq_lens_q[j] ..
 * cu_seq_lens_q[j+1]-1 belong to sequence j, whose K/V are its first
 * Lk_j = cu_seq_lens_k[j+1]-cu_seq_lens_k[j] cached tokens (this step's
 * rows appended beforehand).  Row r of sequence j sits at position
 * Lk_j - Lq_j + r (bottom-right alignment, so a chunk after a cached prefix
 * sees the prefix).  The cu_seq_lens_q/k and host max_seqlen_q/k arguments
 * follow the varlen interface the CB paged kernel takes on every forward
 * (CB sync-driver commit 5f3e1c9, "qwen3_grpo_unified.py fixes"; benchmarks
 * README, "Flash Attention 4 on Blackwell (sm_100)" item 2).
 *
 *   q              bf16 [total_q, num_q_heads, head_dim]        (device, read)
 *   block_tables   int32 [num_seqs, max_pages_per_seq]
 *   cu_seq_lens_q  int32 [num_seqs+1], cu_seq_lens_k int32 [num_seqs+1]
 *   max_seqlen_q   >= every Lq_j (host); max_seqlen_k >= every Lk_j (host)
 *   out            bf16 [total_q, num_q_heads, head_dim]        (device, written)
 *
 * Caller contract: 0 <= Lq_j <= Lk_j <= max_pages_per_seq*page_size.
 *
 * Decode rows may be packed into the same call as one-row sequences
 * (Lq_j = 1, position Lk_j - 1): such a sequence is attended with the
 * decode machinery (its pages split over the workgroup's waves) rather than
 * with 32-row MFMA tiles, so a step mixing decode rows and prompts is one
 * launch per layer (the CB paged kernel likewise takes the whole mixed
 * batch through cu_seq_lens_q on every forward).  At head_dim 512 the
 * one-row sequences take a second launch (the head-dim-split kernel, whose
 * MFMA columns are the group's heads) after the prompts' launch, both on
 * `stream`.
 */
pkv_status pkv_prefill_varlen(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_tables, int32_t max_pages_per_seq,
                              const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
                              int32_t num_seqs, int32_t total_q,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_pages,
                              float scale, int32_t window,
                              uint16_t* out, hipStream_t stream);

/*
 * pkv_prefill_varlen with the key range of long work cut into runs (the
 * flash-decoding split of the keys, applied to the varlen batch).  A short
 * prefill whose workgroups are few -- a handful of chunks with long cached
 * prefixes under a sliding window, beside decode rows, fill a few dozen of
 * the 256 compute units -- spreads its key tiles over more workgroups.
 * Every query block of a prompt or chunk is cut into the same S runs of
 * whole key tiles, S = min(num_splits, tiles of its last block / 4 at head
 * dim 256, 2 at 128 and 64) (no cut below twice that); a one-row sequence
 * (a decode row) has its pages cut the same way with at least four pages
 * per wave and run.  Each run leaves a partial per (query row, head)
 * (running max in log2 units, sum, unnormalised accumulator), and a second
 * launch merges the rows that were cut, in fixed run order; rows that were
 * not cut are written by the first launch.  The result equals
 * pkv_prefill_varlen's within floating-point order and is deterministic
 * for a given num_splits.
 *
 * Arguments are those of pkv_prefill_varlen, plus:
 *   num_splits       1..64; 1 is exactly pkv_prefill_varlen (no workspace)
 *   workspace        device memory of at least
 *                    pkv_prefill_split_workspace_bytes(total_q, num_q_heads,
 *                    head_dim, num_splits) bytes, owned by the caller:
 *                    partials [Tq, Hq, num_splits] (max, sum) and
 *                    [Tq, Hq, num_splits, D] (accumulator), then each row's
 *                    run count; overwritten by every call (it needs no
 *                    clearing); used only when num_splits > 1
 * Errors: as pkv_prefill_varlen; BAD_SHAPE for num_splits outside 1..64;
 * UNSUPPORTED for num_splits > 1 at head_dim 512; NULL_ARG or
 * WORKSPACE_TOO_SMALL for the workspace.
 */
size_t pkv_prefill_split_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                         int32_t num_splits);
pkv_status pkv_prefill_varlen_split(const uint16_t* q, const uint16_t* k_pool,
                                    const uint16_t* v_pool, const int32_t* block_tables,
                                    int32_t max_pages_per_seq, const int32_t* cu_seq_lens_q,
                                    const int32_t* cu_seq_lens_k, int32_t num_seqs, int32_t total_q,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_size, int32_t num_pages, float scale,
                                    int32_t window, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/*
 * Step graphs.  The rollout engine captures one decode step per batch-size
 * bucket (1, 2, 4, 8, ...) during warm-up, dispatches each step to the
 * nearest bucket at or above the live batch, pads it with no-op rows and
 * replays the graph; graph replay is its main lever against launch cost
 * (commit log 1847125, flex_attention paged-KV engine entry, "Why this
 * works" item 3).  Every pkv_* launch above is replay-safe: lengths, tables
 * and slot positions are read from device arrays when the kernels run, and
 * grids depend on host arguments only, which a graph freezes.  A padded
 * decode row is a row with seq_len 0 (its output is zero) and, for
 * pkv_append_mapped, no new tokens (cu_seq_lens_q repeats its last value).
 *
 * pkv_graph_begin starts capturing `stream` (not the legacy null stream;
 * thread-local capture mode): pkv_* calls on it are then recorded, not
 * run.  pkv_graph_end stops the capture and instantiates the graph into
 * *graph (set to NULL on failure; a call that failed during the capture
 * makes pkv_graph_end fail too, and the capture is ended either way).
 * pkv_graph_launch enqueues one replay on any stream of the same device;
 * the buffers it was captured with must stay allocated and must not be
 * resized.  pkv_graph_nodes counts the graph's kernel nodes and its other
 * nodes (memset, copy, ...).  pkv_graph_destroy frees the graph (NULL is
 * accepted); replays already enqueued still complete.
 */
typedef struct pkv_graph_s* pkv_graph;

pkv_status pkv_graph_begin(hipStream_t stream);
pkv_status pkv_graph_end(hipStream_t stream, pkv_graph* graph);
pkv_status pkv_graph_launch(pkv_graph graph, hipStream_t stream);
pkv_status pkv_graph_nodes(pkv_graph graph, int32_t* kernel_nodes, int32_t* other_nodes);
pkv_status pkv_graph_destroy(pkv_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
