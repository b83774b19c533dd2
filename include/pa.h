/*
 * pa.h -- C ABI of the paged K/V cache kernels for AMD Instinct MI355X (gfx950).
 *
 * Three operations make up one decode step over a paged K/V cache:
 *
 *   pa_copy_pages  whole-page copies that implement copy-on-write of shared
 *                  pages (silicon-compiler chapter 15 "A Paged KV Cache and
 *                  Sliding-Window Attention", section "The model": before a
 *                  request writes into a page that others also hold, it copies
 *                  the page and writes into its own copy);
 *   pa_store_kv    the scatter of each step's new K/V rows into their slots
 *                  (mini-sglang part 4, the sections on the KV buffer and its
 *                  store: the pool is viewed as token rows and a slot list
 *                  indexes that view);
 *   pa_decode      single-query attention of every sequence over its rows,
 *                  reached through a per-sequence block table, optionally
 *                  limited to the last W rows (silicon chapter 15, sections
 *                  "The problem" and "The model"; pa_decode_sinks also keeps
 *                  the first rows, "Exercises"; pa_prefill takes several
 *                  query tokens per sequence; pa_update_tables writes a
 *                  step's table changes with one scatter; the dense result it must
 *                  equal is the checkpoint of the tiny-llm page "Paged KV
 *                  Cache", section "Correctness Checkpoint").
 *
 * Common conventions
 *   - Pools: one K pool and one V pool, each [num_pages, page_size, kv_heads,
 *     head_dim] (token-major, the layout of the KV buffer in mini-sglang part 4),
 *     row-major, of element type `dtype`; or head-major, [num_pages, kv_heads,
 *     page_size, head_dim], when the dtype argument carries PA_HEAD_MAJOR.  A
 *     "slot" is page * page_size + offset in both; with token-major pools it is a
 *     row of the flattened view [num_pages * page_size, kv_heads, head_dim].  For
 *     more than one layer, pass each layer's base pointers.
 *   - dtype: PA_F32 (IEEE binary32) or PA_BF16 (bfloat16, upper half of a
 *     binary32), optionally OR-ed with PA_HEAD_MAJOR (see below).  q, new rows
 *     and pools share one element type; decode output is fp32.
 *   - Every pointer argument is caller-owned device memory unless stated.
 *     The library allocates nothing, keeps no state between calls, never
 *     synchronizes, and enqueues all work on `stream` (a hipStream_t; NULL is
 *     the default stream).  Results are valid after stream-ordered completion.
 *     Calls are thread-safe.
 *   - Host-visible arguments are validated and a negative status is returned
 *     without launching anything.  Device-resident index data (tables, slots,
 *     copy lists, context lengths) is not validated on the host, since that
 *     would need a synchronization; the kernels skip any index that falls
 *     outside the pool instead of accessing it, so a bad index yields wrong
 *     numbers, never an out-of-bounds access.
 *   - Alignment: pointers must be aligned to their element size; 16-byte
 *     aligned pools and rows take the vectorized paths.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 };

/*
 * Pool layout flag, OR-ed into the dtype argument of every call that takes the
 * pools: they are head-major, [num_pages, kv_heads, page_size, head_dim].  A
 * page holds page_size * kv_heads * head_dim elements in either layout, so
 * slots, block tables and page copies do not change; only where a (token,
 * kv head) row sits inside its page does.  Head-major puts the rows of one kv
 * head in one contiguous block per page, so an attention pass over one head
 * reads whole blocks instead of one head_dim slice of every token row.  With
 * page_size 1 both layouts are the same bytes.  Every result is bit-identical
 * to the same call on the token-major pool holding the same rows.
 */
#define PA_HEAD_MAJOR 0x100

enum pa_status {
  PA_OK = 0,
  PA_EINVAL = -1,        /* a null pointer, a non-positive size, inconsistent sizes  */
  PA_EUNSUPPORTED = -2,  /* a valid combination this build has no kernel for         */
  PA_EWORKSPACE = -3,    /* decode workspace missing or smaller than required        */
  PA_ELAUNCH = -4,       /* the HIP runtime rejected a launch                         */
  PA_ESCRATCH = -5       /* pa_decode_noalloc: the call needs more than its buffer    */
};

/* Human-readable name of a status code; never NULL. */
const char* pa_status_string(int status);

/*
 * Decode and prefill workspaces.  A call that needs a workspace (see pa_decode)
 * takes device memory whose first PA_WORKSPACE_HEADER bytes hold arrival
 * counters -- one per group of rows whose partial results are combined inside
 * the launch -- and whose remaining bytes hold those partial results.  The
 * counters must be zero when a call starts: allocate the workspace zero-filled,
 * or call pa_reset_workspace once.  A call that runs to completion puts every
 * counter it raised back to zero, and no path writes anything else into the
 * header, so calls of any shape and on any path can share the workspace one
 * after the other.  A call that does not complete (its kernel aborted, the
 * device reset, a fault) can leave counters raised; later calls on that
 * workspace would then return wrong results without an error, so reset the
 * workspace before using it again.  Calls that overlap in time must not share
 * a workspace.
 */
#define PA_WORKSPACE_HEADER 4096

/*
 * pa_reset_workspace -- zero the counter header of a workspace of
 * workspace_bytes bytes (its first min(workspace_bytes, PA_WORKSPACE_HEADER)
 * bytes), in stream order.  The partial-result area needs no clearing.
 *   workspace     device memory, 4-byte aligned; may be NULL only with
 *                 workspace_bytes == 0 (a no-op).
 * Errors: PA_EINVAL for a NULL or misaligned pointer with workspace_bytes > 0,
 * PA_ELAUNCH when the launch is rejected.
 */
int pa_reset_workspace(void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_store_kv -- write new K/V rows into their slots.
 *   k_pool, v_pool  [num_pages, page_size, kv_heads, head_dim] (with
 *                   PA_HEAD_MAJOR: [num_pages, kv_heads, page_size, head_dim]),
 *                   written in place.
 *   k_new, v_new    [num_tokens, kv_heads, head_dim], contiguous.
 *   slot_mapping    device int32 [num_tokens]: flat slot of each row; a negative
 *                   slot skips that row.  Slots must be distinct within a call
 *                   (two rows for one slot: unspecified which one lands).
 * Every element of each row is copied bit for bit; no other byte of the pools
 * changes.  num_tokens == 0 is a no-op.
 * Errors: PA_EINVAL for a non-positive size or an unknown dtype or flag;
 * PA_EUNSUPPORTED when a row (token-major) or a head's row (head-major) is not
 * a multiple of 4 bytes.
 */
int pa_store_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_pages,
                int32_t page_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                void* stream);

/*
 * pa_copy_pages -- pool[dst_pages[i]] = pool[src_pages[i]] for K and V, whole pages.
 *   src_pages, dst_pages  device int32 [num_copies].  Targets must be distinct and
 *                         disjoint from the sources, so the order does not matter.
 * Bit-exact; num_copies == 0 is a no-op.
 */
int pa_copy_pages(void* k_pool, void* v_pool, const int32_t* src_pages,
                  const int32_t* dst_pages, int32_t num_copies, int32_t num_pages,
                  int32_t page_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                  void* stream);

/*
 * pa_decode -- one query token per sequence against its cached rows.
 *   out           fp32 [num_seqs, q_heads, head_dim], written.
 *   q             [num_seqs, q_heads, head_dim], pool dtype.
 *   block_tables  device int32 [num_seqs, bt_stride] (rows beyond num_seqs are
 *                 ignored): entry j is the physical page of logical page j, or
 *                 -1 for a page released by the window.  Logical row i lives at
 *                 page block_tables[s][i / page_size], offset i % page_size.
 *                 A raw token-slot table is the same call with page_size = 1
 *                 and num_pages counted in rows.
 *   context_lens  device int32 [num_seqs]: rows of each sequence, including the
 *                 token being decoded, whose K/V row must already be stored.
 *                 0 gives a zero output row.
 *   window        <= 0: attend rows [0, L); W > 0: rows [L - min(L, W), L).
 *   max_context_len  host upper bound on every context length; <= 0 means
 *                 bt_stride * page_size.  Sizes the workspace and the grid;
 *                 a longer context length is clamped to it.
 *   scale         logit scale (for instance 1/sqrt(head_dim)).
 *   q_heads must be a multiple of kv_heads; query head h reads kv head
 *   h / (q_heads / kv_heads).
 *   Output: out[s][h] = sum_i softmax_i(scale * <q[s][h], K_i>) * V_i over the
 *   attended rows, with fp32 accumulation.
 *   workspace     device scratch of *workspace_bytes bytes.  With workspace ==
 *                 NULL the call only stores the required size in
 *                 *workspace_bytes and returns PA_OK, also when that size is
 *                 0: a call that needs no workspace still takes a non-NULL
 *                 pointer to run.  A non-zero size includes the counter
 *                 header; the header's rules (zero before the first use,
 *                 left zero by every completed call, reset after a call that
 *                 did not complete) are stated above pa_reset_workspace.
 *   Supported: dtype PA_F32 or PA_BF16; head_dim 16, 32, 64, 128 or 256;
 *   q_heads / kv_heads <= 16; any page_size >= 1.
 */
int pa_decode(float* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
              int32_t num_seqs, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
              int32_t num_pages, int32_t page_size, int32_t window, int32_t max_context_len,
              float scale, int32_t dtype, void* workspace, size_t* workspace_bytes,
              void* stream);

/*
 * pa_decode_sinks -- pa_decode with attention sinks (silicon chapter 15,
 * section "Exercises", the attention-sink exercise): besides the window, the
 * first `sinks` rows of every sequence stay attended.
 *   sinks         0 <= sinks < window when window > 0; 0 when window <= 0.
 *                 Once L > window the attended rows are [0, sinks) and
 *                 [L - window + sinks, L) -- still `window` rows; while
 *                 L <= window every row [0, L).  sinks = 0 is pa_decode.
 *                 The block table may read -1 for the pages between the two
 *                 runs (a page holding a sink row or a window row must be
 *                 mapped; rows between them are never read or weighted).
 *   Every other argument, the workspace rules and the supported shapes are
 *   those of pa_decode (a workspace sized for sinks may be larger).
 *   Errors: PA_EINVAL for sinks < 0, or sinks > 0 without a window above it.
 */
int pa_decode_sinks(float* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                    int32_t kv_heads, int32_t head_dim, int32_t num_pages, int32_t page_size,
                    int32_t window, int32_t sinks, int32_t max_context_len, float scale,
                    int32_t dtype, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * pa_decode_hinted -- pa_decode_sinks with hints about the batch that change how
 * the rows are read, never what is computed: the output is bit-identical to
 * pa_decode_sinks with the same arguments.
 *   hints         0 or PA_HINT_UNSHARED: no physical page is attended by two
 *                 sequences of the call (no shared prefix, no fork sharing a
 *                 page), so nothing read has a reuse worth caching; the V rows are
 *                 then loaded with the non-temporal cache hint.  Wrong hints
 *                 cost time, not correctness.  Used by the streaming path (bf16,
 *                 head_dim 128, power-of-two pages, including a raw slot table
 *                 read as pages of one row); ignored elsewhere.
 *   Errors: PA_EINVAL for other hint bits; otherwise those of pa_decode_sinks.
 */
#define PA_HINT_UNSHARED 1
int pa_decode_hinted(float* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t bt_stride,
                     const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                     int32_t kv_heads, int32_t head_dim, int32_t num_pages, int32_t page_size,
                     int32_t window, int32_t sinks, int32_t hints, int32_t max_context_len,
                     float scale, int32_t dtype, void* workspace, size_t* workspace_bytes,
                     void* stream);

/*
 * pa_decode_noalloc -- pa_decode_hinted with no workspace argument and no
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, hosts that forbid allocation during a
 * step).  The workspace is a buffer of PA_NOALLOC_SCRATCH_BYTES bytes held by
 * the library in device memory: one per GPU the library runs on, kept until
 * the process ends.  Its counter header is cleared by the first call on each
 * device (a kernel on `stream`), and every completed call leaves it at zero.
 *   Arguments, results and supported shapes are those of pa_decode_hinted;
 *   the output is bit-identical to pa_decode_hinted with the same arguments.
 *   Every call on a GPU uses that GPU's one buffer: calls that overlap in
 *   time on one GPU (other streams, other threads) race and give wrong
 *   results; a call that does not complete leaves the buffer's counters
 *   raised for every later call in the process.
 *   Calls no hipMalloc, hipFree or other allocating routine.
 * Errors: those of pa_decode_hinted; PA_ESCRATCH when the call would need
 * more than PA_NOALLOC_SCRATCH_BYTES (nothing is launched).
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
int pa_decode_noalloc(float* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                      int32_t kv_heads, int32_t head_dim, int32_t num_pages, int32_t page_size,
                      int32_t window, int32_t sinks, int32_t hints, int32_t max_context_len,
                      float scale, int32_t dtype, void* stream);

/*
 * pa_prefill -- several query tokens per sequence against its cached rows: a
 * chunk of a prompt (the tiny-llm page "Paged KV Cache", section "Prefill
 * with Pages": the chunk's rows are stored into pages, here by pa_store_kv,
 * before its queries attend) or the drafted tokens of a speculative step.
 *   out           fp32 [num_q, q_heads, head_dim], written.
 *   q             [num_q, q_heads, head_dim], pool dtype.
 *   q_start       device int32 [num_seqs + 1], nondecreasing, q_start[0] = 0,
 *                 q_start[num_seqs] = num_q: the query rows of sequence s
 *                 are q_start[s] .. q_start[s+1] - 1, at most max_q_len.
 *   context_lens  device int32 [num_seqs]: rows of each sequence including
 *                 its n query tokens, whose K/V rows must already be stored;
 *                 the queries are its last n rows.
 *   Query i of a sequence (0 <= i < n) sits at row p = L - n + i and attends
 *   rows [p + 1 - min(p + 1, W), p + 1) with a window W > 0, else [0, p + 1):
 *   causal, the window counted from its own row.  A query with p < 0 (more
 *   queries than rows) gets a zero row.  n = 1 everywhere is pa_decode.
 *   max_q_len     host upper bound on the query tokens of one sequence (sizes
 *                 the grid and the workspace); rows beyond it are not written.
 *   The workspace size depends on the shape, max_q_len and the sign of scale:
 *   query it with the arguments of the call.
 *   Every other argument, the workspace rules (the counter header described
 *   above pa_reset_workspace) and the supported shapes are those of
 *   pa_decode; there are no sink rows here.
 *   Errors: PA_EINVAL also for num_q > 0 with num_seqs = 0 or max_q_len <= 0.
 */
int pa_prefill(float* out, const void* q, const int32_t* q_start, const void* k_pool,
               const void* v_pool, const int32_t* block_tables, int32_t bt_stride,
               const int32_t* context_lens, int32_t num_seqs, int32_t num_q,
               int32_t max_q_len, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
               int32_t num_pages, int32_t page_size, int32_t window, int32_t max_context_len,
               float scale, int32_t dtype, void* workspace, size_t* workspace_bytes,
               void* stream);

/*
 * pa_prefill_hinted -- pa_prefill with the hints of pa_decode_hinted, which change
 * how rows are read, never what is computed: the output is bit-identical to
 * pa_prefill with the same arguments.
 *   hints         0 or PA_HINT_UNSHARED (no physical page is attended by two
 *                 sequences of the call): the V rows are loaded with the
 *                 non-temporal cache hint on the streaming path (groups of up to
 *                 two blocks of query tokens); the tile kernel for long chunks,
 *                 whose query tiles share every K/V block, ignores it.
 *   Errors: PA_EINVAL for other hint bits; otherwise those of pa_prefill.
 */
int pa_prefill_hinted(float* out, const void* q, const int32_t* q_start, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q,
                      int32_t max_q_len, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                      int32_t num_pages, int32_t page_size, int32_t window, int32_t hints,
                      int32_t max_context_len, float scale, int32_t dtype, void* workspace,
                      size_t* workspace_bytes, void* stream);

/*
 * pa_update_tables -- one step's table changes as one scatter (the mini-sglang
 * page, part 4, section on writing the page table: new cells are written with
 * one indexed store from host-built index lists, not request by request).
 *   block_tables  device int32 [bt_rows, bt_stride], or NULL: cell
 *                 [rows[i], logical_pages[i]] = pages[i] (pages[i] < 0: -1).
 *   slot_table    device int32 [slot_rows, slot_stride], or NULL: positions
 *                 logical_pages[i] * page_size + k, k < page_size, of row
 *                 rows[i] = pages[i] * page_size + k, or dummy_slot when
 *                 pages[i] < 0 (a whole page of positions, spare capacity
 *                 included, as that page's token expansion writes them).
 *   rows, logical_pages, pages  device int32 [num_updates].
 *   An update outside a table (row, column or position) is skipped for that
 *   table.  Two updates of one cell in one call are a caller error (either
 *   value may remain).  Ownership: every pointer is caller-owned device memory.
 *   Errors: PA_EINVAL for num_updates < 0, page_size <= 0, a non-positive
 *   stride of a table that is passed, or missing index lists.
 */
int pa_update_tables(int32_t* block_tables, int32_t bt_stride, int32_t bt_rows,
                     int32_t* slot_table, int32_t slot_stride, int32_t slot_rows,
                     int32_t dummy_slot, const int32_t* rows, const int32_t* logical_pages,
                     const int32_t* pages, int32_t num_updates, int32_t page_size,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
