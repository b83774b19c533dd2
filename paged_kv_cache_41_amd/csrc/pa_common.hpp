// Shared declarations of the decode kernels: launch arguments and the attended range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Every decode and prefill workspace starts with this many bytes of arrival counters,
// whatever path the call takes: the streaming kernel keeps one int per wavefront range
// there (at most 1024 ranges) and every other path leaves the bytes alone, so a
// workspace used by calls of different shapes or paths never sees partial results where
// a later call expects counters.  Partials start right after the header.
constexpr size_t WS_HEADER = PA_WORKSPACE_HEADER;

struct DecodeArgs {
  float* out;                  // [num_seqs, q_heads, head_dim]
  const void* q;               // [num_seqs, q_heads, head_dim]
  const void* k_pool;          // [num_pages, page_size, kv_heads, head_dim]
  const void* v_pool;
  const int32_t* block_tables; // [num_seqs, bt_stride]
  const int32_t* ctx;          // [num_seqs]
  int bt_stride;
  int num_seqs, q_heads, kv_heads, group;
  int num_pages, page_size, window;
  int sinks;                   // rows at the start kept besides the window (0 <= sinks < window)
  int max_ctx;                 // host bound on context lengths; longer ones are clamped to it
  int max_chunks, chunk;       // rows per chunk; chunks per sequence at most
  float qscale;                // scale * log2(e): logits are kept in base 2
  float* ws_ml;                // partial running max and running sum, pairs
  float* ws_acc;               // partial accumulators, head_dim floats each
  int* ws_arrive;              // streaming path: per-range arrival counters, zero between calls
  int total_waves;             // streaming path: wavefronts sharing the tile list
  // Pool strides in elements of a token row and of a kv head within a page: token-major
  // pool [pages, page_size, kv_heads, head_dim]: kv_heads * head_dim and head_dim;
  // head-major [pages, kv_heads, page_size, head_dim]: head_dim and page_size * head_dim.
  // A page is page_size * kv_heads * head_dim elements in both.
  int row_stride, head_stride;
  int try_aligned;             // streaming path, one query token: launch the kernel that gives
                               // each workgroup whole segments when they are even
  // Several query tokens per sequence (prefill chunk, verify step).  Streaming path: the
  // query rows of sequence s are q_start[s] .. q_start[s+1]-1 of q and out (num_q rows,
  // at most max_q per sequence).  Other paths: every query row is a row of its own, with
  // its sequence in row_seq and its context (its position + 1) in ctx.
  const int32_t* q_start;
  int num_q, max_q;
  int hints;                   // PA_HINT_* bits of the decode call (0: none)
  const int32_t* row_seq;      // nullptr: row s reads the table row of sequence s
};

// The dtype argument of a call that takes a pool: the element type, with PA_HEAD_MAJOR
// set for a head-major pool.  False for an unknown element type or flag.
inline bool split_format(int32_t format, int32_t& dtype, bool& head_major) {
  head_major = (format & PA_HEAD_MAJOR) != 0;
  dtype = format & ~PA_HEAD_MAJOR;
  return dtype == PA_F32 || dtype == PA_BF16;
}

// Element strides of a token row and of a kv head within a page (DecodeArgs).
inline void pool_strides(bool head_major, int page_size, int kv_heads, int head_dim,
                         int& row_stride, int& head_stride) {
  row_stride = head_major ? head_dim : kv_heads * head_dim;
  head_stride = head_major ? page_size * head_dim : head_dim;
}

// Rows attended by a sequence with `ctx` rows: [lo, L) with L = ctx clamped to
// [0, max_ctx]; with a window W > 0 the new token and at most W - 1 before it, i.e.
// lo = L - min(L, W).  The clamp keeps every table index below bt_stride and every
// chunk index below max_chunks whatever the device-resident lengths hold.
__device__ __forceinline__ void live_range(int ctx, int window, int max_ctx, int& L, int& lo,
                                           int& n) {
  L = ctx > 0 ? (ctx < max_ctx ? ctx : max_ctx) : 0;
  lo = (window > 0 && L > window) ? L - window : 0;
  n = L - lo;
}

// The same with attention sinks (the sink exercise of "A Paged KV Cache and Sliding-Window
// Attention", section "Exercises"): once L exceeds the window W, the first S rows and the
// last W - S, i.e. rows [0, sl) and [lo, L) with sl = S and lo = L - W + S; before that
// every row, sl = 0 and lo = 0.  With S = 0 this is live_range.
__device__ __forceinline__ void sink_ranges(int ctx, int window, int sinks, int max_ctx, int& L,
                                            int& sl, int& lo) {
  L = ctx > 0 ? (ctx < max_ctx ? ctx : max_ctx) : 0;
  const bool cut = window > 0 && L > window;
  sl = cut ? sinks : 0;
  lo = cut ? L - window + sinks : 0;
}

// Chunks of `chunk` rows over the two runs: first over [0, sl), then over [lo, L).
__device__ __forceinline__ int chunk_count(int L, int sl, int lo, int chunk) {
  return (sl + chunk - 1) / chunk + (L - lo + chunk - 1) / chunk;
}
__device__ __forceinline__ void chunk_span(int c, int L, int sl, int lo, int chunk, int& tb,
                                           int& te) {
  const int ns = (sl + chunk - 1) / chunk;
  if (c < ns) {
    tb = c * chunk;
    te = min(sl, tb + chunk);
  } else {
    tb = lo + (c - ns) * chunk;
    te = min(L, tb + chunk);
  }
}

}  // namespace pa
