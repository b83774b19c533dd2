// Shared declarations of the decode kernels: launch arguments and the attended range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

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
  int max_ctx;                 // host bound on context lengths; longer ones are clamped to it
  int max_chunks, chunk;       // rows per chunk; chunks per sequence at most
  float qscale;                // scale * log2(e): logits are kept in base 2
  float* ws_ml;                // partial running max and running sum, pairs
  float* ws_acc;               // partial accumulators, head_dim floats each
  int* ws_arrive;              // streaming path: per-range arrival counters, zero between calls
  int total_waves;             // streaming path: wavefronts sharing the tile list
};

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

}  // namespace pa
