// Paged K/V cache kernels for gfx950 (AMD Instinct MI355X, CDNA4) behind the C ABI of pa.h.
//
// Three operations of a decode step over a paged cache:
//   * store_kv   -- scatter of the step's new K/V rows to their slots (mini-sglang
//                   part 4, the KV buffer and its store: the pool is a list of token
//                   rows and a slot list picks the row each new token goes to);
//   * copy_pages -- whole-page copies behind copy-on-write (silicon-compiler chapter 15,
//                   section "The model": a shared page is copied before it is written);
//   * decode     -- single-query attention over the rows a block table reaches, limited
//                   to the last W rows when a window is given (same chapter, sections
//                   "The problem" and "The model"), split over chunks of rows with an
//                   online (running max / running sum) softmax, then merged.
//
// Layout (all row-major): pool [num_pages, page_size, kv_heads, head_dim]; a token row is
// kv_heads * head_dim contiguous elements, a (token, kv head) row head_dim contiguous
// elements.  Logical row i of sequence s lives at page bt[s][i / page_size], offset
// i % page_size.  Element offsets are computed in 64 bits.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pa.h"
#include "pa_common.hpp"
#include "pa_decode_mfma.hpp"
#include "pa_decode_stream.hpp"
#include "pa_prefill_tile.hpp"

namespace pa {

// ------------------------------------------------------------------------------------
// store_kv: one block per new token (grid-stride over tokens).  Rows move in units of U
// (16 bytes when every pointer and the row size allow it, else 4 bytes).  A new row is
// kv_heads pieces of units_per_head units; in the pool, slot page * P + r puts piece h at
// unit page * P * units_per_row + r * row_units + h * head_units (token-major pools pass
// the whole row as one piece).
// ------------------------------------------------------------------------------------
template <typename U>
__global__ __launch_bounds__(256) void store_kv_kernel(
    U* __restrict__ kp, U* __restrict__ vp, const U* __restrict__ kn, const U* __restrict__ vn,
    const int32_t* __restrict__ slots, int num_tokens, int64_t num_slots, int units_per_row,
    int page_size, int units_per_head, int row_units, int head_units) {
  for (int t = blockIdx.x; t < num_tokens; t += gridDim.x) {
    const int slot = slots[t];
    if (slot < 0 || (int64_t)slot >= num_slots) continue;
    const U* ks = kn + (size_t)t * units_per_row;
    const U* vs = vn + (size_t)t * units_per_row;
    const size_t base = (size_t)(slot / page_size) * page_size * units_per_row +
                        (size_t)(slot % page_size) * row_units;
    for (int i = threadIdx.x; i < units_per_row; i += blockDim.x) {
      const int h = i / units_per_head;
      const size_t o = base + (size_t)h * head_units + (i - h * units_per_head);
      kp[o] = ks[i];
      vp[o] = vs[i];
    }
  }
}

// ------------------------------------------------------------------------------------
// copy_pages: blockIdx.y walks the copy list, blockIdx.z picks K (0) or V (1), x and the
// threads stride over the page in units of U.
// ------------------------------------------------------------------------------------
template <typename U>
__global__ __launch_bounds__(256) void copy_pages_kernel(
    U* __restrict__ kp, U* __restrict__ vp, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, int num_copies, int num_pages, int64_t units_per_page) {
  U* pool = blockIdx.z ? vp : kp;
  for (int c = blockIdx.y; c < num_copies; c += gridDim.y) {
    const int s = src[c], d = dst[c];
    if (s < 0 || s >= num_pages || d < 0 || d >= num_pages) continue;
    const U* from = pool + (size_t)s * units_per_page;
    U* to = pool + (size_t)d * units_per_page;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < units_per_page;
         i += (int64_t)gridDim.x * blockDim.x)
      to[i] = from[i];
  }
}

// ------------------------------------------------------------------------------------
// decode, generic VALU path (any dtype, head_dim 16..256, group <= 16, any page size).
//
// One wavefront per (sequence, kv head, chunk).  A (token, kv head) row of head_dim
// elements is spread over LPT lanes holding 16 bytes each, so one wave covers TPW
// tokens per iteration with fully used 16-byte loads.  Logits are reduced across the
// LPT lanes with xor shuffles, leaving every lane of a token with the logits of all
// query heads of the group; the running max is shared by the whole wave, the running
// sum and the output accumulator are kept per token group and summed at the end.
// Logits are in base 2: q is pre-multiplied by scale * log2(e) and exp2 is used.
// ------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&x)[16 / sizeof(T)]);

template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T, int D, int GMAX>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPT = D / EPL;
  constexpr int TPW = 64 / LPT;
  static_assert(D % EPL == 0 && LPT <= 64 && (LPT & (LPT - 1)) == 0, "unsupported head_dim");

  const int lane = threadIdx.x;
  const int Hkv = a.kv_heads;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int c = rest % a.max_chunks;
  const int s = rest / a.max_chunks;
  const int G = a.group;
  const int sub = lane % LPT;
  const int tok = lane / LPT;

  int L, sl, lo;
  sink_ranges(a.ctx[s], a.window, a.sinks, a.max_ctx, L, sl, lo);
  const int nch = chunk_count(L, sl, lo, a.chunk);
  float* outp = a.out + ((size_t)s * a.q_heads + (size_t)g * G) * D + sub * EPL;
  if (nch == 0) {
    if (c == 0 && tok == 0)
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) outp[(size_t)h * D + e] = 0.f;
    return;
  }
  if (c >= nch) return;

  const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)s * a.q_heads + (size_t)g * G) * D + sub * EPL;
  float qv[GMAX][EPL];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      load16<T>(qb + (size_t)h * D, qv[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[h][e] *= a.qscale;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[h][e] = 0.f;
    }
  }
  float m[GMAX], l[GMAX], acc[GMAX][EPL];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const T* kp = reinterpret_cast<const T*>(a.k_pool);
  const T* vp = reinterpret_cast<const T*>(a.v_pool);
  const size_t page_elems = (size_t)a.page_size * Hkv * D;
  const int32_t* btr = a.block_tables + (size_t)(a.row_seq ? a.row_seq[s] : s) * a.bt_stride;
  int t_begin, t_end;
  chunk_span(c, L, sl, lo, a.chunk, t_begin, t_end);

  for (int t0 = t_begin; t0 < t_end; t0 += TPW) {
    const int t = t0 + tok;
    bool valid = t < t_end;
    float kx[EPL], vx[EPL];
    if (valid) {
      const int page = btr[t / a.page_size];
      valid = page >= 0 && page < a.num_pages;
      if (valid) {
        const size_t off = (size_t)page * page_elems + (size_t)(t % a.page_size) * a.row_stride +
                           (size_t)g * a.head_stride + sub * EPL;
        load16<T>(kp + off, kx);
        load16<T>(vp + off, vx);
      }
    }
    if (!valid) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kx[e] = vx[e] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sc = fmaf(qv[h][e], kx[e], sc);
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) sc += __shfl_xor(sc, o, 64);
      if (!valid) sc = -INFINITY;
      float mt = sc;
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
      const float mnew = fmaxf(m[h], mt);
      if (mnew == -INFINITY) continue;
      const float alpha = exp2f(m[h] - mnew);
      const float p = valid ? exp2f(sc - mnew) : 0.f;
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e] * alpha);
      m[h] = mnew;
    }
  }

#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) continue;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) {
      l[h] += __shfl_xor(l[h], o, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
    }
  }
  if (tok != 0) return;
  if (nch == 1) {
    for (int h = 0; h < G; ++h) {
      const float inv = 1.f / l[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) outp[(size_t)h * D + e] = acc[h][e] * inv;
    }
  } else {
    for (int h = 0; h < G; ++h) {
      const size_t part = ((size_t)s * a.q_heads + (size_t)g * G + h) * a.max_chunks + c;
      if (sub == 0) {
        a.ws_ml[2 * part] = m[h];
        a.ws_ml[2 * part + 1] = l[h];
      }
      float* wa = a.ws_acc + part * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) wa[e] = acc[h][e];
    }
  }
}

// ------------------------------------------------------------------------------------
// merge: one block per (sequence, query head) whose rows were split over several chunks.
// out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, chunks in fixed order.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void merge_kernel(DecodeArgs a, int D) {
  const int h = blockIdx.x % a.q_heads;
  const int s = blockIdx.x / a.q_heads;
  int L, sl, lo;
  sink_ranges(a.ctx[s], a.window, a.sinks, a.max_ctx, L, sl, lo);
  const int nch = chunk_count(L, sl, lo, a.chunk);
  if (nch <= 1) return;
  const size_t base = ((size_t)s * a.q_heads + h) * a.max_chunks;
  const float* ml = a.ws_ml + 2 * base;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[2 * c]);
  float den = 0.f;
  for (int c = 0; c < nch; ++c) den += exp2f(ml[2 * c] - M) * ml[2 * c + 1];
  const float inv = 1.f / den;
  const float* acc = a.ws_acc + base * D;
  float* out = a.out + ((size_t)s * a.q_heads + h) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float num = 0.f;
    for (int c = 0; c < nch; ++c) num += exp2f(ml[2 * c] - M) * acc[(size_t)c * D + d];
    out[d] = num * inv;
  }
}

using DecodeFn = void (*)(DecodeArgs);

template <typename T, int D>
DecodeFn pick_generic(int group) {
  if (group <= 1) return decode_generic_kernel<T, D, 1>;
  if (group <= 2) return decode_generic_kernel<T, D, 2>;
  if (group <= 4) return decode_generic_kernel<T, D, 4>;
  if (group <= 8) return decode_generic_kernel<T, D, 8>;
  return decode_generic_kernel<T, D, 16>;
}

template <typename T>
DecodeFn pick_generic_d(int head_dim, int group) {
  switch (head_dim) {
    case 16: return pick_generic<T, 16>(group);
    case 32: return pick_generic<T, 32>(group);
    case 64: return pick_generic<T, 64>(group);
    case 128: return pick_generic<T, 128>(group);
    case 256: return pick_generic<T, 256>(group);
    default: return nullptr;
  }
}

inline int elt_bytes(int dtype) { return dtype == PA_F32 ? 4 : 2; }

// Tiles per wavefront at least: the start-up and the end of a range stay small next to
// its stream (12, 16 and 30 measured no better on the batch-64 and window workloads).
constexpr int stream_tiles_per_wave = 22;

// Wavefronts of the streaming decode: one workgroup of four per compute unit of a 256-CU
// MI355X, so the whole grid is resident at once (a second workgroup per unit measured
// slower: more concurrent streams, each with less of its own data in flight).
constexpr int stream_waves_max = 1024;
static_assert(stream_waves_max * sizeof(int) <= WS_HEADER, "counters must fit the header");

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rows per chunk: a power of two between 16 and 512, about one eighth of the longest
// attended range, so long contexts split into enough chunks to fill the chip and
// short ones stay in one chunk (no merge).
inline int pick_chunk(int max_live) {
  int want = (max_live + 7) / 8;
  int c = 16;
  while (c < want && c < 512) c <<= 1;
  return c;
}

// Rows path: one work item per (row, chunk, kv head) on the chunked matrix-core kernel or
// the VALU kernel, then the merge of rows split over several chunks.
inline int launch_rows(const DecodeArgs& a, DecodeFn generic, bool fast, int head_dim,
                       hipStream_t st) {
  const int64_t blocks = (int64_t)a.num_seqs * a.max_chunks * a.kv_heads;
  if (blocks * 256 > INT32_MAX) return PA_EUNSUPPORTED;
  if (fast) {
    if (mfma::launch(a, st) != 0) return PA_ELAUNCH;
  } else {
    hipLaunchKernelGGL(generic, dim3((unsigned)blocks), dim3(64), 0, st, a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;
  if (a.max_chunks > 1) {
    const int64_t mb = (int64_t)a.num_seqs * a.q_heads;
    if (mb > INT32_MAX) return PA_EUNSUPPORTED;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)mb), dim3(128), 0, st, a, head_dim);
    if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;
  }
  return PA_OK;
}

// Table updates: update i maps logical page logical[i] of table row rows[i] to page
// pages[i] (-1: released) in the block table, and its page_size positions to the page's
// slots (or the dummy slot) in the slot table.  Cells outside a table are skipped.
__global__ __launch_bounds__(64) void update_tables_kernel(
    int32_t* __restrict__ bt, int bt_stride, int bt_rows, int32_t* __restrict__ st,
    int st_stride, int st_rows, int dummy_slot, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ logical, const int32_t* __restrict__ pages, int n, int P) {
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int r = rows[i], j = logical[i], p = pages[i];
    if (bt && threadIdx.x == 0 && r >= 0 && r < bt_rows && j >= 0 && j < bt_stride)
      bt[(size_t)r * bt_stride + j] = p >= 0 ? p : -1;
    if (st && r >= 0 && r < st_rows && j >= 0) {
      for (int k = threadIdx.x; k < P; k += 64) {
        const int64_t pos = (int64_t)j * P + k;
        if (pos < st_stride)
          st[(size_t)r * st_stride + pos] = p >= 0 ? (int32_t)((int64_t)p * P + k) : dummy_slot;
      }
    }
  }
}

// Zero the first n bytes of a workspace (its counter header): 4-byte stores, the odd
// tail bytes by one thread.
__global__ __launch_bounds__(256) void zero_header_kernel(unsigned char* p, int n) {
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  for (int i = threadIdx.x; i < n / 4; i += 256) w[i] = 0u;
  if (threadIdx.x == 0)
    for (int i = n / 4 * 4; i < n; ++i) p[i] = 0;
}

// Query row r of a prefill chunk as a row of its own: its sequence (the last s with
// q_start[s] <= r) and its context, position + 1 (0 when it lies before row 0 or outside
// its sequence's rows).
__global__ __launch_bounds__(256) void prefill_rows_kernel(const int32_t* q_start,
                                                           const int32_t* ctx, int num_seqs,
                                                           int num_q, int max_ctx,
                                                           int32_t* row_seq, int32_t* row_ctx) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= num_q) return;
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int q0 = q_start[lo], n = q_start[lo + 1] - q0, i = r - q0;
  const int c = ctx[lo];
  const int L = c > 0 ? (c < max_ctx ? c : max_ctx) : 0;
  const int p = L - n + i;
  row_seq[r] = lo;
  row_ctx[r] = (i >= 0 && i < n && p >= 0) ? p + 1 : 0;
}

}  // namespace pa

using namespace pa;

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported combination";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_ELAUNCH: return "kernel launch failed";
    case PA_ESCRATCH: return "the call needs more scratch than the no-allocation buffer holds";
    default: return "unknown status";
  }
}

extern "C" int pa_store_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, int32_t num_tokens, int32_t num_pages,
                           int32_t page_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                           void* stream) {
  if (num_tokens < 0 || num_pages <= 0 || page_size <= 0 || kv_heads <= 0 || head_dim <= 0)
    return PA_EINVAL;
  bool head_major;
  if (!split_format(dtype, dtype, head_major)) return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_EINVAL;
  const int64_t head_bytes = (int64_t)head_dim * elt_bytes(dtype);
  const int64_t row_bytes = head_bytes * kv_heads;
  // a head-major pool moves a row head by head: each piece must be whole units
  const int64_t piece = head_major ? head_bytes : row_bytes;
  if (piece % 4) return PA_EUNSUPPORTED;
  const int64_t num_slots = (int64_t)num_pages * page_size;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int grid = num_tokens < 65535 ? num_tokens : 65535;
  int rs, hs;
  pool_strides(head_major, page_size, kv_heads, head_dim, rs, hs);
  const int eb = elt_bytes(dtype);
  if (piece % 16 == 0 && aligned16(k_pool) && aligned16(v_pool) && aligned16(k_new) &&
      aligned16(v_new)) {
    hipLaunchKernelGGL(store_kv_kernel<uint4>, dim3(grid), dim3(128), 0, st,
                       (uint4*)k_pool, (uint4*)v_pool, (const uint4*)k_new, (const uint4*)v_new,
                       slot_mapping, num_tokens, num_slots, (int)(row_bytes / 16), page_size,
                       (int)(piece / 16), rs * eb / 16, hs * eb / 16);
  } else {
    hipLaunchKernelGGL(store_kv_kernel<uint32_t>, dim3(grid), dim3(128), 0, st,
                       (uint32_t*)k_pool, (uint32_t*)v_pool, (const uint32_t*)k_new,
                       (const uint32_t*)v_new, slot_mapping, num_tokens, num_slots,
                       (int)(row_bytes / 4), page_size, (int)(piece / 4), rs * eb / 4,
                       hs * eb / 4);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

extern "C" int pa_copy_pages(void* k_pool, void* v_pool, const int32_t* src_pages,
                             const int32_t* dst_pages, int32_t num_copies, int32_t num_pages,
                             int32_t page_size, int32_t kv_heads, int32_t head_dim,
                             int32_t dtype, void* stream) {
  if (num_copies < 0 || num_pages <= 0 || page_size <= 0 || kv_heads <= 0 || head_dim <= 0)
    return PA_EINVAL;
  bool head_major;   // a page holds the same bytes in either layout: copied whole
  if (!split_format(dtype, dtype, head_major)) return PA_EINVAL;
  if (num_copies == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_pages || !dst_pages) return PA_EINVAL;
  const int64_t page_bytes = (int64_t)page_size * kv_heads * head_dim * elt_bytes(dtype);
  if (page_bytes % 4) return PA_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int gy = num_copies < 65535 ? num_copies : 65535;
  if (page_bytes % 16 == 0 && aligned16(k_pool) && aligned16(v_pool)) {
    const int64_t units = page_bytes / 16;
    const int gx = (int)((units + 256 * 4 - 1) / (256 * 4));
    hipLaunchKernelGGL(copy_pages_kernel<uint4>, dim3(gx, gy, 2), dim3(256), 0, st,
                       (uint4*)k_pool, (uint4*)v_pool, src_pages, dst_pages, num_copies,
                       num_pages, units);
  } else {
    const int64_t units = page_bytes / 4;
    const int gx = (int)((units + 256 * 4 - 1) / (256 * 4));
    hipLaunchKernelGGL(copy_pages_kernel<uint32_t>, dim3(gx, gy, 2), dim3(256), 0, st,
                       (uint32_t*)k_pool, (uint32_t*)v_pool, src_pages, dst_pages, num_copies,
                       num_pages, units);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

static int decode_entry(float* out, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                        int32_t kv_heads, int32_t head_dim, int32_t num_pages,
                        int32_t page_size, int32_t window, int32_t sinks, int32_t hints,
                        int32_t max_context_len, float scale, int32_t dtype, void* workspace,
                        size_t* workspace_bytes, void* stream) {
  if (!workspace_bytes) return PA_EINVAL;
  if (hints & ~PA_HINT_UNSHARED) return PA_EINVAL;
  if (sinks < 0 || (sinks > 0 && (window <= 0 || sinks >= window))) return PA_EINVAL;
  if (num_seqs < 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 || num_pages <= 0 ||
      page_size <= 0 || bt_stride <= 0)
    return PA_EINVAL;
  if (q_heads % kv_heads) return PA_EINVAL;
  bool head_major;
  if (!split_format(dtype, dtype, head_major)) return PA_EINVAL;
  if (!(scale == scale)) return PA_EINVAL;
  const int group = q_heads / kv_heads;
  const int64_t table_rows = (int64_t)bt_stride * page_size;
  if (max_context_len <= 0) max_context_len = table_rows > INT32_MAX ? INT32_MAX : (int32_t)table_rows;
  if ((int64_t)max_context_len > table_rows) return PA_EINVAL;
  if (group > 16) return PA_EUNSUPPORTED;

  DecodeFn generic = dtype == PA_F32 ? pick_generic_d<float>(head_dim, group)
                                     : pick_generic_d<uint16_t>(head_dim, group);
  if (!generic) return PA_EUNSUPPORTED;

  const int max_live = window > 0 && window < max_context_len ? window : max_context_len;
  // sink rows form a run of their own only where the window can cut a context
  const int run_sinks = window > 0 && window < max_context_len ? sinks : 0;
  DecodeArgs a{};
  a.hints = hints;
  a.sinks = window > 0 ? sinks : 0;
  pool_strides(head_major, page_size, kv_heads, head_dim, a.row_stride, a.head_stride);
  // Streaming path over head sets: a tile may take the same rows of hq consecutive kv
  // heads; the kernel then sees kv_heads / hq heads of group x hq query heads each.
  const int hq = stream::head_set(group, kv_heads, page_size);
  const int vkv = kv_heads / hq, vgroup = group * hq;
  if (stream::eligible(dtype, head_dim, vgroup, page_size, num_seqs, bt_stride, vkv,
                       max_live, run_sinks)) {
    // balanced streaming path: wavefronts and chunks sized to the largest possible list
    const int64_t tiles_max = stream::tiles_bound(num_seqs, vkv, max_live, run_sinks);
    // about 22 tiles per wavefront at least (so the start-up and the end of a range stay
    // small next to its stream), at most stream_waves_max
    int64_t waves = tiles_max / stream_tiles_per_wave;
    if (waves > stream_waves_max) waves = stream_waves_max;
    if (waves < stream::NW) waves = stream::NW;
    waves = (waves + stream::NW - 1) / stream::NW * stream::NW;
    // With a window every segment holds at most window / 16 + 1 tiles, so segments are
    // often about equal: a grid of ceil(segs / k) workgroups, k = ceil(segs / 256), gives
    // each workgroup k or k - 1 whole segments, which lets the kernel use its aligned
    // partition (pieces of a cut segment combined in LDS) when the segments are even
    const int64_t segs = (int64_t)num_seqs * vkv;
    if (window > 0 && window < max_context_len && segs >= 64) {
      const int64_t wg_max = stream_waves_max / stream::NW;
      const int64_t k = (segs + wg_max - 1) / wg_max;
      waves = stream::NW * ((segs + k - 1) / k);
      a.try_aligned = 1;
    }
    const size_t need = stream::workspace_bytes((int)waves, vgroup);
    if (!workspace) {
      *workspace_bytes = need;
      return PA_OK;
    }
    if (*workspace_bytes < need) return PA_EWORKSPACE;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_EINVAL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
        !aligned16(workspace))
      return PA_EUNSUPPORTED;
    if ((int64_t)kv_heads * head_dim * 2 * page_size > UINT32_MAX) return PA_EUNSUPPORTED;
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.bt_stride = bt_stride;
    a.ctx = context_lens;
    a.num_seqs = num_seqs;
    a.q_heads = q_heads;
    a.kv_heads = vkv;
    a.group = vgroup;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.window = window > 0 ? window : 0;
    a.max_ctx = max_context_len;
    a.qscale = scale * 1.4426950408889634f;
    a.total_waves = (int)waves;
    stream::carve_workspace(a, workspace, vgroup);
    return stream::launch(a, reinterpret_cast<hipStream_t>(stream), 0, hq) == 0 ? PA_OK
                                                                               : PA_ELAUNCH;
  }
  a.chunk = pick_chunk(max_live);
  const bool fast = mfma::eligible(dtype, head_dim, group, page_size);
  if (fast) a.chunk = mfma::chunk_for(num_seqs, kv_heads, max_live);
  a.max_chunks = run_sinks > 0 ? (run_sinks + a.chunk - 1) / a.chunk +
                                     (max_live - run_sinks + a.chunk - 1) / a.chunk
                                : (max_live + a.chunk - 1) / a.chunk;
  if (a.max_chunks < 1) a.max_chunks = 1;
  const size_t parts = (size_t)num_seqs * q_heads * a.max_chunks;
  const size_t need = WS_HEADER + parts * ((size_t)head_dim + 2) * sizeof(float);
  if (!workspace) {
    *workspace_bytes = need;
    return PA_OK;
  }
  if (*workspace_bytes < need) return PA_EWORKSPACE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_EUNSUPPORTED;

  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.ctx = context_lens;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.window = window > 0 ? window : 0;
  a.max_ctx = max_context_len;
  a.qscale = scale * 1.4426950408889634f;
  a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + WS_HEADER);
  a.ws_acc = a.ws_ml + 2 * parts;

  return launch_rows(a, generic, fast, head_dim, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int pa_decode_sinks(float* out, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
                               int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                               int32_t num_pages, int32_t page_size, int32_t window,
                               int32_t sinks, int32_t max_context_len, float scale,
                               int32_t dtype, void* workspace, size_t* workspace_bytes,
                               void* stream) {
  return decode_entry(out, q, k_pool, v_pool, block_tables, bt_stride, context_lens, num_seqs,
                      q_heads, kv_heads, head_dim, num_pages, page_size, window, sinks, 0,
                      max_context_len, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_hinted(float* out, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_tables,
                                int32_t bt_stride, const int32_t* context_lens,
                                int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                int32_t head_dim, int32_t num_pages, int32_t page_size,
                                int32_t window, int32_t sinks, int32_t hints,
                                int32_t max_context_len, float scale, int32_t dtype,
                                void* workspace, size_t* workspace_bytes, void* stream) {
  return decode_entry(out, q, k_pool, v_pool, block_tables, bt_stride, context_lens, num_seqs,
                      q_heads, kv_heads, head_dim, num_pages, page_size, window, sinks, hints,
                      max_context_len, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" int pa_decode(float* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t bt_stride,
                         const int32_t* context_lens, int32_t num_seqs, int32_t q_heads,
                         int32_t kv_heads, int32_t head_dim, int32_t num_pages,
                         int32_t page_size, int32_t window, int32_t max_context_len, float scale,
                         int32_t dtype, void* workspace, size_t* workspace_bytes, void* stream) {
  return pa_decode_sinks(out, q, k_pool, v_pool, block_tables, bt_stride, context_lens,
                         num_seqs, q_heads, kv_heads, head_dim, num_pages, page_size, window, 0,
                         max_context_len, scale, dtype, workspace, workspace_bytes, stream);
}

static int prefill_entry(float* out, const void* q, const int32_t* q_start,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q, int32_t max_q_len, int32_t q_heads, int32_t kv_heads,
                         int32_t head_dim, int32_t num_pages, int32_t page_size,
                         int32_t window, int32_t hints, int32_t max_context_len, float scale,
                         int32_t dtype, void* workspace, size_t* workspace_bytes,
                         void* stream) {
  if (!workspace_bytes) return PA_EINVAL;
  if (hints & ~PA_HINT_UNSHARED) return PA_EINVAL;
  if (num_seqs < 0 || num_q < 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 ||
      num_pages <= 0 || page_size <= 0 || bt_stride <= 0)
    return PA_EINVAL;
  if (num_q > 0 && (num_seqs == 0 || max_q_len <= 0)) return PA_EINVAL;
  if (q_heads % kv_heads) return PA_EINVAL;
  bool head_major;
  if (!split_format(dtype, dtype, head_major)) return PA_EINVAL;
  if (!(scale == scale)) return PA_EINVAL;
  const int group = q_heads / kv_heads;
  const int64_t table_rows = (int64_t)bt_stride * page_size;
  if (max_context_len <= 0) max_context_len = table_rows > INT32_MAX ? INT32_MAX : (int32_t)table_rows;
  if ((int64_t)max_context_len > table_rows) return PA_EINVAL;
  if (group > 16) return PA_EUNSUPPORTED;
  DecodeFn generic = dtype == PA_F32 ? pick_generic_d<float>(head_dim, group)
                                     : pick_generic_d<uint16_t>(head_dim, group);
  if (!generic) return PA_EUNSUPPORTED;
  if (num_q == 0) {
    if (!workspace) *workspace_bytes = 0;
    return PA_OK;
  }
  const int max_q = max_q_len < num_q ? max_q_len : num_q;
  const int max_live = window > 0 && window < max_context_len ? window : max_context_len;

  DecodeArgs a{};
  pool_strides(head_major, page_size, kv_heads, head_dim, a.row_stride, a.head_stride);
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.window = window > 0 ? window : 0;
  a.max_ctx = max_context_len;
  a.qscale = scale * 1.4426950408889634f;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  // long chunks: a workgroup per tile of 128 query columns, K/V shared through LDS
  if (ptile::eligible(dtype, head_dim, group, page_size, num_seqs, kv_heads, max_q, scale)) {
    if (!workspace) {
      *workspace_bytes = 0;
      return PA_OK;
    }
    if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens)
      return PA_EINVAL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
      return PA_EUNSUPPORTED;
    a.ctx = context_lens;
    a.num_seqs = num_seqs;
    a.q_start = q_start;
    a.num_q = num_q;
    a.max_q = max_q;
    return ptile::launch(a, st) == 0 ? PA_OK : PA_ELAUNCH;
  }

  // keys one group of query tokens may attend
  const int nb = (group & (group - 1)) == 0 ? stream::multi_blocks(group, max_q) : 1;
  const int tpg = 16 / group * nb;
  const int64_t keys64 = window > 0 ? (int64_t)window + tpg - 1 : (int64_t)max_context_len;
  const int keys = (int)(keys64 < max_context_len ? keys64 : max_context_len);
  if (stream::eligible_multi(dtype, head_dim, group, page_size, num_seqs, bt_stride, kv_heads,
                             max_q, keys, nb)) {
    const int64_t tiles_max =
        stream::tiles_bound_multi(num_seqs, kv_heads, group, max_q, keys, nb);
    int64_t waves = tiles_max / stream_tiles_per_wave;
    if (waves > stream_waves_max) waves = stream_waves_max;
    if (waves < stream::NW) waves = stream::NW;
    waves = (waves + stream::NW - 1) / stream::NW * stream::NW;
    // groups of one block with a window: whole segments per workgroup when they are even
    // (as for decode; the bound on the group count sizes the grid, and a batch with fewer
    // groups keeps the flat split)
    const int64_t segs = stream::blocks_bound(num_seqs, group, max_q, nb) * kv_heads;
    if (nb == 1 && window > 0 && window < max_context_len && segs >= 64) {
      const int64_t wg_max = stream_waves_max / stream::NW;
      const int64_t k = (segs + wg_max - 1) / wg_max;
      waves = stream::NW * ((segs + k - 1) / k);
      a.try_aligned = 1;
    }
    const size_t need = stream::workspace_bytes((int)waves, 16 * nb);
    if (!workspace) {
      *workspace_bytes = need;
      return PA_OK;
    }
    if (*workspace_bytes < need) return PA_EWORKSPACE;
    if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens)
      return PA_EINVAL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
        !aligned16(workspace))
      return PA_EUNSUPPORTED;
    if ((int64_t)kv_heads * head_dim * 2 * page_size > UINT32_MAX) return PA_EUNSUPPORTED;
    a.ctx = context_lens;
    a.num_seqs = num_seqs;
    a.q_start = q_start;
    a.num_q = num_q;
    a.max_q = max_q;
    a.total_waves = (int)waves;
    a.hints = hints;
    stream::carve_workspace(a, workspace, 16 * nb);
    return stream::launch(a, st, nb) == 0 ? PA_OK : PA_ELAUNCH;
  }

  // every query row as a row of its own: its sequence and context first, then the rows path
  a.chunk = pick_chunk(max_live);
  const bool fast = mfma::eligible(dtype, head_dim, group, page_size);
  if (fast) a.chunk = mfma::chunk_for(num_q, kv_heads, max_live);
  a.max_chunks = (max_live + a.chunk - 1) / a.chunk;
  if (a.max_chunks < 1) a.max_chunks = 1;
  const size_t rows_bytes = ((size_t)num_q * 2 * sizeof(int32_t) + 255) / 256 * 256;
  const size_t parts = (size_t)num_q * q_heads * a.max_chunks;
  const size_t need = WS_HEADER + rows_bytes + parts * ((size_t)head_dim + 2) * sizeof(float);
  if (!workspace) {
    *workspace_bytes = need;
    return PA_OK;
  }
  if (*workspace_bytes < need) return PA_EWORKSPACE;
  if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens)
    return PA_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_EUNSUPPORTED;
  int32_t* row_seq = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + WS_HEADER);
  int32_t* row_ctx = row_seq + num_q;
  hipLaunchKernelGGL(prefill_rows_kernel, dim3((unsigned)((num_q + 255) / 256)), dim3(256), 0,
                     st, q_start, context_lens, num_seqs, num_q, max_context_len, row_seq,
                     row_ctx);
  if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;
  a.ctx = row_ctx;
  a.row_seq = row_seq;
  a.num_seqs = num_q;
  a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + WS_HEADER +
                                     rows_bytes);
  a.ws_acc = a.ws_ml + 2 * parts;
  return launch_rows(a, generic, fast, head_dim, st);
}

extern "C" int pa_prefill(float* out, const void* q, const int32_t* q_start, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q,
                          int32_t max_q_len, int32_t q_heads, int32_t kv_heads,
                          int32_t head_dim, int32_t num_pages, int32_t page_size,
                          int32_t window, int32_t max_context_len, float scale, int32_t dtype,
                          void* workspace, size_t* workspace_bytes, void* stream) {
  return prefill_entry(out, q, q_start, k_pool, v_pool, block_tables, bt_stride, context_lens,
                       num_seqs, num_q, max_q_len, q_heads, kv_heads, head_dim, num_pages,
                       page_size, window, 0, max_context_len, scale, dtype, workspace,
                       workspace_bytes, stream);
}

extern "C" int pa_prefill_hinted(float* out, const void* q, const int32_t* q_start,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int32_t bt_stride,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q,
                                 int32_t max_q_len, int32_t q_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t num_pages, int32_t page_size,
                                 int32_t window, int32_t hints, int32_t max_context_len,
                                 float scale, int32_t dtype, void* workspace,
                                 size_t* workspace_bytes, void* stream) {
  return prefill_entry(out, q, q_start, k_pool, v_pool, block_tables, bt_stride, context_lens,
                       num_seqs, num_q, max_q_len, q_heads, kv_heads, head_dim, num_pages,
                       page_size, window, hints, max_context_len, scale, dtype, workspace,
                       workspace_bytes, stream);
}

extern "C" int pa_reset_workspace(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u)) return PA_EINVAL;
  const int n = (int)(workspace_bytes < WS_HEADER ? workspace_bytes : WS_HEADER);
  hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<unsigned char*>(workspace), n);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

// ------------------------------------------------------------------------------------
// No-allocation decode: the workspace is a file-scope device array.  Each GPU the library
// runs on holds its own copy (at its own address) until the process ends.  Host code
// never passes the array's name to a kernel: on the host that name is a stand-in, not a
// device address.  The address is taken once per device with hipGetSymbolAddress, with
// that device current, and kept here.
// ------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];       // device address of `scratch`, per device ordinal
bool scratch_zeroed[kMaxDevices];     // its counter header has been cleared once

// This device's scratch, its counter header cleared on first use (stream-ordered before
// the caller's kernels; every completed call leaves the counters at zero after that).
int device_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return PA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ELAUNCH;
    scratch_ptr[dev] = p;
  }
  if (!scratch_zeroed[dev]) {
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(256), 0, st,
                       reinterpret_cast<unsigned char*>(scratch_ptr[dev]), (int)WS_HEADER);
    if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;
    scratch_zeroed[dev] = true;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}
}  // namespace

extern "C" int pa_decode_noalloc(float* out, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int32_t bt_stride, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t num_pages, int32_t page_size,
                                 int32_t window, int32_t sinks, int32_t hints,
                                 int32_t max_context_len, float scale, int32_t dtype,
                                 void* stream) {
  // the size this call's path needs (validates every host-visible argument, no HIP call)
  size_t need = 0;
  int rc = decode_entry(out, q, k_pool, v_pool, block_tables, bt_stride, context_lens, num_seqs,
                        q_heads, kv_heads, head_dim, num_pages, page_size, window, sinks, hints,
                        max_context_len, scale, dtype, nullptr, &need, stream);
  if (rc != PA_OK) return rc;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ESCRATCH;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = device_scratch(st, &ws)) != PA_OK) return rc;
  size_t have = PA_NOALLOC_SCRATCH_BYTES;
  return decode_entry(out, q, k_pool, v_pool, block_tables, bt_stride, context_lens, num_seqs,
                      q_heads, kv_heads, head_dim, num_pages, page_size, window, sinks, hints,
                      max_context_len, scale, dtype, ws, &have, stream);
}

extern "C" int pa_update_tables(int32_t* block_tables, int32_t bt_stride, int32_t bt_rows,
                                int32_t* slot_table, int32_t slot_stride, int32_t slot_rows,
                                int32_t dummy_slot, const int32_t* rows,
                                const int32_t* logical_pages, const int32_t* pages,
                                int32_t num_updates, int32_t page_size, void* stream) {
  if (num_updates < 0 || page_size <= 0) return PA_EINVAL;
  if (block_tables && (bt_stride <= 0 || bt_rows < 0)) return PA_EINVAL;
  if (slot_table && (slot_stride <= 0 || slot_rows < 0)) return PA_EINVAL;
  if (num_updates == 0 || (!block_tables && !slot_table)) return PA_OK;
  if (!rows || !logical_pages || !pages) return PA_EINVAL;
  const int grid = num_updates < 65535 ? num_updates : 65535;
  hipLaunchKernelGGL(update_tables_kernel, dim3(grid), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), block_tables, bt_stride, bt_rows,
                     slot_table, slot_stride, slot_rows, dummy_slot, rows, logical_pages, pages,
                     num_updates, page_size);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}
