// Matrix-core decode path: bf16 pools, head_dim 128, up to 16 query heads per kv head,
// page sizes that are powers of two.
//
// Work item: one workgroup of NW wavefronts per (sequence, kv head, chunk of rows).  The
// chunk's block-table entries are staged in LDS once; wave w then takes the 16-row tiles
// w, w + NW, ... of the chunk, prefetching the next tile's K and V while it computes the
// current one.
//
// Per tile (16 rows of one kv head, 4 KiB of K and 4 KiB of V):
//   * QK^T on the matrix cores: four v_mfma_f32_16x16x32_bf16 with the K tile as the A
//     operand (row = token, lane l holds 64 contiguous bytes of token l % 16) and the
//     group's query vectors as the B operand (column = query head).  The sum over
//     head_dim is order-free, so lane group l / 16 takes head_dim slice
//     [32 (l / 16), 32 (l / 16) + 32) of both operands.  The 16x16 fp32 score tile
//     lands with query head l % 16 in column and tokens 4 (l / 16) .. +3 in the four
//     accumulator registers.
//   * Online softmax in base 2 on that tile: running max per head across the wave
//     (shuffles over lane groups), rescale factor, probabilities, running sum.
//   * The probabilities and the rescale factors go through a small LDS tile to the
//     P.V layout, where lane l owns 16 contiguous bytes (8 columns) of token l / 16 + 4 i
//     of V, i = 0..3: each V row of 256 bytes is read by 16 consecutive lanes.  P.V runs
//     on the vector ALUs in fp32 (the probabilities are never rounded to bf16).
// At the end the waves' (max, sum, accumulator) are combined in LDS; a sequence whose
// rows fit one chunk writes its output directly, others write a partial that the
// merge kernel combines.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa.h"
#include "pa_common.hpp"

namespace pa {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;        // head_dim of this path
constexpr int TILE = 16;       // rows per tile = M of the matrix-core op
constexpr int NW = 4;          // wavefronts per workgroup
constexpr int MAX_CHUNK = 1024;
constexpr int PROW = 20;       // floats per row of the P tile (16 heads + pad)

__device__ __forceinline__ void wave_lds_sync() {
  // LDS traffic of one wavefront is processed in order; this keeps the compiler from
  // moving LDS accesses across the exchange point and waits for issued LDS operations.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

struct Tile {
  uint4 k[4];        // K: token (lane % 16), bytes [64 (lane / 16), +64) of its head row
  uint4 v[4];        // V: token (lane / 16 + 4 i), bytes [16 (lane % 16), +16)
  uint64_t valid;    // bit t: token t0 + t is attended and mapped
};

// Rescale threshold in base-2 logit units: the running reference max is only raised
// when a tile's max exceeds it by more than this, so probabilities stay below 2^8
// and most tiles skip the rescale entirely.  The result is the same softmax: every
// probability and the running sum use one reference until it changes.
constexpr float RESCALE_T = 8.f;

template <int GMAX>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ int s_pages[MAX_CHUNK + 2];
  __shared__ float s_p[NW][TILE + 1][PROW];
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ float s_acc[NW][GMAX][HD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.kv_heads;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int c = rest % a.max_chunks;
  const int s = rest / a.max_chunks;
  const int G = a.group;

  int L, sl, lo;
  sink_ranges(a.ctx[s], a.window, a.sinks, a.max_ctx, L, sl, lo);
  const int nch = chunk_count(L, sl, lo, a.chunk);
  float* out_base = a.out + ((size_t)s * a.q_heads + (size_t)g * G) * HD;
  if (nch == 0) {
    if (c == 0)
      for (int i = tid; i < G * HD; i += 64 * NW) out_base[i] = 0.f;
    return;
  }
  if (c >= nch) return;

  const int P = a.page_size;
  const int lp = 31 - __clz(P);  // page size is a power of two on this path
  int t_begin, t_end;
  chunk_span(c, L, sl, lo, a.chunk, t_begin, t_end);
  const int j0 = t_begin >> lp;
  const int nj = ((t_end - 1) >> lp) - j0 + 1;
  const int32_t* btr = a.block_tables + (size_t)(a.row_seq ? a.row_seq[s] : s) * a.bt_stride;
  for (int i = tid; i < nj; i += 64 * NW) {
    const int pg = btr[j0 + i];
    s_pages[i] = (pg >= 0 && pg < a.num_pages) ? pg : -1;
  }
  __syncthreads();

  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const uint32_t row_bytes = (uint32_t)a.row_stride * 2;
  const uint32_t page_bytes = (uint32_t)Hkv * HD * 2 * (uint32_t)P;
  const int col = lane & 15;           // K token / score head / V 16-byte column block
  const int grp = lane >> 4;           // K head_dim slice / score token group / V token
  const uint32_t head_off = (uint32_t)g * (uint32_t)a.head_stride * 2;
  const uint32_t k_lane = head_off + grp * 64;
  const uint32_t v_lane = head_off + col * 16;
  const int last_page = a.num_pages - 1;

  // query vectors of the group as the B operand: head col, head_dim slice grp
  bf16x8 qb[4];
  {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((size_t)s * a.q_heads + (size_t)g * G + (col < G ? col : 0)) * HD +
                           grp * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 8 * j);
      qb[j] = as_bf16x8(col < G ? v : zero);
    }
  }

  const int ntile = (t_end - t_begin + TILE - 1) / TILE;

  auto row_addr = [&](const char* base, int pg, int t, uint32_t lane_off) {
    // pg is clamped into [0, num_pages) by the callers; a page is < 4 GiB
    return reinterpret_cast<const uint4*>(base + (uint64_t)(uint32_t)pg * page_bytes +
                                          ((uint32_t)(t & (P - 1)) * row_bytes + lane_off));
  };

  // Loads are branch-free so that the compiler can keep several tiles in flight: a row
  // past the end of the chunk, or one whose table entry is unmapped (a caller error
  // inside the attended range), is still read from a clamped in-pool address, and the
  // validity mask keeps it out of the softmax (scores) and out of P.V (values are
  // replaced, not multiplied, so poison in unread pages cannot leak).
  auto load_tile = [&](int tile, Tile& T) {
    const int t0 = t_begin + tile * TILE;
    const int tk = min(t0 + col, t_end - 1);
    const int ek = s_pages[(tk >> lp) - j0];
    T.valid = __ballot(t0 + col < t_end && ek >= 0);
    const uint4* kp = row_addr(kbase, min(max(ek, 0), last_page), tk, k_lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) T.k[j] = kp[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tv = min(t0 + grp + 4 * i, t_end - 1);
      const int ev = s_pages[(tv >> lp) - j0];
      T.v[i] = *row_addr(vbase, min(max(ev, 0), last_page), tv, v_lane);
    }
  };

  float m_ref = -INFINITY;  // reference max of score column col (its query head)
  float l_run = 0.f;
  float acc[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  float(*pt)[PROW] = s_p[w];

  auto compute = [&](const Tile& T) {
    // scores: S[token][head] = K . q
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.k[j]), qb[j], sc, 0, 0, 0);
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (T.valid >> (4 * grp + r)) & 1;
      sv[r] = ok ? sc[r] * a.qscale : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // raise the reference when some head's tile max passes it by more than RESCALE_T
    const bool raise = __ballot(col < G && mt > m_ref + RESCALE_T) != 0;
    if (raise) {
      const float mn = fmaxf(m_ref, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);  // 0 when m_ref = -inf
      l_run *= alpha;
      m_ref = mn;
      if (grp == 0 && col < G) pt[TILE][col] = alpha;
    }
    const float ms = m_ref == -INFINITY ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(sv[r] - ms);
      psum += p;
      if (col < G) pt[4 * grp + r][col] = p;
    }
    l_run += psum;
    wave_lds_sync();

    // P.V on the vector ALUs
    if (raise) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float al = pt[TILE][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
    }
    const bool full = T.valid == ~0ull;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vx[8];
      bf16x8_to_f32(T.v[i], vx);
      if (!full && !((T.valid >> (grp + 4 * i)) & 1)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vx[e] = 0.f;
      }
      const float* prow = pt[grp + 4 * i];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float p = prow[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e]);
      }
    }
    wave_lds_sync();
  };

  // Three register stages: compute one tile while the next two are in flight.  Loads
  // are issued unconditionally; past this wave's last tile they re-read that tile (a
  // cache hit), so no branch separates a load from its use and the compiler can keep
  // the stages in fixed registers.  Only the compute steps are guarded.
  const int ntw = ntile > w ? (ntile - w + NW - 1) / NW : 0;  // tiles of this wave
  if (ntw > 0) {
    auto tile_of = [&](int i) { return w + NW * min(i, ntw - 1); };
    Tile A, B, C;
    load_tile(tile_of(0), A);
    load_tile(tile_of(1), B);
    for (int i = 0; i < ntw; i += 3) {
      load_tile(tile_of(i + 2), C);
      compute(A);
      load_tile(tile_of(i + 3), A);
      if (i + 1 < ntw) compute(B);
      load_tile(tile_of(i + 4), B);
      if (i + 2 < ntw) compute(C);
    }
  }

  // per-wave totals: running sum over the score token groups, accumulator over V token groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16, 64);
      acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
    }
  if (lane < 16) {
    s_m[w][lane] = m_ref;
    s_l[w][lane] = l_run;
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[w][h][lane * 8 + e] = acc[h][e];
  }
  __syncthreads();

  // combine the waves: thread handles (head, column) pairs
  for (int i = tid; i < G * HD; i += 64 * NW) {
    const int h = i / HD, d = i % HD;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, s_m[k][h]);
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const float f = exp2f(s_m[k][h] - M);
        den += f * s_l[k][h];
        num += f * s_acc[k][h][d];
      }
    }
    if (nch == 1) {
      out_base[(size_t)h * HD + d] = den > 0.f ? num / den : 0.f;
    } else {
      const size_t part = ((size_t)s * a.q_heads + (size_t)g * G + h) * a.max_chunks + c;
      if (d == 0) {
        a.ws_ml[2 * part] = M;
        a.ws_ml[2 * part + 1] = den;
      }
      a.ws_acc[part * HD + d] = num;
    }
  }
}

inline bool eligible(int dtype, int head_dim, int group, int page_size) {
  return dtype == PA_BF16 && head_dim == HD && group >= 1 && group <= 16 && page_size > 0 &&
         (page_size & (page_size - 1)) == 0;
}

// Rows per workgroup: aim for about 2048 workgroups when contexts average half the
// longest, in powers of two between 64 and MAX_CHUNK.
inline int chunk_for(int num_seqs, int kv_heads, int max_live) {
  const double want = (double)num_seqs * kv_heads * (max_live / 2.0) / 2048.0;
  int c = 64;
  while (c < want && c < MAX_CHUNK) c <<= 1;
  return c;
}

inline int launch(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)((int64_t)a.num_seqs * a.max_chunks * a.kv_heads);
  if (a.group <= 4)
    hipLaunchKernelGGL(decode_mfma_kernel<4>, dim3(blocks), dim3(64 * NW), 0, st, a);
  else if (a.group <= 8)
    hipLaunchKernelGGL(decode_mfma_kernel<8>, dim3(blocks), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<16>, dim3(blocks), dim3(64 * NW), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mfma
}  // namespace pa
