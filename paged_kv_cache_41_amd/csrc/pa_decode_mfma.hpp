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

  int L, lo, n;
  live_range(a.ctx[s], a.window, a.max_ctx, L, lo, n);
  const int nch = (n + a.chunk - 1) / a.chunk;
  float* out_base = a.out + ((size_t)s * a.q_heads + (size_t)g * G) * HD;
  if (nch == 0) {
    if (c == 0)
      for (int i = tid; i < G * HD; i += 64 * NW) out_base[i] = 0.f;
    return;
  }
  if (c >= nch) return;

  const int P = a.page_size;
  const int lp = 31 - __clz(P);  // page size is a power of two on this path
  const int t_begin = lo + c * a.chunk;
  const int t_end = min(L, t_begin + a.chunk);
  const int j0 = t_begin >> lp;
  const int nj = ((t_end - 1) >> lp) - j0 + 1;
  const int32_t* btr = a.block_tables + (size_t)s * a.bt_stride;
  for (int i = tid; i < nj; i += 64 * NW) {
    const int pg = btr[j0 + i];
    s_pages[i] = (pg >= 0 && pg < a.num_pages) ? pg : -1;
  }
  __syncthreads();

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v_pool);
  const size_t rs = (size_t)Hkv * HD;  // elements per token row
  const size_t head_off = (size_t)g * HD;
  const int col = lane & 15;           // K token / score head / V 16-byte column block
  const int grp = lane >> 4;           // K head_dim slice / score token group / V token

  // query vectors of the group as the B operand: head col, head_dim slice grp
  bf16x8 qb[4];
  {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((size_t)s * a.q_heads + (size_t)g * G + col) * HD + grp * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qb[j] = as_bf16x8(col < G ? *reinterpret_cast<const uint4*>(qrow + 8 * j) : zero);
  }

  const int ntile = (t_end - t_begin + TILE - 1) / TILE;

  auto load_tile = [&](int tile, Tile& T) {
    const int t0 = t_begin + tile * TILE;
    const int tk = t0 + col;
    bool ok = tk < t_end;
    int pg = ok ? s_pages[(tk >> lp) - j0] : -1;
    ok = ok && pg >= 0;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if (ok) {
      const uint16_t* src = kp + ((size_t)pg * P + (tk & (P - 1))) * rs + head_off + grp * 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) T.k[j] = *reinterpret_cast<const uint4*>(src + 8 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) T.k[j] = zero;
    }
    T.valid = __ballot(ok);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = grp + 4 * i;
      const int tv = t0 + tt;
      if ((T.valid >> tt) & 1) {
        const int pv = s_pages[(tv >> lp) - j0];
        T.v[i] = *reinterpret_cast<const uint4*>(
            vp + ((size_t)pv * P + (tv & (P - 1))) * rs + head_off + col * 8);
      } else {
        T.v[i] = zero;
      }
    }
  };

  float m_run = -INFINITY;  // per score column (head col)
  float l_run = 0.f;
  float acc[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  float(*pt)[PROW] = s_p[w];
  Tile cur;
  if (w < ntile) load_tile(w, cur);
  for (int tile = w; tile < ntile; tile += NW) {
    Tile nxt;
    const bool more = tile + NW < ntile;
    if (more) load_tile(tile + NW, nxt);

    // scores: S[token][head] = K . q
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[j]), qb[j], sc, 0, 0, 0);
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (cur.valid >> (4 * grp + r)) & 1;
      sv[r] = ok ? sc[r] * a.qscale : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m_run, mt);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(m_run - ms);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = exp2f(sv[r] - ms);
      psum += p;
      if (col < G) pt[4 * grp + r][col] = p;
    }
    if (grp == 0 && col < G) pt[TILE][col] = alpha;
    l_run = l_run * alpha + psum;
    m_run = mn;
    wave_lds_sync();

    // P.V on the vector ALUs
    float al[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) al[h] = pt[TILE][h];
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vx[8];
      bf16x8_to_f32(cur.v[i], vx);
      const float* prow = pt[grp + 4 * i];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float p = prow[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e]);
      }
    }
    wave_lds_sync();
    if (more) cur = nxt;
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
    s_m[w][lane] = m_run;
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
