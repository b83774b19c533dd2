// Balanced streaming decode: bf16 pools, head_dim 128, up to 16 query heads per kv head,
// page sizes that are powers of two, up to STREAM_BMAX sequences.
//
// Work is the flattened list of 16-row tiles of every (sequence, kv head) segment:
// segment (s, g) covers the tiles of rows [lo_s, L_s) aligned to 16-row boundaries,
// segments are ordered by s then g.  A resident grid of W wavefronts splits that list
// into W contiguous ranges of equal length, so every wavefront streams the same number
// of tiles with no per-item start-up, no empty work items and no ragged tail.  A range
// can cross segment boundaries; the pipeline crosses them too.
//
// Every workgroup first turns the context lengths into per-sequence tile counts and an
// exclusive prefix sum in LDS (workgroup 0 also stores it for the merge kernel).  Each
// wavefront then runs a three-stage software pipeline over its tiles: the block-table
// entry of tile i+3 (one per lane, for token t0 + lane % 16), the K and V rows of tile
// i+2, and the compute of tile i.  All loads are unconditional: a row outside the
// attended range or behind an unmapped entry is read from a clamped address inside the
// pool and masked out of the softmax and P.V; past the end of the range the last tile
// is re-read (a cache hit).
//
// Compute per tile runs on the matrix cores twice.  Scores: four
// v_mfma_f32_16x16x32_bf16 with the K tile as the A operand (row = token, lane l holds
// 64 contiguous bytes of token l % 16; the sum over head_dim is order-free, so lane
// group l / 16 takes head_dim slice [32 (l / 16), +32)) and the group's queries as the
// B operand (column = query head), leaving lane l with the scores of query head l % 16
// for tokens 4 (l / 16) .. +3.  Softmax in base 2 with a lazily raised reference max
// then gives each lane the probabilities of exactly those four tokens for its head,
// which is the A-operand layout of v_mfma_f32_16x16x16_bf16 (row = head, k = token).
// V is loaded so that lane l holds 16 contiguous bytes (8 columns) of tokens
// 4 (l / 16) + j, j = 0..3, at column block l % 16; for each of the 8 columns e of the
// block, v_perm_b32 gathers the four tokens' elements into the B operand (k = token,
// n = column block), so eight P.V products cover all 128 columns with no LDS traffic.
// The probabilities are split into a bf16 high part and a bf16 remainder and both are
// multiplied, so P keeps about 16 significant bits (a bf16 P alone is not accurate
// enough); the accumulators are fp32.  A segment that starts and ends inside one
// wavefront writes its output directly; the first and last segment of a range may be
// cut and are written as partial (max, sum, accumulator) to one of two slots of that
// wavefront, which the merge kernel combines in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa.h"
#include "pa_common.hpp"
#include "pa_decode_mfma.hpp"

namespace pa {
namespace stream {

using mfma::as_bf16x8;
using mfma::bf16x8;
using mfma::f32x4;

typedef short bf16x4 __attribute__((ext_vector_type(4)));   // four bf16 as the MFMA takes them
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int HD = 128;
constexpr int TILE = 16;
constexpr int NW = 4;           // wavefronts per workgroup
constexpr int BMAX = 2048;      // sequences handled by this path
constexpr int GSTRIDE = 16;     // heads per partial slot
constexpr float RESCALE_T = 8.f;
#ifndef STREAM_DEPTH
#define STREAM_DEPTH 2   // tiles of K/V in flight per wavefront while one is computed
#endif

struct Tile {
  uint4 k[4];        // K: token (lane % 16), bytes [64 (lane / 16), +64) of its head row
  uint4 v[4];        // V: token 4 (lane / 16) + j, bytes [16 (lane % 16), +16)
  uint64_t valid;    // bit t (t < 16): token t0 + t is attended and mapped
};

// Two floats rounded to bf16 (nearest even) and packed, low element first.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2v h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Position of a tile in the flattened list, with the fields of its segment.
struct Cur {
  int s, g, k;      // sequence, kv head, tile within the segment
  int tiles;        // tiles of the segment
  int lo, L;        // attended rows [lo, L)
  int t0base;       // first row of tile 0: lo rounded down to a multiple of 16
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int DEPTH, bool PAGE_TILES>
__global__ __launch_bounds__(64 * NW) void decode_stream_kernel(DecodeArgs a) {
  __shared__ int s_cum[BMAX + 1];   // tiles of sequences before s
  __shared__ int s_len[BMAX];       // clamped context length
  __shared__ int s_scan[64 * NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int B = a.num_seqs;
  const int Hkv = a.kv_heads;
  const int G = a.group;

  // ---- per-sequence tile counts and their exclusive prefix sum --------------------------
  {
    const int per = (B + 64 * NW - 1) / (64 * NW);
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int s = tid * per + i;
      if (s < B) {
        int L, lo, n;
        live_range(a.ctx[s], a.window, a.max_ctx, L, lo, n);
        const int t = n > 0 ? ((L - 1) >> 4) - (lo >> 4) + 1 : 0;
        s_len[s] = L;
        s_cum[s] = t;
        local += t;
      }
    }
    s_scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < 64 * NW; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int run = tid > 0 ? s_scan[tid - 1] : 0;
    for (int i = 0; i < per; ++i) {
      const int s = tid * per + i;
      if (s < B) {
        const int t = s_cum[s];
        s_cum[s] = run;
        run += t;
      }
    }
    if (tid == 0) s_cum[B] = s_scan[64 * NW - 1];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += 64 * NW) a.ws_cum[i] = s_cum[i];
  }

  // ---- this wavefront's range of tiles ----------------------------------------------------
  const int64_t T = (int64_t)Hkv * s_cum[B];
  const int W = a.total_waves;
  const int kw = blockIdx.x * NW + w;
  const int ta = (int)((int64_t)kw * T / W);
  const int n = (int)((int64_t)(kw + 1) * T / W) - ta;
  if (lane == 0) {
    a.ws_wave_start[kw] = ta;
    reinterpret_cast<int4*>(a.ws_rec)[kw] = make_int4(-1, 0, 0, 0);
  }
  if (n <= 0) return;

  const int P = a.page_size;
  const int lp = 31 - __clz(P);
  const int last_page = a.num_pages - 1;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const uint32_t row_bytes = (uint32_t)Hkv * HD * 2;
  const uint32_t page_bytes = row_bytes * (uint32_t)P;
  const int col = lane & 15;
  const int grp = lane >> 4;

  auto seg_fields = [&](Cur& c) {
    c.tiles = uni(s_cum[c.s + 1] - s_cum[c.s]);
    c.L = uni(s_len[c.s]);
    c.lo = (a.window > 0 && c.L > a.window) ? c.L - a.window : 0;
    c.t0base = (c.lo >> 4) << 4;
  };
  // one past the flattened index of the segment's last tile
  auto seg_end_flat = [&](const Cur& c) {
    return Hkv * s_cum[c.s] + (c.g + 1) * c.tiles;
  };
  // locate flattened tile ta
  Cur cc;
  {
    int lo_s = 0, hi_s = B - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if ((int64_t)Hkv * s_cum[mid] <= ta) lo_s = mid; else hi_s = mid - 1;
    }
    cc.s = uni(lo_s);
    seg_fields(cc);
    const int within = ta - Hkv * s_cum[cc.s];
    cc.g = uni(within / cc.tiles);
    cc.k = uni(within % cc.tiles);
  }
  // advance to the next tile; `more` is false at the last tile of the range (the cursor
  // then stays, so the stages re-read it)
  auto advance = [&](Cur& c, bool more) {
    if (!more) return;
    if (c.k + 1 < c.tiles) {
      c.k += 1;
      return;
    }
    c.k = 0;
    c.g += 1;
    if (c.g == Hkv) {
      c.g = 0;
      do { c.s += 1; } while (s_cum[c.s + 1] == s_cum[c.s]);
      c.s = uni(c.s);
      seg_fields(c);
    }
  };

  // Table entries.  With pages of at least 16 rows the tile lies in one page: one entry,
  // read through the scalar path (constant address space), whose completion is counted
  // apart from the vector loads, so waiting for it never drains the K/V tiles in flight.
  // Smaller pages need one entry per token (lane col holds token t0 + col's).
  const __attribute__((address_space(4))) int32_t* bt_const =
      (const __attribute__((address_space(4))) int32_t*)a.block_tables;
  auto table_entry = [&](const Cur& c) {
    if constexpr (PAGE_TILES) {
      const int t = min(max(c.t0base + c.k * TILE, c.lo), c.L - 1);
      // num_seqs * bt_stride < 2^31 on this path, so the index fits one scalar register
      return bt_const[uni(c.s * a.bt_stride + (t >> lp))];
    } else {
      const int t = min(max(c.t0base + c.k * TILE + col, c.lo), c.L - 1);
      return a.block_tables[(size_t)c.s * a.bt_stride + (t >> lp)];
    }
  };

  auto row_addr = [&](const char* base, int pg, int t, uint32_t lane_off) {
    return reinterpret_cast<const uint4*>(base + (uint64_t)(uint32_t)pg * page_bytes +
                                          ((uint32_t)(t & (P - 1)) * row_bytes + lane_off));
  };

  // K rows of token t0 + col (64 B at slice grp), V rows of tokens t0 + 4 grp + j (16 B
  // at column block col); e = table entry of token t0 + col
  // Per-lane byte offsets that do not change from tile to tile when a tile lies inside one
  // page (page size >= 16: tiles start at multiples of 16): K of token col, V of tokens
  // 4 grp + j.
  constexpr bool page_tiles = PAGE_TILES;
  const uint32_t k_lane_off = (uint32_t)col * row_bytes + grp * 64;
  const uint32_t v_lane_off = (uint32_t)(4 * grp) * row_bytes + col * 16;

  auto load_tile = [&](const Cur& c, int e, Tile& Tl) {
    const int t0 = c.t0base + c.k * TILE;
    if constexpr (page_tiles) {
      // one page for the whole tile: a uniform base address plus constant lane offsets
      const int pg = uni(e);
      const bool mapped = pg >= 0 && pg <= last_page;
      const int lo_off = max(c.lo - t0, 0), hi_off = min(c.L - t0, TILE);
      const uint32_t bits = ((1u << hi_off) - 1u) & ~((1u << lo_off) - 1u);
      Tl.valid = mapped ? (uint64_t)bits : 0ull;
      const uint64_t base = (uint64_t)(uint32_t)min(max(pg, 0), last_page) * page_bytes +
                            (uint32_t)(t0 & (P - 1)) * row_bytes + (uint32_t)c.g * HD * 2;
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + base + k_lane_off);
#pragma unroll
      for (int j = 0; j < 4; ++j) Tl.k[j] = kp[j];
      const char* vb = vbase + base + v_lane_off;
#pragma unroll
      for (int j = 0; j < 4; ++j) Tl.v[j] = *reinterpret_cast<const uint4*>(vb + j * row_bytes);
      return;
    }
    const int tk = t0 + col;
    Tl.valid = __ballot(tk >= c.lo && tk < c.L && e >= 0 && e <= last_page) & 0xffffull;
    const uint32_t hoff = (uint32_t)c.g * HD * 2;
    const int tkc = min(max(tk, c.lo), c.L - 1);
    const uint4* kp = row_addr(kbase, min(max(e, 0), last_page), tkc, hoff + grp * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) Tl.k[j] = kp[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ev = __shfl(e, 4 * grp + j, 64);
      const int tv = min(max(t0 + 4 * grp + j, c.lo), c.L - 1);
      Tl.v[j] = *row_addr(vbase, min(max(ev, 0), last_page), tv, hoff + col * 16);
    }
  };

  // ---- per-segment state -----------------------------------------------------------------
  // m_ref: reference max of score column col (query head col), the same in every lane
  // group; l_run: this lane's share of the running sum (its four tokens); oacc[e][r]:
  // output of query head 4 grp + r at column 8 col + e.
  bf16x8 qb[4];
  float m_ref = -INFINITY, l_run = 0.f;
  f32x4 oacc[8];
  bool first_seg = true;     // the segment being computed is the first of this range
  bool started_here = false; // ... and this wavefront computed its tile 0

  auto begin_segment = [&](const Cur& c) {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((size_t)c.s * a.q_heads + (size_t)c.g * G + (col < G ? col : 0)) * HD +
                           grp * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 8 * j);
      qb[j] = as_bf16x8(col < G ? v : zero);
    }
    // Wait here, on this rare path, for the query rows: otherwise the compiler would
    // have to assume the load may still be outstanding wherever the query registers
    // are read and drain every prefetched tile before each tile's compute.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    m_ref = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    started_here = c.k == 0;
  };

  auto end_segment = [&](const Cur& c, bool complete) {
    float lt = l_run;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    float lr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lr[r] = __shfl(lt, 4 * grp + r, 64);
    if (complete) {
      float* out = a.out + ((size_t)c.s * a.q_heads + (size_t)c.g * G) * HD + col * 8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) {
          const float inv = lr[r] > 0.f ? 1.f / lr[r] : 0.f;
          float4* o = reinterpret_cast<float4*>(out + (size_t)h * HD);
          o[0] = make_float4(oacc[0][r] * inv, oacc[1][r] * inv, oacc[2][r] * inv, oacc[3][r] * inv);
          o[1] = make_float4(oacc[4][r] * inv, oacc[5][r] * inv, oacc[6][r] * inv, oacc[7][r] * inv);
        }
      }
    } else {
      const int slot = first_seg ? 0 : 1;
      const size_t pi = (size_t)kw * 2 + slot;
      if (lane < G) {
        a.ws_ml[(pi * GSTRIDE + lane) * 2] = m_ref;
        a.ws_ml[(pi * GSTRIDE + lane) * 2 + 1] = lt;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) {
          float4* o = reinterpret_cast<float4*>(a.ws_acc + (pi * GSTRIDE + h) * HD + col * 8);
          o[0] = make_float4(oacc[0][r], oacc[1][r], oacc[2][r], oacc[3][r]);
          o[1] = make_float4(oacc[4][r], oacc[5][r], oacc[6][r], oacc[7][r]);
        }
      }
      if (started_here && lane == 0) {
        // this wavefront holds the first piece of a segment cut at its range end: leave
        // the merge kernel a record (segment, slot of this piece, wavefront of the last
        // piece: the one whose range holds the segment's last tile)
        const int64_t seg_end = seg_end_flat(c);
        const int k2 = (int)((seg_end * W - 1) / T);
        reinterpret_cast<int4*>(a.ws_rec)[kw] = make_int4(c.s * Hkv + c.g, slot, k2, 0);
      }
    }
    first_seg = false;
  };

  auto compute = [&](const Tile& Tl, const Cur& c, int i) {
    if (i == 0 || c.k == 0) begin_segment(c);
    // scores S[token][head] = K . q
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Tl.k[j]), qb[j], sc, 0, 0, 0);
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (Tl.valid >> (4 * grp + r)) & 1;
      sv[r] = ok ? sc[r] * a.qscale : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    // raise the reference when some head's tile max passes it by more than RESCALE_T;
    // this lane's own max decides whether any does, so the cross-lane max is only taken
    // on the (rare) raise
    if (__ballot(col < G && mt > m_ref + RESCALE_T) != 0) {
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m_ref, mt);
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - mn);
      l_run *= alpha;
      m_ref = mn;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[e][r] *= ar;
      }
    }
    const float ms = m_ref == -INFINITY ? 0.f : m_ref;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = col < G ? __builtin_amdgcn_exp2f(sv[r] - ms) : 0.f;
      l_run += p[r];
    }
    // P as the A operand (row = head col, k = token 4 grp + r), split into a bf16 high
    // part and the bf16-rounded remainder
    const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
    const uint32_t l01 = pack_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = pack_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const bf16x4 phi = __builtin_bit_cast(bf16x4, make_uint2(h01, h23));
    const bf16x4 plo = __builtin_bit_cast(bf16x4, make_uint2(l01, l23));
    // Rows outside the attended range get probability 0, but their V may be anything
    // (rows of the last page past the sequence end are never written): replace them by
    // zeros, since 0 * NaN would poison the product.
    uint4 vt[4] = {Tl.v[0], Tl.v[1], Tl.v[2], Tl.v[3]};
    if (Tl.valid != 0xffffull) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!((Tl.valid >> (4 * grp + j)) & 1)) vt[j] = make_uint4(0, 0, 0, 0);
    }
    const uint32_t v0[4] = {vt[0].x, vt[0].y, vt[0].z, vt[0].w};
    const uint32_t v1[4] = {vt[1].x, vt[1].y, vt[1].z, vt[1].w};
    const uint32_t v2[4] = {vt[2].x, vt[2].y, vt[2].z, vt[2].w};
    const uint32_t v3[4] = {vt[3].x, vt[3].y, vt[3].z, vt[3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // column 8 col + e of the four tokens: the B operand (k = token, n = column block)
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b01 = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], sel);
      const uint32_t b23 = __builtin_amdgcn_perm(v3[e >> 1], v2[e >> 1], sel);
      const bf16x4 bv = __builtin_bit_cast(bf16x4, make_uint2(b01, b23));
      oacc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, oacc[e], 0, 0, 0);
      oacc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, oacc[e], 0, 0, 0);
    }
    const bool seg_last = c.k == c.tiles - 1;
    if (seg_last || i == n - 1) end_segment(c, seg_last && started_here);
  };

  // ---- pipeline: table entry DEPTH+1 tiles ahead, K/V DEPTH tiles ahead, compute ------
  // The K/V buffers form a ring of DEPTH+1 tiles indexed by compile-time constants (the
  // inner loop is fully unrolled), so every stage keeps fixed registers.
  Cur cl = cc, ct = cc;  // load cursor, table cursor
  int jl = 0, jt = 0;    // their tile indices within the range
  auto adv_t = [&]() { advance(ct, jt < n - 1); jt += jt < n - 1; };
  auto adv_l = [&]() { advance(cl, jl < n - 1); jl += jl < n - 1; };
  Tile buf[DEPTH + 1];
  int e_next = table_entry(ct);
  adv_t();
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    const int e_use = e_next;
    e_next = table_entry(ct);
    adv_t();
    load_tile(cl, e_use, buf[u]);
    adv_l();
  }
  for (int i = 0; i < n; i += DEPTH + 1) {
#pragma unroll
    for (int u = 0; u <= DEPTH; ++u) {
      const int e_use = e_next;
      e_next = table_entry(ct);
      adv_t();
      load_tile(cl, e_use, buf[(u + DEPTH) % (DEPTH + 1)]);
      adv_l();
      if (i + u < n) {
        compute(buf[u], cc, i + u);
        advance(cc, i + u + 1 < n);
      }
    }
  }
}

// Combines the partials of segments cut between wavefronts (one block per wavefront
// whose range opens a cut segment: it holds the first piece, the following wavefronts
// hold the rest in slot 0), and zeroes the output rows of empty sequences.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_BATCH = 8;   // pieces whose partials are loaded together

__global__ __launch_bounds__(MERGE_THREADS) void merge_stream_kernel(DecodeArgs a) {
  const int Hkv = a.kv_heads, G = a.group;
  const int W = a.total_waves;
  const int k1 = blockIdx.x;
  if (k1 >= W) {
    // zero rows: blocks W .. W + num_seqs - 1, one per sequence
    const int s = k1 - W;
    if (a.ws_cum[s + 1] != a.ws_cum[s]) return;
    float* out = a.out + (size_t)s * a.q_heads * HD;
    for (int i = threadIdx.x; i < a.q_heads * HD; i += blockDim.x) out[i] = 0.f;
    return;
  }
  const int4 rec = reinterpret_cast<const int4*>(a.ws_rec)[k1];
  if (rec.x < 0) return;
  const int s = rec.x / Hkv, g = rec.x % Hkv;
  const int np = rec.z - k1 + 1;  // pieces: wavefronts k1 .. k2
  float* out = a.out + ((size_t)s * a.q_heads + (size_t)g * G) * HD;
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int h = i / HD, d = i % HD;
    // running max, rescaled sum and accumulator over the pieces in order; the loads of a
    // batch of pieces are independent and issued together
    float M = -INFINITY, den = 0.f, num = 0.f;
    for (int p0 = 0; p0 < np; p0 += MERGE_BATCH) {
      float mm[MERGE_BATCH], ll[MERGE_BATCH], xx[MERGE_BATCH];
#pragma unroll
      for (int q = 0; q < MERGE_BATCH; ++q) {
        const int p = p0 + q;
        const size_t pi = (size_t)(k1 + p) * 2 + (p == 0 ? rec.y : 0);
        const bool ok = p < np;
        mm[q] = ok ? a.ws_ml[(pi * GSTRIDE + h) * 2] : -INFINITY;
        ll[q] = ok ? a.ws_ml[(pi * GSTRIDE + h) * 2 + 1] : 0.f;
        xx[q] = ok ? a.ws_acc[(pi * GSTRIDE + h) * HD + d] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < MERGE_BATCH; ++q) {
        if (mm[q] == -INFINITY) continue;
        const float mn = fmaxf(M, mm[q]);
        const float fo = exp2f(M - mn), fn = exp2f(mm[q] - mn);
        den = den * fo + ll[q] * fn;
        num = num * fo + xx[q] * fn;
        M = mn;
      }
    }
    out[(size_t)h * HD + d] = den > 0.f ? num / den : 0.f;
  }
}

inline bool eligible(int dtype, int head_dim, int group, int page_size, int num_seqs,
                     int bt_stride) {
  return dtype == PA_BF16 && head_dim == HD && group >= 1 && group <= 16 && page_size > 0 &&
         (page_size & (page_size - 1)) == 0 && num_seqs >= 1 && num_seqs <= BMAX &&
         (int64_t)num_seqs * bt_stride < ((int64_t)1 << 31);
}

// Workspace: per wavefront two partial slots of GSTRIDE heads and a merge record, then
// the per-sequence prefix sums, then the first tile of every wavefront's range.
inline size_t workspace_bytes(int total_waves, int num_seqs) {
  const size_t slots = (size_t)total_waves * 2 * GSTRIDE;
  return slots * 2 * sizeof(float) + slots * HD * sizeof(float) + (size_t)total_waves * 16 +
         (size_t)(num_seqs + 1) * 4 + (size_t)total_waves * 4 + 256;
}

inline int launch(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.total_waves / NW);
  if (a.page_size >= TILE)
    hipLaunchKernelGGL((decode_stream_kernel<STREAM_DEPTH, true>), dim3(blocks), dim3(64 * NW), 0,
                       st, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<STREAM_DEPTH, false>), dim3(blocks), dim3(64 * NW),
                       0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(merge_stream_kernel, dim3((unsigned)(a.total_waves + a.num_seqs)),
                     dim3(MERGE_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace stream
}  // namespace pa
