// Prefill chunks: several query tokens per sequence, many of them (bf16 pools, head_dim
// 128, G = q_heads / kv_heads a power of two up to 16, page sizes that are powers of two,
// a positive scale).
//
// One workgroup of four wavefronts per (sequence, kv head, tile of 128 score columns); a
// column is one query head of one query token (column c: head c % G of token c / G of the
// tile), so a tile holds 128 / G query tokens.  Wavefront w takes two blocks of 16
// columns, 32 w .. 32 w + 31, so every K and V fragment it reads from LDS feeds both.
// The workgroup walks the key rows its tile's queries attend, from the window start of
// its first query to its last query's own row, 32 rows at a time: the K and V rows of the
// next 32 are loaded by all 256 lanes (each lane 32 bytes of K and of V) while the current
// ones are computed, and written to one of two LDS buffers, so every K/V byte is read from
// memory once per tile and shared by its 128 columns.  Two workgroups share a compute
// unit.  Each wavefront reads the keys and values from LDS in matrix-core operand
// layouts: scores with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 of head_dim, B = 16
// columns' queries), base-2 online softmax with a lazily raised reference max, P.V with
// v_mfma_f32_16x16x32_f16 over 32 keys (P rounded to fp16; V converted to fp16 when it is
// staged into LDS and read back with transposing LDS reads, ds_read_b64_tr_b16, which hand
// each lane one head_dim column of four key rows), and the running sums as the same product
// against ones.  Each column is masked to its own query's rows
// (causal, the window counted from its row); the blocks every column attends run in a
// loop of their own without masks.  A workgroup covers its tile's whole key range, so
// there is no split and nothing to merge; every key row loaded lies in [window start of
// the first query, last query's row], which are rows some query attends, so every table
// entry read is a mapped page.  Units of work start longest first.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa.h"
#include "pa_common.hpp"
#include "pa_decode_mfma.hpp"

namespace pa {
namespace ptile {

using mfma::as_bf16x8;
using mfma::bf16x8;
using mfma::f32x4;
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int HD = 128;
#ifndef PTILE_KT
#define PTILE_KT 32
#endif
constexpr int KT = PTILE_KT;      // key rows per block
constexpr int NKB = KT / 16;      // blocks of 16 rows in a matrix-core product
static_assert(NKB % 2 == 0, "P.V takes the key blocks in pairs");
constexpr int TPR = 256 / KT;     // lanes loading one key row
constexpr int UPT = KT / 16;      // 16-byte pieces of K (and of V) each lane loads
#ifndef PTILE_CB
#define PTILE_CB 2
#endif
constexpr int CB = PTILE_CB;      // blocks of 16 score columns per wavefront
constexpr int COLS = 64 * CB;     // score columns per workgroup
#ifndef PTILE_WG_PER_CU
#define PTILE_WG_PER_CU (CB == 1 ? 3 : 2)
#endif
#ifndef PTILE_DIE_MAJOR
#define PTILE_DIE_MAJOR 1
#endif
// LDS holds a key row in 256 bytes, its 16-byte chunks permuted within the row: chunk ch
// of row r sits at chunk ch ^ swz(r).  The LDS has 64 banks of 4 bytes and serves 256
// bytes per cycle: sixteen lanes of a 16-byte access, thirty-two of an 8-byte one.  swz
// takes all sixteen values on rows 16k .. 16k + 15 (a K read: one chunk of sixteen rows)
// and, on rows 8k .. 8k + 7, values whose bits 1-3 differ (a transposing V read: chunks
// 2e and 2e + 1 of eight rows), so neither touches a bank twice; the staging writes
// (sixteen lanes: half a row each of two rows, the halves crossed between even and odd
// rows) land on sixteen different chunks too.
constexpr int ROWB = 256;
__device__ __forceinline__ int swz(int row) { return ((row << 1) & 15) | ((row >> 3) & 1); }
// byte offset of 16-byte chunk `ch` (0..15) of key row `row` in an LDS buffer
__device__ __forceinline__ int lds_off(int row, int ch) {
  return row * ROWB + ((ch ^ swz(row)) << 4);
}
constexpr float RESCALE_T = 8.f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2v h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// P.V runs in fp16: P rounded to nearest (11 significant bits), V converted from bf16 when
// it is staged into LDS (exact for every bf16 value in fp16's normal range, 2^-14 to 65504;
// smaller ones keep an absolute error below 2^-25).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 x) {
  return make_uint4(pack_f16(bf16_lo(x.x), bf16_hi(x.x)), pack_f16(bf16_lo(x.y), bf16_hi(x.y)),
                    pack_f16(bf16_lo(x.z), bf16_hi(x.z)), pack_f16(bf16_lo(x.w), bf16_hi(x.w)));
}

#ifndef PTILE_LPT
#define PTILE_LPT 1
#endif
constexpr int LPT_MAX = 256;    // sequences ordered longest first (more: in index order)

// OFF32: pools under 4 GiB with pages and page counts under 2^24 bytes and pages: K/V rows
// are read through buffer resources with 32-bit offsets formed by 24-bit multiplies, in
// place of 64-bit address arithmetic for every load.
template <bool OFF32>
__global__ __launch_bounds__(256, PTILE_WG_PER_CU) void prefill_tile_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_k[2][KT * ROWB];
  __shared__ __attribute__((aligned(16))) char lds_v[2][KT * ROWB];
#if PTILE_LPT
  __shared__ int lpt_key[LPT_MAX];
  __shared__ int lpt_seq[LPT_MAX];
#endif

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int lg = 31 - __clz(G);
  const int Hkv = a.kv_heads;
  const int tpt = COLS >> lg;                       // query tokens per tile
  const int QT = (a.max_q + tpt - 1) / tpt;         // tiles per sequence at most
  // Workgroups go to the eight dies round-robin (workgroup b to die b % 8); numbering the
  // work die-major gives each die a contiguous run of it, so the query tiles of one
  // (sequence, kv head), which read the same key rows, share that die's L2.
  int wid = blockIdx.x;
#if PTILE_DIE_MAJOR
  {
    const int nb = gridDim.x, x = wid & 7, i = wid >> 3, q = nb >> 3, r = nb & 7;
    wid = x * q + min(x, r) + i;
  }
#endif
  const int qt = wid % QT;
  int sg = wid / QT;
#if PTILE_LPT
  if (a.num_seqs <= LPT_MAX) {
    // Longest first: workgroups start in number order within a die, and the work per
    // (sequence, kv head) unit follows its attended rows, which vary widely; starting the
    // longest units first keeps a long one from running alone at the end.  Units are taken
    // in order of their sequence's attended rows (ties by index) and dealt round-robin over
    // the dies' runs of work: run x holds units x, x + 8, x + 16, ... of that order.
    const int B = a.num_seqs;
    for (int t = tid; t < B; t += 256) {
      const int q0t = a.q_start[t];
      int nq = a.q_start[t + 1] - q0t;
      if (q0t < 0 || q0t > a.num_q) nq = 0;
      nq = max(0, min(min(nq, a.num_q - q0t), a.max_q));
      const int ct = a.ctx[t];
      const int Lt = ct > 0 ? (ct < a.max_ctx ? ct : a.max_ctx) : 0;
      lpt_key[t] = nq > 0 ? (a.window > 0 ? min(Lt, a.window + nq) : Lt) : -1;
    }
    __syncthreads();
    for (int t = tid; t < B; t += 256) {
      const int kt = lpt_key[t];
      int r = 0;
      for (int u = 0; u < B; ++u) {
        const int ku = lpt_key[u];
        r += (ku > kt) | ((ku == kt) & (u < t));
      }
      lpt_seq[r] = t;
    }
    __syncthreads();
    const int U = B * Hkv, q8 = U >> 3, r8 = U & 7;
    int x, i;
    if (sg < r8 * (q8 + 1)) {
      x = sg / (q8 + 1);
      i = sg % (q8 + 1);
    } else {
      x = r8 + (sg - r8 * (q8 + 1)) / q8;
      i = (sg - r8 * (q8 + 1)) % q8;
    }
    const int k = x + 8 * i;
    sg = lpt_seq[k / Hkv] * Hkv + k % Hkv;
  }
#endif
  const int g = sg % Hkv;
  const int s = sg / Hkv;

  // the sequence's query rows, clamped to the bounds the host passed
  const int q0 = a.q_start[s];
  int n = a.q_start[s + 1] - q0;
  if (q0 < 0 || q0 > a.num_q) n = 0;
  n = max(0, min(min(n, a.num_q - q0), a.max_q));
  const int tk0 = qt * tpt;
  if (tk0 >= n) return;                             // uniform over the workgroup
  const int nt = min(tpt, n - tk0);
  const int ctx = a.ctx[s];
  const int L = ctx > 0 ? (ctx < a.max_ctx ? ctx : a.max_ctx) : 0;
  const int p0 = L - n + tk0;                       // row of the tile's first query
  const int kend = max(p0 + nt, 0);                 // one past its last query's row
  const int lo = a.window > 0 ? max(p0 + 1 - a.window, 0) : 0;
  float* out = a.out + ((size_t)(q0 + tk0) * a.q_heads + (size_t)g * G) * HD;
  if (kend <= lo) {
    // every query of the tile lies before row 0: zero rows
    for (int i = tid; i < nt * G * HD; i += 256) {
      const int t = i / (G * HD), r = i - t * G * HD;
      out[(size_t)t * a.q_heads * HD + r] = 0.f;
    }
    return;
  }

  // this lane's column of block cb: head (c & (G - 1)) of query token c >> lg of the tile,
  // c = 16 (CB w + cb) + col
  bool cval[CB];
  int pc[CB], pc_lo[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int tq = (16 * (CB * w + cb) + col) >> lg;
    cval[cb] = tq < nt;
    pc[cb] = p0 + tq;
    pc_lo[cb] = a.window > 0 ? pc[cb] - a.window : (-0x7fffffff - 1);
  }
  // a block of rows [k0, k0 + KT) with k0 + KT - 1 <= pmin and k0 > plo is attended by all
  const int pmin = p0;
  const int plo = a.window > 0 ? p0 + nt - 1 - a.window : (-0x7fffffff - 1);

  bf16x8 qb[CB][4];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    const int c = 16 * (CB * w + cb) + col;
    const int tq = cval[cb] ? c >> lg : 0;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(a.q) +
        ((size_t)(q0 + tk0 + tq) * a.q_heads + (size_t)g * G + (c & (G - 1))) * HD + grp * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[cb][j] = as_bf16x8(cval[cb] ? qrow[j] : zero);
  }

  const int P = a.page_size;
  const int lp = 31 - __clz(P);
  const uint32_t row_bytes = (uint32_t)a.row_stride * 2;
  const uint32_t page_bytes = (uint32_t)Hkv * HD * 2 * (uint32_t)P;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * a.head_stride * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * a.head_stride * 2;
  const int32_t* btr = a.block_tables + (size_t)s * a.bt_stride;
  const int last_page = a.num_pages - 1;

  // loading: lane tid takes key row kk = tid / TPR of the block, 16-byte pieces
  // part + TPR (i ^ (kk & 1)) of it, i < UPT
  const int kk = tid / TPR, part = tid % TPR, hx = kk & 1;
  const int kt0 = lo & ~(KT - 1);
  const int nblk = (kend - 1 - kt0) / KT + 1;
  // (the key of block b is written out in each lambda: a lambda that calls another one
  // keeps its closure in scratch memory)
  auto entry = [&](int b) __attribute__((always_inline)) { return btr[min(max(kt0 + b * KT + kk, lo), kend - 1) >> lp]; };
  // (the rows travel in named registers: arrays or structs shared between the lambdas
  // and the loop stayed in scratch memory)
  uint4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3;
  // (OFF32) the pools as buffer resources, and this lane's byte offsets of its pieces
  // within a key row of its head
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.k_pool), 0, (int)((uint32_t)a.num_pages * page_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.v_pool), 0, (int)((uint32_t)a.num_pages * page_bytes), 0x00020000);
  const uint32_t piece0 = (uint32_t)g * (uint32_t)a.head_stride * 2u + part * 16;
  auto ld = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t o) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 0));
  };
  auto load = [&](int b, int e) __attribute__((always_inline)) {
    const int key = min(max(kt0 + b * KT + kk, lo), kend - 1);
    const int pg = min(max(e, 0), last_page);
    if constexpr (OFF32) {
      const uint32_t o = __umul24((uint32_t)pg, page_bytes) +
                         __umul24((uint32_t)(key & (P - 1)), row_bytes) + piece0;
      rk0 = ld(rsk, o + TPR * 16 * (0 ^ hx));
      rk1 = ld(rsk, o + TPR * 16 * (1 ^ hx));
      rv0 = ld(rsv, o + TPR * 16 * (0 ^ hx));
      rv1 = ld(rsv, o + TPR * 16 * (1 ^ hx));
      if constexpr (UPT > 2) {
        rk2 = ld(rsk, o + TPR * 16 * (2 ^ hx));
        rk3 = ld(rsk, o + TPR * 16 * (3 ^ hx));
        rv2 = ld(rsv, o + TPR * 16 * (2 ^ hx));
        rv3 = ld(rsv, o + TPR * 16 * (3 ^ hx));
      }
      return;
    }
    const size_t off = (size_t)(uint32_t)pg * page_bytes + (size_t)(key & (P - 1)) * row_bytes +
                       part * 16;
    const uint4* kp = reinterpret_cast<const uint4*>(kbase + off);
    const uint4* vp = reinterpret_cast<const uint4*>(vbase + off);
    rk0 = kp[TPR * (0 ^ hx)];
    rk1 = kp[TPR * (1 ^ hx)];
    rv0 = vp[TPR * (0 ^ hx)];
    rv1 = vp[TPR * (1 ^ hx)];
    if constexpr (UPT > 2) {
      rk2 = kp[TPR * (2 ^ hx)];
      rk3 = kp[TPR * (3 ^ hx)];
      rv2 = vp[TPR * (2 ^ hx)];
      rv3 = vp[TPR * (3 ^ hx)];
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    char* kd = lds_k[buf];
    char* vd = lds_v[buf];
    *reinterpret_cast<uint4*>(kd + lds_off(kk, part + TPR * (0 ^ hx))) = rk0;
    *reinterpret_cast<uint4*>(kd + lds_off(kk, part + TPR * (1 ^ hx))) = rk1;
    *reinterpret_cast<uint4*>(vd + lds_off(kk, part + TPR * (0 ^ hx))) = bf16x8_to_f16(rv0);
    *reinterpret_cast<uint4*>(vd + lds_off(kk, part + TPR * (1 ^ hx))) = bf16x8_to_f16(rv1);
    if constexpr (UPT > 2) {
      *reinterpret_cast<uint4*>(kd + lds_off(kk, part + TPR * (2 ^ hx))) = rk2;
      *reinterpret_cast<uint4*>(kd + lds_off(kk, part + TPR * (3 ^ hx))) = rk3;
      *reinterpret_cast<uint4*>(vd + lds_off(kk, part + TPR * (2 ^ hx))) = bf16x8_to_f16(rv2);
      *reinterpret_cast<uint4*>(vd + lds_off(kk, part + TPR * (3 ^ hx))) = bf16x8_to_f16(rv3);
    }
  };

  // lsum[cb][r]: running sum of column 4 grp + r's probabilities (as rounded to fp16), on
  // the matrix cores: P times a block of ones, in the layout of the accumulators
  float m_ref[CB];
  f32x4 lsum[CB];
  f32x4 oacc[CB][8];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m_ref[cb] = -INFINITY;
    lsum[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[cb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // compute block b from LDS buffer buf (a constant at every call, so the buffer's offset
  // folds into the LDS instructions); MASKED: some column does not attend every row
  auto compute = [&](auto masked, int b, int buf) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int k0 = kt0 + b * KT;
    const char* Ks = lds_k[buf];
    const char* Vs = lds_v[buf];
    // scores of the block's rows: lane (col, grp) gets rows 16 kb + 4 grp + r of column col
    // of each column block.  All K fragments of the block are read first, so their LDS
    // latency overlaps, and serve every column block.
    uint4 kf[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kf[kb][j] = *reinterpret_cast<const uint4*>(Ks + lds_off(kb * 16 + col, 4 * grp + j));
    f32x4 sc[CB][NKB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sc[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sc[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kb][j]), qb[cb][j],
                                                               sc[cb][kb], 0, 0, 0);
      }
    // The P.V operand of head_dim 16 e .. 16 e + 15, read now (in flight during the
    // softmax) with transposing LDS reads: in each group of 16 lanes, lane L reads 4
    // consecutive values of key row 4 grp + L / 4 at head_dim 16 e + 4 (L % 4), and the read
    // hands lane L the values of its head_dim 16 e + L from the group's four key rows.
    bf16x4 vb[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vb[kb][e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) bf16x4*)(
                Vs + lds_off(kb * 16 + 4 * grp + (col >> 2), 2 * e + ((col >> 1) & 1)) +
                8 * (col & 1)));
    // Scores stay unscaled: the scale (times log2 e, positive on this path) multiplies the
    // block max once and enters each exponent through one fused multiply-add.  Masked
    // blocks set the scores of rows a column does not attend to -inf with selects.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float sv[NKB][4];
      float mr = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (MASKED) {
            const int t = k0 + kb * 16 + 4 * grp + r;
            const bool ok = (t <= pc[cb]) & (t > pc_lo[cb]);
            sv[kb][r] = ok ? sc[cb][kb][r] : -INFINITY;
          } else {
            sv[kb][r] = sc[cb][kb][r];
          }
          mr = fmaxf(mr, sv[kb][r]);
        }
      float mt = mr * a.qscale;
      if (__ballot(cval[cb] && mt > m_ref[cb] + RESCALE_T) != 0) {
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m_ref[cb], mt);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref[cb] - mn);
        m_ref[cb] = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * grp + r, 64);
          lsum[cb][r] *= ar;
#pragma unroll
          for (int e = 0; e < 8; ++e) oacc[cb][e][r] *= ar;
        }
      }
      const float ms = m_ref[cb] == -INFINITY ? 0.f : m_ref[cb];
      // P.V over 32 keys per product (v_mfma_f32_16x16x32_f16): the A operand of lane
      // (col, grp) holds column col's probabilities of keys 4 grp + r of two 16-row blocks,
      // and the B operand the same keys' values (the two transposing reads of those
      // blocks, fp16 in LDS), so both sides take the keys in the same order.  The running
      // sum is the same product against ones: the probabilities as rounded to fp16, so
      // each output row is an exact convex combination of value rows with the weights the
      // products used.
#pragma unroll
      for (int kp = 0; kp < NKB / 2; ++kp) {
        uint32_t hw[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = 2 * kp + h;
          float p[4];
#pragma unroll
          // (a column past the tile's queries has zero queries and finite values
          // throughout, and its output row is never written)
          for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], a.qscale, -ms));
          hw[2 * h] = pack_f16(p[0], p[1]);
          hw[2 * h + 1] = pack_f16(p[2], p[3]);
        }
        const f16x8 pv = __builtin_bit_cast(f16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
        lsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv, ones, lsum[cb], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint2 v0 = __builtin_bit_cast(uint2, vb[2 * kp][e]);
          const uint2 v1 = __builtin_bit_cast(uint2, vb[2 * kp + 1][e]);
          const f16x8 bv = __builtin_bit_cast(f16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
          oacc[cb][e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv, bv, oacc[cb][e], 0, 0, 0);
        }
      }
    }
  };

  // pipeline: block b computed from LDS while block b + 1 is loaded into registers, then
  // written to the other buffer; the table entry is read one block further ahead
  // (past the last block the loads repeat it: in range, and never staged)
  const int bl = nblk - 1;
  load(0, entry(0));
  int e1 = entry(min(1, bl));
  stage(0);
  load(min(1, bl), e1);
  int e2 = entry(min(2, bl));
  __syncthreads();
  // Blocks [pb1, pb2) are attended by every column (past the window start of the last
  // query, up to the first query's row) and take no masks; the blocks before and after
  // them do.  Three loops, so that each holds one copy of the block's code.
  const int pb1 = min(plo < kt0 ? 0 : (plo - kt0) / KT + 1, nblk);
  const int pb2 = min(max(max(pmin - kt0 + 1, 0) / KT, pb1), nblk);
  int b = 0;
  for (; b < pb1; ++b) {
    compute(std::true_type{}, b, b & 1);
    if (b + 1 < nblk) {
      stage((b + 1) & 1);
      load(min(b + 2, bl), e2);
      e2 = entry(min(b + 3, bl));
    }
    __syncthreads();
  }
  for (; b < pb2; ++b) {
    compute(std::false_type{}, b, b & 1);
    if (b + 1 < nblk) {
      stage((b + 1) & 1);
      load(min(b + 2, bl), e2);
      e2 = entry(min(b + 3, bl));
    }
    __syncthreads();
  }
  for (; b < nblk; ++b) {
    compute(std::true_type{}, b, b & 1);
    if (b + 1 < nblk) {
      stage((b + 1) & 1);
      load(min(b + 2, bl), e2);
      e2 = entry(min(b + 3, bl));
    }
    __syncthreads();
  }

  // output: lane (col, grp) holds columns 4 grp + r of each column block at head_dim
  // 16 e + col
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = lsum[cb][r];
      const int h = 16 * (CB * w + cb) + 4 * grp + r;
      if ((h >> lg) < nt) {
        const float inv = lr > 0.f ? 1.f / lr : 0.f;
        float* o = out + ((size_t)(h >> lg) * a.q_heads + (h & (G - 1))) * HD + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[16 * e] = oacc[cb][e][r] * inv;
      }
    }
  }
}

// Tiles per sequence at most and the grid; the path serves chunks of at least 48 query
// columns (12 tokens at G = 4: below that the streaming kernel, which does not pad the
// columns to a 128-column tile, is faster) with a workgroup for every slot of the chip.
constexpr int MIN_COLS = 48;
constexpr int MIN_GRID = 256 * PTILE_WG_PER_CU;
inline int64_t grid_size(int num_seqs, int kv_heads, int group, int max_q) {
  const int tpt = COLS / group;
  return (int64_t)num_seqs * kv_heads * ((max_q + tpt - 1) / tpt);
}
inline bool eligible(int dtype, int head_dim, int group, int page_size, int num_seqs,
                     int kv_heads, int max_q, float scale) {
  return scale > 0.f && dtype == PA_BF16 && head_dim == HD && group >= 1 && group <= 16 &&
         (group & (group - 1)) == 0 && page_size > 0 && (page_size & (page_size - 1)) == 0 &&
         num_seqs >= 1 && (int64_t)max_q * group >= MIN_COLS &&
         grid_size(num_seqs, kv_heads, group, max_q) >= MIN_GRID &&
         grid_size(num_seqs, kv_heads, group, max_q) < ((int64_t)1 << 31);
}

inline int launch(const DecodeArgs& a, hipStream_t st) {
  const int64_t blocks = grid_size(a.num_seqs, a.kv_heads, a.group, a.max_q);
  const uint64_t page_bytes = (uint64_t)a.kv_heads * HD * 2 * (uint64_t)a.page_size;
  const bool off32 = page_bytes < (1u << 24) && (uint64_t)a.num_pages < (1u << 24) &&
                     (uint64_t)a.num_pages * page_bytes < ((uint64_t)1 << 32);
  if (off32)
    hipLaunchKernelGGL(prefill_tile_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_tile_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace ptile
}  // namespace pa
