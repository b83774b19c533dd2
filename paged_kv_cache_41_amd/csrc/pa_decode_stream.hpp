// Balanced streaming decode: bf16 pools, head_dim 128, up to 16 query heads per kv head,
// page sizes that are powers of two, up to BMAX sequences.
//
// Work is the flattened list of 16-row tiles of every (sequence, kv head) segment:
// segment (s, g) covers the tiles of its attended rows aligned to 16-row boundaries (with
// attention sinks, the sink rows' tiles and then the window's), segments ordered by s then
// g.  A resident grid of W wavefronts splits that list into W contiguous ranges of equal
// length, so every wavefront streams the same number of tiles with no per-item start-up,
// no empty work items and no ragged tail.  A range can cross segment boundaries; the
// pipeline crosses them too.
//
// Every workgroup first turns the context lengths into per-sequence tile counts and an
// exclusive prefix sum in LDS.  Each wavefront then runs a three-stage software pipeline
// over its tiles: the block-table entry of tile i+D+1 (one per tile, read through the
// scalar unit, for pages of at least 16 rows; one per lane for smaller pages), the K and V
// rows of tile i+D, and the compute of tile i (D = STREAM_DEPTH tiles in flight).  All
// loads are unconditional: a row outside the attended range or behind an unmapped entry is
// read from a clamped address inside the pool and masked out of the softmax and P.V; past
// the end of the range the last tile is re-read (a cache hit).
//
// Compute per tile runs on the matrix cores twice.  Scores: four
// v_mfma_f32_16x16x32_bf16 with the K tile as the A operand (row = token; the sum over
// head_dim is order-free, so in product j lane l takes the 8 elements at 32 j + 8 (l / 16)
// of token l % 16, and each load reads 64 contiguous bytes of every token) and the
// group's queries, in the same order, as the B operand (column = query head), leaving
// lane l with the scores of query head l % 16
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
// wavefront: in LDS when every piece lies in the wavefront's workgroup (the wavefront
// holding the first piece combines them after a workgroup barrier), else in device
// memory (the wavefront that finishes the segment's last piece to arrive combines them).
// Either way the pieces are combined in range order with the same arithmetic.
//
// Several query tokens per sequence (MULTI, NB > 0): the score columns are NB blocks of
// 16 / G consecutive query tokens times the G heads of the group, so a segment is (group
// of query tokens, kv head) and covers the rows the group's first query may attend up to
// its last query's own row; each column is masked to its own query's rows (causal, window
// counted from that query), and the NB blocks share every K/V tile and V operand gather.
//
// Head sets (HQ > 1, one query token, pages under 16 rows): a tile holds the same 16 rows
// of HQ consecutive kv heads, read with one set of per-lane table entries, and a segment is
// (sequence, head set).  The scores of head h are its four products against a copy of the
// query operand that keeps only head h's columns (zero elsewhere), all accumulated into
// the one score tile; in P.V, head h's values meet a copy of P that keeps only the rows
// (columns) of head h.  Everything else sees one head of HQ x G query heads.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <type_traits>

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
constexpr float RESCALE_T = 8.f;
constexpr int COMBINE_BATCH = 4;   // pieces whose partials are loaded together
#ifndef STREAM_DEPTH
#define STREAM_DEPTH 1   // tiles of K/V in flight per wavefront while one is computed (two
                         // measured 1-1.7 us slower on the batch-64 and window workloads:
                         // more bytes in flight per compute unit only lengthen the queues)
#endif
#ifndef STREAM_MULTI_DEPTH
#define STREAM_MULTI_DEPTH 1   // the same with several query tokens per sequence (its
                               // registers go to the query groups)
#endif

// A tile holds the rows of HQ kv heads (a head set); head h's K and V are in k[4 h + j]
// and v[4 h + j].
template <int HQ>
struct Tile {
  uint4 k[4 * HQ];   // K: token (lane % 16), bytes [64 j + 16 (lane / 16), +16) of its
                     // head row in k[j]
  uint4 v[4 * HQ];   // V: token 4 (lane / 16) + j, bytes [16 (lane % 16), +16)
  uint4 q[4];        // query column lane % 16, the same bytes as k: loaded with the
                     // tile that opens a segment piece only (groups of more than one block
                     // read their queries at the segment start instead)
  uint32_t valid;    // bit t (t < 16): token t0 + t is attended and mapped (uniform)
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
  int s, g, k;      // sequence (block of query tokens with MULTI), kv head, tile within it
  int tr;           // block-table row
  int tiles;        // tiles of the segment
  int sl, lo, L;    // attended rows [0, sl) and [lo, L)
  int sk;           // tiles of the sink rows: tiles 0 .. sk-1 start at rows 0, 16, ...
  int t0base;       // added to 16 k for the later tiles: the window's tiles start at row
                    // 16 max(sk, lo / 16)
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Device-scope accesses for the partials handed between wavefronts of one launch: buffer
// instructions with the sc1 cache policy (stores written through to the point where every
// compute unit reads them, loads that skip the caches of the compute unit and of its die),
// 8 or 16 bytes per lane.  The descriptor covers the partial area only; the hardware
// drops accesses past it.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int CPOL_DEVICE = 16;    // sc1
struct DevBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ DevBuf(void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ void store4(uint32_t off, float4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0,
                                           CPOL_DEVICE);
  }
  __device__ __forceinline__ void store2(uint32_t off, float2 v) const {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, (int)off, 0,
                                          CPOL_DEVICE);
  }
  __device__ __forceinline__ float4 load4(uint32_t off) const {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0,
                                                                            CPOL_DEVICE));
  }
  __device__ __forceinline__ float2 load2(uint32_t off) const {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0,
                                                                           CPOL_DEVICE));
  }
};

// ---- ranges of the flattened tile list ---------------------------------------------------
// With T tiles in the list and W wavefronts, the first R = min(W, T) wavefronts take one
// range each: range r is [r T / R, (r + 1) T / R), never empty.  Range order is list order,
// so the pieces of a segment cut by range boundaries lie in consecutive ranges.
__device__ __forceinline__ int range_start(int T, int R, int r) {
  return (int)((int64_t)r * T / R);
}
// the range holding tile x
__device__ __forceinline__ int range_of(int T, int R, int x) {
  return (int)(((int64_t)(x + 1) * R - 1) / T);
}

// Aligned partition (single-query decode): when the segments are about equal, each
// workgroup takes an equal count of whole segments (its first tile in st_wgb), and its four
// wavefronts split that range in equal parts.  No segment then crosses a workgroup, and the pieces of a cut segment are
// combined through LDS after a workgroup barrier, with no device-scope exchange.
__shared__ int st_wgb[BMAX / 4 + 1];
// partial (max and sum of every column, then the accumulators) of each wavefront's first
// and last segment piece, in the aligned partition
__shared__ float st_part[NW][2][16 * (2 + HD)];
struct Part {
  bool aligned;
  int T, R;        // flat: R equal ranges of the T tiles
  __device__ __forceinline__ int start(int r) const {
    if (!aligned) return range_start(T, R, r);
    const int g = r >> 2, q = r & 3, A = st_wgb[g];
    return q == 0 ? A : A + (int)((int64_t)q * (st_wgb[g + 1] - A) / 4);   // (r = R: g = NWG)
  }
  __device__ __forceinline__ int of(int x) const {
    if (!aligned) return range_of(T, R, x);
    int lo = 0, hi = R / 4 - 1;   // the workgroup whose range holds x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (st_wgb[mid] <= x) lo = mid; else hi = mid - 1;
    }
    int r = 4 * lo + 3;
    while (start(r) > x) --r;
    return r;
  }
};

// Table entries of a tile whose rows lie in several pages: lane (col, grp)'s K row and
// its four V rows.
struct RowPages {
  int k;
  int v[4];
};

// What the load and compute stages need of one tile.
enum : int {
  RANGE_FIRST = 1,   // first tile of the range
  RANGE_LAST = 2,    // last tile of the range
  SEG_FIRST = 4,     // tile 0 of its segment
  SEG_LAST = 8,      // last tile of its segment
  IDLE = 16,         // past the end of the range: loaded (a repeat) but not computed
};
struct Desc {
  int s, g;          // sequence (block of query tokens with MULTI), kv head
  int tr;            // block-table row
  int t0;            // first row of the tile
  int sl, lo, L;     // attended rows [0, sl) and [lo, L) of the sequence
  int flags;
};

// Per-sequence tile prefix sums and clamped lengths, built by every workgroup at the start.
__shared__ int st_cum[BMAX + 1];   // tiles of sequences before s (st_cum[B] = all)
__shared__ int st_len[BMAX];       // clamped context length
__shared__ int st_scan[NW];       // wavefront totals of the scan
__shared__ int st_scan2[NW];      // ... of the second array scanned with it
// MULTI: per sequence, its first group of query tokens and its first tile (prefix sums)
__shared__ int st_bseq[BMAX + 1];
__shared__ int st_tseq[BMAX + 1];
// MULTI: per block of query tokens, its sequence, first query row, position of its first
// query (negative when the sequence has more queries than rows), tokens and first key row
__shared__ int st_seq[BMAX];
__shared__ int st_q0[BMAX];
__shared__ int st_p0[BMAX];
__shared__ int st_nt[BMAX];
__shared__ int st_lo[BMAX];

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts by 1, 2, 4 and 8 lanes
// inside each row of 16 (lanes shifted in from outside the row add 0), then the last lane
// of row 0 added to row 1 and of row 2 to row 3, then the last lane of row 1 (the total of
// rows 0 and 1) added to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2, 3
  return v;
}

// Largest of a non-negative value over the 64 lanes of a wavefront, in every lane (the same
// row shifts and broadcasts, with max for +).
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// Exclusive prefix sums over two LDS count arrays a1[0..n) and a2[0..n) by the whole
// workgroup, in one pass (two barriers); a1[n] and a2[n] receive the totals.
__device__ __forceinline__ void wg_exclusive_scan2(int* a1, int* a2, int n, int tid, int lane,
                                                   int w) {
  const int per = (n + 64 * NW - 1) / (64 * NW);
  int l1 = 0, l2 = 0;
  for (int i = 0; i < per; ++i) {
    const int x = tid * per + i;
    if (x < n) {
      l1 += a1[x];
      l2 += a2[x];
    }
  }
  const int i1 = wave_inclusive_sum(l1), i2 = wave_inclusive_sum(l2);
  if (lane == 63) {
    st_scan[w] = i1;
    st_scan2[w] = i2;
  }
  __syncthreads();
  int b1 = 0, b2 = 0;
  for (int i = 0; i < w; ++i) {
    b1 += st_scan[i];
    b2 += st_scan2[i];
  }
  int r1 = b1 + i1 - l1, r2 = b2 + i2 - l2;
  for (int i = 0; i < per; ++i) {
    const int x = tid * per + i;
    if (x < n) {
      const int t1 = a1[x], t2 = a2[x];
      a1[x] = r1;
      a2[x] = r2;
      r1 += t1;
      r2 += t2;
    }
  }
  if (tid == 64 * NW - 1) {
    a1[n] = b1 + i1;
    a2[n] = b2 + i2;
  }
  __syncthreads();
}

// The front of a wavefront's pipeline: walks its range one tile per step, then stays on
// the last tile, marked idle.
template <bool MULTI>
struct Front {
  Cur f;
  int rem;            // tiles of the range from the front on (1: the front is on its last)
  bool first;         // the front is on the first tile of the range
  bool idle;
  int B, Hkv, window, sinks;

  __device__ __forceinline__ void seg_fields() {
    f.tiles = uni(st_cum[f.s + 1] - st_cum[f.s]);
    f.L = uni(st_len[f.s]);
    if constexpr (MULTI) {
      f.tr = uni(st_seq[f.s]);
      f.sl = 0;
      f.lo = uni(st_lo[f.s]);
      f.sk = 0;
      f.t0base = (f.lo >> 4) << 4;
      return;
    }
    f.tr = f.s;
    const bool cut = window > 0 && f.L > window;
    f.sl = cut ? sinks : 0;
    f.lo = cut ? f.L - window + sinks : 0;
    f.sk = (f.sl + 15) >> 4;
    f.t0base = (max(f.sk, f.lo >> 4) - f.sk) << 4;
  }
  // position of flattened tile x
  __device__ __forceinline__ void locate(int x) {
    // the last s with Hkv st_cum[s] <= x: st_cum does not decrease, so those s are 0 .. s*;
    // the lanes count them among every step-th entry (step = ceil(B / 64)), then among the
    // step entries from the chunk that holds s* (one LDS read and one ballot each)
    const int lane = threadIdx.x & 63;
    const int step = (B + 63) >> 6;
    const int s1 = lane * step;
    const int c1 = __popcll(__ballot(s1 < B && Hkv * st_cum[s1 < B ? s1 : 0] <= x));
    const int cs = (c1 - 1) * step;
    const int s2 = cs + lane;
    const int c2 =
        __popcll(__ballot(lane < step && s2 < B && Hkv * st_cum[s2 < B ? s2 : 0] <= x));
    f.s = uni(cs + c2 - 1);
    seg_fields();
    const int within = x - Hkv * st_cum[f.s];
    f.g = uni(within / f.tiles);
    f.k = uni(within % f.tiles);
  }
  // next tile of the list; one is known to follow (segments of empty sequences are skipped)
  __device__ __forceinline__ void step() {
    if (f.k + 1 < f.tiles) {
      f.k += 1;
      return;
    }
    f.k = 0;
    f.g += 1;
    if (f.g == Hkv) {
      f.g = 0;
      int s = f.s;
      do { s += 1; } while (st_cum[s + 1] == st_cum[s]);
      f.s = uni(s);
      seg_fields();
    }
  }
  __device__ __forceinline__ Desc desc() const {
    Desc d;
    d.s = f.s;
    d.tr = f.tr;
    d.g = f.g;
    d.t0 = f.k * TILE + (f.k >= f.sk ? f.t0base : 0);
    d.sl = f.sl;
    d.lo = f.lo;
    d.L = f.L;
    d.flags = idle ? IDLE
                   : ((first ? RANGE_FIRST : 0) | (rem == 1 ? RANGE_LAST : 0) |
                      (f.k == 0 ? SEG_FIRST : 0) | (f.k == f.tiles - 1 ? SEG_LAST : 0));
    return d;
  }
  __device__ __forceinline__ void next() {
    if (idle) return;
    first = false;
    if (rem > 1) {
      step();
      rem -= 1;
    } else {
      idle = true;
    }
  }
};

// NB = 0: one query token per sequence.  NB > 0 (MULTI): several query tokens per
// sequence, taken in groups of NB blocks of 16 / G tokens; a group's NB x 16 score
// columns share every K/V tile a wavefront loads.
// VNT: the V rows are loaded with the non-temporal cache hint (pages not shared, so no
// reuse to keep); K keeps the default policy, since its four loads per row share lines.
// HQ > 1 (one query token only): a tile holds the same rows of HQ consecutive kv heads, and
// a segment is (sequence, head set); the host passes kv_heads / HQ sets of group x HQ query
// heads each, so that everything but the loads and the products sees one wider head.
template <int DEPTH, bool PAGE_TILES, int NB, bool VNT = false, bool ALIGN = false, int HQ = 1>
__global__ __launch_bounds__(64 * NW) void decode_stream_kernel(DecodeArgs a) {
  static_assert(HQ == 1 || NB == 0, "head sets with one query token only");
  using Tile = pa::stream::Tile<HQ>;
  constexpr bool MULTI = NB > 0;
  constexpr int NBX = MULTI ? NB : 1;
  // WGL: a cut segment whose pieces all lie in this workgroup's ranges hands its partials
  // over in LDS (slots of 16 columns: one block of columns at most)
  constexpr bool WGL = NB <= 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.kv_heads;
  const int G = a.group;
  // score columns in use: the G heads, or (MULTI) NB x 16 / G query tokens of G heads each;
  // column c is then head c % G of the group's query token c / G
  const int C = MULTI ? 16 * NB : G;
  const int lg = MULTI ? 31 - __clz(G) : 0;   // G is a power of two with MULTI
  int B = a.num_seqs;                         // segments per kv head: sequences or groups

  if constexpr (MULTI) {
    // ---- groups of NB x 16 / G query tokens.  One thread per sequence counts its groups
    // and their tiles; one workgroup scan gives each sequence its first group and its
    // first tile; the same thread then writes its groups' records and first tiles -------
    const int tpb = (16 >> lg) * NB;
    // sequence s: first query row, query count (clamped to the call's bounds), length
    auto seq_fields = [&](int s, int& q0, int& n, int& L) {
      q0 = a.q_start[s];
      n = a.q_start[s + 1] - q0;
      if (q0 < 0 || q0 > a.num_q) n = 0;
      n = max(0, min(min(n, a.num_q - q0), a.max_q));
      const int ctx = a.ctx[s];
      L = ctx > 0 ? (ctx < a.max_ctx ? ctx : a.max_ctx) : 0;
    };
    // group b of such a sequence: its tokens, the position of its first query, one past
    // the last query's row, the first row any of its queries attends, and its tiles
    struct Group { int nt, p0, kend, lo, tiles; };
    auto group = [&](int n, int L, int b) {
      Group g;
      g.nt = min(tpb, n - b * tpb);
      g.p0 = L - n + b * tpb;
      g.kend = max(g.p0 + g.nt, 0);
      g.lo = a.window > 0 ? max(g.p0 + 1 - a.window, 0) : 0;
      g.tiles = g.kend > 0 ? ((g.kend - 1) >> 4) - (g.lo >> 4) + 1 : 0;
      return g;
    };
    int f_q0 = 0, f_n = 0, f_L = 0;   // of sequence tid, kept for the records
    for (int s = tid; s < B; s += 64 * NW) {
      int q0, n, L;
      seq_fields(s, q0, n, L);
      if (s == tid) {
        f_q0 = q0;
        f_n = n;
        f_L = L;
      }
      const int nb = (n + tpb - 1) / tpb;
      int tiles = 0;
      for (int b = 0; b < nb; ++b) tiles += group(n, L, b).tiles;
      st_bseq[s] = nb;
      st_tseq[s] = tiles;
    }
    __syncthreads();
    wg_exclusive_scan2(st_bseq, st_tseq, B, tid, lane, w);
    const int VB = st_bseq[B];
    for (int s = tid; s < B; s += 64 * NW) {
      int q0 = f_q0, n = f_n, L = f_L;
      if (s != tid) seq_fields(s, q0, n, L);
      const int base = st_bseq[s], nb = st_bseq[s + 1] - base;
      int first = st_tseq[s];
      for (int b = 0; b < nb; ++b) {
        const int v = base + b;
        const Group g = group(n, L, b);
        st_seq[v] = s;
        st_q0[v] = q0 + b * tpb;
        st_p0[v] = g.p0;
        st_nt[v] = g.nt;
        st_lo[v] = g.lo;
        st_len[v] = g.kend;
        st_cum[v] = first;
        first += g.tiles;
      }
    }
    if (tid == 0) st_cum[VB] = st_tseq[B];
    __syncthreads();
    B = VB;
    // query rows of groups with nothing to attend are zero
    for (int v = blockIdx.x; v < B; v += gridDim.x) {
      if (st_cum[v + 1] != st_cum[v]) continue;
      float* out = a.out + (size_t)st_q0[v] * a.q_heads * HD;
      for (int i = tid; i < st_nt[v] * a.q_heads * HD; i += 64 * NW) out[i] = 0.f;
    }
  } else {
  // ---- per-sequence tile counts and their exclusive prefix sum --------------------------
  {
    const int per = (B + 64 * NW - 1) / (64 * NW);
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int s = tid * per + i;
      if (s < B) {
        int L, sl, lo;
        sink_ranges(a.ctx[s], a.window, a.sinks, a.max_ctx, L, sl, lo);
        // sink tiles, then the window's tiles from the first one past them
        const int sk = (sl + 15) >> 4;
        const int t = L > 0 ? sk + ((L - 1) >> 4) - max(sk, lo >> 4) + 1 : 0;
        st_len[s] = L;
        st_cum[s] = t;
        local += t;
      }
    }
    // inclusive scan within the wavefront, then the wavefront totals in LDS
    const int incl = wave_inclusive_sum(local);
    if (lane == 63) st_scan[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += st_scan[i];
    int run = base + incl - local;
    for (int i = 0; i < per; ++i) {
      const int s = tid * per + i;
      if (s < B) {
        const int t = st_cum[s];
        st_cum[s] = run;
        run += t;
      }
    }
    if (tid == 64 * NW - 1) st_cum[B] = base + incl;
    __syncthreads();
  }
  // output rows of sequences with nothing to attend are zero
  for (int s = blockIdx.x; s < B; s += gridDim.x) {
    if (st_cum[s + 1] != st_cum[s]) continue;
    float* out = a.out + (size_t)s * a.q_heads * HD;
    for (int i = tid; i < a.q_heads * HD; i += 64 * NW) out[i] = 0.f;
  }
  }

  // ---- the partition and this wavefront's range ----------------------------------------
  const int T = uni(Hkv * st_cum[B]);
  Part part_of{false, T, min(a.total_waves, T)};
  if constexpr (ALIGN) {
    // Aligned partition: workgroup g takes segments g NSEG / NWG to (g + 1) NSEG / NWG - 1
    // (NSEG = B Hkv, split by count: even segments give even workgroups, with no drift);
    // it is used when no workgroup then holds more than 1/16 above the mean.  Every
    // workgroup computes the same split, so all take the same decision.  The tile list
    // holds the kv heads of sequence s one after the other from Hkv st_cum[s] on, each
    // with st_cum[s + 1] - st_cum[s] tiles.
    const int NWG = gridDim.x;
    if (NWG * NW == a.total_waves && NWG <= BMAX / 4 && T >= NWG) {
      const bool narrow = (int64_t)NWG * B * Hkv < ((int64_t)1 << 31);
      for (int g = tid; g <= NWG; g += 64 * NW) {
        const int j = narrow ? (int)((uint32_t)(g * B * Hkv) / (uint32_t)NWG)
                             : (int)((int64_t)g * B * Hkv / NWG);
        const int sq = j / Hkv, h = j - sq * Hkv;
        st_wgb[g] = sq >= B ? T : Hkv * st_cum[sq] + h * (st_cum[sq + 1] - st_cum[sq]);
      }
      __syncthreads();
      // every wavefront finds the largest workgroup itself (the same value in all)
      int big = 0;
      for (int g = lane; g < NWG; g += 64) big = max(big, st_wgb[g + 1] - st_wgb[g]);
      big = wave_max_nonneg(big);
      const int mean = (T + NWG - 1) / NWG;
      part_of.aligned = big <= mean + mean / 16;
      if (part_of.aligned) part_of.R = a.total_waves;
    }
  }
  const int R = part_of.R;
  const int kw = blockIdx.x * NW + w;
  // With WGL every wavefront of the workgroup reaches the barrier ahead of the combines in
  // LDS, so one without a range (more wavefronts than tiles) only skips the stream.
  const bool has_range = part_of.aligned || kw < R;
  if (!WGL && !has_range) return;
  const int ta = has_range ? part_of.start(kw) : 0;
  const int n = has_range ? part_of.start(kw + 1) - ta : 0;

  const int P = a.page_size;
  const int lp = 31 - __clz(P);
  const int last_page = a.num_pages - 1;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  const uint32_t row_bytes = (uint32_t)a.row_stride * 2;      // one token's row of a head
  const uint32_t head_bytes = (uint32_t)a.head_stride * 2;    // one kv head within a page
  const uint32_t page_bytes = (uint32_t)(Hkv * HQ) * HD * 2 * (uint32_t)P;
  const int col = lane & 15;
  const int grp = lane >> 4;

  Front<MULTI> fr;
  fr.B = B;
  fr.Hkv = Hkv;
  fr.window = a.window;
  fr.sinks = a.sinks;
  if (n > 0) fr.locate(ta);   // (an aligned range may be empty)
  fr.rem = n;
  fr.first = true;
  fr.idle = false;

  // Table entries.  With pages of at least 16 rows the tile lies in one page: one entry,
  // read through the scalar path (constant address space), whose completion is counted
  // apart from the vector loads, so waiting for it never drains the K/V tiles in flight.
  // Smaller pages need one entry per token (lane col holds token t0 + col's).  Rows outside
  // the attended ones are clamped to one that is, so their entries are mapped pages.
  const __attribute__((address_space(4))) int32_t* bt_const =
      (const __attribute__((address_space(4))) int32_t*)a.block_tables;
  // Table entries of a tile.  Pages of at least 16 rows: the one page of the tile, read
  // through the scalar unit.  Smaller pages: each lane reads the page of its K row (token
  // t0 + col) and those of its four V rows (tokens t0 + 4 grp + j) itself, one tile ahead,
  // so the V addresses need no lane shuffle while the tile's loads wait to issue.
  auto table_entry = [&](const Desc& d) {
    if constexpr (PAGE_TILES) {
      const int t = d.t0 < d.sl ? d.t0 : min(max(d.t0, d.lo), d.L - 1);
      // num_seqs * bt_stride < 2^31 on this path, so the index fits one scalar register
      return bt_const[uni(d.tr * a.bt_stride + (t >> lp))];
    } else {
      const int32_t* row = a.block_tables + (size_t)d.tr * a.bt_stride;
      auto clamp_row = [&](int tc) { return tc < d.sl ? tc : min(max(tc, d.lo), d.L - 1); };
      RowPages e;
      e.k = row[clamp_row(d.t0 + col) >> lp];
#pragma unroll
      for (int j = 0; j < 4; ++j) e.v[j] = row[clamp_row(d.t0 + 4 * grp + j) >> lp];
      return e;
    }
  };

  auto row_addr = [&](const char* base, int pg, int t, uint32_t lane_off) {
    return reinterpret_cast<const uint4*>(base + (uint64_t)(uint32_t)pg * page_bytes +
                                          ((uint32_t)(t & (P - 1)) * row_bytes + lane_off));
  };

  // K rows of token t0 + col (16 B at byte 64 j + 16 grp for product j: the four lanes of
  // a token read 64 contiguous bytes per load), V rows of tokens t0 + 4 grp + j (16 B at
  // column block col).  When a tile lies inside one page (page size >= 16: tiles start
  // at multiples of 16) the per-lane byte offsets are the same for every tile.
  const uint32_t k_lane_off = (uint32_t)col * row_bytes + grp * 16;
  const uint32_t v_lane_off = (uint32_t)(4 * grp) * row_bytes + col * 16;

  auto load_tile = [&](const Desc& d, const auto& e, Tile& Tl) {
    const int t0 = d.t0;
    if (NB <= 1 && (uni(d.flags) & (RANGE_FIRST | SEG_FIRST))) {
      // the query rows of the group, fetched with the tile so that waiting for them is
      // waiting for this tile; lanes past the group read head 0 and are zeroed later
      size_t qr;
      if constexpr (MULTI) {
        // column col: query token col / G of the block, head col % G of the group
        const int tq = (col >> lg) < st_nt[d.s] ? (col >> lg) : 0;
        qr = (size_t)(st_q0[d.s] + tq) * a.q_heads + (size_t)d.g * G + (col & (G - 1));
      } else {
        qr = (size_t)d.s * a.q_heads + (size_t)d.g * G + (col < G ? col : 0);
      }
      const uint4* qrow = reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint16_t*>(a.q) + qr * HD + grp * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) Tl.q[j] = qrow[4 * j];
    }
    if constexpr (PAGE_TILES) {
      // one page for the whole tile: a uniform base address plus constant lane offsets
      // (the descriptor's fields are the same in every lane: read as such, the mask and
      // the base address are scalar work)
      const int pg = uni(e);
      const int ut0 = uni(t0), ulo = uni(d.lo), uL = uni(d.L), usl = uni(d.sl), ug = uni(d.g);
      const bool mapped = pg >= 0 && pg <= last_page;
      const int lo_off = min(max(ulo - ut0, 0), TILE), hi_off = min(uL - ut0, TILE);
      const int sl_off = min(max(usl - ut0, 0), TILE);
      const uint32_t bits = ((1u << hi_off) - 1u) & (~((1u << lo_off) - 1u) | ((1u << sl_off) - 1u));
      Tl.valid = mapped ? bits : 0u;
      const uint64_t base = (uint64_t)(uint32_t)min(max(pg, 0), last_page) * page_bytes +
                            (uint32_t)(ut0 & (P - 1)) * row_bytes +
                            (uint32_t)(ug * HQ) * head_bytes;
#pragma unroll
      for (int h = 0; h < HQ; ++h) {
        const uint4* kp = reinterpret_cast<const uint4*>(kbase + base + h * head_bytes + k_lane_off);
#pragma unroll
        for (int j = 0; j < 4; ++j) Tl.k[4 * h + j] = kp[4 * j];
      }
#pragma unroll
      for (int h = 0; h < HQ; ++h) {
        const char* vb = vbase + base + h * head_bytes + v_lane_off;
        if constexpr (VNT) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            Tl.v[4 * h + j] = __builtin_bit_cast(
                uint4, __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vb + j * row_bytes)));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            Tl.v[4 * h + j] = *reinterpret_cast<const uint4*>(vb + j * row_bytes);
        }
      }
    } else {
    const int tk = t0 + col;
    Tl.valid = (uint32_t)(__ballot((tk < d.sl || tk >= d.lo) && tk < d.L && e.k >= 0 &&
                                   e.k <= last_page) & 0xffffull);
    const uint32_t hoff = (uint32_t)(d.g * HQ) * head_bytes;
    const int tkc = tk < d.sl ? tk : min(max(tk, d.lo), d.L - 1);
#pragma unroll
    for (int h = 0; h < HQ; ++h) {
      const uint4* kp =
          row_addr(kbase, min(max(e.k, 0), last_page), tkc, hoff + h * head_bytes + grp * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) Tl.k[4 * h + j] = kp[4 * j];
    }
#pragma unroll
    for (int h = 0; h < HQ; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tr = t0 + 4 * grp + j;
      const int tv = tr < d.sl ? tr : min(max(tr, d.lo), d.L - 1);
      const uint4* vp = row_addr(vbase, min(max(e.v[j], 0), last_page), tv,
                                 hoff + h * head_bytes + col * 16);
      if constexpr (VNT)
        Tl.v[4 * h + j] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vp)));
      else
        Tl.v[4 * h + j] = *vp;
    }
    }
  };

  // ---- per-segment state -----------------------------------------------------------------
  // m_ref: reference max of score column col (query head col), the same in every lane
  // group; l_run: this lane's share of the running sum (its four tokens); oacc[e][r]:
  // output of query head 4 grp + r at column 8 col + e.
  // One set per block of 16 columns (decode: one).
  bf16x8 qb[NBX][4];
  float m_ref[NBX], l_run[NBX];
  f32x4 oacc[NBX][8];
  // (HQ > 1) the query operand of head h of the set: the lane's column's query where that
  // column is one of head h's, zero elsewhere, so that head h's products add nothing to
  // the other heads' columns
  bf16x8 qm[HQ > 1 ? HQ : 1][4];
  const int hc = HQ > 1 ? col / (G / HQ) : 0;   // head of the set column col belongs to
  bool first_seg = true;     // the segment being computed is the first of the range
  bool started_here = false; // ... and its tile 0 lies in this range
  // this lane's score column of each block is in use; (MULTI) the rows its query may
  // attend are (pc_lo, pc]
  bool cval[NBX];
  int pc[NBX], pc_lo[NBX];
  // (MULTI) a tile of rows [t0, t0 + 16) with t0 + 15 <= seg_pmin and t0 > seg_plo is
  // attended by every query of the segment's group
  int seg_pmin = 0, seg_plo = 0;
#pragma unroll
  for (int i = 0; i < NBX; ++i) {
    m_ref[i] = -INFINITY;
    l_run[i] = 0.f;
    cval[i] = col < G;
    pc[i] = pc_lo[i] = 0;
  }
  // partial area: the (max, sum) pair of every slot and column, then their accumulators
  const uint32_t nslots = (uint32_t)a.total_waves * 2 * C;
  const DevBuf part(a.ws_ml, nslots * (2 + HD) * 4);
  auto ml_off = [&](uint32_t idx) { return idx * 8; };
  auto acc_off = [&](uint32_t idx) { return nslots * 8 + idx * HD * 4; };
  // cut segments this range holds a piece of: its first segment (piece in slot 0) and its
  // last (slot 1); segment index s * Hkv + g and the ranges of its first and last piece
  bool cut0 = false, cut1 = false;
  int seg0 = 0, k1_0 = 0, k2_0 = 0, seg1 = 0, k1_1 = 0, k2_1 = 0;
  // the pieces of a cut segment, ranges k1 .. k2, all lie in this workgroup (ranges
  // NW blockIdx .. NW blockIdx + NW - 1): its partials go through LDS
  auto in_workgroup = [&](int k1, int k2) {
    return part_of.aligned || (WGL && k1 / NW == k2 / NW);
  };

  auto begin_segment = [&](const Desc& d, const Tile& Tl) {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if constexpr (MULTI) {
      const int nt = st_nt[d.s], p0 = st_p0[d.s], q0 = st_q0[d.s];
      seg_pmin = uni(p0);
      seg_plo = uni(a.window > 0 ? p0 + nt - 1 - a.window : (-0x7fffffff - 1));
#pragma unroll
      for (int i = 0; i < NBX; ++i) {
        const int tq = ((i * 16 + col) >> lg);   // query token of this lane's column
        cval[i] = tq < nt;
        pc[i] = p0 + tq;
        pc_lo[i] = a.window > 0 ? pc[i] - a.window : (-0x7fffffff - 1);
        if constexpr (NB > 1) {
          // the group's queries, read here (a wait for them drains the loads in flight,
          // once per segment)
          const uint4* qrow = reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(a.q) +
              ((size_t)(q0 + (cval[i] ? tq : 0)) * a.q_heads + (size_t)d.g * G +
               (col & (G - 1))) * HD + grp * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) qb[i][j] = as_bf16x8(cval[i] ? qrow[4 * j] : zero);
        }
      }
    }
    if constexpr (NB <= 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) qb[0][j] = as_bf16x8(cval[0] ? Tl.q[j] : zero);
      if constexpr (HQ > 1) {
#pragma unroll
        for (int h = 0; h < HQ; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) qm[h][j] = as_bf16x8(hc == h && cval[0] ? Tl.q[j] : zero);
      }
    }
#pragma unroll
    for (int i = 0; i < NBX; ++i) {
      m_ref[i] = -INFINITY;
      l_run[i] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[i][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    started_here = (uni(d.flags) & SEG_FIRST) != 0;
  };

  auto end_segment = [&](const Desc& d, bool complete) {
    float* out = a.out + ((size_t)d.s * a.q_heads + (size_t)d.g * G) * HD + col * 8;
    int ncols = G;
    if constexpr (MULTI) {
      out = a.out + ((size_t)st_q0[d.s] * a.q_heads + (size_t)d.g * G) * HD + col * 8;
      ncols = st_nt[d.s] << lg;
    }
    // a piece of a segment cut by a range boundary: partial (max, sum, accumulator) to
    // slot 0 (the range's first segment) or 1 (its last), stored at device scope (written
    // through to the point where every compute unit reads it)
    const size_t pi = (size_t)kw * 2 + (first_seg ? 0 : 1);
    int k1 = 0, k2 = 0;
    if (!complete) {
      const int tiles = st_cum[d.s + 1] - st_cum[d.s];
      const int seg_start = Hkv * st_cum[d.s] + d.g * tiles;
      k1 = part_of.of(seg_start);
      k2 = part_of.of(seg_start + tiles - 1);
    }
    const bool in_lds = in_workgroup(k1, k2);
#pragma unroll
    for (int i = 0; i < NBX; ++i) {
      float lt = l_run[i];
      lt += __shfl_xor(lt, 16, 64);
      lt += __shfl_xor(lt, 32, 64);
      float lr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lr[r] = __shfl(lt, 4 * grp + r, 64);
      if (complete) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = i * 16 + 4 * grp + r;
          if (h < ncols) {
            const float inv = lr[r] > 0.f ? 1.f / lr[r] : 0.f;
            // MULTI: column h is head h % G of query token h / G (rows q_heads apart)
            const size_t row = MULTI ? (size_t)(h >> lg) * a.q_heads + (h & (G - 1)) : (size_t)h;
            float4* o = reinterpret_cast<float4*>(out + row * HD);
            const f32x4* ac = oacc[i];
            o[0] = make_float4(ac[0][r] * inv, ac[1][r] * inv, ac[2][r] * inv, ac[3][r] * inv);
            o[1] = make_float4(ac[4][r] * inv, ac[5][r] * inv, ac[6][r] * inv, ac[7][r] * inv);
          }
        }
      } else if (in_lds) {
        // every piece of the segment lies in this workgroup: the partial stays in LDS for
        // the workgroup's combine (one block of 16 columns: NB is at most 1 here)
        float* pl = st_part[w][first_seg ? 0 : 1];
        if (lane < C) {
          pl[2 * lane] = m_ref[i];
          pl[2 * lane + 1] = lt;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * grp + r;
          if (h < C) {
            float* pa = pl + 2 * C + h * HD + col * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) pa[e] = oacc[i][e][r];
          }
        }
      } else {
        const int c0 = i * 16;
        if (lane < min(C - c0, 16))
          part.store2(ml_off((uint32_t)(pi * C + c0 + lane)), make_float2(m_ref[i], lt));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = c0 + 4 * grp + r;
          if (h < C) {
            const uint32_t o = acc_off((uint32_t)(pi * C + h)) + col * 32;
            const f32x4* ac = oacc[i];
            part.store4(o, make_float4(ac[0][r], ac[1][r], ac[2][r], ac[3][r]));
            part.store4(o + 16, make_float4(ac[4][r], ac[5][r], ac[6][r], ac[7][r]));
          }
        }
      }
    }
    if (!complete) {
      if (first_seg) {
        cut0 = true;
        seg0 = d.s * Hkv + d.g;
        k1_0 = k1;
        k2_0 = k2;
      } else {
        cut1 = true;
        seg1 = d.s * Hkv + d.g;
        k1_1 = k1;
        k2_1 = k2;
      }
    }
    first_seg = false;
  };

  auto compute = [&](const Tile& Tl, const Desc& d) {
    // the tile's flags and row mask are the same in every lane: read them as such, so
    // the branches on them are scalar
    const int flags = uni(d.flags);
    const uint32_t valid = (uint32_t)uni((int)Tl.valid);
    if (flags & (RANGE_FIRST | SEG_FIRST)) begin_segment(d, Tl);
    // scores S[token][column] = K . q, one product per block of 16 columns
    f32x4 sc[NBX];
#pragma unroll
    for (int i = 0; i < NBX; ++i) {
      sc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (HQ > 1) {
        // head h's keys against the queries of head h's columns (zero in the others)
#pragma unroll
        for (int h = 0; h < HQ; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Tl.k[4 * h + j]), qm[h][j],
                                                            sc[i], 0, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Tl.k[j]), qb[i][j], sc[i],
                                                          0, 0, 0);
      }
    }
    // a tile whose rows every column attends needs no masks (most tiles of long contexts)
    bool plain = valid == 0xffffu;
    if constexpr (MULTI) plain = plain && d.t0 + 15 <= seg_pmin && d.t0 > seg_plo;
    bf16x4 phi[NBX], plo[NBX];
#pragma unroll
    for (int i = 0; i < NBX; ++i) {
      float sv[4];
      float mt = -INFINITY;
      if (plain) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = sc[i][r] * a.qscale;
          mt = fmaxf(mt, sv[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bool ok = (valid >> (4 * grp + r)) & 1;
          if constexpr (MULTI) {
            const int t = d.t0 + 4 * grp + r;
            ok = ok && t <= pc[i] && t > pc_lo[i];
          }
          sv[r] = ok ? sc[i][r] * a.qscale : -INFINITY;
          mt = fmaxf(mt, sv[r]);
        }
      }
      // raise the reference when some column's tile max passes it by more than RESCALE_T;
      // this lane's own max decides whether any does, so the cross-lane max is only taken
      // on the (rare) raise
      if (__ballot(cval[i] && mt > m_ref[i] + RESCALE_T) != 0) {
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m_ref[i], mt);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref[i] - mn);
        l_run[i] *= alpha;
        m_ref[i] = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
          for (int e = 0; e < 8; ++e) oacc[i][e][r] *= ar;
        }
      }
      const float ms = m_ref[i] == -INFINITY ? 0.f : m_ref[i];
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = cval[i] ? __builtin_amdgcn_exp2f(sv[r] - ms) : 0.f;
        l_run[i] += p[r];
      }
      // P as the A operand (row = column col, k = token 4 grp + r), split into a bf16 high
      // part and the bf16-rounded remainder
      const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
      const uint32_t l01 = pack_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
      phi[i] = __builtin_bit_cast(bf16x4, make_uint2(h01, h23));
      plo[i] = __builtin_bit_cast(bf16x4, make_uint2(l01, l23));
    }
    // Rows outside the attended range get probability 0, but their V may be anything
    // (rows of the last page past the sequence end are never written): replace them by
    // zeros, since 0 * NaN would poison the product.
#pragma unroll
    for (int h = 0; h < HQ; ++h) {
      uint4 vt[4] = {Tl.v[4 * h], Tl.v[4 * h + 1], Tl.v[4 * h + 2], Tl.v[4 * h + 3]};
      if (valid != 0xffffu) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!((valid >> (4 * grp + j)) & 1)) vt[j] = make_uint4(0, 0, 0, 0);
      }
      const uint32_t v0[4] = {vt[0].x, vt[0].y, vt[0].z, vt[0].w};
      const uint32_t v1[4] = {vt[1].x, vt[1].y, vt[1].z, vt[1].w};
      const uint32_t v2[4] = {vt[2].x, vt[2].y, vt[2].z, vt[2].w};
      const uint32_t v3[4] = {vt[3].x, vt[3].y, vt[3].z, vt[3].w};
      // (HQ > 1) head h's values only for the rows of P (columns) that are head h's
      bf16x4 ph[NBX], pl[NBX];
#pragma unroll
      for (int i = 0; i < NBX; ++i) {
        const bf16x4 z = {0, 0, 0, 0};
        ph[i] = HQ == 1 || hc == h ? phi[i] : z;
        pl[i] = HQ == 1 || hc == h ? plo[i] : z;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // column 8 col + e of the four tokens: the B operand (k = token, n = column block),
        // gathered once and used by every block
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t b01 = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], sel);
        const uint32_t b23 = __builtin_amdgcn_perm(v3[e >> 1], v2[e >> 1], sel);
        const bf16x4 bv = __builtin_bit_cast(bf16x4, make_uint2(b01, b23));
#pragma unroll
        for (int i = 0; i < NBX; ++i) {
          oacc[i][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph[i], bv, oacc[i][e], 0, 0, 0);
          oacc[i][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl[i], bv, oacc[i][e], 0, 0, 0);
        }
      }
    }
    if (flags & (SEG_LAST | RANGE_LAST))
      end_segment(d, (flags & SEG_LAST) && started_here);
  };

  // ---- pipeline: table entry DEPTH+1 tiles ahead, K/V DEPTH tiles ahead, compute ------
  // The K/V buffers and their descriptors form a ring of DEPTH+1 slots indexed by
  // compile-time constants (the inner loop is fully unrolled), so every stage keeps fixed
  // registers.  Past the end of the range the front repeats its last tile marked IDLE: it
  // is re-read (a cache hit) and skipped.
  Tile buf[DEPTH + 1];
  Desc dsc[DEPTH + 1];
  if (n > 0) {
  Desc d_next = fr.desc();
  auto e_next = table_entry(d_next);
  fr.next();
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    const Desc d_use = d_next;
    const auto e_use = e_next;
    d_next = fr.desc();
    e_next = table_entry(d_next);
    fr.next();
    load_tile(d_use, e_use, buf[u]);
    dsc[u] = d_use;
  }
  for (;;) {
#pragma unroll
    for (int u = 0; u <= DEPTH; ++u) {
      const Desc d_use = d_next;
      const auto e_use = e_next;
      d_next = fr.desc();
      e_next = table_entry(d_next);
      fr.next();
      load_tile(d_use, e_use, buf[(u + DEPTH) % (DEPTH + 1)]);
      dsc[(u + DEPTH) % (DEPTH + 1)] = d_use;
      if (!(uni(dsc[u].flags) & IDLE)) compute(buf[u], dsc[u]);
    }
    if (uni(dsc[DEPTH].flags) & IDLE) break;
  }
  }

  // One wavefront combines a segment, CPP columns per pass: lane l of the NL lanes doing
  // it takes head_dim QPL floats of column l / LPC (+ CPP per pass), LPC = NL / CPP; the
  // partials of COMBINE_BATCH pieces are loaded together.  Decode (at most 16 columns,
  // usually a few) takes 4 columns per pass, several query tokens (16 or 32 columns) 8.
  // A decode wavefront that combines both of its segments gives each one half of its
  // lanes, so that the loads of the two combines are in flight together.
  constexpr int CPP = MULTI || HQ > 1 ? 8 : 4;
  auto combine = [&](auto nl_c, int sl, int seg, int k1, int k2) {
    constexpr int NL = decltype(nl_c)::value;
    constexpr int LPC = NL / CPP;             // lanes per column
    constexpr int QPL = HD / LPC / 4;         // float4 per lane
    const int s = seg / Hkv, g = seg % Hkv;
    const int tiles = st_cum[s + 1] - st_cum[s];
    const int seg_start = Hkv * st_cum[s] + g * tiles;
    // in range k1 the segment is the first one (slot 0) only if it starts the range
    const int slot1 = seg_start == part_of.start(k1) ? 0 : 1;
    float* out = a.out + ((size_t)s * a.q_heads + (size_t)g * G) * HD;
    int ncols = G;
    if constexpr (MULTI) {
      out = a.out + ((size_t)st_q0[s] * a.q_heads + (size_t)g * G) * HD;
      ncols = st_nt[s] << lg;
    }
    const int cd = (sl % LPC) * (QPL * 4);
    const bool in_lds = in_workgroup(k1, k2);
    for (int h = sl / LPC; h < ncols; h += CPP) {
      float M = -INFINITY, den = 0.f;
      float4 nm[QPL];
#pragma unroll
      for (int q = 0; q < QPL; ++q) nm[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k0 = k1; k0 <= k2; k0 += COMBINE_BATCH) {
        float2 ml[COMBINE_BATCH];
        float4 x[COMBINE_BATCH][QPL];
#pragma unroll
        for (int b = 0; b < COMBINE_BATCH; ++b) {
          const int k = min(k0 + b, k2);
          if (in_lds) {
            // the piece of wavefront k - NW blockIdx of this workgroup, from LDS
            const float* pl = st_part[k - (int)blockIdx.x * NW][k == k1 ? slot1 : 0];
            ml[b] = make_float2(pl[2 * h], pl[2 * h + 1]);
            const float* src = pl + 2 * C + h * HD + cd;
#pragma unroll
            for (int q = 0; q < QPL; ++q)
              x[b][q] = make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
            continue;
          }
          const size_t pi = (size_t)k * 2 + (k == k1 ? slot1 : 0);
          ml[b] = part.load2(ml_off((uint32_t)pi * C + h));
          const uint32_t o = acc_off((uint32_t)pi * C + h) + cd * 4;
#pragma unroll
          for (int q = 0; q < QPL; ++q) x[b][q] = part.load4(o + 16 * q);
        }
#pragma unroll
        for (int b = 0; b < COMBINE_BATCH; ++b) {
          const float mm = ml[b].x;
          if (k0 + b > k2 || mm == -INFINITY) continue;
          const float mn = fmaxf(M, mm);
          const float fo = exp2f(M - mn), fn = exp2f(mm - mn);
          den = den * fo + ml[b].y * fn;
#pragma unroll
          for (int q = 0; q < QPL; ++q) {
            nm[q].x = nm[q].x * fo + x[b][q].x * fn;
            nm[q].y = nm[q].y * fo + x[b][q].y * fn;
            nm[q].z = nm[q].z * fo + x[b][q].z * fn;
            nm[q].w = nm[q].w * fo + x[b][q].w * fn;
          }
          M = mn;
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const size_t row = MULTI ? (size_t)(h >> lg) * a.q_heads + (h & (G - 1)) : (size_t)h;
      float4* o = reinterpret_cast<float4*>(out + row * HD + cd);
#pragma unroll
      for (int q = 0; q < QPL; ++q)
        o[q] = make_float4(nm[q].x * inv, nm[q].y * inv, nm[q].z * inv, nm[q].w * inv);
    }
    if (sl == 0 && !in_lds)
      __hip_atomic_store(a.ws_arrive + k1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // ---- cut segments -----------------------------------------------------------------------
  // A segment whose pieces all lie in this workgroup's ranges (always, with the aligned
  // partition; with the flat one, when its ranges are among this workgroup's four) hands
  // its partials over in LDS and is combined after a barrier by the wavefront holding its
  // first piece.  A segment cut across workgroups is combined by the piece that arrives
  // last: each piece counts itself on the counter of the segment's first range once its
  // partial is written; the one that completes the count reads every piece's partial,
  // combines them in range order, and puts the counter back to zero for the next call.
  // Those partials and counters move only through device-scope accesses (stores written
  // through, loads that skip the caches of the compute unit and of its die), and the count
  // is raised only after this wavefront's partial stores have completed (vmcnt reaches 0),
  // so a wavefront that sees the full count reads complete partials.  No cache-wide
  // write-back or invalidate is needed: nothing is exchanged through ordinary cached
  // stores.  Either way the pieces are combined in range order with the same arithmetic.
  if (part_of.aligned) {
    // every piece of a cut segment lies in this workgroup: after the barrier the wavefront
    // holding a segment's first piece combines it from LDS.  A workgroup with fewer tiles
    // than wavefronts has empty ranges, which can lie between a segment's first and last
    // pieces: they publish a running max of -inf, a piece the combine skips.
    if (n == 0 && lane < C) {
      st_part[w][0][2 * lane] = -INFINITY;
      st_part[w][1][2 * lane] = -INFINITY;
    }
    __syncthreads();
    const bool own0 = cut0 && k1_0 == kw, own1 = cut1 && k1_1 == kw;
    if (!MULTI && own0 && own1) {
      const bool hi = lane >= 32;
      combine(std::integral_constant<int, 32>{}, lane & 31, hi ? seg1 : seg0,
              hi ? k1_1 : k1_0, hi ? k2_1 : k2_0);
    } else {
      if (own0) combine(std::integral_constant<int, 64>{}, lane, seg0, k1_0, k2_0);
      if (own1) combine(std::integral_constant<int, 64>{}, lane, seg1, k1_1, k2_1);
    }
    return;
  }
  // segments cut across workgroups: through the device-scope counters and partials
  const bool dev0 = cut0 && !in_workgroup(k1_0, k2_0), dev1 = cut1 && !in_workgroup(k1_1, k2_1);
  if (dev0 || dev1) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // all counters: every store above has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int arrived0 = 0, arrived1 = 0;
    if (lane == 0) {
      if (dev0)
        arrived0 = __hip_atomic_fetch_add(a.ws_arrive + k1_0, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      if (dev1)
        arrived1 = __hip_atomic_fetch_add(a.ws_arrive + k1_1, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    }
    arrived0 = __builtin_amdgcn_readlane(arrived0, 0);
    arrived1 = __builtin_amdgcn_readlane(arrived1, 0);
    const bool last0 = dev0 && arrived0 == k2_0 - k1_0;
    const bool last1 = dev1 && arrived1 == k2_1 - k1_1;
    if (!MULTI && last0 && last1) {
      const bool hi = lane >= 32;
      combine(std::integral_constant<int, 32>{}, lane & 31, hi ? seg1 : seg0, hi ? k1_1 : k1_0,
              hi ? k2_1 : k2_0);
    } else {
      if (last0) combine(std::integral_constant<int, 64>{}, lane, seg0, k1_0, k2_0);
      if (last1) combine(std::integral_constant<int, 64>{}, lane, seg1, k1_1, k2_1);
    }
  }
  if constexpr (WGL) {
    // segments whose pieces all lie in this workgroup: once every wavefront has left its
    // stream (and written its pieces to LDS), the wavefront holding a segment's first piece
    // combines it.  Every wavefront of the workgroup reaches this barrier.
    __syncthreads();
    const bool own0 = cut0 && !dev0 && k1_0 == kw, own1 = cut1 && !dev1 && k1_1 == kw;
    if (!MULTI && own0 && own1) {
      const bool hi = lane >= 32;
      combine(std::integral_constant<int, 32>{}, lane & 31, hi ? seg1 : seg0,
              hi ? k1_1 : k1_0, hi ? k2_1 : k2_0);
    } else {
      if (own0) combine(std::integral_constant<int, 64>{}, lane, seg0, k1_0, k2_0);
      if (own1) combine(std::integral_constant<int, 64>{}, lane, seg1, k1_1, k2_1);
    }
  }
}

// Tiles of the whole list at most: max_live attended rows per sequence, of which `sinks`
// may form a run of their own at the start.
inline int64_t tiles_bound(int num_seqs, int kv_heads, int max_live, int sinks) {
  const int per = sinks > 0 ? (sinks + 15) / 16 + (max_live - sinks + 15) / 16 + 1
                            : (max_live + 15) / 16 + 1;
  return (int64_t)num_seqs * kv_heads * per;
}

inline bool eligible(int dtype, int head_dim, int group, int page_size, int num_seqs,
                     int bt_stride, int kv_heads, int max_live, int sinks) {
  return dtype == PA_BF16 && head_dim == HD && group >= 1 && group <= 16 && page_size > 0 &&
         (page_size & (page_size - 1)) == 0 && num_seqs >= 1 && num_seqs <= BMAX &&
         (int64_t)num_seqs * bt_stride < ((int64_t)1 << 31) &&
         tiles_bound(num_seqs, kv_heads, max_live, sinks) < ((int64_t)1 << 30);
}

// Several query tokens per sequence: groups of nb blocks of 16 / group tokens, each
// attending at most `keys` rows (the window plus the group's other tokens, or the whole
// context).  Longer chunks take more blocks per group, so that more query columns share
// every K/V tile.
inline int multi_blocks(int group, int max_q) {
  // four blocks (64 columns) would need more registers than a wavefront has
  return max_q <= 16 / group ? 1 : 2;
}
inline int64_t blocks_bound(int num_seqs, int group, int max_q, int nb) {
  const int tpg = 16 / group * nb;
  return (int64_t)num_seqs * ((max_q + tpg - 1) / tpg);
}
inline int64_t tiles_bound_multi(int num_seqs, int kv_heads, int group, int max_q, int keys,
                                 int nb) {
  return blocks_bound(num_seqs, group, max_q, nb) * kv_heads * ((keys + 15) / 16 + 1);
}
inline bool eligible_multi(int dtype, int head_dim, int group, int page_size, int num_seqs,
                           int bt_stride, int kv_heads, int max_q, int keys, int nb) {
  return dtype == PA_BF16 && head_dim == HD && group >= 1 && group <= 16 &&
         (group & (group - 1)) == 0 && page_size > 0 && (page_size & (page_size - 1)) == 0 &&
         num_seqs >= 1 && max_q >= 1 && blocks_bound(num_seqs, group, max_q, nb) <= BMAX &&
         (int64_t)num_seqs * bt_stride < ((int64_t)1 << 31) &&
         tiles_bound_multi(num_seqs, kv_heads, group, max_q, keys, nb) < ((int64_t)1 << 30);
}

// Workspace: the arrival counters in the common header (zero between calls; one per
// range, at most WS_HEADER / 4 ranges), then per wavefront two partial slots of `cols`
// score columns (running max and sum, accumulator): the group's heads, or 16 with
// several query tokens per sequence.
inline size_t workspace_bytes(int total_waves, int cols) {
  const size_t slots = (size_t)total_waves * 2 * cols;
  return WS_HEADER + slots * 2 * sizeof(float) + slots * HD * sizeof(float);
}
inline void carve_workspace(DecodeArgs& a, void* workspace, int cols) {
  const size_t slots = (size_t)a.total_waves * 2 * cols;
  a.ws_arrive = reinterpret_cast<int*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + WS_HEADER);
  a.ws_acc = a.ws_ml + slots * 2;
}

template <int NB, bool ALIGN, int HQ>
inline void launch_variant(const DecodeArgs& a, hipStream_t st, dim3 grid, dim3 block) {
  constexpr int D = NB > 0 ? STREAM_MULTI_DEPTH : STREAM_DEPTH;
  const bool unshared = (a.hints & PA_HINT_UNSHARED) != 0;
  if constexpr (HQ == 1) {   // (head sets serve pages under 16 rows only)
    if (a.page_size >= TILE) {
      if (unshared)
        hipLaunchKernelGGL((decode_stream_kernel<D, true, NB, true, ALIGN, 1>), grid, block, 0,
                           st, a);
      else
        hipLaunchKernelGGL((decode_stream_kernel<D, true, NB, false, ALIGN, 1>), grid, block, 0,
                           st, a);
      return;
    }
  }
  if (unshared)
    hipLaunchKernelGGL((decode_stream_kernel<D, false, NB, true, ALIGN, HQ>), grid, block, 0,
                       st, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<D, false, NB, false, ALIGN, HQ>), grid, block, 0,
                       st, a);
}

// Only a kernel built with ALIGN tries the aligned partition, so the others carry none of
// its branches.  (Its LDS partials hold one block of 16 columns: NB at most 1.)
template <int NB, int HQ>
inline void launch_nb(const DecodeArgs& a, hipStream_t st, dim3 grid, dim3 block) {
  if (NB <= 1 && a.try_aligned)
    launch_variant<NB, NB <= 1, HQ>(a, st, grid, block);
  else
    launch_variant<NB, false, HQ>(a, st, grid, block);
}

// Kv heads per tile of the one-token path.  With pages under 16 rows every lane reads the
// table entries of its own rows for each tile, and a tile of four (or two) kv heads reads
// them once for all of its heads, whose columns fill the 16 of a product together (group
// x heads at most 16); 4-5% faster on the raw slot-table workload, at every group size
// measured.  With pages of 16 rows or more (one scalar entry per tile) tiles of several
// heads ran slower, so those keep one head.  The choice is the same in both pool layouts,
// which therefore give the same bits.
inline int head_set(int group, int kv_heads, int page_size) {
  if (page_size >= TILE) return 1;
  if (group * 4 <= 16 && kv_heads % 4 == 0) return 4;
  return group * 2 <= 16 && kv_heads % 2 == 0 ? 2 : 1;
}

// nb = 0: one query token per sequence (hq kv heads per tile: 1, 2 or 4); 1 or 2: blocks
// per group of query tokens
inline int launch(const DecodeArgs& a, hipStream_t st, int nb, int hq = 1) {
  const dim3 grid((unsigned)(a.total_waves / NW)), block(64 * NW);
  if (nb != 0 && hq != 1) return -1;
  switch (nb * 8 + hq) {
    case 1: launch_nb<0, 1>(a, st, grid, block); break;
    case 2: launch_nb<0, 2>(a, st, grid, block); break;
    case 4: launch_nb<0, 4>(a, st, grid, block); break;
    case 9: launch_nb<1, 1>(a, st, grid, block); break;
    case 17: launch_nb<2, 1>(a, st, grid, block); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace stream
}  // namespace pa
