// Main Branch ("MiniMax Sparse Attention" explainer, section 05 part 2).
//
// KV-outer partial attention: each non-local KV block is loaded once per
// work item and the queries that selected it are gathered through the
// inverted index; G heads x several query positions are packed into MFMA
// row tiles (query concatenation); hot blocks are cut along the query
// dimension into work items planned before launch (pre-scheduled
// chunking); each (query, head, block) partial goes to a pre-assigned slot
// (two-phase forward).
//
// Combine: one work-group per (query block, group) loads that block's K/V,
// computes the local block -- the query's own block, the only one with a
// causal mask -- exactly on MFMA with a hi/lo split of P, and merges it with
// the query's non-local partials through their log-sum-exp in ascending
// slot (= block) order.  Keeping the local block out of the partial buffer
// saves its round trip through HBM and keeps rows i < 128, which see only
// their local block, in fp32 all the way.
//
// Partial precision: O_s in bf16 (the pages' IO accounting is bf16), lse_s
// in fp32.  Workspace layouts (d_h = DH, G heads per group):
//   Os    bf16 [Nq][k-1][H_kv][DH/4][G][4]   non-local slot s of position iq
//   lse_s fp32 [Nq][k-1][H_q]
// plus one spare slot after the last, written (never read) by MFMA rows
// past the end of a work item.
// One (position, slot, group) partial is G * DH contiguous values, and
// within it four consecutive d of consecutive heads are adjacent, so the G
// heads of a position that one MFMA tile holds store G * 8 contiguous
// bytes per instruction, and the combine reads them back the same way.
#include "common.h"
#include "lds_rows.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

// ---------------------------------------------------------------------------
// Work list.  Bucket (r, b) of the CSR holds first the queries whose local
// block is b (positions inside block b, all of which select it), then the
// queries that picked b as a non-local block.  For the attention the first
// part is handled by the combine and only the second is cut into items of
// at most `chunk` positions; with `with_local` (the index KL pass) the
// whole bucket is.  Item = {bucket, start offset into col, count, 0}.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bucket_items(int64_t bucket, int32_t rp0, int32_t rp1, int nblk,
                                             int64_t q_start, int64_t Nq, int chunk,
                                             bool with_local, int32_t& n_loc, int32_t& n_non) {
  const int b = (int)(bucket % nblk);
  const int32_t cnt = rp1 - rp0;
  const int64_t lo = max(q_start, (int64_t)b * kBlock);
  const int64_t hi = min(q_start + Nq, (int64_t)(b + 1) * kBlock);
  n_loc = hi > lo && !with_local ? (int32_t)(hi - lo) : 0;
  n_non = cnt - n_loc;
}

// Items go out heaviest first -- every full item (exactly `chunk` positions)
// in bucket order, then the buckets' remainders -- so the work-groups that
// fetch items last get short ones.  n_items[0] = item count; n_items[1] is
// the attention kernel's fetch counter, cleared here.  Each thread takes a
// contiguous run of buckets and reads their row_ptr entries sixteen at a
// time, so each pass costs a few memory round trips.
__global__ __launch_bounds__(1024) void build_items_kernel(const int32_t* __restrict__ row_ptr,
                                                           int64_t nb, int nblk, int64_t q_start,
                                                           int64_t Nq, int chunk, bool with_local,
                                                           int4* __restrict__ items,
                                                           int32_t* __restrict__ n_items) {
  constexpr int RB = 16;
  __shared__ int32_t full[1024], rest[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(nb, 1024);
  const int64_t lo = min(nb, per * t), hi = min(nb, per * (t + 1));
  // row_ptr[x0 .. x0+RB] of the run's next batch
  auto batch = [&](int64_t x0, int32_t (&rp)[RB + 1]) {
#pragma unroll
    for (int u = 0; u <= RB; ++u) rp[u] = x0 + u <= hi ? row_ptr[x0 + u] : 0;
  };
  int32_t nf = 0, nr = 0;
  for (int64_t x0 = lo; x0 < hi; x0 += RB) {
    int32_t rp[RB + 1];
    batch(x0, rp);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (x0 + u < hi) {
        int32_t n_loc, n_non;
        bucket_items(x0 + u, rp[u], rp[u + 1], nblk, q_start, Nq, chunk, with_local, n_loc,
                     n_non);
        nf += n_non / chunk;
        nr += n_non % chunk != 0;
      }
    }
  }
  full[t] = nf;
  rest[t] = nr;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t vf = t >= o ? full[t - o] : 0, vr = t >= o ? rest[t - o] : 0;
    __syncthreads();
    full[t] += vf;
    rest[t] += vr;
    __syncthreads();
  }
  const int32_t n_full = full[1023];
  int32_t pf = t ? full[t - 1] : 0, pr = n_full + (t ? rest[t - 1] : 0);
  for (int64_t x0 = lo; x0 < hi; x0 += RB) {
    int32_t rp[RB + 1];
    batch(x0, rp);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (x0 + u < hi) {
        int32_t n_loc, n_non;
        bucket_items(x0 + u, rp[u], rp[u + 1], nblk, q_start, Nq, chunk, with_local, n_loc,
                     n_non);
        const int32_t start = rp[u] + n_loc;
        int32_t done = 0;
        for (; done + chunk <= n_non; done += chunk)
          items[pf++] = make_int4((int)(x0 + u), start + done, chunk, 0);
        if (done < n_non) items[pr++] = make_int4((int)(x0 + u), start + done, n_non - done, 0);
      }
    }
  }
  if (t == 1023) {
    n_items[0] = n_full + rest[1023];
    n_items[1] = 0;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces.
//
// LDS: K block row-major [128][DH] (16-byte chunks XOR-swizzled by row) and
// V block transposed [DH][128 + 4] (rows padded by 8 bytes, so the 32 rows a
// wave reads at one key offset spread over the banks; the padding keeps
// every V^T address a per-lane base plus a compile-time offset), plus the
// item's query positions and slots.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16): S^T = K . Q^T puts keys on the
// rows, so each lane holds 16 keys of one tile row (row = lane % 32): row
// max and sum are in-lane plus one swap of the lane halves.  O^T = V^T . P^T
// keeps the row on the lane as well.  The d dimension of QK^T is permuted
// identically on both operands (lane half h takes d in [h*DH/2,
// (h+1)*DH/2)), which leaves the dot products unchanged.
// ---------------------------------------------------------------------------
constexpr int kVtPitch = kBlock + 4;  // elements per V^T row

template <int DH>
struct AttnSmem {
  __bf16 k[kBlock * DH];
  __bf16 vt[DH * kVtPitch];
  int32_t pos[kMaxItem];  // the item's query positions (its slice of col)
  uint8_t sl[kMaxItem];   // and their slots
};

__device__ __forceinline__ int vt_off(int d, int key) { return d * kVtPitch + key; }

// K and V of block (group r, keys key0..key0+127); keys >= Nk read as 0.
// Every global load is issued before the first LDS store, so the block
// arrives in one memory round trip.
template <int DH>
__device__ __forceinline__ void stage_kv(AttnSmem<DH>& sm, const __bf16* __restrict__ K,
                                         const __bf16* __restrict__ V, int r, int H_kv,
                                         int64_t key0, int64_t Nk, int t) {
  constexpr int CH = DH / 8;                   // 16-byte chunks per K row
  constexpr int KL = kBlock * CH / 256;        // K chunks per thread
  constexpr int VL = (kBlock / 4) * CH / 256;  // V (4 keys x 8 d) pieces per thread
  bf16x8 kr[KL], vr[VL][4];
#pragma unroll
  for (int u = 0; u < KL; ++u) {
    const int id = t + 256 * u, row = id / CH, c = id % CH;
    kr[u] = key0 + row < Nk
                ? *reinterpret_cast<const bf16x8*>(K + ((key0 + row) * H_kv + r) * DH + 8 * c)
                : bf16x8{};
  }
#pragma unroll
  for (int u = 0; u < VL; ++u) {
    const int id = t + 256 * u, kq = id % (kBlock / 4), c = id / (kBlock / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t key = key0 + 4 * kq + e;
      vr[u][e] = key < Nk ? *reinterpret_cast<const bf16x8*>(V + (key * H_kv + r) * DH + 8 * c)
                          : bf16x8{};
    }
  }
#pragma unroll
  for (int u = 0; u < KL; ++u) {
    const int id = t + 256 * u, row = id / CH, c = id % CH;
    *reinterpret_cast<bf16x8*>(&sm.k[row * DH + 8 * (c ^ row_swz<DH>(row))]) = kr[u];
  }
#pragma unroll
  for (int u = 0; u < VL; ++u) {
    const int id = t + 256 * u, kq = id % (kBlock / 4), c = id / (kBlock / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 w = {vr[u][0][e], vr[u][1][e], vr[u][2][e], vr[u][3][e]};
      *reinterpret_cast<bf16x4*>(&sm.vt[vt_off(8 * c + e, 4 * kq)]) = w;
    }
  }
}

// Row of a 32-row tile held by this lane: item row R = tile*32 + n is
// (position R / G of the item, head R % G of the group).  R / G is taken as
// trunc((R + 1/2) * inv_G) in fp32 with inv_G = fp32(1 / G): the true
// quotient plus 1/(2G) stays at least 1/(2G) >= 1/128 away from the next
// integer, far beyond the rounding error for R < 2^17 and G <= 64 (rows per
// item <= 2048 * 64); it keeps the integer division and its spilled
// reciprocal out of the tile loop.
struct TileRow {
  int pos;  // absolute query position (< 2^31)
  int hq, sl;
  bool ok;
};

template <int DH>
__device__ __forceinline__ TileRow tile_row(const AttnSmem<DH>& sm, int nrows, int tile, int r,
                                            int G, float inv_G, int n) {
  // rows past the end read the item's first query row (always in range,
  // also when Q is addressed from the start of a cached-prefill chunk)
  TileRow t{sm.pos[0], r * G, 0, false};
  const int R = tile * 32 + n;
  if (R < nrows) {
    const int p = (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G);
    t.pos = sm.pos[p];
    t.sl = sm.sl[p];
    t.hq = r * G + (R - p * G);
    t.ok = true;
  }
  return t;
}

// Q operand of the lane's row (MFMA B: 16 d x 32 rows per k-step).  The
// contraction order is permuted alike here and in k_frag: k-step s, lane
// half h takes d = 16s + 8h .. 16s + 8h + 7, so the two lanes of a row read
// neighbouring 16-byte pieces and a load instruction touches 32 cache lines
// (32 bytes of each) instead of 64 (Main Branch 171.3 -> 167.4 ms per 1M
// step).  Rows past the item's end carry the item's first query row
// (tile_row), which lies inside the chunk and so is valid memory: a row only
// feeds its own MFMA column, and such rows are never stored.
template <int DH>
__device__ __forceinline__ void load_q(bf16x8 (&qb)[DH / 16], const __bf16* __restrict__ Q,
                                       const TileRow& t, int H_q, int h) {
  const __bf16* qrow = Q + ((int64_t)t.pos * H_q + t.hq) * DH + 8 * h;
#pragma unroll
  for (int s = 0; s < DH / 16; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
}

// K fragment (MFMA A: 32 keys x 16 d) of key group g, k-step s, in the
// contraction order of load_q (d = 16s + 8h ..).
template <int DH>
__device__ __forceinline__ bf16x8 k_frag(const AttnSmem<DH>& sm, int g, int s, int h, int n) {
  const int krow = 32 * g + n;
  return *reinterpret_cast<const bf16x8*>(
      &sm.k[krow * DH + 8 * ((2 * s + h) ^ row_swz<DH>(krow))]);
}

// V^T fragment (MFMA A: 32 d x 16 keys) for d = 32*dg + n and the keys of
// P^T step (g, u): MFMA k-index 8h'+e is key 32g+16u+4h'+e (e < 4) or
// 32g+16u+8+4h'+(e-4), which is accumulator 8u+e of the S^T group g.
template <int DH>
__device__ __forceinline__ bf16x8 v_frag(const AttnSmem<DH>& sm, int dg, int g, int u, int h,
                                         int n) {
  const int d = 32 * dg + n, kb0 = 32 * g + 16 * u + 4 * h;
  const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(&sm.vt[vt_off(d, kb0)]);
  const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(&sm.vt[vt_off(d, kb0 + 8)]);
  return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
}

// ---------------------------------------------------------------------------
// KV-outer partial attention of non-local work items.  64-row tiles per
// wave, as two 32-row halves c = 0, 1 that share every K and V^T fragment
// read from LDS (each fragment feeds two MFMAs).  P is kept in bf16
// registers and O is produced in halves of d so the accumulators fit two
// waves per SIMD.
//
// Memory pipeline: the next tile's Q rows are fetched into the Q registers
// once the softmax is done, then this tile's partials are stored; the loop
// is rotated so that the next tile's S^T follows the stores in straight-
// line code, and every store is unconditional (rows past the item's end
// write to the spare slot `spare` instead), so the wait for the Q rows
// leaves the stores in flight.
// ---------------------------------------------------------------------------
template <int DH>
__device__ __forceinline__ void s_tile(const AttnSmem<DH>& sm, const bf16x8 (&qb)[2][DH / 16],
                                       f32x16 (&sacc)[2][4], int h, int n) {
  constexpr int S = DH / 16;
#pragma unroll
  for (int g0 = 0; g0 < 4; g0 += 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) sacc[c][g0] = sacc[c][g0 + 1] = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int g = g0; g < g0 + 2; ++g) {
        const bf16x8 a = k_frag<DH>(sm, g, s, h, n);
#pragma unroll
        for (int c = 0; c < 2; ++c) sacc[c][g] = mfma32(a, qb[c][s], sacc[c][g]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int DH>
__device__ __forceinline__ void attn_item(const AttnSmem<DH>& sm, const __bf16* __restrict__ Q,
                                          int nrows, int wave, int r, int G, float inv_G,
                                          int H_q, int H_kv, int k, int64_t q_start,
                                          int64_t spare, float scale_log2,
                                          __bf16* __restrict__ Os, float* __restrict__ lse_s,
                                          int h, int n) {
  constexpr int S = DH / 16;
  constexpr int NDG = DH / 32;
  const int ntile = (nrows + 63) / 64;
  if (wave >= ntile) return;
  TileRow row[2];
  bf16x8 qb[2][S];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    row[c] = tile_row<DH>(sm, nrows, 2 * wave + c, r, G, inv_G, n);
    load_q<DH>(qb[c], Q, row[c], H_q, h);
  }
  f32x16 sacc[2][4];
  s_tile<DH>(sm, qb, sacc, h, n);
  for (int tile = wave;;) {
    // ---- softmax: P in bf16, row sums l ---------------------------------------
    bf16x8 pb[2][4][2];
    float mb[2], l[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float m = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 16; ++j) m = fmaxf(m, sacc[c][g][j]);
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      mb[c] = m * scale_log2;
      float ls = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(sacc[c][g][8 * u + e] * scale_log2 - mb[c]);
            ls += p;
            pb[c][g][u][e] = f2bf(p);
          }
      l[c] = ls + __shfl_xor(ls, 32, kWave);
    }
    // ---- prefetch the next tile's Q into qb -----------------------------------
    const bool more = tile + 4 < ntile;
    // with no next tile the (unused) load still goes out: point it at the
    // item's first query row, which is always in range
    TileRow nrow[2] = {{sm.pos[0], r * G, 0, false}, {sm.pos[0], r * G, 0, false}};
    if (more) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        nrow[c] = tile_row<DH>(sm, nrows, 2 * (tile + 4) + c, r, G, inv_G, n);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) load_q<DH>(qb[c], Q, nrow[c], H_q, h);
    // ---- O^T = V^T . P^T in halves of d, stored as bf16 partials -------------
    // Partial (iq, slot) of the row, or the spare slot for rows past the end.
    int64_t ps[2];
    float inv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      ps[c] = row[c].ok ? (int64_t)(row[c].pos - (int)q_start) * (k - 1) + row[c].sl : spare;
      inv[c] = 1.f / l[c];
    }
#pragma unroll
    for (int half = 0; half < NDG / 2; ++half) {
      f32x16 oacc[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) oacc[c][0] = oacc[c][1] = f32x16{};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int dd = 0; dd < 2; ++dd) {
            const bf16x8 a = v_frag<DH>(sm, 2 * half + dd, g, u, h, n);
#pragma unroll
            for (int c = 0; c < 2; ++c) oacc[c][dd] = mfma32(a, pb[c][g][u], oacc[c][dd]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // d = 32dg + 8qd + 4h + e  ->  d-quad 8dg + 2qd + h; the lane's h and
        // head go into the pointer, the rest is a wave-uniform offset.
        __bf16* dst = Os + (ps[c] * H_kv + r) * (DH / 4) * G * 4 +
                      (row[c].hq - r * G + h * G) * 4;
#pragma unroll
        for (int dd = 0; dd < 2; ++dd)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<bf16x4*>(dst + (8 * (2 * half + dd) + 2 * qd) * G * 4) =
                bf16x4{f2bf(oacc[c][dd][4 * qd] * inv[c]),
                       f2bf(oacc[c][dd][4 * qd + 1] * inv[c]),
                       f2bf(oacc[c][dd][4 * qd + 2] * inv[c]),
                       f2bf(oacc[c][dd][4 * qd + 3] * inv[c])};
      }
      __builtin_amdgcn_sched_barrier(0);  // one half's accumulators live at a time
    }
    // Both lane halves hold the row's lse; both store it (same value).
#pragma unroll
    for (int c = 0; c < 2; ++c)
      lse_s[ps[c] * H_q + row[c].hq] = (mb[c] + log2f(l[c])) * 0.69314718055994531f;
    if (!more) break;
    tile += 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) row[c] = nrow[c];
    s_tile<DH>(sm, qb, sacc, h, n);
  }
}

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_kv_outer_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ items, int32_t* __restrict__ n_items, int64_t q_start,
    int64_t Nk, int H_q, int H_kv, int G, float inv_G, int nblk, int k, int64_t spare,
    float scale_log2, __bf16* __restrict__ Os, float* __restrict__ lse_s) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnSmem<DH>& sm = *reinterpret_cast<AttnSmem<DH>*>(smem_raw);
  __shared__ int32_t next;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int32_t total = n_items[0];
  // Persistent work-groups fetch items in list order until the list is
  // exhausted; every wave of a work-group sees the same fetched index.
  for (;;) {
    if (t == 0) next = atomicAdd(&n_items[1], 1);
    __syncthreads();
    const int32_t item_id = next;
    if (item_id >= total) return;
    const int4 it = items[item_id];
    const int bucket = it.x, start = it.y, count = it.z;
    const int r = bucket / nblk, b = bucket % nblk;
    // Per-thread addresses are rebuilt for every item from a thread index
    // the compiler cannot see through: hoisted out of this loop they would
    // be spilled, and each reload would wait for every load in flight.
    int tl = t;
    asm volatile("" : "+v"(tl));
    for (int p = tl; p < count; p += 256) {
      sm.pos[p] = col[start + p];
      sm.sl[p] = slot[start + p];
    }
    stage_kv<DH>(sm, K, V, r, H_kv, (int64_t)b * kBlock, Nk, tl);
    __syncthreads();
    const int ll = tl & 63;
    attn_item<DH>(sm, Q, count * G, wave, r, G, inv_G, H_q, H_kv, k, q_start, spare,
                  scale_log2, Os, lse_s, ll >> 5, ll & 31);
    __syncthreads();  // LDS and `next` are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// Combine with the local block.  Work-group = (query block b, group r): the
// chunk's positions inside block b, times the G heads of group r, in 32-row
// tiles.  Per tile: S^T over the block with the causal mask key <= i, P
// split as hi + lo bf16 (two MFMAs, ~fp32 accuracy), O_loc and lse_loc in
// registers; then the row's non-local partials (slots 0 .. n_sel-2) and the
// local block (slot n_sel-1) are merged in ascending slot order:
//   M = max lse, w_s = exp(lse_s - M), O = sum w_s O_s / sum w_s,
//   lse = M + ln sum w_s.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256, 2) void combine_local_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    int64_t q_start, int64_t Nq, int64_t Nk, int H_q, int H_kv, int G, float inv_G, int k,
    float scale_log2, const __bf16* __restrict__ Os, const float* __restrict__ lse_s,
    float* __restrict__ O, float* __restrict__ lse) {
  constexpr int S = DH / 16;
  constexpr int NDG = DH / 32;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnSmem<DH>& sm = *reinterpret_cast<AttnSmem<DH>*>(smem_raw);
  const int r = blockIdx.x;
  const int64_t b = q_start / kBlock + blockIdx.y;
  const int64_t p0 = max(q_start, b * kBlock), p1 = min(q_start + Nq, (b + 1) * kBlock);
  const int npos = (int)(p1 - p0);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int h = lane >> 5, n = lane & 31;
  const int n_sel = (int)min((int64_t)k, b + 1);
  for (int p = t; p < npos; p += 256) {
    sm.pos[p] = (int)(p0 + p);
    sm.sl[p] = 0;
  }
  const int64_t key0 = b * kBlock;
  stage_kv<DH>(sm, K, V, r, H_kv, key0, Nk, t);
  __syncthreads();

  const int nrows = npos * G;
  const int ntile = (nrows + 31) / 32;
  for (int tile = wave; tile < ntile; tile += 4) {
    const TileRow row = tile_row<DH>(sm, nrows, tile, r, G, inv_G, n);
    // ---- local block: S^T with the causal mask --------------------------------
    f32x16 sacc[4];
    {
      bf16x8 qb[S];
      load_q<DH>(qb, Q, row, H_q, h);
#pragma unroll
      for (int g0 = 0; g0 < 4; g0 += 2) {
        sacc[g0] = sacc[g0 + 1] = f32x16{};
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int g = g0; g < g0 + 2; ++g)
            sacc[g] = mfma32(k_frag<DH>(sm, g, s, h, n), qb[s], sacc[g]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // key 32g + acc_row(j, h) is visible iff it is <= pos - key0; acc_row
    // is 4h plus a constant, so compare the constant with a per-lane limit.
    const int lim = (row.ok ? (int)(row.pos - key0) : kBlock - 1) - 4 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (32 * g + acc_row(j, 0) > lim) sacc[g][j] = -INFINITY;
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, sacc[g][j]);
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    const float mb = m * scale_log2;
    f32x16 oacc[NDG];
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg) oacc[dg] = f32x16{};
    float l = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 phi, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[g][8 * u + e] * scale_log2 - mb);
          l += p;
          phi[e] = f2bf(p);
          plo[e] = f2bf(p - bf2f(phi[e]));
        }
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) {
          const bf16x8 a = v_frag<DH>(sm, dg, g, u, h, n);
          oacc[dg] = mfma32(a, phi, oacc[dg]);
          oacc[dg] = mfma32(a, plo, oacc[dg]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l += __shfl_xor(l, 32, kWave);
    if (!row.ok) continue;

    // ---- merge with the non-local partials ------------------------------------
    // nns = n_sel - 1 non-local slots (uniform over the work-group).  Their
    // lse values are requested together (addresses clamped to the row's
    // last slot, so every load is in bounds and none is predicated) for the
    // max; the partials are then accumulated in ascending slot order.
    const int iq = row.pos - (int)q_start;
    const float lse_loc = (mb + log2f(l)) * 0.69314718055994531f;
    const int nns = n_sel - 1;
    const float* ls = lse_s + (int64_t)iq * (k - 1) * H_q + row.hq;
    float M = lse_loc;
    if (nns > 0) {
      float lv[kMaxK - 1];
#pragma unroll
      for (int s = 0; s < kMaxK - 1; ++s) lv[s] = ls[min(s, nns - 1) * H_q];
#pragma unroll
      for (int s = 0; s < kMaxK - 1; ++s) M = fmaxf(M, lv[s]);
    }
    float acc[NDG][16];
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[dg][j] = 0.f;
    float den = 0.f;
    const __bf16* src =
        Os + ((int64_t)iq * (k - 1) * H_kv + r) * (DH / 4) * G * 4 + (row.hq - r * G) * 4;
    for (int s = 0; s < nns; ++s) {
      const float w = __expf(ls[s * H_q] - M);
      den += w;
      const __bf16* ps = src + (int64_t)s * (DH / 4) * H_q * 4;
      bf16x4 x[NDG][4];
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          x[dg][qd] = *reinterpret_cast<const bf16x4*>(ps + (8 * dg + 2 * qd + h) * G * 4);
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[dg][4 * qd + e] += w * bf2f(x[dg][qd][e]);
    }
    // the local block (the highest block id) last: O_loc = oacc / l
    const float w_loc = __expf(lse_loc - M);
    den += w_loc;
    const float wl = w_loc / l;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[dg][j] += wl * oacc[dg][j];
    const float inv = 1.f / den;
    float* dst = O + ((int64_t)iq * H_q + row.hq) * DH;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = acc[dg][4 * qd + e] * inv;
        *reinterpret_cast<f32x4*>(dst + 32 * dg + 8 * qd + 4 * h) = o;
      }
    if (lse && h == 0) lse[(int64_t)iq * H_q + row.hq] = M + __logf(den);
  }
}

int attn_max_chunk() { return kMaxItem; }

int64_t attn_max_items(int64_t nb, int64_t nnz, int chunk) { return nb + nnz / chunk + 1; }

hipError_t launch_build_items(const int32_t* row_ptr, int64_t nb, int nblk, int64_t q_start,
                              int64_t Nq, int chunk, bool with_local, int4* items,
                              int32_t* n_items, hipStream_t stream) {
  build_items_kernel<<<1, 1024, 0, stream>>>(row_ptr, nb, nblk, q_start, Nq, chunk, with_local,
                                             items, n_items);
  return hipGetLastError();
}

template <typename Kern>
static hipError_t allow_lds(Kern* kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

static bool attn_lds_ready = false;

static hipError_t attn_prepare() {
  // The d_h = 128 kernels need more than 64 KiB of LDS per work-group.
  if (attn_lds_ready) return hipSuccess;
  hipError_t e = allow_lds(&attn_kv_outer_kernel<128>, sizeof(AttnSmem<128>));
  if (e == hipSuccess) e = allow_lds(&attn_kv_outer_kernel<64>, sizeof(AttnSmem<64>));
  if (e == hipSuccess) e = allow_lds(&combine_local_kernel<128>, sizeof(AttnSmem<128>));
  if (e == hipSuccess) e = allow_lds(&combine_local_kernel<64>, sizeof(AttnSmem<64>));
  if (e == hipSuccess) attn_lds_ready = true;
  return e;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_attn(const void* Q, const void* K, const void* V, const int32_t* col,
                       const uint8_t* slot, const int4* items, int32_t* n_items,
                       int64_t max_items, int64_t q_start, int64_t Nq, int64_t Nk, int H_q,
                       int H_kv, int d_h, int nblk, int k, float scale, void* Os, float* lse_s,
                       hipStream_t stream) {
  hipError_t e = attn_prepare();
  if (e != hipSuccess) return e;
  if (k < 2) return hipSuccess;  // no non-local blocks
  const int G = H_q / H_kv;
  const int64_t spare = Nq * (k - 1);  // the slot after the last real one
  const float inv_G = 1.f / (float)G;
  const float scale_log2 = scale * 1.4426950408889634f;
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* v = static_cast<const __bf16*>(V);
  auto* os = static_cast<__bf16*>(Os);
  // Two resident work-groups per CU (the kernel's occupancy).
  dim3 grid((unsigned)std::min<int64_t>(max_items, 2 * (int64_t)device_cus())), block(256);
  if (d_h == 128)
    attn_kv_outer_kernel<128><<<grid, block, sizeof(AttnSmem<128>), stream>>>(
        q, kk, v, col, slot, items, n_items, q_start, Nk, H_q, H_kv, G, inv_G, nblk, k, spare,
        scale_log2, os, lse_s);
  else if (d_h == 64)
    attn_kv_outer_kernel<64><<<grid, block, sizeof(AttnSmem<64>), stream>>>(
        q, kk, v, col, slot, items, n_items, q_start, Nk, H_q, H_kv, G, inv_G, nblk, k, spare,
        scale_log2, os, lse_s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine(const void* Q, const void* K, const void* V, const void* Os,
                          const float* lse_s, int64_t q_start, int64_t Nq, int64_t Nk, int H_q,
                          int H_kv, int d_h, int k, float scale, float* O, float* lse,
                          hipStream_t stream) {
  hipError_t e = attn_prepare();
  if (e != hipSuccess) return e;
  const int G = H_q / H_kv;
  const float inv_G = 1.f / (float)G;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int64_t nqb = (q_start + Nq - 1) / kBlock - q_start / kBlock + 1;
  // group fastest: the H_kv work-groups of a query block run together and
  // read each (position, slot) partial record, all groups side by side,
  // at once (0.5 % faster per 1M step than query blocks fastest)
  dim3 grid((unsigned)H_kv, (unsigned)nqb), block(256);
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* v = static_cast<const __bf16*>(V);
  auto* os = static_cast<const __bf16*>(Os);
  if (d_h == 128)
    combine_local_kernel<128><<<grid, block, sizeof(AttnSmem<128>), stream>>>(
        q, kk, v, q_start, Nq, Nk, H_q, H_kv, G, inv_G, k, scale_log2, os, lse_s, O, lse);
  else if (d_h == 64)
    combine_local_kernel<64><<<grid, block, sizeof(AttnSmem<64>), stream>>>(
        q, kk, v, q_start, Nq, Nk, H_q, H_kv, G, inv_G, k, scale_log2, os, lse_s, O, lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
