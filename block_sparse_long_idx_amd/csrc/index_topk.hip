// Index Branch kernels: index-score GEMM with block max-pooling, and the
// exp-free Top-k over pooled block scores.
//
// Method: "MiniMax Sparse Attention" explainer
// (minimax-sparse-attention-danialwang.pages.dev), Figure 1 caption (index
// score -> Block Max Pooling -> Top-k per query and GQA group, local block
// forced) and section 05 part 1 (Top-k on raw scores, since softmax keeps
// their order; per-lane register heaps merged across the lanes).
#include "common.h"
#include "msa_internal.h"

namespace msa {

// ---------------------------------------------------------------------------
// Score GEMM + block max-pool.
//
// Work-group = (group r, tile of 64*NW query positions); NW = 4 or 8 waves
// x 64 queries (8 when the grid still fills the chip: each staged key block
// then serves twice the queries).
// The WG sweeps key blocks kb = 0 .. lb(last query)-1 in ascending order:
// each block's 128 index keys are copied once into LDS by direct
// global->LDS loads (double-buffered) and shared by the 4 waves.  A wave computes S^T = K_blk . Q^T with keys as
// MFMA rows and its queries as columns, so every lane's 16 accumulators are
// 16 keys of one query: the 128-key max is an in-lane max plus one swap
// between the two lane halves.  Only blocks strictly before a query's local
// block are ever consumed (the local block is forced, never ranked), and
// those blocks are entirely in the past, so no causal mask is needed.
//
// Output P[r][q - q_start][kb] fp32, row pitch ldp (multiple of 4).  Entries
// for kb >= lb(q) are unspecified.
// The d_idx dimension is permuted identically on both operands: lane half h
// covers d in [h*D/2, (h+1)*D/2), k-step s takes 8 of them.  A dot product
// does not depend on the order of its terms, so the scores are unchanged.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int kswz(int row) {
  // XOR swizzle of the 16-byte chunk index inside a key row: the 16 rows that
  // one 128-bit LDS read cycle serves (16 lanes x 16 B = 256 B) then hit 16
  // distinct 16-byte bank groups.
  return D == 32 ? ((row >> 2) & 3) : D == 64 ? ((row >> 1) & 7) : (row & 15);
}

// The sweep shared by both Index-Branch variants.  For every key block kb
// it hands the pooled scores of the lane's own queries to `sink(kb, v)`.
// A wave takes CG column groups of 32 queries (32*CG queries); lane half h
// owns the queries of column groups h, h+2, ..: q_own[j] = qw0 + 32*(2j+h)
// + n, v[j] its score.
template <int D, int NW, int CG, typename Sink>
__device__ __forceinline__ void index_sweep(const __bf16* __restrict__ q_idx,
                                            const __bf16* __restrict__ k_idx, int64_t q_start,
                                            int64_t Nq, int H_kv, int r, int tile,
                                            __bf16 (*lds)[128 * D], Sink& sink) {
  static_assert(CG == 2 || CG == 4, "column groups per wave");
  constexpr int S = D / 16;   // MFMA k-steps
  constexpr int CH = D / 8;   // 16-byte chunks per key row
  constexpr int QW = 32 * CG;  // queries per wave
  constexpr int NQ = CG / 2;   // queries per lane
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int h = lane >> 5, n = lane & 31;
  const int64_t q_end = q_start + Nq;
  const int64_t q0 = q_start + (int64_t)tile * (QW * NW);
  const int64_t qw0 = q0 + wave * QW;
  const int64_t q_last = min(q0 + QW * NW - 1, q_end - 1);
  const int kb_end = (int)(q_last / kBlock);
  const int kb_end_w = qw0 < q_end ? (int)(min(qw0 + QW - 1, q_end - 1) / kBlock) : 0;

  // Query operand (MFMA B: 16 d x 32 queries), CG column groups.
  bf16x8 qb[CG][S];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int64_t q = qw0 + 32 * c + n;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (q < q_end)
        qb[c][s] = *reinterpret_cast<const bf16x8*>(
            q_idx + (q * H_kv + r) * D + (D / 2) * h + 8 * s);
      else
        qb[c][s] = bf16x8{};
    }
  }

  // Key block kb -> LDS buffer `buf` by direct global->LDS loads (no
  // registers): each wave-instruction fills one contiguous KiB, lane i
  // writing bytes 16i..16i+15, i.e. key rows v*RPI .. v*RPI+RPI-1; a lane
  // fetches the global chunk that the swizzled layout keeps at its LDS spot.
  constexpr int RPI = 1024 / (2 * D);      // key rows per wave-instruction
  constexpr int PER_WAVE = 128 / RPI / NW;  // wave-instructions per wave per block
  auto dma = [&](int kb, int buf) {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int v = wave * PER_WAVE + u;
      const int row = v * RPI + lane / CH, cs = lane % CH;
      const __bf16* src =
          k_idx + (((int64_t)kb * kBlock + row) * H_kv + r) * D + 8 * (cs ^ kswz<D>(row));
      __builtin_amdgcn_global_load_lds(src, &lds[buf][v * 512], 16, 0, 0);
    }
  };
  // Two buffers: block kb+1 is fetched while block kb is scored.  (A third
  // buffer, fetching two blocks ahead, measured no faster.)
  if (kb_end > 0) dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // block 0 and the query operand
  __syncthreads();

  // The sink takes block kb-1's pooled scores while block kb's MFMAs are in
  // flight, so its VALU work can issue under them.
  int kb_prev = -1;
  float v_prev[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) v_prev[j] = -INFINITY;
  for (int kb = 0; kb < kb_end; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < kb_end) dma(kb + 1, buf ^ 1);
    if (kb < kb_end_w) {
      float m[CG];
#pragma unroll
      for (int c = 0; c < CG; ++c) m[c] = -INFINITY;
      if constexpr (CG == 2) {
        // key-row groups in pairs: the second group's MFMAs overlap the
        // first group's max-pool
#pragma unroll
        for (int g0 = 0; g0 < 4; g0 += 2) {
          f32x16 acc[2][2];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int row = 32 * (g0 + g) + n;
            bf16x8 a[S];
#pragma unroll
            for (int s = 0; s < S; ++s)
              a[s] = *reinterpret_cast<const bf16x8*>(
                  &lds[buf][row * D + 8 * (((D / 16) * h + s) ^ kswz<D>(row))]);
            acc[g][0] = acc[g][1] = f32x16{};
#pragma unroll
            for (int s = 0; s < S; ++s) {
              acc[g][0] = mfma32(a[s], qb[0][s], acc[g][0]);
              acc[g][1] = mfma32(a[s], qb[1][s], acc[g][1]);
            }
          }
          if (g0 == 0 && kb_prev >= 0) sink(kb_prev, kb_end_w, v_prev);
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              m[0] = fmaxf(m[0], acc[g][0][j]);
              m[1] = fmaxf(m[1], acc[g][1][j]);
            }
        }
      } else {
        // Key-row group g, k-step s in sequence: each LDS fragment feeds CG
        // MFMAs, and the next fragment is read while they run (one
        // fragment ahead, so its LDS latency hides under CG MFMAs and only
        // two fragments are live).
        auto frag = [&](int st) {
          const int row = 32 * (st / S) + n;
          return *reinterpret_cast<const bf16x8*>(
              &lds[buf][row * D + 8 * (((D / 16) * h + st % S) ^ kswz<D>(row))]);
        };
        f32x16 acc[CG];
        bf16x8 a_cur = frag(0);
#pragma unroll
        for (int st = 0; st < 4 * S; ++st) {
          const int s = st % S;
          const bf16x8 a_nxt = st + 1 < 4 * S ? frag(st + 1) : a_cur;
          if (s == 0) {
#pragma unroll
            for (int c = 0; c < CG; ++c) acc[c] = f32x16{};
          }
#pragma unroll
          for (int c = 0; c < CG; ++c) acc[c] = mfma32(a_cur, qb[c][s], acc[c]);
          if (st == 0 && kb_prev >= 0) sink(kb_prev, kb_end_w, v_prev);
          if (s == S - 1) {
#pragma unroll
            for (int c = 0; c < CG; ++c)
#pragma unroll
              for (int j = 0; j < 16; ++j) m[c] = fmaxf(m[c], acc[c][j]);
          }
          a_cur = a_nxt;
        }
      }
      kb_prev = kb;
      // Lane half h keeps column groups 2j+h: it sends across its partial
      // max of the other group of each pair and takes the other half's
      // partial max of its own.  The selects are bit operations on a lane
      // mask, which keeps the hand-over in registers.
      const uint32_t hm = h ? 0xffffffffu : 0u;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const uint32_t a = __float_as_uint(m[2 * j]), b = __float_as_uint(m[2 * j + 1]);
        const float mine = __uint_as_float((b & hm) | (a & ~hm));
        const float other = __uint_as_float((a & hm) | (b & ~hm));
        v_prev[j] = fmaxf(mine, __shfl_xor(other, 32, kWave));
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of block kb+1 is in LDS
    __syncthreads();
  }
  if (kb_prev >= 0) sink(kb_prev, kb_end_w, v_prev);
}

// Work-group -> (group r, query tile).  Work-groups are dispatched to the
// 8 XCDs round-robin by linear id; when H_kv divides 8, all tiles of a
// group land on the same 8/H_kv XCDs, so the tiles that sweep that group's
// key blocks concurrently share them through one L2.  Heaviest tiles (the
// longest causal rows) first.  Returns false for the padding work-groups.
__device__ __forceinline__ bool index_tile_of(int w, int ntiles, int H_kv, int& r, int& tile) {
  int ti;
  if (8 % H_kv == 0) {
    const int per = 8 / H_kv;
    r = (w % 8) / per;
    ti = (w / 8) * per + (w % per);
  } else {
    r = w % H_kv;
    ti = w / H_kv;
  }
  tile = ntiles - 1 - ti;
  return ti < ntiles;
}

__host__ __forceinline__ int index_grid(int ntiles, int H_kv) {
  const int per = (8 % H_kv == 0) ? 8 / H_kv : 1;
  return (int)ceil_div(ntiles, per) * per * H_kv;
}

// Sink of the two-kernel variant: stores the pooled scores into
// P[r][q - q_start][kb], 16 blocks (64 contiguous bytes) at a time.  The
// rows of neighbouring lanes lie a whole row pitch apart, so narrower
// stores would leave every written line partly filled and multiply the
// HBM write traffic.  The last group stops at the quad holding block
// kb_end_w - 1, inside the row (the pitch is a multiple of 4).
struct PoolStore {
  float* prow;
  bool own_ok;
  float pend[16];
  __device__ __forceinline__ void operator()(int kb, int kb_end_w, const float (&v)[1]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) pend[e] = (kb & 15) == e ? v[0] : pend[e];  // no dynamic index
    if (own_ok && ((kb & 15) == 15 || kb == kb_end_w - 1)) {
      f32x4* dst = reinterpret_cast<f32x4*>(prow + (kb & ~15));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * q <= (kb & 15))
          dst[q] = f32x4{pend[4 * q], pend[4 * q + 1], pend[4 * q + 2], pend[4 * q + 3]};
    }
  }
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void index_pool_kernel(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx,
    int64_t q_start, int64_t Nq, int H_kv, int ntiles, float* __restrict__ P,
    int64_t ldp) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][128 * D];
  int r, tile;
  if (!index_tile_of(blockIdx.x, ntiles, H_kv, r, tile)) return;
  const int lane = threadIdx.x & 63;
  const int64_t q_own = q_start + (int64_t)tile * (64 * NW) + (threadIdx.x >> 6) * 64 +
                        32 * (lane >> 5) + (lane & 31);
  PoolStore sink{P + ((int64_t)r * Nq + (q_own - q_start)) * ldp, q_own < q_start + Nq, {}};
  index_sweep<D, NW, 2>(q_idx, k_idx, q_start, Nq, H_kv, r, tile, lds, sink);
}

// Sink of the fused variant: a running Top-LM list of (score, block) per
// query, sorted by score, descending.  Blocks arrive in ascending order and
// a new score must beat an equal one strictly, so among equal scores the
// lower block stays ahead (ties go to the lower block index).
// Inserting v moves every entry it beats one place down: the new score at
// place j is the median of (old j-1, v, old j), since the list is sorted;
// the block ids follow the same two comparisons.  Places 0..LM/2 can only
// change when v beats the entry at LM/2, so that half is skipped (by the
// whole wave) when no lane's v reaches it: late in the sweep most new
// entries land near the bottom of the list.
template <int LM, int NQ>
struct TopkKeep {
  int lb_own[NQ];
  float sc[NQ][LM];
  int bk[NQ][LM];
  __device__ __forceinline__ void place(int q, int j, float v, int kb) {
    const bool up = v > sc[q][j - 1];
    const bool here = v > sc[q][j];
    bk[q][j] = up ? bk[q][j - 1] : (here ? kb : bk[q][j]);
    sc[q][j] = __builtin_amdgcn_fmed3f(sc[q][j - 1], v, sc[q][j]);
  }
  __device__ __forceinline__ void operator()(int kb, int, const float (&vin)[NQ]) {
    constexpr int SP = LM / 2;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      // A block that must not enter (the local block or later) becomes -inf.
      const float v = kb < lb_own[q] ? vin[q] : -INFINITY;
      if (v > sc[q][LM - 1]) {
#pragma unroll
        for (int j = LM - 1; j > SP; --j) place(q, j, v, kb);
        if (v > sc[q][SP]) {
#pragma unroll
          for (int j = SP; j > 0; --j) place(q, j, v, kb);
          bk[q][0] = v > sc[q][0] ? kb : bk[q][0];
          sc[q][0] = fmaxf(v, sc[q][0]);
        }
      }
    }
  }
};

template <int D, int NW, int CG, int LM>
__global__ __launch_bounds__(64 * NW) void index_topk_fused_kernel(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx, int64_t q_start,
    int64_t Nq, int H_kv, int ntiles, int k, int32_t* __restrict__ sel) {
  constexpr int NQ = CG / 2;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][128 * D];
  int r, tile;
  if (!index_tile_of(blockIdx.x, ntiles, H_kv, r, tile)) return;
  const int lane = threadIdx.x & 63;
  const int64_t qw0 = q_start + (int64_t)tile * (32 * CG * NW) + (threadIdx.x >> 6) * (32 * CG);
  TopkKeep<LM, NQ> keep;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t q_own = qw0 + 32 * (2 * q + (lane >> 5)) + (lane & 31);
    keep.lb_own[q] = q_own < q_start + Nq ? (int)(q_own / kBlock) : 0;
#pragma unroll
    for (int j = 0; j < LM; ++j) {
      keep.sc[q][j] = -INFINITY;
      keep.bk[q][j] = -1;
    }
  }
  index_sweep<D, NW, CG>(q_idx, k_idx, q_start, Nq, H_kv, r, tile, lds, keep);
  const int K1 = k - 1;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t q_own = qw0 + 32 * (2 * q + (lane >> 5)) + (lane & 31);
    if (q_own >= q_start + Nq) continue;
    int32_t* out = sel + ((q_own - q_start) * H_kv + r) * k;
    const int lb = keep.lb_own[q];
    if (lb <= K1) {
      for (int t = 0; t < k; ++t) out[t] = t <= lb ? t : -1;
      continue;
    }
    // the K1 best blocks in ascending order, then the local block (largest id)
#pragma unroll
    for (int j = 0; j < LM; ++j) {
      if (j < K1) {
        int rank = 0;
#pragma unroll
        for (int i = 0; i < LM; ++i) rank += (i < K1) & (keep.bk[q][i] < keep.bk[q][j]);
        out[rank] = keep.bk[q][j];
      }
    }
    out[K1] = lb;
  }
}

// Waves per index work-group: 8 when 512-query tiles still give at least
// one work-group per CU, else 4.  d_idx = 128 keeps 4: its accumulators and
// query operand need more registers than two waves per SIMD leave.
static int index_waves(int64_t Nq, int H_kv, int d_idx) {
  return d_idx < 128 && ceil_div(Nq, (int64_t)512) * H_kv >= device_cus() ? 8 : 4;
}

template <int D, int NW>
static void launch_pool_dn(const __bf16* qi, const __bf16* ki, int64_t q_start, int64_t Nq,
                           int H_kv, float* P, int64_t ldp, hipStream_t stream) {
  const int ntiles = (int)ceil_div(Nq, (int64_t)(64 * NW));
  index_pool_kernel<D, NW><<<index_grid(ntiles, H_kv), 64 * NW, 0, stream>>>(
      qi, ki, q_start, Nq, H_kv, ntiles, P, ldp);
}

template <int D>
static void launch_pool_d(const __bf16* qi, const __bf16* ki, int64_t q_start, int64_t Nq,
                          int H_kv, float* P, int64_t ldp, hipStream_t stream) {
  if (D < 128 && index_waves(Nq, H_kv, D) == 8)
    launch_pool_dn<D, D < 128 ? 8 : 4>(qi, ki, q_start, Nq, H_kv, P, ldp, stream);
  else
    launch_pool_dn<D, 4>(qi, ki, q_start, Nq, H_kv, P, ldp, stream);
}

hipError_t launch_index_pool(const void* q_idx, const void* k_idx, int64_t q_start,
                             int64_t Nq, int H_kv, int d_idx, float* P, int64_t ldp,
                             hipStream_t stream) {
  auto* qi = static_cast<const __bf16*>(q_idx);
  auto* ki = static_cast<const __bf16*>(k_idx);
  switch (d_idx) {
    case 32: launch_pool_d<32>(qi, ki, q_start, Nq, H_kv, P, ldp, stream); break;
    case 64: launch_pool_d<64>(qi, ki, q_start, Nq, H_kv, P, ldp, stream); break;
    case 128: launch_pool_d<128>(qi, ki, q_start, Nq, H_kv, P, ldp, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exp-free Top-k, one wavefront per (query, group) row of pooled scores.
//
// Candidates are the blocks b < lb strictly before the local block.  Each
// candidate becomes a unique 64-bit key (order-preserving score bits, then
// ~b so that on equal scores the lower block ranks higher); the k-1 largest
// keys are selected, the local block is added and the k ids are written in
// ascending order.
//
// A row of at most 128 candidates is held whole, two per lane.  A longer row
// is read once, in steps of 1,024 blocks.  After each step every lane's
// best score so far is the score of one of its blocks, so at least k-1
// candidates reach the (k-1)-th largest of those 64 bests, tau, and no block
// scoring below tau can be among the k-1 best.  The step's blocks scoring
// at least tau are packed into LDS in the order the wave meets them (a
// ballot and each lane's count of the set bits below it); once the pack is
// more than half full, the keys that fell below a risen tau are dropped
// before the next step packs.  Few blocks usually pass: up to 128 of them
// sit two per lane at the end, and the wave pops the best k-1 keys one at a
// time (a cross-lane max per pop, by DPP and ds_swizzle exchanges).  When
// more pass (rows with many equal scores), a second read lets every lane
// keep its best LM keys scoring at least the final tau in a sorted register
// list, and the pops take the heads of the lists.
// ---------------------------------------------------------------------------
template <int LM>
__device__ __forceinline__ void list_insert(uint64_t (&lst)[LM], uint64_t key) {
#pragma unroll
  for (int j = LM - 1; j > 0; --j) {
    const uint64_t up = lst[j - 1];
    lst[j] = key > up ? up : (key > lst[j] ? key : lst[j]);
  }
  lst[0] = key > lst[0] ? key : lst[0];
}

__device__ __forceinline__ uint64_t block_key(float s, int b) {
  return ((uint64_t)ord_f32(s) << 32) | (uint32_t)(~b);
}

// the score whose order key is o (the inverse of ord_f32)
__device__ __forceinline__ float f32_of_ord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// lanes below this one whose bit is set in the wave mask m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The maximum (MAX) or minimum over the 64 lanes, wave-uniform: DPP within
// each 16-lane row, the four rows joined by readlane (no LDS traffic).
template <bool MAX, int CTRL>
__device__ __forceinline__ uint32_t dpp_pick_u32(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
  return MAX ? max(x, y) : min(x, y);
}

template <bool MAX>
__device__ __forceinline__ uint32_t wave_pick_u32(uint32_t x) {
  x = dpp_pick_u32<MAX, 0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_pick_u32<MAX, 0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_pick_u32<MAX, 0x141>(x);  // row_half_mirror
  x = dpp_pick_u32<MAX, 0x140>(x);  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return MAX ? max(max(a, b), max(c, d)) : min(min(a, b), min(c, d));
}

// The r-th largest (MAX) or smallest of the lanes' values, a value counted
// once per lane that holds it; lanes holding `none` take no part, and
// `none` is returned when fewer than r lanes do.  Each round takes the
// cross-lane extreme and retires the lanes that hold it.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_rank_u32(uint32_t x, int r) {
  constexpr uint32_t none = MAX ? 0u : 0xFFFFFFFFu;
  for (;;) {
    const uint32_t top = wave_pick_u32<MAX>(x);
    const int held = __builtin_popcountll(__builtin_amdgcn_ballot_w64(x == top));
    if (held >= r || top == none) return top;
    r -= held;
    if (x == top) x = none;
  }
}

// A step reads kTopkLoads scores per lane, blocks b0 + 64u + lane, so that
// all of a step's loads are in flight together.  Blocks at or past lb load
// block lb - 1 (no branch around the load) and read as -inf.
constexpr int kTopkLoads = 16;
constexpr int kTopkStep = kWave * kTopkLoads;
constexpr int kTopkPack = 2 * kWave;  // packed keys per wave, two per lane

__device__ __forceinline__ void load_step(const float* __restrict__ prow, int b0, int lb,
                                          int lane, float (&v)[kTopkLoads]) {
#pragma unroll
  for (int u = 0; u < kTopkLoads; ++u) {
    const int b = b0 + kWave * u + lane;
    const float x = prow[min(b, lb - 1)];
    v[u] = b < lb ? x : -__builtin_inff();
  }
}

// k1 pops of the cross-lane max over two sorted keys per lane (hd >= tl; 0
// is below every key): lane p < k1 receives the p-th best block id.
__device__ __forceinline__ void pop_pairs(uint64_t hd, uint64_t tl, int k1, int lane,
                                          int& mine) {
  for (int p = 0; p < k1; ++p) {
    const uint64_t bk = wave_max_u64(hd);
    if (hd == bk) {
      hd = tl;
      tl = 0;
    }
    if (lane == p) mine = (int)(~(uint32_t)bk);
  }
}

template <int LM>
__device__ __forceinline__ void topk_row(const float* __restrict__ prow, int lb, int k,
                                         int32_t* __restrict__ out, int lane,
                                         uint64_t* __restrict__ cand) {
  const int K1 = k - 1;
  if (lb <= K1) {  // every visible block is selected
    if (lane < k) out[lane] = lane <= lb ? lane : -1;
    return;
  }
  int mine = lb;  // lane K1 keeps the local block
  if (K1 > 0 && lb <= 2 * kWave) {
    // Short row: every block is a candidate, blocks lane and lane + 64.
    const int b2 = lane + kWave;
    uint64_t hd = lane < lb ? block_key(prow[lane], lane) : 0;
    uint64_t tl = b2 < lb ? block_key(prow[min(b2, lb - 1)], b2) : 0;
    pop_pairs(tl > hd ? tl : hd, tl > hd ? hd : tl, K1, lane, mine);
  } else if (K1 > 0) {
    // One read.  Every lane owns a block of the first step (lb > 128).
    float best = -__builtin_inff();  // the lane's best score so far
    int n = 0;  // keys packed so far, the same in every lane
    uint32_t to = 0;  // order key of tau
    float tau = -__builtin_inff();
    for (int b0 = 0; b0 < lb; b0 += kTopkStep) {
      float v[kTopkLoads];
      load_step(prow, b0, lb, lane, v);
#pragma unroll
      for (int u = 0; u < kTopkLoads; ++u) best = fmaxf(best, v[u]);
      // fmaxf returns one of its operands, so each lane's best is the score
      // of one of its blocks, and tau, the K1-th largest lane best, is
      // reached by at least K1 blocks.  Usually only the lanes at or above
      // the previous tau can hold it: with c of them (K1 <= c < 2 K1) it is
      // their (c - K1 + 1)-th smallest, a few rounds from below.
      const uint32_t bo = ord_f32(best);
      const int c = b0 ? __builtin_popcountll(__builtin_amdgcn_ballot_w64(bo >= to)) : 0;
      if (c >= K1 && c < 2 * K1)
        to = wave_rank_u32<false>(bo >= to ? bo : 0xFFFFFFFFu, c - K1 + 1);
      else
        to = wave_rank_u32<true>(bo, K1);
      tau = to ? f32_of_ord(to) : -__builtin_inff();
      if (n > kTopkPack / 2 && n <= kTopkPack) {
        // drop the packed keys that fell below tau
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t c0 = lane < n ? cand[lane] : 0;
        const uint64_t c1 = lane + kWave < n ? cand[lane + kWave] : 0;
        const bool k0 = c0 && f32_of_ord((uint32_t)(c0 >> 32)) >= tau;
        const bool k1 = c1 && f32_of_ord((uint32_t)(c1 >> 32)) >= tau;
        const uint64_t m0 = __builtin_amdgcn_ballot_w64(k0);
        const uint64_t m1 = __builtin_amdgcn_ballot_w64(k1);
        const int n0 = __builtin_popcountll(m0);
        if (k0) cand[lanes_below(m0)] = c0;
        if (k1) cand[n0 + lanes_below(m1)] = c1;
        n = n0 + __builtin_popcountll(m1);
      }
      // pack this step's blocks scoring >= tau, in the order the wave meets
      // them; a count past kTopkPack marks the pack as overflowed
#pragma unroll
      for (int u = 0; u < kTopkLoads; ++u) {
        const int b = b0 + kWave * u + lane;
        const bool pass = b < lb && v[u] >= tau;
        const uint64_t m = __builtin_amdgcn_ballot_w64(pass);
        if (m) {
          const int pos = n + lanes_below(m);
          if (pass && pos < kTopkPack) cand[pos] = block_key(v[u], b);
          n += __builtin_popcountll(m);
        }
      }
    }
    // The wave's LDS accesses complete in order; the fences keep the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (n <= kTopkPack) {
      const uint64_t c0 = lane < n ? cand[lane] : 0;
      const uint64_t c1 = lane + kWave < n ? cand[lane + kWave] : 0;
      pop_pairs(c1 > c0 ? c1 : c0, c1 > c0 ? c0 : c1, K1, lane, mine);
    } else {
      // the pack overflowed: read the row again, each lane keeping its best
      // LM keys among the blocks scoring >= the final tau
      uint64_t lst[LM];
#pragma unroll
      for (int j = 0; j < LM; ++j) lst[j] = 0;
      for (int b0 = 0; b0 < lb; b0 += kTopkStep) {
        float v[kTopkLoads];
        load_step(prow, b0, lb, lane, v);
#pragma unroll
        for (int u = 0; u < kTopkLoads; ++u) {
          const int b = b0 + kWave * u + lane;
          const uint64_t key = block_key(v[u], b);
          if (b < lb && v[u] >= tau && key > lst[LM - 1]) list_insert<LM>(lst, key);
        }
      }
      for (int p = 0; p < K1; ++p) {
        const uint64_t bk = wave_max_u64(lst[0]);
        if (lst[0] == bk) {
#pragma unroll
          for (int j = 0; j < LM - 1; ++j) lst[j] = lst[j + 1];
          lst[LM - 1] = 0;
        }
        if (lane == p) mine = (int)(~(uint32_t)bk);
      }
    }
  }
  // ascending order: rank of each of the k ids among lanes 0..k-1
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const int o = __builtin_amdgcn_readlane(mine, j);
    rank += o < mine;
  }
  if (lane < k) out[rank] = mine;
}

// rows: prefill = H_kv * Nq rows of P[r][iq][*]; decode = B * H_kv rows of
// P[b][r][*] whose local block is nblk_dec - 1.
template <int LM>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ P, int64_t ldp,
                                                   int64_t nrows, int64_t Nq, int H_kv,
                                                   int64_t q_start, int nblk_dec, int k,
                                                   int32_t* __restrict__ sel) {
  __shared__ uint64_t cand[4][kTopkPack];
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrows) return;
  int lb;
  int32_t* out;
  if (nblk_dec > 0) {
    lb = nblk_dec - 1;
    out = sel + row * k;  // row = b * H_kv + r  ->  sel[b][r][:]
  } else {
    const int r = (int)(row / Nq);
    const int64_t iq = row % Nq;
    lb = (int)((q_start + iq) / kBlock);
    out = sel + (iq * H_kv + r) * k;
  }
  topk_row<LM>(P + row * ldp, lb, k, out, lane, cand[threadIdx.x >> 6]);
}

static hipError_t launch_topk(const float* P, int64_t ldp, int64_t nrows, int64_t Nq,
                              int H_kv, int64_t q_start, int nblk_dec, int k, int32_t* sel,
                              hipStream_t stream) {
  dim3 grid((unsigned)ceil_div(nrows, 4)), block(256);
  if (k <= 8)
    topk_kernel<7><<<grid, block, 0, stream>>>(P, ldp, nrows, Nq, H_kv, q_start, nblk_dec, k, sel);
  else if (k <= 16)
    topk_kernel<15><<<grid, block, 0, stream>>>(P, ldp, nrows, Nq, H_kv, q_start, nblk_dec, k, sel);
  else
    topk_kernel<31><<<grid, block, 0, stream>>>(P, ldp, nrows, Nq, H_kv, q_start, nblk_dec, k, sel);
  return hipGetLastError();
}

hipError_t launch_topk_prefill(const float* P, int64_t ldp, int64_t q_start, int64_t Nq,
                               int H_kv, int k, int32_t* sel, hipStream_t stream) {
  return launch_topk(P, ldp, (int64_t)H_kv * Nq, Nq, H_kv, q_start, 0, k, sel, stream);
}

hipError_t launch_topk_decode(const float* P, int64_t ldp, int B, int H_kv, int nblk, int k,
                              int32_t* sel, hipStream_t stream) {
  return launch_topk(P, ldp, (int64_t)B * H_kv, 1, H_kv, 0, nblk, k, sel, stream);
}

template <int D, int NW, int CG>
static void launch_fused_dn(const __bf16* qi, const __bf16* ki, int64_t q_start, int64_t Nq,
                            int H_kv, int k, int32_t* sel, hipStream_t stream) {
  const int ntiles = (int)ceil_div(Nq, (int64_t)(32 * CG * NW));
  dim3 grid(index_grid(ntiles, H_kv)), block(64 * NW);
  if (k <= 8)
    index_topk_fused_kernel<D, NW, CG, 7><<<grid, block, 0, stream>>>(qi, ki, q_start, Nq, H_kv, ntiles, k, sel);
  else if (k <= 16)
    index_topk_fused_kernel<D, NW, CG, 15><<<grid, block, 0, stream>>>(qi, ki, q_start, Nq, H_kv, ntiles, k, sel);
  else
    index_topk_fused_kernel<D, NW, CG, 31><<<grid, block, 0, stream>>>(qi, ki, q_start, Nq, H_kv, ntiles, k, sel);
}

template <int D>
static void launch_fused_d(const __bf16* qi, const __bf16* ki, int64_t q_start, int64_t Nq,
                           int H_kv, int k, int32_t* sel, hipStream_t stream) {
  // 128 queries per wave (each staged key block then serves 1024 queries)
  // while 1024-query tiles still give every CU a work-group; the lists of
  // k > 16 would not fit the registers of two queries per lane
  if (D <= 64 && k <= 16 && ceil_div(Nq, (int64_t)1024) * H_kv >= device_cus())
    launch_fused_dn<D, 8, D <= 64 ? 4 : 2>(qi, ki, q_start, Nq, H_kv, k, sel, stream);
  else if (D < 128 && index_waves(Nq, H_kv, D) == 8)
    launch_fused_dn<D, D < 128 ? 8 : 4, 2>(qi, ki, q_start, Nq, H_kv, k, sel, stream);
  else
    launch_fused_dn<D, 4, 2>(qi, ki, q_start, Nq, H_kv, k, sel, stream);
}

hipError_t launch_index_topk_fused(const void* q_idx, const void* k_idx, int64_t q_start,
                                   int64_t Nq, int H_kv, int d_idx, int k, int32_t* sel,
                                   hipStream_t stream) {
  auto* qi = static_cast<const __bf16*>(q_idx);
  auto* ki = static_cast<const __bf16*>(k_idx);
  switch (d_idx) {
    case 32: launch_fused_d<32>(qi, ki, q_start, Nq, H_kv, k, sel, stream); break;
    case 64: launch_fused_d<64>(qi, ki, q_start, Nq, H_kv, k, sel, stream); break;
    case 128: launch_fused_d<128>(qi, ki, q_start, Nq, H_kv, k, sel, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
