// Main Branch backward ("MiniMax Sparse Attention" explainer, section 02:
// the Main Branch is exact softmax attention over the selected blocks, so
// its gradients are those of softmax attention restricted to each row's
// token set T; section 03: the selection is not differentiable, so nothing
// flows back into the Index Branch from here).
//
// Per row (query i, head h of group r), with p the forward's probabilities
// (recomputed from the saved lse), D = dO . O:
//   dp_j = dO . V_j,  ds_j = p_j (dp_j - D)
//   dQ = scale * sum_j ds_j K_j,  dK_j += scale * ds_j Q,  dV_j += p_j dO
// Both passes run KV-outer on the forward's inverted index (local positions
// included, with the causal mask), like the forward:
//   dQ:    work items of <= chunk positions of one bucket; 32-row tiles
//          (rows = (position, head) pairs) on the lanes: S^T = K Q^T,
//          dP^T = V dO^T, dS in registers, dQ^T = K^T dS^T; a bf16 partial
//          per (i, h, slot), summed per (i, h) in ascending slot order.
//   dK/dV: one work-group per non-empty bucket, its four waves owning 32
//          keys each and sweeping all the bucket's rows in 32-row tiles with
//          keys on the lanes: S = Q K^T, dP = dO V^T, then dV += P^T dO and
//          dK += dS^T Q contract over the rows.  Each key's sums are complete
//          inside one work-group, so they are added to dK/dV once, with no
//          partial buffers and no atomics.
#include "common.h"
#include "lds_rows.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTp = kBlock + 4;  // pitch of a transposed [d][128 keys] block
constexpr int kRp = 32 + 4;      // pitch of a transposed [d][32 rows] tile

// A fragment (MFMA A or B: 32 rows x 16 d at k-step s) of a row-major
// swizzled block; lane half h covers d in [h*D/2, (h+1)*D/2).
template <int D>
__device__ __forceinline__ bf16x8 rm_frag(const __bf16* blk, int row, int s, int h) {
  return *reinterpret_cast<const bf16x8*>(
      &blk[row * D + 8 * (((D / 16) * h + s) ^ row_swz<D>(row))]);
}

// Fragment with the contraction over 16 "rows" of a transposed block
// t[d][pitch]: lane half h takes rows c0 + 4h + {0..3} and c0 + 8 + 4h +
// {0..3}, which is the order in which an accumulator's entries 8u..8u+7
// hold rows 16u.. (so an accumulator can be the other operand).
template <int PITCH>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* t, int d, int c0, int h) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&t[d * PITCH + c0 + 4 * h]);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&t[d * PITCH + c0 + 8 + 4 * h]);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// K, V of block (r, key0..): row-major swizzled; rows >= Nk read as 0.
template <int DH>
__device__ __forceinline__ void stage_rm2(__bf16* kd, __bf16* vd, const __bf16* __restrict__ K,
                                          const __bf16* __restrict__ V, int r, int H_kv,
                                          int64_t key0, int64_t Nk, int t, int nthreads) {
  constexpr int CH = DH / 8;
  for (int id0 = 0; id0 < kBlock * CH; id0 += 4 * nthreads) {
    bf16x8 kr[4], vr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = id0 + t + nthreads * u, row = id / CH, c = id % CH;
      const bool in = id < kBlock * CH && key0 + row < Nk;
      const int64_t off = ((key0 + row) * H_kv + r) * DH + 8 * c;
      kr[u] = in ? *reinterpret_cast<const bf16x8*>(K + off) : bf16x8{};
      vr[u] = in ? *reinterpret_cast<const bf16x8*>(V + off) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = id0 + t + nthreads * u, row = id / CH, c = id % CH;
      if (id < kBlock * CH) {
        *reinterpret_cast<bf16x8*>(&kd[row * DH + 8 * (c ^ row_swz<DH>(row))]) = kr[u];
        *reinterpret_cast<bf16x8*>(&vd[row * DH + 8 * (c ^ row_swz<DH>(row))]) = vr[u];
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// D = dO . O per (row, head): 16 lanes per row, one 8-wide chunk each.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* __restrict__ dO,
                                                        const float* __restrict__ O,
                                                        int64_t rows, int d_h,
                                                        float* __restrict__ D) {
  const int cpr = d_h / 8;  // 8 or 16 lanes per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / cpr;
  const int c = (int)(gid % cpr);
  float s = 0.f;
  if (row < rows) {
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * d_h + 8 * c);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + row * d_h + 8 * c);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + row * d_h + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(bf2f(g[e]), o0[e], s);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(bf2f(g[4 + e]), o1[e], s);
  }
  for (int o = 1; o < cpr; o <<= 1) s += __shfl_xor(s, o, kWave);
  if (row < rows && c == 0) D[row] = s;
}

// ---------------------------------------------------------------------------
// dQ pass.
template <int DH>
struct BwdQSmem {
  __bf16 k[kBlock * DH];   // row-major, swizzled
  __bf16 v[kBlock * DH];   // row-major, swizzled
  __bf16 kt[DH * kTp];     // K transposed, padded
  int32_t pos[kMaxItem];
  uint8_t sl[kMaxItem];
};

template <int DH>
__global__ __launch_bounds__(512) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ items, int32_t* __restrict__ n_items, int64_t q_start, int64_t Nk,
    int H_q, int H_kv, int G, float inv_G, int nblk, int k, int64_t spare, float scale_log2,
    __bf16* __restrict__ part) {
  constexpr int S = DH / 16, NDG = DH / 32, NW = 8;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  BwdQSmem<DH>& sm = *reinterpret_cast<BwdQSmem<DH>*>(smem_raw);
  __shared__ int32_t next;
  const int t = threadIdx.x, wave = t >> 6;
  const int32_t total = n_items[0];
  for (;;) {
    if (t == 0) next = atomicAdd(&n_items[1], 1);
    __syncthreads();
    const int32_t item_id = next;
    if (item_id >= total) return;
    const int4 it = items[item_id];
    const int bucket = it.x, start = it.y, count = it.z;
    const int r = bucket / nblk, b = bucket % nblk;
    int tl = t;  // per-item addresses are rebuilt, not hoisted and spilled
    asm volatile("" : "+v"(tl));
    for (int p = tl; p < count; p += 64 * NW) {
      sm.pos[p] = col[start + p];
      sm.sl[p] = slot[start + p];
    }
    stage_rm2<DH>(sm.k, sm.v, K, V, r, H_kv, (int64_t)b * kBlock, Nk, tl, 64 * NW);
    __syncthreads();
    // K^T from the staged rows: each thread moves 4 keys x 8 d
    for (int id = tl; id < (kBlock / 4) * (DH / 8); id += 64 * NW) {
      const int kq = id % (kBlock / 4), c = id / (kBlock / 4);
      bf16x8 rw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = 4 * kq + u;
        rw[u] = *reinterpret_cast<const bf16x8*>(&sm.k[row * DH + 8 * (c ^ row_swz<DH>(row))]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<bf16x4*>(&sm.kt[(8 * c + e) * kTp + 4 * kq]) =
            bf16x4{rw[0][e], rw[1][e], rw[2][e], rw[3][e]};
    }
    __syncthreads();

    const int lane = tl & 63, h = lane >> 5, n = lane & 31;
    const int nrows = count * G;
    const int ntile = (nrows + 31) / 32;
    for (int tile = wave; tile < ntile; tile += NW) {
      const int R = tile * 32 + n;
      const bool ok = R < nrows;
      const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
      const int pos = sm.pos[pp];
      const int hq = r * G + (ok ? R - pp * G : 0);
      const int64_t iq = pos - q_start;
      const int lim = ok ? pos - b * kBlock : -1;  // visible keys 0..lim
      bf16x8 qb[S], gb[S];
      const __bf16* qrow = Q + ((int64_t)pos * H_q + hq) * DH + (DH / 2) * h;
      const __bf16* grow = dO + (iq * H_q + hq) * DH + (DH / 2) * h;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 8 * s);
        gb[s] = *reinterpret_cast<const bf16x8*>(grow + 8 * s);
      }
      const float l2 = lse[iq * H_q + hq] * kLog2e;
      const float Dv = D[iq * H_q + hq];
      // per key group: S^T -> P, dP^T -> dS, packed as the next MFMA's B
      // operand (keys on the accumulator rows, the row on the lane).  The
      // LDS index goes through an opaque copy of n so the fragment reads are
      // not hoisted out of the tile loop into registers.
      int nn = n;
      asm volatile("" : "+v"(nn));
      bf16x8 dsb[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x16 sa = {}, pa = {};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          sa = mfma32(rm_frag<DH>(sm.k, 32 * g + nn, s, h), qb[s], sa);
          pa = mfma32(rm_frag<DH>(sm.v, 32 * g + nn, s, h), gb[s], pa);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 8 * u + e;
            const float p = 32 * g + acc_row(j, h) <= lim
                                ? __builtin_amdgcn_exp2f(sa[j] * scale_log2 - l2)
                                : 0.f;
            dsb[g][u][e] = f2bf(p * (pa[j] - Dv));
          }
      }
      // dQ^T = K^T dS^T, stored as a bf16 partial (rows past the end: spare slot)
      const int64_t ps = ok ? iq * k + sm.sl[pp] : spare;
      __bf16* dst = part + (ps * H_kv + r) * (DH / 4) * G * 4 + (hq - r * G + h * G) * 4;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        f32x16 acc = {};
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc = mfma32(tr_frag<kTp>(sm.kt, 32 * dg + nn, 32 * g + 16 * u, h), dsb[g][u], acc);
        // d = 32dg + 8qd + 4h + e  ->  d-quad 8dg + 2qd + h
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<bf16x4*>(dst + (8 * dg + 2 * qd) * G * 4) =
              bf16x4{f2bf(acc[4 * qd]), f2bf(acc[4 * qd + 1]), f2bf(acc[4 * qd + 2]),
                     f2bf(acc[4 * qd + 3])};
      }
    }
    __syncthreads();  // LDS and `next` are reused by the next item
  }
}

// dQ[i, h] = scale * sum over the row's slots (ascending) of the partials.
template <int DH>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const __bf16* __restrict__ part,
                                                            int64_t q_start, int64_t Nq,
                                                            int H_q, int H_kv, int k,
                                                            float scale, float* __restrict__ dQ) {
  // one thread per (iq, h, d-quad)
  const int G = H_q / H_kv;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= Nq * H_q * (DH / 4)) return;
  const int dq = (int)(gid % (DH / 4));
  const int64_t ih = gid / (DH / 4);
  const int h = (int)(ih % H_q);
  const int64_t iq = ih / H_q;
  const int r = h / G;
  const int n_sel = (int)min((int64_t)k, (q_start + iq) / kBlock + 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_sel; ++s) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(
        part + ((iq * k + s) * H_kv + r) * (DH / 4) * G * 4 + (int64_t)dq * G * 4 + (h - r * G) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += bf2f(x[e]);
  }
  // d-quad dq holds d = 4*dq .. 4*dq+3
  *reinterpret_cast<f32x4*>(dQ + (iq * H_q + h) * DH + 4 * dq) =
      f32x4{acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
}

// ---------------------------------------------------------------------------
// dK/dV pass: units = non-empty buckets, the largest first.
__global__ __launch_bounds__(1024) void build_units_kernel(const int32_t* __restrict__ row_ptr,
                                                           int64_t nb, int heavy,
                                                           int4* __restrict__ units,
                                                           int32_t* __restrict__ n_units) {
  __shared__ int32_t big[1024], small[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(nb, 1024);
  const int64_t lo = min(nb, per * t), hi = min(nb, per * (t + 1));
  int32_t nbg = 0, nsm = 0;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t cnt = row_ptr[x + 1] - row_ptr[x];
    nbg += cnt >= heavy;
    nsm += cnt > 0 && cnt < heavy;
  }
  big[t] = nbg;
  small[t] = nsm;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t vb = t >= o ? big[t - o] : 0, vs = t >= o ? small[t - o] : 0;
    __syncthreads();
    big[t] += vb;
    small[t] += vs;
    __syncthreads();
  }
  const int32_t n_big = big[1023];
  int32_t pb = t ? big[t - 1] : 0, ps = n_big + (t ? small[t - 1] : 0);
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t cnt = row_ptr[x + 1] - row_ptr[x];
    if (cnt >= heavy)
      units[pb++] = make_int4((int)x, row_ptr[x], cnt, 0);
    else if (cnt > 0)
      units[ps++] = make_int4((int)x, row_ptr[x], cnt, 0);
  }
  if (t == 1023) {
    n_units[0] = n_big + small[1023];
    n_units[1] = 0;
  }
}

template <int DH>
struct BwdKvSmem {
  __bf16 k[kBlock * DH];  // row-major, swizzled
  __bf16 v[kBlock * DH];
  __bf16 qr[32 * DH];     // the tile's Q rows, row-major swizzled
  __bf16 gr[32 * DH];     // the tile's dO rows
  __bf16 qt[DH * kRp];    // the same, transposed
  __bf16 gt[DH * kRp];
  int32_t lim[32];        // per tile row: last visible key of the block
  float l2[32];           // lse * log2(e)
  float dv[32];           // D = dO . O
};

template <int DH>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    const int32_t* __restrict__ col, const int4* __restrict__ units,
    int32_t* __restrict__ n_units, int64_t q_start, int64_t Nk, int H_q, int H_kv, int G,
    float inv_G, int nblk, float scale, float scale_log2, float* __restrict__ dK,
    float* __restrict__ dV) {
  constexpr int S = DH / 16, NDG = DH / 32, CH = DH / 8;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  BwdKvSmem<DH>& sm = *reinterpret_cast<BwdKvSmem<DH>*>(smem_raw);
  __shared__ int32_t next;
  const int t = threadIdx.x, wave = t >> 6;
  const int32_t total = n_units[0];
  for (;;) {
    if (t == 0) next = atomicAdd(&n_units[1], 1);
    __syncthreads();
    const int32_t unit_id = next;
    if (unit_id >= total) return;
    const int4 un = units[unit_id];
    const int bucket = un.x, start = un.y, count = un.z;
    const int r = bucket / nblk, b = bucket % nblk;
    int tl = t;
    asm volatile("" : "+v"(tl));
    stage_rm2<DH>(sm.k, sm.v, K, V, r, H_kv, (int64_t)b * kBlock, Nk, tl, 256);
    const int lane = tl & 63, h = lane >> 5, n = lane & 31;
    const int kw = 32 * wave;  // this wave's keys kw .. kw+31
    f32x16 ak[NDG], av[NDG];
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg) ak[dg] = av[dg] = f32x16{};
    const int nrows = count * G;
    for (int R0 = 0; R0 < nrows; R0 += 32) {
      __syncthreads();  // previous tile's LDS reads are done (and K/V staged)
      // stage the tile's 32 rows of Q and dO, both layouts
      for (int id = tl; id < 32 * CH * 2; id += 256) {
        const int which = id / (32 * CH), rc = id % (32 * CH), rr = rc / CH, c = rc % CH;
        const int R = R0 + rr;
        bf16x8 x = {};
        if (R < nrows) {
          const int pp = (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G);
          const int pos = col[start + pp];
          const int hq = r * G + (R - pp * G);
          x = which == 0
                  ? *reinterpret_cast<const bf16x8*>(Q + ((int64_t)pos * H_q + hq) * DH + 8 * c)
                  : *reinterpret_cast<const bf16x8*>(dO + ((pos - q_start) * H_q + hq) * DH +
                                                     8 * c);
        }
        __bf16* rmj = which == 0 ? sm.qr : sm.gr;
        __bf16* trj = which == 0 ? sm.qt : sm.gt;
        *reinterpret_cast<bf16x8*>(&rmj[rr * DH + 8 * (c ^ row_swz<DH>(rr))]) = x;
#pragma unroll
        for (int e = 0; e < 8; ++e) trj[(8 * c + e) * kRp + rr] = x[e];
      }
      if (tl < 32) {
        const int R = R0 + tl;
        int lm = -1;
        float l = 0.f, dd = 0.f;
        if (R < nrows) {
          const int pp = (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G);
          const int pos = col[start + pp];
          const int hq = r * G + (R - pp * G);
          const int64_t iq = pos - q_start;
          lm = pos - b * kBlock;
          l = lse[iq * H_q + hq] * kLog2e;
          dd = D[iq * H_q + hq];
        }
        sm.lim[tl] = lm;
        sm.l2[tl] = l;
        sm.dv[tl] = dd;
      }
      __syncthreads();
      // S = Q K^T and dP = dO V^T for the wave's 32 keys (key on the lane)
      f32x16 sa = {}, pa = {};
#pragma unroll
      for (int s = 0; s < S; ++s) {
        sa = mfma32(rm_frag<DH>(sm.qr, n, s, h), rm_frag<DH>(sm.k, kw + n, s, h), sa);
        pa = mfma32(rm_frag<DH>(sm.gr, n, s, h), rm_frag<DH>(sm.v, kw + n, s, h), pa);
      }
      bf16x8 pA[2], dA[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = acc_row(8 * u + e, h);
          const float p = kw + n <= sm.lim[row]
                              ? __builtin_amdgcn_exp2f(sa[8 * u + e] * scale_log2 - sm.l2[row])
                              : 0.f;
          pA[u][e] = f2bf(p);
          dA[u][e] = f2bf(p * (pa[8 * u + e] - sm.dv[row]));
        }
      // dV += P^T dO and dK += dS^T Q, contracting over the tile's rows
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          av[dg] = mfma32(pA[u], tr_frag<kRp>(sm.gt, 32 * dg + n, 16 * u, h), av[dg]);
          ak[dg] = mfma32(dA[u], tr_frag<kRp>(sm.qt, 32 * dg + n, 16 * u, h), ak[dg]);
        }
    }
    // add the bucket's sums: accumulator rows are keys, the lane is d
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t key = (int64_t)b * kBlock + kw + acc_row(j, h);
        if (key < Nk) {
          const int64_t off = (key * H_kv + r) * DH + 32 * dg + n;
          dK[off] += scale * ak[dg][j];
          dV[off] += av[dg][j];
        }
      }
    __syncthreads();  // `next` is reused
  }
}

// ---------------------------------------------------------------------------
static bool bwd_lds_ready = false;

template <typename Kern>
static hipError_t bwd_allow(Kern* kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

static hipError_t bwd_prepare() {
  if (bwd_lds_ready) return hipSuccess;
  hipError_t e = bwd_allow(&bwd_dq_kernel<128>, sizeof(BwdQSmem<128>));
  if (e == hipSuccess) e = bwd_allow(&bwd_dq_kernel<64>, sizeof(BwdQSmem<64>));
  if (e == hipSuccess) e = bwd_allow(&bwd_dkdv_kernel<128>, sizeof(BwdKvSmem<128>));
  if (e == hipSuccess) e = bwd_allow(&bwd_dkdv_kernel<64>, sizeof(BwdKvSmem<64>));
  if (e == hipSuccess) bwd_lds_ready = true;
  return e;
}

int64_t bwd_max_units(int64_t nb) { return nb + 1; }

hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                           const float* lse, const void* dO, const int32_t* row_ptr,
                           const int32_t* col, const uint8_t* slot, const int4* items,
                           int32_t* n_items, int64_t max_items, int4* units, int32_t* n_units,
                           int64_t q_start, int64_t Nq, int64_t Nk, int H_q, int H_kv, int d_h,
                           int nblk, int k, float scale, float* Dbuf, void* dq_part, float* dQ,
                           float* dK, float* dV, hipStream_t stream) {
  hipError_t e = bwd_prepare();
  if (e != hipSuccess) return e;
  const int G = H_q / H_kv;
  const float inv_G = 1.f / (float)G;
  const float scale_log2 = scale * kLog2e;
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* v = static_cast<const __bf16*>(V);
  auto* g = static_cast<const __bf16*>(dO);
  auto* part = static_cast<__bf16*>(dq_part);
  const int64_t rows = Nq * H_q;
  const int cpr = d_h / 8;
  bwd_delta_kernel<<<(unsigned)ceil_div(rows * cpr, (int64_t)256), 256, 0, stream>>>(
      g, O, rows, d_h, Dbuf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t spare = Nq * k;
  const int nb = H_kv * nblk;
  dim3 qgrid((unsigned)std::min<int64_t>(max_items, device_cus()));
  dim3 rgrid((unsigned)ceil_div(rows * (d_h / 4), (int64_t)256));
  build_units_kernel<<<1, 1024, 0, stream>>>(row_ptr, nb, 1024, units, n_units);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 kvgrid((unsigned)std::min<int64_t>(bwd_max_units(nb), device_cus()));
  if (d_h == 128) {
    bwd_dq_kernel<128><<<qgrid, 512, sizeof(BwdQSmem<128>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, items, n_items, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale_log2, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<128><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k,
                                                         scale, dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dkdv_kernel<128><<<kvgrid, 256, sizeof(BwdKvSmem<128>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G, nblk,
        scale, scale_log2, dK, dV);
  } else if (d_h == 64) {
    bwd_dq_kernel<64><<<qgrid, 512, sizeof(BwdQSmem<64>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, items, n_items, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale_log2, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<64><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k, scale,
                                                        dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dkdv_kernel<64><<<kvgrid, 256, sizeof(BwdKvSmem<64>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G, nblk,
        scale, scale_log2, dK, dV);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
