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
// One KV-outer pass over the forward's inverted index (local positions
// included, with the causal mask).  A work unit is one bucket (group r,
// block b), or a fixed-size slice of a large one.  Its work-group keeps the
// block's K and V in registers (each of the four waves owns 32 keys) and
// sweeps the unit's rows -- (position, head) pairs -- in 32-row tiles that
// are double-buffered in LDS, row-major for S = Q K^T and dP = dO V^T and
// transposed for dV += P^T dO and dK += dS^T Q (the contractions over
// rows).  Each tile's dS goes through LDS so that the waves, now owning 32
// d each, form dQ^T = K^T dS^T over all 128 keys; that is stored as a bf16
// partial per (i, h, slot) and summed per (i, h) in ascending slot order by
// a second kernel.  A whole bucket adds its dK/dV sums to the outputs at
// the end; the slices of a split bucket write fp32 partials that a third
// kernel sums in slice order.  Deterministic, no atomics on the outputs.
#include "common.h"
#include "lds_rows.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRp = 32 + 4;       // pitch of a transposed [d][32 rows] tile
constexpr int kDsp = kBlock + 4;  // pitch of the [32 rows][128 keys] dS tile
constexpr int kUnitRows = 16384;  // rows per work unit, at most
constexpr int kUnitPos = 1024;    // positions per work unit, at most

// A fragment (MFMA A or B: 32 rows x 16 d at k-step s) of a row-major
// swizzled tile; lane half h covers d in [h*D/2, (h+1)*D/2).
template <int D>
__device__ __forceinline__ bf16x8 rm_frag(const __bf16* blk, int row, int s, int h) {
  return *reinterpret_cast<const bf16x8*>(
      &blk[row * D + 8 * (((D / 16) * h + s) ^ row_swz<D>(row))]);
}

// Fragment with the contraction over 16 entries c0.. of a row of t[.][PITCH]:
// lane half h takes entries c0 + 4h + {0..3} and c0 + 8 + 4h + {0..3}, which
// is the order in which an accumulator's registers 8u..8u+7 hold rows 16u..
// (so an accumulator can be the other operand).
template <int PITCH>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* t, int d, int c0, int h) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&t[d * PITCH + c0 + 4 * h]);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&t[d * PITCH + c0 + 8 + 4 * h]);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace

int bwd_unit_positions(int G) { return std::min(kUnitPos, std::max(1, kUnitRows / G)); }

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
// Work units: every non-empty bucket, split into slices of at most `upos`
// positions when larger.  Units of split buckets and buckets of at least
// upos/2 entries come first.  A split bucket also gets a record (bucket,
// first partial, slices) for the dK/dV partial sum.
__global__ __launch_bounds__(1024) void build_bwd_units_kernel(
    const int32_t* __restrict__ row_ptr, int64_t nb, int upos, int4* __restrict__ units,
    int32_t* __restrict__ n_units, int4* __restrict__ splits, int32_t* __restrict__ n_splits) {
  __shared__ int4 sc[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(nb, (int64_t)1024);
  const int64_t lo = min(nb, per * t), hi = min(nb, per * (t + 1));
  int4 c = make_int4(0, 0, 0, 0);  // large units, small units, split buckets, slices
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t cnt = row_ptr[x + 1] - row_ptr[x];
    const int32_t nu = (cnt + upos - 1) / upos;
    if (nu > 1) {
      c.x += nu;
      c.z += 1;
      c.w += nu;
    } else if (2 * cnt >= upos) {
      c.x += 1;
    } else if (cnt > 0) {
      c.y += 1;
    }
  }
  sc[t] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int4 v = t >= o ? sc[t - o] : make_int4(0, 0, 0, 0);
    __syncthreads();
    const int4 m = sc[t];
    sc[t] = make_int4(m.x + v.x, m.y + v.y, m.z + v.z, m.w + v.w);
    __syncthreads();
  }
  const int4 tot = sc[1023];
  const int4 ex = t ? sc[t - 1] : make_int4(0, 0, 0, 0);
  int32_t ub = ex.x, us = tot.x + ex.y, sp = ex.z, pi = ex.w;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t s0 = row_ptr[x], cnt = row_ptr[x + 1] - s0;
    const int32_t nu = (cnt + upos - 1) / upos;
    if (nu > 1) {
      splits[sp++] = make_int4((int)x, pi, nu, 0);
      for (int32_t s = 0; s < nu; ++s)
        units[ub++] = make_int4((int)x, s0 + s * upos, min(upos, cnt - s * upos), pi + s);
      pi += nu;
    } else if (2 * cnt >= upos) {
      units[ub++] = make_int4((int)x, s0, cnt, -1);
    } else if (cnt > 0) {
      units[us++] = make_int4((int)x, s0, cnt, -1);
    }
  }
  if (t == 1023) {
    n_units[0] = tot.x + tot.y;
    n_units[1] = 0;
    n_splits[0] = tot.z;
  }
}

template <int DH>
struct BwdSmem {
  __bf16 qr[2][32 * DH];    // the tile's Q rows, row-major swizzled
  __bf16 gr[2][32 * DH];    // the tile's dO rows
  __bf16 qt[3][DH * kRp];   // the same, transposed [d][row] (three tiles live)
  __bf16 gt[3][DH * kRp];
  __bf16 ds[2][32 * kDsp];  // dS [row][key], for dQ
  __bf16 pt[2][kBlock * kRp];   // P^T [key][row], for the second d-half's dV
  __bf16 dst[2][kBlock * kRp];  // dS^T [key][row], for its dK
  int32_t lim[2][32];       // per tile row: last visible key of the block (-1: none)
  float l2[2][32];          // lse * log2(e)
  float dv[2][32];          // D = dO . O
  int32_t pos[kUnitPos];    // the unit's query positions
  uint8_t sl[kUnitPos];     // and the block's slot in each one's selection
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Eight waves per work-group, two per SIMD, in producer/consumer pairs
// over the same 32 keys kw = 32 (w mod 4):
//  - waves 0-3 (first d-half) form S = Q K^T and dP = dO V^T, the softmax
//    and dS for tile T, add its P^T dO and dS^T Q into dV/dK for d < DH/2,
//    and leave dS, P^T and dS^T in LDS;
//  - waves 4-7 take tile T-1 from LDS after the barrier: dV/dK for the
//    second d-half, and dQ^T = K^T dS^T for their 32-wide d-slice (K^T in
//    registers).
// No MFMA or softmax is done twice, and each SIMD holds one wave of each
// kind, so one's softmax and LDS waits overlap the other's MFMAs.
template <int DH>
__global__ __launch_bounds__(512) void bwd_fused_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ units, int32_t* __restrict__ n_units, int64_t q_start, int64_t Nk,
    int H_q, int H_kv, int G, float inv_G, int nblk, int k, int64_t spare, float scale,
    float scale_log2, __bf16* __restrict__ part, float* __restrict__ kvpart,
    float* __restrict__ dK, float* __restrict__ dV) {
  constexpr int S = DH / 16, NDG = DH / 32, NDH = NDG / 2, CH = DH / 8;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  BwdSmem<DH>& sm = *reinterpret_cast<BwdSmem<DH>*>(smem_raw);
  __shared__ int32_t next;
  const int t = threadIdx.x, wave = t >> 6;
  const int32_t total = n_units[0];
  for (;;) {
    if (t == 0) next = atomicAdd(&n_units[1], 1);
    __syncthreads();
    const int32_t unit_id = next;
    if (unit_id >= total) return;
    const int4 un = units[unit_id];
    const int bucket = un.x, start = un.y, count = un.z, pidx = un.w;
    const int r = bucket / nblk, b = bucket % nblk;
    int tl = t;  // per-unit addresses are rebuilt, not hoisted and spilled
    asm volatile("" : "+v"(tl));
    {
      // count <= kUnitPos = 2 * 512: all loads first, then the LDS stores
      int32_t pv[kUnitPos / 512];
      uint8_t sv[kUnitPos / 512];
#pragma unroll
      for (int u = 0; u < kUnitPos / 512; ++u) {
        const int p = tl + 512 * u;
        pv[u] = col[start + min(p, count - 1)];
        sv[u] = slot[start + min(p, count - 1)];
      }
#pragma unroll
      for (int u = 0; u < kUnitPos / 512; ++u) {
        const int p = tl + 512 * u;
        if (p < count) {
          sm.pos[p] = pv[u];
          sm.sl[p] = sv[u];
        }
      }
    }
    const int lane = tl & 63, h = lane >> 5, n = lane & 31;
    const int kq = wave & 3, dh = wave >> 2;
    const int kw = 32 * kq;  // this wave's keys kw .. kw+31; its d-slice for dQ
    const int64_t key0 = (int64_t)b * kBlock;
    // Static operands in one register array, by role: producers hold the
    // wave's keys as the B operand of S (fr[0..S)) and dP (fr[S..2S)), d
    // split by lane half; consumers hold K^T of their d-slice over all 128
    // keys as the A operand of dQ^T (fr[0..8)).
    bf16x8 fr[2 * S];
#pragma unroll
    for (int s = 0; s < 2 * S; ++s) fr[s] = bf16x8{};
    if (dh == 0) {
      const int64_t key = key0 + kw + n;
      const bool in = key < Nk;
      const int64_t off = ((in ? key : key0) * H_kv + r) * DH + (DH / 2) * h;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        fr[s] = *reinterpret_cast<const bf16x8*>(K + off + 8 * s);
        fr[S + s] = *reinterpret_cast<const bf16x8*>(V + off + 8 * s);
      }
#pragma unroll
      for (int s = 0; s < 2 * S; ++s) fr[s] = in ? fr[s] : bf16x8{};
    } else if (kw < DH) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t key = key0 + 16 * u + (e < 4 ? 4 * h + e : 8 + 4 * h + (e - 4));
          const __bf16 xv = K[((key < Nk ? key : key0) * H_kv + r) * DH + kw + n];
          fr[u][e] = key < Nk ? xv : f2bf(0.f);
        }
    }
    // every fragment load of the unit has landed before the tile loop, so no
    // wait inside the loop has to cover them
    __builtin_amdgcn_s_waitcnt(0);

    // tile staging: thread -> (tensor, 2-row group, 16-byte chunk)
    const int which = tl / (16 * CH);  // 0: Q, 1: dO, 2+: none (wave-uniform)
    const int it = tl % (16 * CH), rp = it / CH, c = it % CH;
    const int nrows = count * G;
    const int ntile = (nrows + 31) / 32;
    const int hq0 = r * G;
    bf16x8 x[2];
    int vmask = 0, mlim = -1;
    float ml2 = 0.f, mdv = 0.f;
    // Every thread issues the same global loads (idle staging threads and
    // rows past the end read a valid row), so the compiler can count the
    // loads and stores in flight instead of waiting for all of them.
    auto load = [&](int T) {
      vmask = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int R = 32 * T + 2 * rp + u;
        const bool ok = which < 2 && R < nrows;
        const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
        const int64_t pos = sm.pos[pp];
        const int hq = hq0 + (ok ? R - pp * G : 0);
        const __bf16* src = which == 0 ? Q + (pos * H_q + hq) * DH
                                       : dO + ((pos - q_start) * H_q + hq) * DH;
        x[u] = *reinterpret_cast<const bf16x8*>(src + 8 * c);
        vmask |= (int)ok << u;
      }
      {
        const int R = 32 * T + (tl & 31);
        const bool ok = R < nrows;
        const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
        const int64_t pos = sm.pos[pp];
        const int hq = hq0 + (ok ? R - pp * G : 0);
        const int64_t ih = (pos - q_start) * H_q + hq;
        ml2 = lse[ih];
        mdv = D[ih];
        mlim = ok ? (int)(pos - key0) : -1;
      }
    };
    auto store = [&](int T) {
      const int b2 = T & 1, b3 = T % 3;
      if (which < 2) {
        __bf16* rm = which == 0 ? sm.qr[b2] : sm.gr[b2];
        __bf16* tr = which == 0 ? sm.qt[b3] : sm.gt[b3];
        bf16x8 y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) y[u] = (vmask >> u) & 1 ? x[u] : bf16x8{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 2 * rp + u;
          *reinterpret_cast<bf16x8*>(&rm[row * DH + 8 * (c ^ row_swz<DH>(row))]) = y[u];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<bf16x2*>(&tr[(8 * c + e) * kRp + 2 * rp]) = bf16x2{y[0][e], y[1][e]};
      }
      if (tl < 32) {
        sm.lim[b2][tl] = mlim;
        sm.l2[b2][tl] = ml2 * kLog2e;
        sm.dv[b2][tl] = mdv;
      }
    };
    // consumer work on tile T (its producers' LDS output is complete): dV/dK
    // of the second d-half, then dQ^T of the wave's d-slice stored as the
    // rows' bf16 partials.  With T < 0 (nothing to consume) the MFMAs are
    // skipped and zeros go to the spare slot, so the stores stay uniform.
    f32x16 ak[NDH], av[NDH];
    auto consume = [&](int T, int nn) {
      const bool live = T >= 0;
      const int b2 = T & 1, b3 = (T + 3) % 3;
      f32x16 acc = {};
      if (live) {
#pragma unroll
        for (int i = 0; i < NDH; ++i) {
          const int dg = NDH + i;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            av[i] = mfma32(tr_frag<kRp>(sm.pt[b2], kw + nn, 16 * u, h),
                           tr_frag<kRp>(sm.gt[b3], 32 * dg + nn, 16 * u, h), av[i]);
            ak[i] = mfma32(tr_frag<kRp>(sm.dst[b2], kw + nn, 16 * u, h),
                           tr_frag<kRp>(sm.qt[b3], 32 * dg + nn, 16 * u, h), ak[i]);
          }
        }
        if (kw < DH) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            acc = mfma32(fr[u], tr_frag<kDsp>(sm.ds[b2], nn, 16 * u, h), acc);
        }
      }
      const int R = 32 * T + n;
      const bool ok = live && kw < DH && R < nrows;
      const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
      const int64_t ps = ok ? (sm.pos[pp] - q_start) * k + sm.sl[pp] : spare;
      const int hl = ok ? R - pp * G : 0;
      __bf16* dstp = part + (ps * H_kv + r) * (DH / 4) * G * 4 + hl * 4;
      // accumulator rows are d = kw + 8qd + 4h + {0..3}: d-quad 8kq + 2qd + h
      const int dq0 = ok ? 8 * kq : 0;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<bf16x4*>(dstp + (int64_t)(dq0 + 2 * qd + h) * G * 4) =
            bf16x4{f2bf(acc[4 * qd]), f2bf(acc[4 * qd + 1]), f2bf(acc[4 * qd + 2]),
                   f2bf(acc[4 * qd + 3])};
    };

    __syncthreads();  // positions staged
    load(0);
    store(0);
    if (ntile > 1) load(1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NDH; ++i) ak[i] = av[i] = f32x16{};
    for (int T = 0; T < ntile; ++T) {
      const int b2 = T & 1, b3 = T % 3;
      // LDS indices go through an opaque copy of n so that the fragment
      // reads stay inside the loop rather than being hoisted into registers
      int nn = n;
      asm volatile("" : "+v"(nn));
      if (dh == 0) {
        // S = Q K^T and dP = dO V^T for the wave's 32 keys (key on the lane)
        f32x16 sa = {}, pa = {};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          sa = mfma32(rm_frag<DH>(sm.qr[b2], nn, s, h), fr[s], sa);
          pa = mfma32(rm_frag<DH>(sm.gr[b2], nn, s, h), fr[S + s], pa);
        }
        bf16x8 pA[2], dA[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int row = acc_row(8 * u + e, h);
            const int lm = sm.lim[b2][row];
            const float l2 = sm.l2[b2][row], dv = sm.dv[b2][row];
            const float ex = __builtin_amdgcn_exp2f(sa[8 * u + e] * scale_log2 - l2);
            const float p = kw + n <= lm ? ex : 0.f;
            pA[u][e] = f2bf(p);
            dA[u][e] = f2bf(p * (pa[8 * u + e] - dv));
          }
        // dV += P^T dO and dK += dS^T Q over the tile's rows, first d-half
#pragma unroll
        for (int i = 0; i < NDH; ++i) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            av[i] = mfma32(pA[u], tr_frag<kRp>(sm.gt[b3], 32 * i + nn, 16 * u, h), av[i]);
            ak[i] = mfma32(dA[u], tr_frag<kRp>(sm.qt[b3], 32 * i + nn, 16 * u, h), ak[i]);
          }
        }
        // dS [row][key] for dQ; P^T and dS^T [key][row] for the consumers:
        // registers 8u + 4q' .. +3 hold rows 16u + 8q' + 4h .. +3
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sm.ds[b2][acc_row(8 * u + e, h) * kDsp + kw + nn] = dA[u][e];
#pragma unroll
          for (int qh = 0; qh < 2; ++qh) {
            const int row0 = 16 * u + 8 * qh + 4 * h;
            *reinterpret_cast<bf16x4*>(&sm.pt[b2][(kw + nn) * kRp + row0]) =
                bf16x4{pA[u][4 * qh], pA[u][4 * qh + 1], pA[u][4 * qh + 2], pA[u][4 * qh + 3]};
            *reinterpret_cast<bf16x4*>(&sm.dst[b2][(kw + nn) * kRp + row0]) =
                bf16x4{dA[u][4 * qh], dA[u][4 * qh + 1], dA[u][4 * qh + 2], dA[u][4 * qh + 3]};
          }
        }
        // producers store no dQ; the same (zero, spare-slot) stores as the
        // consumers keep the memory counters uniform
        consume(-1, nn);
      } else {
        consume(T - 1, nn);
      }
      (void)b3;
      // the next tile's rows into the free buffers, then fetch the one after
      if (T + 1 < ntile) {
        store(T + 1);
        if (T + 2 < ntile) load(T + 2);
      }
      __syncthreads();
    }
    if (dh == 1) consume(ntile - 1, n);
    // the unit's dK/dV sums: accumulator rows are keys, the lane is d
    if (pidx < 0) {
#pragma unroll
      for (int i = 0; i < NDH; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t key = key0 + kw + acc_row(j, h);
          if (key < Nk) {
            const int64_t off = (key * H_kv + r) * DH + 32 * (NDH * dh + i) + n;
            dK[off] += scale * ak[i][j];
            dV[off] += av[i][j];
          }
        }
    } else {
      float* pk = kvpart + (int64_t)pidx * 2 * kBlock * DH;
#pragma unroll
      for (int i = 0; i < NDH; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kr = kw + acc_row(j, h), d = 32 * (NDH * dh + i) + n;
          pk[kr * DH + d] = ak[i][j];
          pk[(kBlock + kr) * DH + d] = av[i][j];
        }
    }
  }
}

// dQ[i, h] = scale * sum over the row's slots (ascending) of the partials.
// Thread -> (row i, group r, d-quad, head in group), head fastest: a
// partial row group [d_h/4][G][4] is then read contiguously by consecutive
// threads, and each head's dQ row gets whole 64-byte runs.
template <int DH>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const __bf16* __restrict__ part,
                                                            int64_t q_start, int64_t Nq,
                                                            int H_q, int H_kv, int k,
                                                            float scale, float* __restrict__ dQ) {
  const int G = H_q / H_kv;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= Nq * H_q * (DH / 4)) return;
  const int hl = (int)(gid % G);
  const int64_t rest = gid / G;
  const int dq = (int)(rest % (DH / 4));
  const int64_t ir = rest / (DH / 4);
  const int r = (int)(ir % H_kv);
  const int64_t iq = ir / H_kv;
  const int n_sel = (int)min((int64_t)k, (q_start + iq) / kBlock + 1);
  const __bf16* src = part + ((iq * k) * H_kv + r) * (DH / 4) * G * 4 + ((int64_t)dq * G + hl) * 4;
  const int64_t slot_stride = (int64_t)H_kv * (DH / 4) * G * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // each partial is read once: non-temporal loads, four slots in flight
#pragma unroll 4
  for (int s = 0; s < n_sel; ++s) {
    const bf16x4 x =
        __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(src + s * slot_stride));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += bf2f(x[e]);
  }
  // d-quad dq holds d = 4*dq .. 4*dq+3
  *reinterpret_cast<f32x4*>(dQ + (iq * H_q + r * G + hl) * DH + 4 * dq) =
      f32x4{acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
}

// dK/dV of split buckets: the slices' partials summed in slice order.
template <int DH>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(
    const int4* __restrict__ splits, const int32_t* __restrict__ n_splits,
    const float* __restrict__ kvpart, int H_kv, int nblk, int64_t Nk, float scale,
    float* __restrict__ dK, float* __restrict__ dV) {
  const int32_t ns = n_splits[0];
  for (int32_t si = blockIdx.x; si < ns; si += gridDim.x) {
    const int4 sp = splits[si];
    const int r = sp.x / nblk, b = sp.x % nblk;
    for (int e = 4 * (int)threadIdx.x; e < kBlock * DH; e += 4 * 256) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < sp.z; ++s) {
        const float* pk = kvpart + (int64_t)(sp.y + s) * 2 * kBlock * DH;
        const f32x4 a = *reinterpret_cast<const f32x4*>(pk + e);
        const f32x4 v = *reinterpret_cast<const f32x4*>(pk + kBlock * DH + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sk[q] += a[q];
          sv[q] += v[q];
        }
      }
      const int64_t key = (int64_t)b * kBlock + e / DH;
      if (key < Nk) {
        const int64_t off = (key * H_kv + r) * DH + e % DH;
        f32x4 ok = *reinterpret_cast<const f32x4*>(dK + off);
        f32x4 ov = *reinterpret_cast<const f32x4*>(dV + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ok[q] += scale * sk[q];
          ov[q] += sv[q];
        }
        *reinterpret_cast<f32x4*>(dK + off) = ok;
        *reinterpret_cast<f32x4*>(dV + off) = ov;
      }
    }
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
  hipError_t e = bwd_allow(&bwd_fused_kernel<128>, sizeof(BwdSmem<128>));
  if (e == hipSuccess) e = bwd_allow(&bwd_fused_kernel<64>, sizeof(BwdSmem<64>));
  if (e == hipSuccess) bwd_lds_ready = true;
  return e;
}

BwdBounds bwd_bounds(int64_t nb, int64_t nnz, int G) {
  const int64_t upos = bwd_unit_positions(G);
  BwdBounds w;
  w.max_units = nb + nnz / upos + 1;
  w.max_splits = nnz / (upos + 1) + 1;
  w.max_slices = 2 * (nnz / upos) + 1;
  return w;
}

hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                           const float* lse, const void* dO, const int32_t* row_ptr,
                           const int32_t* col, const uint8_t* slot, int4* units,
                           int32_t* n_units, int4* splits, int32_t* n_splits,
                           const BwdBounds& bounds, int64_t q_start, int64_t Nq, int64_t Nk,
                           int H_q, int H_kv, int d_h, int nblk, int k, float scale,
                           float* Dbuf, void* dq_part, float* kvpart, float* dQ, float* dK,
                           float* dV, hipStream_t stream) {
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
  build_bwd_units_kernel<<<1, 1024, 0, stream>>>(row_ptr, nb, bwd_unit_positions(G), units,
                                                 n_units, splits, n_splits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid((unsigned)std::min<int64_t>(bounds.max_units, device_cus()));
  dim3 rgrid((unsigned)ceil_div(rows * (d_h / 4), (int64_t)256));
  dim3 sgrid((unsigned)std::min<int64_t>(bounds.max_splits, 2 * device_cus()));
  if (d_h == 128) {
    bwd_fused_kernel<128><<<grid, 512, sizeof(BwdSmem<128>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale, scale_log2, part, kvpart, dK, dV);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<128><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k,
                                                         scale, dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_kv_reduce_kernel<128><<<sgrid, 256, 0, stream>>>(splits, n_splits, kvpart, H_kv, nblk,
                                                         Nk, scale, dK, dV);
  } else if (d_h == 64) {
    bwd_fused_kernel<64><<<grid, 512, sizeof(BwdSmem<64>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale, scale_log2, part, kvpart, dK, dV);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<64><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k, scale,
                                                        dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_kv_reduce_kernel<64><<<sgrid, 256, 0, stream>>>(splits, n_splits, kvpart, H_kv, nblk,
                                                        Nk, scale, dK, dV);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
