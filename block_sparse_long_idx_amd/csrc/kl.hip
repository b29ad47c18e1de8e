// Index-alignment KL, forward value ("MiniMax Sparse Attention" explainer,
// section 03 "KL Loss"; section 05 part 2 on keeping the LSE from the
// forward pass).
//
// For query i and group r, on the token set T of the selected blocks
// (j <= i), the student is the softmax of the index scores q_idx . k_idx
// and the teacher is the mean over the group's G query heads of their Main
// Branch attention probabilities; the loss is KL(teacher || student).
// With the forward's per-head log-sum-exp the teacher probabilities are
// final without a second softmax pass:
//   t_j = (1/G) sum_h exp(scale * Q[i,h] . K[j,r] - lse[i,h])
// and, writing s_j for the index score and L for ln sum_{j in T} exp(s_j),
//   KL = sum_j t_j ln t_j - sum_j t_j s_j + L        (sum_j t_j = 1).
// All three sums split over the selected blocks, so the pass runs KV-outer
// on the same inverted index as the Main Branch: one work item = one key
// block and the queries that selected it (local positions included, with
// the causal mask), producing per (i, r, slot) the partials
//   A = sum t ln t,  B = sum t s,  L_b = ln sum exp(s)
// which a second kernel merges in ascending slot order.
#include "common.h"
#include "lds_rows.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

constexpr float kLog2e = 1.4426950408889634f;

template <int DH, int DI>
struct KlSmem {
  __bf16 k[kBlock * DH];   // K of the block, rows swizzled
  __bf16 ki[kBlock * DI];  // k_idx of the block, rows swizzled
  int32_t pos[kMaxItem];
  uint8_t sl[kMaxItem];
};

// Rows key0.. of a [N][H_kv][D] tensor for group r into a swizzled [128][D]
// LDS block; rows >= Nk read as 0.  Loads are issued before the stores.
template <int D>
struct RowStage {
  static constexpr int CH = D / 8;
  static constexpr int L = kBlock * CH / 256;
  bf16x8 v[L];
  __device__ __forceinline__ void load(const __bf16* __restrict__ src, int r, int H_kv,
                                       int64_t key0, int64_t Nk, int t) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int id = t + 256 * u, row = id / CH, c = id % CH;
      v[u] = key0 + row < Nk
                 ? *reinterpret_cast<const bf16x8*>(src + ((key0 + row) * H_kv + r) * D + 8 * c)
                 : bf16x8{};
    }
  }
  __device__ __forceinline__ void store(__bf16* dst, int t) const {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int id = t + 256 * u, row = id / CH, c = id % CH;
      *reinterpret_cast<bf16x8*>(dst + row * D + 8 * (c ^ row_swz<D>(row))) = v[u];
    }
  }
};

// MFMA A fragment (32 keys x 16 d) of key group g, k-step s from a swizzled
// block; at k-step s lane half h covers d = 16s + 8h .. 16s + 8h + 7.  The
// query operands take the same order, so the two lanes of a row read
// neighbouring 16-byte pieces and each load instruction touches half as
// many cache lines as with a contiguous half-row per lane.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const __bf16* blk, int g, int s, int h, int n) {
  const int row = 32 * g + n;
  return *reinterpret_cast<const bf16x8*>(&blk[row * D + 8 * ((2 * s + h) ^ row_swz<D>(row))]);
}

// One work item: 32-position tiles, positions on the MFMA columns (S^T =
// K . Q^T), so every lane holds 16 keys of one position and the teacher's
// head mean is an element-wise sum over per-head MFMA passes.
template <int DH, int DI>
__device__ __forceinline__ void kl_item(const KlSmem<DH, DI>& sm, const __bf16* __restrict__ Q,
                                        const __bf16* __restrict__ q_idx,
                                        const float* __restrict__ lse, int count, int wave,
                                        int r, int b, int G, int H_q, int H_kv, int k,
                                        int64_t q_start, float scale_log2,
                                        float* __restrict__ part, int h, int n) {
  constexpr int S = DH / 16, SI = DI / 16;
  const int ntile = (count + 31) / 32;
  const float inv_G = 1.f / (float)G;
  for (int tile = wave; tile < ntile; tile += 4) {
    const int p = tile * 32 + n;
    const bool ok = p < count;
    const int i = sm.pos[ok ? p : 0];  // columns past the end repeat position 0
    const int lim = i - b * kBlock;    // keys 0..lim of the block are visible
    f32x16 t[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) t[g] = f32x16{};
    // Unmasked per-head sums (keys past the query are dropped below); the
    // K fragments are read from LDS again for every head: an index the
    // compiler cannot see through keeps them from being hoisted out of the
    // head loop into registers.
    // Each head's Q row and lse are requested one head ahead, so their
    // latency hides under the previous head's MFMAs and exps (the last head
    // requests its own row again).
    auto ldq = [&](int hh, bf16x8* dst, float& l2o) {
      const int hq = r * G + hh;
      const __bf16* qrow = Q + ((int64_t)i * H_q + hq) * DH + 8 * h;
#pragma unroll
      for (int s = 0; s < S; ++s) dst[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
      l2o = lse[(int64_t)(i - (int)q_start) * H_q + hq];
    };
    bf16x8 qb[S];
    float l2r;
    ldq(0, qb, l2r);
    for (int hh = 0; hh < G; ++hh) {
      int nn = n;
      asm volatile("" : "+v"(nn));
      bf16x8 qn[S];
      float l2n;
      ldq(min(hh + 1, G - 1), qn, l2n);
      // the next head's loads stay ahead of this head's LDS reads and MFMAs
      asm volatile("" ::: "memory");
      const float l2 = l2r * kLog2e;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x16 sacc = {};
#pragma unroll
        for (int s = 0; s < S; ++s) sacc = mfma32(row_frag<DH>(sm.k, g, s, h, nn), qb[s], sacc);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          t[g][j] += __builtin_amdgcn_exp2f(sacc[j] * scale_log2 - l2);
      }
      // ... and land by the end of this head's work
#pragma unroll
      for (int s = 0; s < S; ++s) asm volatile("" : "+v"(qn[s]));
      asm volatile("" : "+v"(l2n));
#pragma unroll
      for (int s = 0; s < S; ++s) qb[s] = qn[s];
      l2r = l2n;
    }
    // student scores s = q_idx . k_idx over the block
    const __bf16* qirow = q_idx + ((int64_t)i * H_kv + r) * DI + 8 * h;
    bf16x8 qi[SI];
#pragma unroll
    for (int s = 0; s < SI; ++s) qi[s] = *reinterpret_cast<const bf16x8*>(qirow + 16 * s);
    f32x16 sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sc[g] = f32x16{};
#pragma unroll
      for (int s = 0; s < SI; ++s) sc[g] = mfma32(row_frag<DI>(sm.ki, g, s, h, n), qi[s], sc[g]);
    }
    // per-position partials over the lane's 64 keys, then the lane pair
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (32 * g + acc_row(j, h) <= lim) m = fmaxf(m, sc[g][j]);
    float z = 0.f, A = 0.f, B = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (32 * g + acc_row(j, h) > lim) continue;
        z += __builtin_amdgcn_exp2f((sc[g][j] - m) * kLog2e);
        const float tt = t[g][j] * inv_G;
        if (tt > 0.f) A += tt * __logf(tt);
        B += tt * sc[g][j];
      }
    const float mp = __shfl_xor(m, 32, kWave), zp = __shfl_xor(z, 32, kWave);
    const float Ap = __shfl_xor(A, 32, kWave), Bp = __shfl_xor(B, 32, kWave);
    const float M = fmaxf(m, mp);  // finite: key 0 of the block is always visible
    const float Z = z * __builtin_amdgcn_exp2f((m - M) * kLog2e) +
                    zp * __builtin_amdgcn_exp2f((mp - M) * kLog2e);
    if (ok && h == 0) {
      float* dst = part + (((int64_t)(i - (int)q_start) * H_kv + r) * k + sm.sl[p]) * 3;
      dst[0] = A + Ap;
      dst[1] = B + Bp;
      dst[2] = M + __logf(Z);
    }
  }
}

template <int DH, int DI>
__global__ __launch_bounds__(256, 2) void kl_kv_outer_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ q_idx,
    const __bf16* __restrict__ k_idx, const float* __restrict__ lse,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ items, int32_t* __restrict__ n_items, int64_t q_start, int64_t Nk,
    int H_q, int H_kv, int G, int nblk, int k, float scale_log2, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  KlSmem<DH, DI>& sm = *reinterpret_cast<KlSmem<DH, DI>*>(smem_raw);
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
    int tl = t;  // rebuilt per item, not hoisted and spilled
    asm volatile("" : "+v"(tl));
    for (int p = tl; p < count; p += 256) {
      sm.pos[p] = col[start + p];
      sm.sl[p] = slot[start + p];
    }
    {
      RowStage<DH> ks;
      RowStage<DI> kis;
      ks.load(K, r, H_kv, (int64_t)b * kBlock, Nk, tl);
      kis.load(k_idx, r, H_kv, (int64_t)b * kBlock, Nk, tl);
      ks.store(sm.k, tl);
      kis.store(sm.ki, tl);
    }
    __syncthreads();
    const int ll = tl & 63;
    kl_item<DH, DI>(sm, Q, q_idx, lse, count, wave, r, b, G, H_q, H_kv, k, q_start, scale_log2,
                    part, ll >> 5, ll & 31);
    __syncthreads();  // LDS and `next` are reused by the next item
  }
}

// Per (query, group): the selection's slots in ascending order,
//   KL = sum_s A_s - sum_s B_s + ln sum_s exp(L_s).
__global__ __launch_bounds__(256) void kl_merge_kernel(const float* __restrict__ part,
                                                       int64_t q_start, int64_t Nq, int H_kv,
                                                       int k, float* __restrict__ kl) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;  // iq * H_kv + r
  if (u >= Nq * H_kv) return;
  const int64_t i = q_start + u / H_kv;
  const int n_sel = (int)min((int64_t)k, i / kBlock + 1);
  const float* ps = part + u * k * 3;
  float A = 0.f, B = 0.f, M = -INFINITY;
  for (int s = 0; s < n_sel; ++s) {
    A += ps[3 * s];
    B += ps[3 * s + 1];
    M = fmaxf(M, ps[3 * s + 2]);
  }
  float Z = 0.f;
  for (int s = 0; s < n_sel; ++s) Z += __expf(ps[3 * s + 2] - M);
  kl[u] = A - B + (M + __logf(Z));
}

// Deterministic sum of n values: work-group w adds elements
// [w*4096, (w+1)*4096) in a fixed tree into sums[w]; then one work-group
// adds sums[0..nw) in the same fixed way into *out.
__device__ __forceinline__ double block_sum_f64(double v) {
  __shared__ double red[256];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(256) void sum_stage1_kernel(const float* __restrict__ x, int64_t n,
                                                         double* __restrict__ sums) {
  const int64_t base = (int64_t)blockIdx.x * 4096;
  double v = 0.0;
  for (int e = 0; e < 16; ++e) {
    const int64_t idx = base + threadIdx.x * 16 + e;
    if (idx < n) v += (double)x[idx];
  }
  const double s = block_sum_f64(v);
  if (threadIdx.x == 0) sums[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void sum_stage2_kernel(const double* __restrict__ sums,
                                                         int64_t nw, double* __restrict__ out) {
  double v = 0.0;
  for (int64_t idx = threadIdx.x; idx < nw; idx += 256) v += sums[idx];
  const double s = block_sum_f64(v);
  if (threadIdx.x == 0) *out = s;
}

int64_t kl_sum_partials(int64_t n) { return ceil_div(n, (int64_t)4096); }

static bool kl_lds_ready = false;

template <int DH, int DI>
static hipError_t allow_kl_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&kl_kv_outer_kernel<DH, DI>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)sizeof(KlSmem<DH, DI>));
}

template <int DH, int DI>
static hipError_t launch_kl_dd(const __bf16* q, const __bf16* kk, const __bf16* qi,
                               const __bf16* ki, const float* lse, const int32_t* col,
                               const uint8_t* slot, const int4* items, int32_t* n_items,
                               int64_t max_items, int64_t q_start, int64_t Nk, int H_q, int H_kv,
                               int nblk, int k, float scale_log2, float* part,
                               hipStream_t stream) {
  const int G = H_q / H_kv;
  // persistent: two resident work-groups per CU
  dim3 grid((unsigned)std::min<int64_t>(max_items, 2 * (int64_t)device_cus())), block(256);
  kl_kv_outer_kernel<DH, DI><<<grid, block, sizeof(KlSmem<DH, DI>), stream>>>(
      q, kk, qi, ki, lse, col, slot, items, n_items, q_start, Nk, H_q, H_kv, G, nblk, k,
      scale_log2, part);
  return hipGetLastError();
}

template <int DH>
static hipError_t launch_kl_d(int d_idx, const __bf16* q, const __bf16* kk, const __bf16* qi,
                              const __bf16* ki, const float* lse, const int32_t* col,
                              const uint8_t* slot, const int4* items, int32_t* n_items,
                              int64_t max_items, int64_t q_start, int64_t Nk, int H_q, int H_kv,
                              int nblk, int k, float scale_log2, float* part,
                              hipStream_t stream) {
  switch (d_idx) {
    case 32:
      return launch_kl_dd<DH, 32>(q, kk, qi, ki, lse, col, slot, items, n_items, max_items,
                                  q_start, Nk, H_q, H_kv, nblk, k, scale_log2, part, stream);
    case 64:
      return launch_kl_dd<DH, 64>(q, kk, qi, ki, lse, col, slot, items, n_items, max_items,
                                  q_start, Nk, H_q, H_kv, nblk, k, scale_log2, part, stream);
    case 128:
      return launch_kl_dd<DH, 128>(q, kk, qi, ki, lse, col, slot, items, n_items, max_items,
                                   q_start, Nk, H_q, H_kv, nblk, k, scale_log2, part, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_index_kl(const void* Q, const void* K, const void* q_idx, const void* k_idx,
                           const float* lse, const int32_t* col, const uint8_t* slot,
                           const int4* items, int32_t* n_items, int64_t max_items,
                           int64_t q_start, int64_t Nq, int64_t Nk, int H_q, int H_kv, int d_h,
                           int d_idx, int nblk, int k, float scale, float* part, float* kl,
                           double* sums, double* kl_sum, hipStream_t stream) {
  if (!kl_lds_ready) {
    hipError_t e = allow_kl_lds<128, 32>();
    if (e == hipSuccess) e = allow_kl_lds<128, 64>();
    if (e == hipSuccess) e = allow_kl_lds<128, 128>();
    if (e == hipSuccess) e = allow_kl_lds<64, 32>();
    if (e == hipSuccess) e = allow_kl_lds<64, 64>();
    if (e == hipSuccess) e = allow_kl_lds<64, 128>();
    if (e != hipSuccess) return e;
    kl_lds_ready = true;
  }
  const float scale_log2 = scale * kLog2e;
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* qi = static_cast<const __bf16*>(q_idx);
  auto* ki = static_cast<const __bf16*>(k_idx);
  hipError_t e;
  if (d_h == 128)
    e = launch_kl_d<128>(d_idx, q, kk, qi, ki, lse, col, slot, items, n_items, max_items, q_start,
                         Nk, H_q, H_kv, nblk, k, scale_log2, part, stream);
  else if (d_h == 64)
    e = launch_kl_d<64>(d_idx, q, kk, qi, ki, lse, col, slot, items, n_items, max_items, q_start,
                        Nk, H_q, H_kv, nblk, k, scale_log2, part, stream);
  else
    e = hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int64_t rows = Nq * H_kv;
  kl_merge_kernel<<<(unsigned)ceil_div(rows, (int64_t)256), 256, 0, stream>>>(part, q_start, Nq,
                                                                              H_kv, k, kl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (kl_sum) {
    const int64_t nw = kl_sum_partials(rows);
    sum_stage1_kernel<<<(unsigned)nw, 256, 0, stream>>>(kl, rows, sums);
    sum_stage2_kernel<<<1, 256, 0, stream>>>(sums, nw, kl_sum);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace msa
