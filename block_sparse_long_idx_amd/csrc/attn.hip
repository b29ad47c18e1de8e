// Main Branch, KV-outer ("MiniMax Sparse Attention" explainer, section 05
// part 2): each KV block is loaded once per work item and the queries that
// selected it are gathered through the inverted index; G heads x several
// query positions are packed into one 128-row MFMA tile (query
// concatenation); hot blocks are cut along the query dimension into work
// items planned before launch (pre-scheduled chunking); each (query, head,
// block) partial goes to a pre-assigned slot and a combine kernel merges
// the slots through their log-sum-exp (two-phase forward).
//
// Partial precision: non-local blocks store O_s in bf16 (the pages' IO
// accounting is bf16) with lse_s in fp32; the local block -- the only one
// with a causal mask and the only one for rows i < 128, where few tokens can
// make |O| large -- is computed with a hi/lo split of P and stored in fp32.
#include "common.h"
#include "msa_internal.h"

namespace msa {

// ---------------------------------------------------------------------------
// Work list.  Bucket (r, b) of the CSR holds first the queries whose local
// block is b (positions inside block b, all of which select it), then the
// queries that picked b as a non-local block.  Items: one "local" item for
// the first part, then non-local items of at most `chunk` positions.
// Item = {bucket, start offset into col, count, is_local}.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bucket_items(int64_t bucket, const int32_t* row_ptr, int nblk,
                                             int64_t q_start, int64_t Nq, int chunk,
                                             int32_t& n_loc, int32_t& n_non, int32_t& items) {
  const int b = (int)(bucket % nblk);
  const int32_t cnt = row_ptr[bucket + 1] - row_ptr[bucket];
  const int64_t lo = max(q_start, (int64_t)b * kBlock);
  const int64_t hi = min(q_start + Nq, (int64_t)(b + 1) * kBlock);
  n_loc = hi > lo ? (int32_t)(hi - lo) : 0;
  n_non = cnt - n_loc;
  items = (n_loc > 0) + (n_non + chunk - 1) / chunk;
}

__global__ __launch_bounds__(1024) void build_items_kernel(const int32_t* __restrict__ row_ptr,
                                                           int64_t nb, int nblk, int64_t q_start,
                                                           int64_t Nq, int chunk,
                                                           int4* __restrict__ items,
                                                           int32_t* __restrict__ n_items) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(nb, 1024);
  const int64_t lo = min(nb, per * t), hi = min(nb, per * (t + 1));
  int32_t s = 0;
  for (int64_t x = lo; x < hi; ++x) {
    int32_t a, c, it;
    bucket_items(x, row_ptr, nblk, q_start, Nq, chunk, a, c, it);
    s += it;
  }
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t pos = t ? part[t - 1] : 0;
  for (int64_t x = lo; x < hi; ++x) {
    int32_t n_loc, n_non, it;
    bucket_items(x, row_ptr, nblk, q_start, Nq, chunk, n_loc, n_non, it);
    int32_t start = row_ptr[x];
    if (n_loc > 0) {
      items[pos++] = make_int4((int)x, start, n_loc, 1);
      start += n_loc;
    }
    for (int32_t done = 0; done < n_non; done += chunk) {
      items[pos++] = make_int4((int)x, start + done, min(chunk, n_non - done), 0);
    }
  }
  if (t == 1023) *n_items = part[1023];
}

// ---------------------------------------------------------------------------
// Partial attention of one work item.
//
// LDS: K block row-major [128][DH] (16-byte chunks XOR-swizzled by row) and
// V block transposed [DH][128 + 4] (rows padded by 8 bytes, so the 32 rows a
// wave reads at one key offset spread over the banks; the padding keeps
// every V^T address a per-lane base plus a compile-time offset).
// Each wave takes 32-row tiles; row R of the item = (position R / G, head
// R % G of the group).  S^T = K . Q^T puts keys on MFMA rows so every lane
// holds 16 keys of one row (row = lane % 32): the row max/sum are in-lane
// plus one swap of lane halves.  O^T = V^T . P^T keeps the row on the lane,
// so the 1/l normalisation is in-lane as well.
// ---------------------------------------------------------------------------
constexpr int kVtPitch = kBlock + 4;  // elements per V^T row

template <int DH>
struct AttnSmem {
  __bf16 k[kBlock * DH];
  __bf16 vt[DH * kVtPitch];
};

__device__ __forceinline__ int vt_off(int d, int key) { return d * kVtPitch + key; }

// One 32-row tile of a work item (rows = (position, head) pairs).
template <int DH, bool LOCAL>
__device__ __forceinline__ void attn_tile(const AttnSmem<DH>& sm, const __bf16* __restrict__ Q,
                                          const int32_t* __restrict__ col,
                                          const uint8_t* __restrict__ slot, int start, int nrows,
                                          int tile, int r, int G, int H_q, int k, int64_t key0,
                                          int64_t q_start, float scale_log2,
                                          __bf16* __restrict__ Os, float* __restrict__ lse_s,
                                          float* __restrict__ Oloc, int h, int n) {
  constexpr int S = DH / 16;    // k-steps of the QK^T MFMA chain
  constexpr int NDG = DH / 32;  // 32-wide d groups of O
  // ---- gather this lane's row: position, head, slot -------------------------
  const int R = tile * 32 + n;
  const bool row_ok = R < nrows;
  int64_t pos = 0;
  int hq = 0, sl = 0;
  if (row_ok) {
    const int p = R / G;
    pos = col[start + p];
    sl = slot[start + p];
    hq = r * G + R % G;
  }

  // ---- S^T = K . Q^T: 4 groups of 32 keys ------------------------------------
  f32x16 sacc[4];
  {
    bf16x8 qb[S];
    const __bf16* qrow = Q + (pos * H_q + hq) * DH + (DH / 2) * h;
#pragma unroll
    for (int s = 0; s < S; ++s)
      qb[s] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 8 * s) : bf16x8{};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sacc[g] = f32x16{};
      const int krow = 32 * g + n;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &sm.k[krow * DH + 8 * (((DH / 16) * h + s) ^ (krow & 7))]);
        sacc[g] = mfma32(a, qb[s], sacc[g]);
      }
      __builtin_amdgcn_sched_barrier(0);  // bound the LDS reads in flight
    }
  }

  // ---- softmax over the block (scale folded into exp2) ---------------------
  if (LOCAL) {
    // key 32g + acc_row(j, h) is visible iff it is <= pos - key0; acc_row
    // is 4h plus a constant, so compare the constant with a per-lane limit.
    const int lim = (row_ok ? (int)(pos - key0) : kBlock - 1) - 4 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (32 * g + acc_row(j, 0) > lim) sacc[g][j] = -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, sacc[g][j]);
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  const float mb = m * scale_log2;

  // ---- O^T = V^T . P^T, P formed one 16-key step at a time ----------------
  // P^T operand of step (g, u): MFMA k-index 8h'+e is key 32g+16u+4h'+e
  // (e < 4) or 32g+16u+8+4h'+(e-4), which is accumulator 8u+e of sacc[g].
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
        if (LOCAL) plo[e] = f2bf(p - bf2f(phi[e]));
      }
      const int kb0 = 32 * g + 16 * u + 4 * h;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        const int d = 32 * dg + n;
        const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(&sm.vt[vt_off(d, kb0)]);
        const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(&sm.vt[vt_off(d, kb0 + 8)]);
        const bf16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        oacc[dg] = mfma32(a, phi, oacc[dg]);
        if (LOCAL) oacc[dg] = mfma32(a, plo, oacc[dg]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  l += __shfl_xor(l, 32, kWave);

  // ---- write the partial ----------------------------------------------------
  if (!row_ok) return;
  const float inv = 1.f / l;
  const int64_t iq = pos - q_start;
  if (LOCAL) {
    float* dst = Oloc + (iq * H_q + hq) * DH;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(dst + 32 * dg + 8 * qd + 4 * h) =
            f32x4{oacc[dg][4 * qd] * inv, oacc[dg][4 * qd + 1] * inv,
                  oacc[dg][4 * qd + 2] * inv, oacc[dg][4 * qd + 3] * inv};
  } else {
    __bf16* dst = Os + ((iq * (k - 1) + sl) * H_q + hq) * DH;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<bf16x4*>(dst + 32 * dg + 8 * qd + 4 * h) =
            bf16x4{f2bf(oacc[dg][4 * qd] * inv), f2bf(oacc[dg][4 * qd + 1] * inv),
                   f2bf(oacc[dg][4 * qd + 2] * inv), f2bf(oacc[dg][4 * qd + 3] * inv)};
  }
  if (h == 0) lse_s[(iq * k + sl) * H_q + hq] = (mb + log2f(l)) * 0.69314718055994531f;
}

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_kv_outer_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ items, const int32_t* __restrict__ n_items, int64_t q_start,
    int64_t Nk, int H_q, int H_kv, int G, int nblk, int k, float scale_log2,
    __bf16* __restrict__ Os, float* __restrict__ lse_s, float* __restrict__ Oloc) {
  constexpr int CH = DH / 8;  // 16-byte chunks per K row
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnSmem<DH>& sm = *reinterpret_cast<AttnSmem<DH>*>(smem_raw);

  const int item_id = blockIdx.x;
  if (item_id >= *n_items) return;
  const int4 it = items[item_id];
  const int bucket = it.x, start = it.y, count = it.z;
  const bool local = it.w != 0;
  const int r = bucket / nblk, b = bucket % nblk;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int h = lane >> 5, n = lane & 31;
  const int64_t key0 = (int64_t)b * kBlock;

  // ---- stage K (row-major, swizzled) and V^T --------------------------------
  for (int id = t; id < kBlock * CH; id += 256) {
    const int row = id / CH, c = id % CH;
    bf16x8 v = {};
    if (key0 + row < Nk)
      v = *reinterpret_cast<const bf16x8*>(K + ((key0 + row) * H_kv + r) * DH + 8 * c);
    *reinterpret_cast<bf16x8*>(&sm.k[row * DH + 8 * (c ^ (row & 7))]) = v;
  }
  for (int id = t; id < (kBlock / 4) * CH; id += 256) {
    const int kq = id % (kBlock / 4), c = id / (kBlock / 4);  // 4 keys x 8 d
    bf16x8 rows[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t key = key0 + 4 * kq + u;
      rows[u] = key < Nk ? *reinterpret_cast<const bf16x8*>(V + (key * H_kv + r) * DH + 8 * c)
                         : bf16x8{};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 w = {rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
      *reinterpret_cast<bf16x4*>(&sm.vt[vt_off(8 * c + e, 4 * kq)]) = w;
    }
  }
  __syncthreads();

  const int nrows = count * G;
  const int ntile = (nrows + 31) / 32;
  for (int tile = wave; tile < ntile; tile += 4) {
    if (local)
      attn_tile<DH, true>(sm, Q, col, slot, start, nrows, tile, r, G, H_q, k, key0, q_start,
                          scale_log2, Os, lse_s, Oloc, h, n);
    else
      attn_tile<DH, false>(sm, Q, col, slot, start, nrows, tile, r, G, H_q, k, key0, q_start,
                           scale_log2, Os, lse_s, Oloc, h, n);
  }
}

// ---------------------------------------------------------------------------
// Combine: for each (position, head) merge its n_sel = min(k, lb+1) partials
// in ascending slot order (= ascending block; the local block is last):
//   M = max lse_s, w_s = exp(lse_s - M), O = sum w_s O_s / sum w_s,
//   lse = M + ln sum w_s.
// One work-group per position; 4 threads per head, DH/4 dims each.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void combine_kernel(const __bf16* __restrict__ Os,
                                                      const float* __restrict__ lse_s,
                                                      const float* __restrict__ Oloc,
                                                      int64_t q_start, int H_q, int k,
                                                      float* __restrict__ O,
                                                      float* __restrict__ lse) {
  constexpr int DQ = DH / 4;
  const int64_t iq = blockIdx.x;
  const int64_t i = q_start + iq;
  const int n_sel = (int)min((int64_t)k, i / kBlock + 1);
  for (int hq = threadIdx.x / 4; hq < H_q; hq += 64) {
    const int d0 = (threadIdx.x & 3) * DQ;
    const float* ls = lse_s + iq * k * H_q + hq;
    float M = -INFINITY;
    for (int s = 0; s < n_sel; ++s) M = fmaxf(M, ls[(int64_t)s * H_q]);
    float acc[DQ];
#pragma unroll
    for (int d = 0; d < DQ; ++d) acc[d] = 0.f;
    float den = 0.f;
    for (int s = 0; s < n_sel - 1; ++s) {
      const float w = __expf(ls[(int64_t)s * H_q] - M);
      den += w;
      const __bf16* src = Os + ((iq * (k - 1) + s) * H_q + hq) * DH + d0;
#pragma unroll
      for (int v = 0; v < DQ / 8; ++v) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(src + 8 * v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * v + e] += w * bf2f(x[e]);
      }
    }
    {
      const float w = __expf(ls[(int64_t)(n_sel - 1) * H_q] - M);
      den += w;
      const float* src = Oloc + (iq * H_q + hq) * DH + d0;
#pragma unroll
      for (int v = 0; v < DQ / 4; ++v) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * v + e] += w * x[e];
      }
    }
    const float inv = 1.f / den;
    float* dst = O + (iq * H_q + hq) * DH + d0;
#pragma unroll
    for (int v = 0; v < DQ / 4; ++v)
      *reinterpret_cast<f32x4*>(dst + 4 * v) =
          f32x4{acc[4 * v] * inv, acc[4 * v + 1] * inv, acc[4 * v + 2] * inv,
                acc[4 * v + 3] * inv};
    if (lse && (threadIdx.x & 3) == 0) lse[iq * H_q + hq] = M + __logf(den);
  }
}

int64_t attn_max_items(int64_t nb, int64_t nnz, int chunk) {
  return 2 * nb + nnz / chunk + 1;
}

hipError_t launch_build_items(const int32_t* row_ptr, int64_t nb, int nblk, int64_t q_start,
                              int64_t Nq, int chunk, int4* items, int32_t* n_items,
                              hipStream_t stream) {
  build_items_kernel<<<1, 1024, 0, stream>>>(row_ptr, nb, nblk, q_start, Nq, chunk, items,
                                             n_items);
  return hipGetLastError();
}

static bool attn_lds_ready = false;

hipError_t attn_prepare() {
  // The d_h = 128 kernel needs a little over 64 KiB of LDS per work-group.
  if (attn_lds_ready) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kv_outer_kernel<128>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)sizeof(AttnSmem<128>));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kv_outer_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(AttnSmem<64>));
  if (e == hipSuccess) attn_lds_ready = true;
  return e;
}

hipError_t launch_attn(const void* Q, const void* K, const void* V, const int32_t* col,
                       const uint8_t* slot, const int4* items, const int32_t* n_items,
                       int64_t max_items, int64_t q_start, int64_t Nk, int H_q, int H_kv,
                       int d_h, int nblk, int k, float scale, void* Os, float* lse_s,
                       float* Oloc, hipStream_t stream) {
  hipError_t e = attn_prepare();
  if (e != hipSuccess) return e;
  const int G = H_q / H_kv;
  const float scale_log2 = scale * 1.4426950408889634f;
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* v = static_cast<const __bf16*>(V);
  auto* os = static_cast<__bf16*>(Os);
  dim3 grid((unsigned)max_items), block(256);
  if (d_h == 128)
    attn_kv_outer_kernel<128><<<grid, block, sizeof(AttnSmem<128>), stream>>>(q, kk, v, col, slot, items, n_items,
                                                          q_start, Nk, H_q, H_kv, G, nblk, k,
                                                          scale_log2, os, lse_s, Oloc);
  else if (d_h == 64)
    attn_kv_outer_kernel<64><<<grid, block, sizeof(AttnSmem<64>), stream>>>(q, kk, v, col, slot, items, n_items,
                                                         q_start, Nk, H_q, H_kv, G, nblk, k,
                                                         scale_log2, os, lse_s, Oloc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine(const void* Os, const float* lse_s, const float* Oloc,
                          int64_t q_start, int64_t Nq, int H_q, int d_h, int k, float* O,
                          float* lse, hipStream_t stream) {
  auto* os = static_cast<const __bf16*>(Os);
  if (d_h == 128)
    combine_kernel<128><<<(unsigned)Nq, 256, 0, stream>>>(os, lse_s, Oloc, q_start, H_q, k, O,
                                                          lse);
  else if (d_h == 64)
    combine_kernel<64><<<(unsigned)Nq, 256, 0, stream>>>(os, lse_s, Oloc, q_start, H_q, k, O,
                                                         lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
