// Decode: one new query per sequence, at the last cache row, so it sees the
// whole cache and its local block is the last block.  Same Index Branch and
// Main Branch as the prefill row ("MiniMax Sparse Attention" explainer,
// section 02 and Figure 1 caption; the pages report a decode speed-up in
// Figure 4 without a kernel design).  Layout Q-outer, split-K:
//   (1) split scan of k_idx: every wavefront scores a run of blocks against
//       the sequence's index query and max-pools them (HBM streaming);
//   (2) exp-free Top-k over the pooled row (shared Top-k kernel);
//   (3) one work-group per (sequence, group, selected block): exact softmax
//       of the G heads over that block -> fp32 partial (O_s, lse_s);
//   (4) merge of the k partials in ascending block order through their
//       log-sum-exp.
#include "common.h"
#include "lds_rows.h"
#include "msa_internal.h"

namespace msa {

// (1) Split scan.  A wavefront streams one 128-token block at a time as
// contiguous 1 KiB loads (lane l takes elements 8l..8l+7 of every KiB), so
// each load instruction is fully coalesced.  Those 8 values belong to one
// (token, group) segment of D values held by D/8 consecutive lanes: a
// partial dot product in-lane (bf16 dot2), the segment sum by xor-shuffles,
// then a running max over the block's tokens.  Requires H_kv * D to divide
// 512 (a KiB holds whole tokens).  Only blocks before the local block.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float dot8(bf16x8 x, const bf16x2 (&q)[4]) {
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bf16x2 xp = {x[2 * p], x[2 * p + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(xp, q[p], s, false);
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(256) void decode_scan_kernel(const __bf16* __restrict__ q_idx,
                                                          const __bf16* __restrict__ k_idx,
                                                          int64_t N, int H_kv, int nblk,
                                                          int blocks_per_wave,
                                                          float* __restrict__ P, int64_t ldp) {
  constexpr int SEG = D / 8;  // lanes per (token, group) segment
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int TE = H_kv * D;          // elements per token
  const int e_lane = 8 * lane;
  const int r = (e_lane % TE) / D, d0 = e_lane % D;
  bf16x2 q[4];
  {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(q_idx + ((int64_t)b * H_kv + r) * D + d0);
#pragma unroll
    for (int p = 0; p < 4; ++p) q[p] = bf16x2{x[2 * p], x[2 * p + 1]};
  }
  const __bf16* kseq = k_idx + (int64_t)b * N * TE + e_lane;
  const int iters = kBlock * TE / 512;  // KiB loads per block (a multiple of 8)
  const int nb_scan = nblk - 1;        // non-local blocks
  const int blk0 = ((int)blockIdx.x * 4 + wave) * blocks_per_wave;
  const int blk1 = min(nb_scan, blk0 + blocks_per_wave);
  for (int blk = blk0; blk < blk1; ++blk) {
    const __bf16* base = kseq + (int64_t)blk * kBlock * TE;
    float m = -INFINITY;
    for (int u0 = 0; u0 < iters; u0 += 8) {
      // the cache's index keys are read exactly once: non-temporal loads
      // (measured 5.7 -> 6.5 TB/s on the 32 x 1M scan)
      bf16x8 x[8];
#pragma unroll
      for (int v = 0; v < 8; ++v)
        x[v] = __builtin_nontemporal_load(
            reinterpret_cast<const bf16x8*>(base + (int64_t)512 * (u0 + v)));
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        float s = dot8(x[v], q);
#pragma unroll
        for (int o = 1; o < SEG; o <<= 1) s += __shfl_xor(s, o, kWave);
        m = fmaxf(m, s);
      }
    }
    // lanes at the same offset inside a token hold the same group
    for (int o = TE / 8; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if (lane < TE / 8 && lane % SEG == 0) P[((int64_t)b * H_kv + r) * ldp + blk] = m;
  }
}

// (3) Partial attention of the G heads of group r over one selected block:
// one work-group per (sequence, group, selected block).  The block's K and V
// are staged in LDS with coalesced 16-byte loads (K rows XOR-swizzled by
// 16-byte chunk, so 16 lanes reading 16 consecutive rows at one chunk hit
// distinct banks), q in fp32.  Scores: thread (key = t % 128, half = t / 128)
// takes heads half, half + 2, ...; softmax: one wave per head; PV: thread
// (d pair, head group) accumulates up to four heads per pass, reading each
// V pair once for all of them.
template <int DH>
__global__ __launch_bounds__(256) void decode_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ sel, int64_t N, int H_q, int H_kv, int k, float scale_log2,
    float* __restrict__ Opart, float* __restrict__ lse_part) {
  constexpr int CH = DH / 8;            // 16-byte chunks per row
  constexpr int LD = kBlock * CH / 256;  // chunks of K (and of V) per thread
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  __bf16* ks = reinterpret_cast<__bf16*>(dsm);           // [128][DH], swizzled
  __bf16* vs = ks + kBlock * DH;                           // [128][DH]
  float* qs = reinterpret_cast<float*>(vs + kBlock * DH);  // [G][DH]
  const int s_id = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int G = H_q / H_kv;
  // Scores [G][128] fp32: over K once K is scored when one pass covers every
  // head (G <= 16), else after q.
  constexpr int HB = 8;  // heads per scoring pass per thread (two thread halves)
  const bool alias = G <= 2 * HB;
  float* ss = alias ? reinterpret_cast<float*>(dsm) : qs + G * DH;
  const int32_t blk = sel[((int64_t)b * H_kv + r) * k + s_id];
  if (blk < 0) return;
  const int t = threadIdx.x;
  const int64_t key0 = (int64_t)blk * kBlock;
  const __bf16* Kb = K + (int64_t)b * N * H_kv * DH;
  const __bf16* Vb = V + (int64_t)b * N * H_kv * DH;
  {
    // every load of the block is issued before the first LDS store
    bf16x8 kx[LD], vx[LD];
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int id = t + 256 * u, row = id / CH, c = id % CH;
      const int64_t j = key0 + row;
      kx[u] = vx[u] = bf16x8{};
      if (j < N) {
        kx[u] = *reinterpret_cast<const bf16x8*>(Kb + (j * H_kv + r) * DH + 8 * c);
        vx[u] = *reinterpret_cast<const bf16x8*>(Vb + (j * H_kv + r) * DH + 8 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int id = t + 256 * u, row = id / CH, c = id % CH;
      *reinterpret_cast<bf16x8*>(ks + row * DH + 8 * (c ^ row_swz<DH>(row))) = kx[u];
      *reinterpret_cast<bf16x8*>(vs + row * DH + 8 * c) = vx[u];
    }
  }
  for (int e = t; e < G * CH; e += 256) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(q + ((int64_t)b * H_q + r * G) * DH + 8 * e);
#pragma unroll
    for (int u = 0; u < 8; ++u) qs[8 * e + u] = bf2f(x[u]);
  }
  __syncthreads();

  // ---- scores ----------------------------------------------------------------
  {
    const int key = t & (kBlock - 1), half = t >> 7;
    const bool valid = key0 + key < N;
    float sc[HB];
    for (int h0 = half; h0 < G; h0 += 2 * HB) {
#pragma unroll
      for (int j = 0; j < HB; ++j) sc[j] = 0.f;
      for (int c = 0; c < CH; ++c) {
        const bf16x8 kx =
            *reinterpret_cast<const bf16x8*>(ks + key * DH + 8 * (c ^ row_swz<DH>(key)));
        float kf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kf[u] = bf2f(kx[u]);
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          const int h = h0 + 2 * j;
          if (h < G) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(qs + h * DH + 8 * c);
            const f32x4 d = *reinterpret_cast<const f32x4*>(qs + h * DH + 8 * c + 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              sc[j] = fmaf(a[u], kf[u], sc[j]);
              sc[j] = fmaf(d[u], kf[4 + u], sc[j]);
            }
          }
        }
      }
      if (!alias) {
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          const int h = h0 + 2 * j;
          if (h < G) ss[h * kBlock + key] = valid ? sc[j] * scale_log2 : -INFINITY;
        }
      }
    }
    if (alias) {  // one pass: wait until every thread is done reading K
      __syncthreads();
      if (half < G) {
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          const int h = half + 2 * j;
          if (h < G) ss[h * kBlock + key] = valid ? sc[j] * scale_log2 : -INFINITY;
        }
      }
    }
  }
  __syncthreads();
  // ---- softmax per head (one wave per head), probabilities in place --------
  const int wave = t >> 6, lane = t & 63;
  for (int hh = wave; hh < G; hh += 4) {
    float* row = ss + hh * kBlock;
    const float a = row[lane], c = row[lane + 64];
    const float m = wave_max_f32(fmaxf(a, c));
    const float pa = exp2f(a - m), pc = exp2f(c - m);
    const float l = wave_sum_f32(pa + pc);
    row[lane] = pa / l;
    row[lane + 64] = pc / l;
    if (lane == 0)
      lse_part[(((int64_t)b * H_q + r * G + hh) * k) + s_id] = (m + log2f(l)) * 0.69314718055994531f;
  }
  __syncthreads();
  // ---- O_s[h][d] = sum_key p[h][key] V[key][d] -------------------------------
  {
    constexpr int NDP = DH / 2;      // d pairs
    constexpr int NHG = 256 / NDP;   // head groups
    constexpr int HP = 4;            // heads per pass per thread
    const int dp = t % NDP, hg = t / NDP;
    for (int h0 = hg; h0 < G; h0 += NHG * HP) {
      float a0[HP], a1[HP];
#pragma unroll
      for (int j = 0; j < HP; ++j) a0[j] = a1[j] = 0.f;
      for (int key = 0; key < kBlock; key += 4) {
        float v0[4], v1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vs + (key + u) * DH + 2 * dp);
          v0[u] = __uint_as_float(w << 16);
          v1[u] = __uint_as_float(w & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < HP; ++j) {
          const int h = h0 + NHG * j;
          if (h < G) {
            const f32x4 p = *reinterpret_cast<const f32x4*>(ss + h * kBlock + key);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              a0[j] = fmaf(p[u], v0[u], a0[j]);
              a1[j] = fmaf(p[u], v1[u], a1[j]);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < HP; ++j) {
        const int h = h0 + NHG * j;
        if (h < G) {
          float* dst = Opart + (((int64_t)b * H_q + r * G + h) * k + s_id) * DH + 2 * dp;
          *reinterpret_cast<float2*>(dst) = float2{a0[j], a1[j]};
        }
      }
    }
  }
}

// (4) merge in ascending slot order.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ Opart,
                                                           const float* __restrict__ lse_part,
                                                           int H_q, int d_h, int k, int n_sel,
                                                           float* __restrict__ O,
                                                           float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;  // b * H_q + h
  const float* ls = lse_part + bh * k;
  float M = -INFINITY;
  for (int s = 0; s < n_sel; ++s) M = fmaxf(M, ls[s]);
  float den = 0.f;
  for (int s = 0; s < n_sel; ++s) den += __expf(ls[s] - M);
  for (int d = threadIdx.x; d < d_h; d += 256) {
    float acc = 0.f;
    for (int s = 0; s < n_sel; ++s)
      acc += __expf(ls[s] - M) * Opart[(bh * k + s) * d_h + d];
    O[bh * d_h + d] = acc / den;
  }
  if (lse && threadIdx.x == 0) lse[bh] = M + __logf(den);
}

hipError_t launch_decode_scan(const void* q_idx, const void* k_idx, int B, int64_t N, int H_kv,
                              int d_idx, int nblk, float* P, int64_t ldp, hipStream_t stream) {
  const int bpw = 4;
  const int waves = (int)ceil_div(max(nblk - 1, 1), bpw);
  dim3 grid((unsigned)ceil_div(waves, 4), B), block(256);
  auto* qi = static_cast<const __bf16*>(q_idx);
  auto* ki = static_cast<const __bf16*>(k_idx);
  switch (d_idx) {
    case 32:
      decode_scan_kernel<32><<<grid, block, 0, stream>>>(qi, ki, N, H_kv, nblk, bpw, P, ldp);
      break;
    case 64:
      decode_scan_kernel<64><<<grid, block, 0, stream>>>(qi, ki, N, H_kv, nblk, bpw, P, ldp);
      break;
    case 128:
      decode_scan_kernel<128><<<grid, block, 0, stream>>>(qi, ki, N, H_kv, nblk, bpw, P, ldp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_attn(const void* q, const void* K, const void* V, const int32_t* sel,
                              int B, int64_t N, int H_q, int H_kv, int d_h, int k, float scale,
                              float* Opart, float* lse_part, hipStream_t stream) {
  const int G = H_q / H_kv;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(k, H_kv, B), block(256);
  // K, V, q and (when they do not go over K) the scores
  const size_t lds = 2 * sizeof(__bf16) * kBlock * d_h + sizeof(float) * (size_t)G * d_h +
                     (G <= 16 ? 0 : sizeof(float) * (size_t)G * kBlock);
  static bool lds_ready = false;  // up to 128 KiB (G = 64): above the default 64 KiB
  if (!lds_ready) {
    const size_t most = 2 * sizeof(__bf16) * kBlock * 128 + sizeof(float) * 64 * (128 + kBlock);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_attn_kernel<128>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_attn_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e != hipSuccess) return e;
    lds_ready = true;
  }
  auto* qq = static_cast<const __bf16*>(q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* vv = static_cast<const __bf16*>(V);
  if (d_h == 128)
    decode_attn_kernel<128><<<grid, block, lds, stream>>>(qq, kk, vv, sel, N, H_q, H_kv, k,
                                                          scale_log2, Opart, lse_part);
  else if (d_h == 64)
    decode_attn_kernel<64><<<grid, block, lds, stream>>>(qq, kk, vv, sel, N, H_q, H_kv, k,
                                                         scale_log2, Opart, lse_part);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(const float* Opart, const float* lse_part, int B, int H_q,
                               int d_h, int k, int n_sel, float* O, float* lse,
                               hipStream_t stream) {
  decode_merge_kernel<<<(unsigned)((int64_t)B * H_q), 256, 0, stream>>>(Opart, lse_part, H_q,
                                                                         d_h, k, n_sel, O, lse);
  return hipGetLastError();
}

}  // namespace msa
