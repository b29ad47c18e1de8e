// Index Branch front-end ("MiniMax Sparse Attention" explainer, Figure 1
// caption: the hidden states pass a linear projection and then "Norm &
// RoPE" to give the light-weight Q^idx and K^idx; section 06: the model's
// RoPE width is 64).  For token i at position pos0 + i and GQA group r:
//   y = hidden[i] . W[r*d_idx .. (r+1)*d_idx)^T          (fp32 accumulation)
//   y = y * gamma / sqrt(mean(y^2) + eps)                (RMS norm per group)
//   (y_j, y_{j+R/2}) turned by pos * theta^(-2j/R), j < R/2, R = rope_dim
// and stored as bf16.  The pages name the norm and RoPE without fixing
// their form; these are the plain readings (rotate-half pairing).
//
// One MFMA GEMM per projection with the norm and rotation in its epilogue:
// a work-group computes 256 rows x 256 output columns (eight waves, 64 x
// 128 each, two per SIMD), staging 64-wide slabs of the contraction in LDS by direct
// global->LDS loads (two buffers, 16-byte chunks XOR-swizzled by row pair).  The
// q and k work-groups of one row tile run on the same XCD, so the second
// read of those hidden rows hits that XCD's L2.  Angles are reduced to a
// fraction of a turn in fp64 before the hardware sine and cosine, so large
// positions keep their accuracy.
#include "common.h"
#include "msa_internal.h"

#include <type_traits>

namespace msa {

namespace {

constexpr int NWR = 4;                    // waves along the rows (x 2 along the columns)
constexpr int FM = 64 * NWR, FN = 256, FK = 64;

struct FeSmem {
  __bf16 a[2][FM * FK];  // hidden rows [row][64]
  __bf16 b[2][FN * FK];  // weight rows (output columns) [col][64]
};

// The 16-byte chunks of a 128-byte slab row sit XOR-swizzled by
// (row >> 1) & 7: two rows share a 256-byte bank row, and a fragment read
// serves 16 consecutive rows at a time, so (row parity, swizzled chunk)
// must differ across them (swizzling by row & 7 put rows r and r + 8 on
// the same banks: 3.0e8 conflict cycles per 1M launch, 3.88 -> 3.71 ms).
__device__ __forceinline__ int fe_swz(int row) { return (row >> 1) & 7; }

// MFMA operand fragment (32 rows x 16 of the contraction at sub-step s).
__device__ __forceinline__ bf16x8 fe_frag(const __bf16* t, int row, int s, int h) {
  const int c = 2 * s + h;
  return *reinterpret_cast<const bf16x8*>(&t[row * FK + 8 * (c ^ fe_swz(row))]);
}

}  // namespace

// 128 KiB of LDS: one work-group of eight waves per CU, two per SIMD.
template <int DI, int R>
__global__ __launch_bounds__(128 * NWR) void index_frontend_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ Wq, const __bf16* __restrict__ Wk,
    const float* __restrict__ gq, const float* __restrict__ gk, __bf16* __restrict__ oq,
    __bf16* __restrict__ ok, int64_t N, int64_t pos0, int d_model, int ncols, int n_rt,
    double log2_theta, float eps) {
  static_assert(DI == 32 || DI == 64 || DI == 128, "d_idx");
  static_assert(R == 0 || R == 32 || (R == 64 && DI >= 64), "rope_dim");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FeSmem& sm = *reinterpret_cast<FeSmem*>(smem_raw);
  // work-group b runs on XCD b % 8; (b, b + 8) are the q and k halves of one
  // row tile
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const bool isk = slot & 1;
  const int rt = (slot >> 1) * 8 + xcd;
  if (rt >= n_rt) return;
  const __bf16* W = isk ? Wk : Wq;
  const float* gamma = isk ? gk : gq;
  __bf16* out = isk ? ok : oq;
  const int64_t row0 = (int64_t)rt * FM;
  const int col0 = blockIdx.y * FN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, h = lane >> 5, n = lane & 31;
  const int wr = wave % NWR, wc = wave / NWR;

  // Each wave instruction fills 1 KiB = 8 rows of 64; lane i writes chunk
  // position i % 8 of row i / 8, so it fetches the chunk that lands there.
  auto dma = [&](int kk, int buf) {
#pragma unroll
    for (int q = 0; q < FM / 8 / (2 * NWR); ++q) {
      const int v = wave * (FM / 8 / (2 * NWR)) + q;
      const int rr = 8 * v + (lane >> 3), p = lane & 7;
      const int64_t grow = min(row0 + rr, N - 1);
      const __bf16* src = X + grow * d_model + (int64_t)kk * FK + 8 * (p ^ fe_swz(rr));
      __builtin_amdgcn_global_load_lds(src, &sm.a[buf][v * 512], 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < FN / 8 / (2 * NWR); ++q) {
      const int v = wave * (FN / 8 / (2 * NWR)) + q;
      const int rr = 8 * v + (lane >> 3), p = lane & 7;
      const int64_t gcol = min(col0 + rr, ncols - 1);
      const __bf16* src = W + gcol * d_model + (int64_t)kk * FK + 8 * (p ^ fe_swz(rr));
      __builtin_amdgcn_global_load_lds(src, &sm.b[buf][v * 512], 16, 0, 0);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x16{};
  const int nk = d_model / FK;
  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const int buf = kk & 1;
    if (kk + 1 < nk) dma(kk + 1, buf ^ 1);
#pragma unroll
    for (int s = 0; s < FK / 16; ++s) {
      bf16x8 af[2], bf[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) af[rb] = fe_frag(sm.a[buf], wr * 64 + rb * 32 + n, s, h);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) bf[cb] = fe_frag(sm.b[buf], wc * 128 + cb * 32 + n, s, h);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma32(af[rb], bf[cb], acc[rb][cb]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of slab kk+1 is in LDS
    __syncthreads();
  }

  // Epilogue.  acc[rb][cb][j] is row wr*64 + rb*32 + acc_row(j, h), column
  // wc*128 + cb*32 + n; a group's DI columns are CPG whole 32-column blocks
  // of this wave (the tile's column offsets are multiples of DI).
  constexpr int CPG = DI / 32;
  float gm[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) gm[cb] = gamma[(cb * 32 + n) % DI];
  // rotation frequency of this lane's pair index
  // (in turns: theta^(-2j/R) / (2 pi), j = this lane's pair index)
  constexpr int HALF = R > 0 ? R / 2 : 1;
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  const double turns_per_pos =
      R > 0 ? exp2(-(2.0 * (double)(n % HALF) / (double)(2 * HALF)) * log2_theta) * kInvTwoPi
            : 0.0;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t row = row0 + wr * 64 + rb * 32 + acc_row(j, h);
      float cs = 1.f, sn = 0.f;
      if constexpr (R > 0) {
        // the angle in turns, reduced to [0, 1) in fp64; v_sin/v_cos take turns
        const double ang = (double)(pos0 + row) * turns_per_pos;
        const float fr = (float)(ang - floor(ang));
        sn = __builtin_amdgcn_sinf(fr);
        cs = __builtin_amdgcn_cosf(fr);
      }
      // the wave's groups, with compile-time block indices
      auto group = [&](auto g0c) {
        constexpr int g0 = decltype(g0c)::value;
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < CPG; ++u) ss = fmaf(acc[rb][g0 + u][j], acc[rb][g0 + u][j], ss);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o, kWave);
        const float rn = 1.f / sqrtf(ss * (1.f / DI) + eps);
        float y[CPG];
#pragma unroll
        for (int u = 0; u < CPG; ++u) y[u] = acc[rb][g0 + u][j] * rn * gm[g0 + u];
        if constexpr (R == 64) {
          // pair (column n of block g0, column n of block g0 + 1)
          const float a = y[0], bq = y[1];
          y[0] = a * cs - bq * sn;
          y[1] = bq * cs + a * sn;
        } else if constexpr (R == 32) {
          // pair (n, n + 16) inside block g0
          const float o = __shfl_xor(y[0], 16, kWave);
          y[0] = n < 16 ? y[0] * cs - o * sn : y[0] * cs + o * sn;
        }
        if (row < N) {
#pragma unroll
          for (int u = 0; u < CPG; ++u) {
            const int col = col0 + wc * 128 + (g0 + u) * 32 + n;
            if (col < ncols) out[row * ncols + col] = f2bf(y[u]);
          }
        }
      };
      group(std::integral_constant<int, 0>{});
      if constexpr (CPG <= 2) group(std::integral_constant<int, CPG>{});
      if constexpr (CPG == 1) {
        group(std::integral_constant<int, 2>{});
        group(std::integral_constant<int, 3>{});
      }
    }
}

// ---------------------------------------------------------------------------
static bool fe_ready = false;

template <int DI, int R>
static hipError_t fe_allow() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&index_frontend_kernel<DI, R>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(FeSmem));
}

static hipError_t fe_prepare() {
  if (fe_ready) return hipSuccess;
  hipError_t e = fe_allow<32, 0>();
  if (e == hipSuccess) e = fe_allow<32, 32>();
  if (e == hipSuccess) e = fe_allow<64, 0>();
  if (e == hipSuccess) e = fe_allow<64, 32>();
  if (e == hipSuccess) e = fe_allow<64, 64>();
  if (e == hipSuccess) e = fe_allow<128, 0>();
  if (e == hipSuccess) e = fe_allow<128, 32>();
  if (e == hipSuccess) e = fe_allow<128, 64>();
  if (e == hipSuccess) fe_ready = true;
  return e;
}

hipError_t launch_index_frontend(const void* hidden, const void* Wq, const void* Wk,
                                 const float* gq, const float* gk, int64_t N, int64_t pos0,
                                 int d_model, int H_kv, int d_idx, int rope_dim,
                                 double log2_theta, float eps, void* q_idx, void* k_idx,
                                 hipStream_t stream) {
  hipError_t e = fe_prepare();
  if (e != hipSuccess) return e;
  const int ncols = H_kv * d_idx;
  const int n_rt = (int)ceil_div(N, (int64_t)FM);
  // 16 work-groups per 8 row tiles (q and k of each), padded to whole groups
  dim3 grid((unsigned)(ceil_div((int64_t)n_rt, (int64_t)8) * 16), (unsigned)ceil_div(ncols, FN));
  auto* x = static_cast<const __bf16*>(hidden);
  auto* wq = static_cast<const __bf16*>(Wq);
  auto* wk = static_cast<const __bf16*>(Wk);
  auto* oq = static_cast<__bf16*>(q_idx);
  auto* ok = static_cast<__bf16*>(k_idx);
  const size_t lds = sizeof(FeSmem);
#define MSA_FE(DI, R)                                                                      \
  index_frontend_kernel<DI, R><<<grid, 128 * NWR, lds, stream>>>(x, wq, wk, gq, gk, oq, ok, N,  \
                                                           pos0, d_model, ncols, n_rt,    \
                                                           log2_theta, eps)
  if (d_idx == 32 && rope_dim == 0) MSA_FE(32, 0);
  else if (d_idx == 32 && rope_dim == 32) MSA_FE(32, 32);
  else if (d_idx == 64 && rope_dim == 0) MSA_FE(64, 0);
  else if (d_idx == 64 && rope_dim == 32) MSA_FE(64, 32);
  else if (d_idx == 64 && rope_dim == 64) MSA_FE(64, 64);
  else if (d_idx == 128 && rope_dim == 0) MSA_FE(128, 0);
  else if (d_idx == 128 && rope_dim == 32) MSA_FE(128, 32);
  else if (d_idx == 128 && rope_dim == 64) MSA_FE(128, 64);
  else return hipErrorInvalidValue;
#undef MSA_FE
  return hipGetLastError();
}

}  // namespace msa
