// Inverted index: selection table (query -> blocks) turned into a CSR over
// (group, block) buckets (block -> queries), as KV-outer execution needs
// ("MiniMax Sparse Attention" explainer, section 05 part 2: each KV block
// gathers the queries that selected it).
//
// Deterministic, no ordering atomics: the query range is cut into tiles of
// kTile positions; (1) per tile and group an LDS histogram over blocks,
// (2) for every bucket an exclusive scan over tiles plus the bucket totals,
// (3) an exclusive scan of the totals -> row_ptr, (4) per tile and group a
// scatter that walks the tile's queries in ascending order with an LDS
// cursor per block.  Inside a bucket positions therefore come out ascending.
#include "common.h"
#include "msa_internal.h"

namespace msa {

constexpr int kTile = 256;

// (1) hist[tile][r][b] = number of queries of the tile whose group-r row
//     selects block b.
__global__ __launch_bounds__(256) void csr_hist_kernel(const int32_t* __restrict__ sel,
                                                       int64_t Nq, int H_kv, int k, int nblk,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int tile = blockIdx.x, r = blockIdx.y;
  for (int b = threadIdx.x; b < nblk; b += 256) cnt[b] = 0;
  __syncthreads();
  const int64_t iq0 = (int64_t)tile * kTile;
  for (int e = threadIdx.x; e < kTile * k; e += 256) {
    const int64_t iq = iq0 + e / k;
    if (iq < Nq) {
      const int32_t b = sel[(iq * H_kv + r) * k + e % k];
      if (b >= 0) atomicAdd(&cnt[b], 1);
    }
  }
  __syncthreads();
  int32_t* dst = hist + ((int64_t)tile * H_kv + r) * nblk;
  for (int b = threadIdx.x; b < nblk; b += 256) dst[b] = cnt[b];
}

// (2) per bucket: exclusive prefix over tiles (in place) and the total.
__global__ __launch_bounds__(256) void csr_tile_scan_kernel(int32_t* __restrict__ hist,
                                                            int ntiles, int64_t nb,
                                                            int32_t* __restrict__ total) {
  const int64_t bucket = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (bucket >= nb) return;
  int32_t run = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int32_t v = hist[(int64_t)t * nb + bucket];
    hist[(int64_t)t * nb + bucket] = run;
    run += v;
  }
  total[bucket] = run;
}

// (3) single work-group exclusive scan: out[x] = sum_{y<x} in[y], out[n] = total.
__global__ __launch_bounds__(1024) void exclusive_scan_kernel(const int32_t* __restrict__ in,
                                                              int64_t n,
                                                              int32_t* __restrict__ out) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(n, 1024);
  const int64_t lo = min(n, per * t), hi = min(n, per * (t + 1));
  int32_t s = 0;
  for (int64_t x = lo; x < hi; ++x) s += in[x];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = t ? part[t - 1] : 0;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t v = in[x];
    out[x] = run;
    run += v;
  }
  if (t == 1023) out[n] = part[1023];
}

// (4) scatter: one wavefront per (tile, group).  Lane s handles slot s of
//     the current query; the k blocks of one query are distinct, so the
//     lanes never touch the same cursor, and queries are walked in order.
__global__ __launch_bounds__(64) void csr_scatter_kernel(const int32_t* __restrict__ sel,
                                                         int64_t q_start, int64_t Nq, int H_kv,
                                                         int k, int nblk,
                                                         const int32_t* __restrict__ hist,
                                                         const int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col,
                                                         uint8_t* __restrict__ slot) {
  extern __shared__ int32_t cur[];
  const int tile = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int32_t* hb = hist + ((int64_t)tile * H_kv + r) * nblk;
  const int32_t* rp = row_ptr + (int64_t)r * nblk;
  for (int b = lane; b < nblk; b += 64) cur[b] = hb[b] + rp[b];
  __syncthreads();
  const int64_t iq0 = (int64_t)tile * kTile;
  const int64_t iq1 = min(Nq, iq0 + kTile);
  for (int64_t iq = iq0; iq < iq1; ++iq) {
    if (lane < k) {
      const int32_t b = sel[(iq * H_kv + r) * k + lane];
      if (b >= 0) {
        const int32_t pos = cur[b];
        cur[b] = pos + 1;
        col[pos] = (int32_t)(q_start + iq);
        slot[pos] = (uint8_t)lane;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

size_t invert_scratch_bytes(int64_t Nq, int H_kv, int nblk) {
  const int64_t ntiles = ceil_div(Nq, kTile);
  const int64_t nb = (int64_t)H_kv * nblk;
  return sizeof(int32_t) * (size_t)(ntiles * nb + nb);
}

hipError_t launch_invert(const int32_t* sel, int64_t q_start, int64_t Nq, int H_kv, int k,
                         int nblk, int32_t* row_ptr, int32_t* col, uint8_t* slot,
                         void* scratch, hipStream_t stream) {
  const int ntiles = (int)ceil_div(Nq, kTile);
  const int64_t nb = (int64_t)H_kv * nblk;
  int32_t* hist = static_cast<int32_t*>(scratch);
  int32_t* total = hist + (int64_t)ntiles * nb;
  const size_t lds = sizeof(int32_t) * (size_t)nblk;
  csr_hist_kernel<<<dim3(ntiles, H_kv), 256, lds, stream>>>(sel, Nq, H_kv, k, nblk, hist);
  csr_tile_scan_kernel<<<(unsigned)ceil_div(nb, 256), 256, 0, stream>>>(hist, ntiles, nb, total);
  exclusive_scan_kernel<<<1, 1024, 0, stream>>>(total, nb, row_ptr);
  csr_scatter_kernel<<<dim3(ntiles, H_kv), 64, lds, stream>>>(sel, q_start, Nq, H_kv, k, nblk,
                                                               hist, row_ptr, col, slot);
  return hipGetLastError();
}

}  // namespace msa
